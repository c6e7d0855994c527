// BabyBear, p = 2^31 - 2^27 + 1 (the WHIR forum post, section 2), for the Reed-Solomon
// encoding transform.  Elements are 32-bit words below p, held in Montgomery form with
// R = 2^32 (the post's section 3.4): x is stored as x 2^32 mod p.
//
// Every element fits one 32-bit register, so unlike BN254 there is no digit layer: a sum
// or difference is an add and a min (the wrapped value is the larger one), and a product
// by a fixed twiddle uses Shoup's precomputed quotient (w' = floor(w 2^32 / p)): one high
// and two low 32-bit multiplies and a correction.  With w a plain integer the product
// keeps x's Montgomery factor, so the transform never leaves the interface's form.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#ifndef G16_HD
#define G16_HD __host__ __device__ __forceinline__
#endif

namespace g16 {

constexpr uint32_t kBbP = 0x78000001u;  // 2^31 - 2^27 + 1
constexpr uint32_t kBbGen = 31u;        // the smallest generator of the multiplicative group
constexpr uint32_t kBbTwoAdicity = 27u;

// a + b and a - b for a, b < p.  a + b < 2p < 2^32, so the reduced value is the smaller of
// s and s - p (s - p wraps above s when s < p); likewise a - b + p.
G16_HD uint32_t bb_add(uint32_t a, uint32_t b) {
    const uint32_t s = a + b, t = s - kBbP;
    return s < t ? s : t;
}
G16_HD uint32_t bb_sub(uint32_t a, uint32_t b) {
    const uint32_t d = a - b, t = d + kBbP;
    return d < t ? d : t;
}

// x w mod p for x < 2^32 and a fixed w < p with w' = floor(w 2^32 / p): q = floor(x w' /
// 2^32) is floor(x w / p) or one less, so x w - q p lies in [0, 2p) and its low 32 bits
// are exact.
G16_HD uint32_t bb_shoup(uint32_t x, uint32_t w, uint32_t wp) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t q = __umulhi(x, wp);
#else
    const uint32_t q = (uint32_t)(((uint64_t)x * wp) >> 32);
#endif
    const uint32_t r = x * w - q * kBbP;
    const uint32_t t = r - kBbP;
    return r < t ? r : t;
}

G16_HD uint32_t bb_shoup_companion(uint32_t w) {
    return (uint32_t)(((uint64_t)w << 32) / kBbP);
}

// x wm 2^-32 mod p for x, wm < p (Montgomery's REDC with R = 2^32): with wm = w 2^32 mod p
// the product of x by w in the data's Montgomery form, from a 4-byte twiddle instead of
// Shoup's 8-byte pair (two more instructions).  m = lo (-p^-1) mod 2^32 makes lo + (m p)
// mod 2^32 zero, so (x wm + m p) / 2^32 = hi + mulhi(m, p) + (lo != 0), below
// p^2 / 2^32 + p < 2p.
constexpr uint32_t kBbPNeg = 0x77ffffffu;  // -p^-1 mod 2^32
static_assert((uint32_t)(kBbP * kBbPNeg) == 0xffffffffu, "kBbPNeg");
G16_HD uint32_t bb_mont_mul(uint32_t x, uint32_t wm) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t lo = x * wm, hi = __umulhi(x, wm);
    const uint32_t m = lo * kBbPNeg;
    const uint32_t u = hi + __umulhi(m, kBbP) + (lo != 0u ? 1u : 0u);
#else
    const uint64_t t = (uint64_t)x * wm;
    const uint32_t m = (uint32_t)t * kBbPNeg;
    const uint32_t u = (uint32_t)((t + (uint64_t)m * kBbP) >> 32);
#endif
    const uint32_t v = u - kBbP;
    return u < v ? u : v;
}

// Plain modular product and power (table building and host code).
G16_HD uint32_t bb_mul_plain(uint32_t a, uint32_t b) {
    return (uint32_t)(((uint64_t)a * b) % kBbP);
}
G16_HD uint32_t bb_pow_plain(uint32_t a, uint64_t e) {
    uint32_t r = 1u;
    while (e) {
        if (e & 1u) r = bb_mul_plain(r, a);
        a = bb_mul_plain(a, a);
        e >>= 1;
    }
    return r;
}

// A primitive 2^L-th root of unity (L <= 27): 31^((p - 1) / 2^L).
G16_HD uint32_t bb_root(uint32_t L) { return bb_pow_plain(kBbGen, (uint64_t)(kBbP - 1u) >> L); }

}  // namespace g16
