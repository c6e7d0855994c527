// BN254 base field Fp (the curve's coordinates) for gfx950: 256-bit Montgomery
// arithmetic on 8 x 32-bit limbs, R = 2^256.
//
// The MSM_CU page takes its curve field from a header the page does not show; this one
// is written from the mathematics, with the same algorithm as the scalar field (fr.hpp):
// Montgomery multiplication in the coarsely integrated operand scanning order (Koc,
// Acar, Kaliski, IEEE Micro 1996), each limb product one v_mad_u64_u32 and one
// add-with-carry, every function returning the canonical representative in [0, p).
// p < 2^254, so a + b < 2^255 never carries out of limb 7 and the CIOS running value
// stays below 2p + p 2^32 < 2^287 (limb 8 absorbs the overflow).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fr.hpp"  // G16_HD, addc, subb, neg_inv32

namespace g16 {

struct Fp {
    uint32_t w[8];
};

// p = 0x30644e72e131a029b85045b68181585d97816a916871ca8d3c208c16d87cfd47
G16_HD constexpr uint32_t p_limb(int i) {
    return i == 0 ? 0xd87cfd47u : i == 1 ? 0x3c208c16u : i == 2 ? 0x6871ca8du
         : i == 3 ? 0x97816a91u : i == 4 ? 0x8181585du : i == 5 ? 0xb85045b6u
         : i == 6 ? 0xe131a029u : 0x30644e72u;
}
constexpr uint32_t kPNPrime = neg_inv32(0xd87cfd47u);
static_assert(uint32_t(0xd87cfd47u * kPNPrime) == 0xffffffffu, "kPNPrime is -p^-1 mod 2^32");

// R mod p (Montgomery one) and R^2 mod p.
G16_HD constexpr uint32_t p_one_limb(int i) {
    return i == 0 ? 0xc58f0d9du : i == 1 ? 0xd35d438du : i == 2 ? 0xf5c70b3du
         : i == 3 ? 0x0a78eb28u : i == 4 ? 0x7879462cu : i == 5 ? 0x666ea36fu
         : i == 6 ? 0x9a07df2fu : 0x0e0a77c1u;
}
G16_HD constexpr uint32_t p_r2_limb(int i) {
    return i == 0 ? 0x538afa89u : i == 1 ? 0xf32cfc5bu : i == 2 ? 0xd44501fbu
         : i == 3 ? 0xb5e71911u : i == 4 ? 0x0a417ff6u : i == 5 ? 0x47ab1effu
         : i == 6 ? 0xcab8351fu : 0x06d89f71u;
}

G16_HD Fp fp_zero() {
    Fp z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z.w[i] = 0u;
    return z;
}

G16_HD Fp fp_one() {
    Fp z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z.w[i] = p_one_limb(i);
    return z;
}

G16_HD bool fp_is_zero(const Fp& a) {
    uint32_t d = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d |= a.w[i];
    return d == 0u;
}

G16_HD bool fp_eq(const Fp& a, const Fp& b) {
    uint32_t d = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d |= a.w[i] ^ b.w[i];
    return d == 0u;
}

// t in [0, 2p) -> t mod p
G16_HD Fp fp_reduce_once(const Fp& t) {
    Fp d;
    uint32_t borrow = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d.w[i] = subb(t.w[i], p_limb(i), borrow);
    Fp out;
#pragma unroll
    for (int i = 0; i < 8; ++i) out.w[i] = borrow ? t.w[i] : d.w[i];
    return out;
}

G16_HD Fp fp_add(const Fp& a, const Fp& b) {
    Fp s;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.w[i] = addc(a.w[i], b.w[i], c);
    return fp_reduce_once(s);
}

G16_HD Fp fp_sub(const Fp& a, const Fp& b) {
    Fp d, e;
    uint32_t borrow = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d.w[i] = subb(a.w[i], b.w[i], borrow);
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) e.w[i] = addc(d.w[i], p_limb(i), c);
    Fp out;
#pragma unroll
    for (int i = 0; i < 8; ++i) out.w[i] = borrow ? e.w[i] : d.w[i];
    return out;
}

G16_HD Fp fp_neg(const Fp& a) { return fp_sub(fp_zero(), a); }
G16_HD Fp fp_dbl(const Fp& a) { return fp_add(a, a); }

// Montgomery product a b 2^-256 mod p (CIOS), canonical in and out.
G16_HD Fp fp_mul(const Fp& a, const Fp& b) {
    uint32_t t[9];
#pragma unroll
    for (int j = 0; j < 9; ++j) t[j] = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint64_t pr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pr[j] = (uint64_t)a.w[j] * b.w[i] + t[j];
        uint32_t c = 0;
        t[0] = (uint32_t)pr[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) t[j] = addc((uint32_t)pr[j], (uint32_t)(pr[j - 1] >> 32), c);
        t[8] = t[8] + (uint32_t)(pr[7] >> 32) + c;
        const uint32_t m = t[0] * kPNPrime;
        uint64_t q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = (uint64_t)m * p_limb(j) + t[j];
        c = 0;
#pragma unroll
        for (int j = 1; j < 8; ++j) t[j - 1] = addc((uint32_t)q[j], (uint32_t)(q[j - 1] >> 32), c);
        t[7] = t[8] + (uint32_t)(q[7] >> 32) + c;
        t[8] = 0u;
    }
    Fp out;
#pragma unroll
    for (int j = 0; j < 8; ++j) out.w[j] = t[j];
    return fp_reduce_once(out);
}

G16_HD Fp fp_sqr(const Fp& a) { return fp_mul(a, a); }

G16_HD Fp fp_to_mont(const Fp& x) {
    Fp r2;
#pragma unroll
    for (int i = 0; i < 8; ++i) r2.w[i] = p_r2_limb(i);
    return fp_mul(x, r2);
}

G16_HD Fp fp_from_mont(const Fp& a) {
    Fp one = fp_zero();
    one.w[0] = 1u;
    return fp_mul(a, one);
}

// a^(p-2) = a^-1 (Fermat; 0 -> 0), Montgomery in and out.
G16_HD Fp fp_inv(const Fp& a) {
    Fp acc = fp_one();
    for (int bit = 255; bit >= 0; --bit) {
        acc = fp_sqr(acc);
        uint32_t e = p_limb(bit >> 5);
        if ((bit >> 5) == 0) e -= 2u;  // low limb of p - 2 (p's low limb is odd and large)
        if ((e >> (bit & 31)) & 1u) acc = fp_mul(acc, a);
    }
    return acc;
}

}  // namespace g16
