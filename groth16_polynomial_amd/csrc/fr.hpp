// BN254 scalar field Fr for gfx950: 256-bit Montgomery arithmetic on 8 x 32-bit limbs.
//
// The pages do not show their field layer (the NTT_CU and POINTWISE_CU pages call
// fr_mul, fr_add, fr_sub and fr_from_mont from a header that is not on the page), so
// this one is written from the mathematics:
//   * Montgomery multiplication, R = 2^256 (P. L. Montgomery, "Modular multiplication
//     without trial division", Math. Comp. 1985), in the coarsely integrated operand
//     scanning order (Koc, Acar, Kaliski, "Analyzing and comparing Montgomery
//     multiplication algorithms", IEEE Micro 1996);
//   * each row of limb products is formed as 64-bit values lo + hi * 2^32 by one
//     multiply-add each (a[j] * b + t[j] never overflows 64 bits), and the high words
//     are folded into the next limb by one add-with-carry chain, so a limb product
//     costs one v_mad_u64_u32 and one v_addc_co_u32;
//   * every function returns the canonical representative in [0, r): the pages'
//     backends agree bit for bit, which requires canonical stored values.
//
// Elements are 32-byte little-endian integers (limb 0 least significant), the layout
// of a 4 x 64-bit Montgomery-form element read as 8 x 32-bit words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define G16_HD __host__ __device__ __forceinline__

namespace g16 {

struct Fr {
    uint32_t w[8];
};

// r = 0x30644e72e131a029b85045b68181585d2833e84879b9709143e1f593f0000001
G16_HD constexpr uint32_t r_limb(int i) {
    return i == 0 ? 0xf0000001u : i == 1 ? 0x43e1f593u : i == 2 ? 0x79b97091u
         : i == 3 ? 0x2833e848u : i == 4 ? 0x8181585du : i == 5 ? 0xb85045b6u
         : i == 6 ? 0xe131a029u : 0x30644e72u;
}

// -r^-1 mod 2^32 by Newton iteration on the low limb (x <- x (2 - r0 x) doubles the
// number of correct low bits; r0 is odd, and x = r0 is correct to 3 bits).
G16_HD constexpr uint32_t neg_inv32(uint32_t r0) {
    uint32_t x = r0;
    for (int i = 0; i < 5; ++i) x = x * (2u - r0 * x);
    return 0u - x;
}
constexpr uint32_t kNPrime = neg_inv32(0xf0000001u);
static_assert(uint32_t(0xf0000001u * kNPrime) == 0xffffffffu, "kNPrime is -r^-1 mod 2^32");

// R mod r (Montgomery one) and R^2 mod r, little-endian 32-bit limbs.
G16_HD constexpr uint32_t one_limb(int i) {
    return i == 0 ? 0x4ffffffbu : i == 1 ? 0xac96341cu : i == 2 ? 0x9f60cd29u
         : i == 3 ? 0x36fc7695u : i == 4 ? 0x7879462eu : i == 5 ? 0x666ea36fu
         : i == 6 ? 0x9a07df2fu : 0x0e0a77c1u;
}
G16_HD constexpr uint32_t r2_limb(int i) {
    return i == 0 ? 0xae216da7u : i == 1 ? 0x1bb8e645u : i == 2 ? 0xe35c59e3u
         : i == 3 ? 0x53fe3ab1u : i == 4 ? 0x53bb8085u : i == 5 ? 0x8c49833du
         : i == 6 ? 0x7f4e44a5u : 0x0216d0b1u;
}

G16_HD Fr fr_zero() {
    Fr z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z.w[i] = 0u;
    return z;
}

G16_HD Fr fr_mont_one() {
    Fr z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z.w[i] = one_limb(i);
    return z;
}

G16_HD Fr fr_r2() {
    Fr z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z.w[i] = r2_limb(i);
    return z;
}

G16_HD bool fr_is_equal(const Fr& a, const Fr& b) {
    uint32_t d = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d |= a.w[i] ^ b.w[i];
    return d == 0u;
}

// x + y + carry -> (sum, carry out); lowers to v_add_co_u32 / v_addc_co_u32.
G16_HD uint32_t addc(uint32_t x, uint32_t y, uint32_t& carry) {
    uint32_t co;
    uint32_t s = __builtin_addc(x, y, carry, &co);
    carry = co;
    return s;
}

// x - y - borrow -> (difference, borrow out in {0, 1}).
G16_HD uint32_t subb(uint32_t x, uint32_t y, uint32_t& borrow) {
    uint32_t bo;
    uint32_t d = __builtin_subc(x, y, borrow, &bo);
    borrow = bo;
    return d;
}

// t in [0, 2r) -> t mod r.
G16_HD Fr fr_reduce_once(const Fr& t) {
    Fr d;
    uint32_t borrow = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d.w[i] = subb(t.w[i], r_limb(i), borrow);
    Fr out;
#pragma unroll
    for (int i = 0; i < 8; ++i) out.w[i] = borrow ? t.w[i] : d.w[i];
    return out;
}

// (a + b) mod r for canonical a, b.  a + b < 2r < 2^255, so no carry leaves limb 7.
G16_HD Fr fr_add(const Fr& a, const Fr& b) {
    Fr s;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.w[i] = addc(a.w[i], b.w[i], c);
    return fr_reduce_once(s);
}

// (a - b) mod r for canonical a, b.
G16_HD Fr fr_sub(const Fr& a, const Fr& b) {
    Fr d, e;
    uint32_t borrow = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d.w[i] = subb(a.w[i], b.w[i], borrow);
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) e.w[i] = addc(d.w[i], r_limb(i), c);
    Fr out;
#pragma unroll
    for (int i = 0; i < 8; ++i) out.w[i] = borrow ? e.w[i] : d.w[i];
    return out;
}

// Montgomery product a * b * 2^-256 mod r for canonical a, b (CIOS).
//
// Invariant: at the top of iteration i the running value t (limbs t0..t8) is < 2r.
// Adding a * b_i keeps it below 2r + r 2^32 < 2^287, so limb 8 absorbs the overflow;
// adding m r (m chosen so the low limb cancels) and dropping that limb divides by
// 2^32 and returns t below 2r, so limb 8 is zero again after the shift.
G16_HD Fr fr_mul(const Fr& a, const Fr& b) {
    uint32_t t[9];
#pragma unroll
    for (int j = 0; j < 9; ++j) t[j] = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // t += a * b_i
        uint64_t p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = (uint64_t)a.w[j] * b.w[i] + t[j];
        uint32_t c = 0;
        t[0] = (uint32_t)p[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) t[j] = addc((uint32_t)p[j], (uint32_t)(p[j - 1] >> 32), c);
        t[8] = t[8] + (uint32_t)(p[7] >> 32) + c;
        // t = (t + m r) / 2^32 with m = t0 * (-r^-1) mod 2^32
        uint32_t m = t[0] * kNPrime;
        uint64_t q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = (uint64_t)m * r_limb(j) + t[j];
        c = 0;
#pragma unroll
        for (int j = 1; j < 8; ++j) t[j - 1] = addc((uint32_t)q[j], (uint32_t)(q[j - 1] >> 32), c);
        t[7] = t[8] + (uint32_t)(q[7] >> 32) + c;
        t[8] = 0u;
    }
    Fr out;
#pragma unroll
    for (int j = 0; j < 8; ++j) out.w[j] = t[j];
    return fr_reduce_once(out);
}

// Montgomery reduction a * 2^-256 mod r: Montgomery form -> standard form.  For a < r
// the result is already below r (the sum a + m r stays below r 2^256 + r).
G16_HD Fr fr_from_mont(const Fr& a) {
    uint32_t t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = a.w[j];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t m = t[0] * kNPrime;
        uint64_t q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) q[j] = (uint64_t)m * r_limb(j) + t[j];
        uint32_t c = 0;
#pragma unroll
        for (int j = 1; j < 8; ++j) t[j - 1] = addc((uint32_t)q[j], (uint32_t)(q[j - 1] >> 32), c);
        t[7] = (uint32_t)(q[7] >> 32) + c;
    }
    Fr out;
#pragma unroll
    for (int j = 0; j < 8; ++j) out.w[j] = t[j];
    return fr_reduce_once(out);
}

// 29-bit digit mask and 2^261 mod r (standard form), used by the digit layer (fr29.hpp)
// to build table entries.
constexpr uint32_t kM29 = (1u << 29) - 1u;

G16_HD constexpr uint32_t c261_limb(int i) {
    return i == 0 ? 0x8fffff57u : i == 1 ? 0x2fd4e156u : i == 2 ? 0xa494b01au
         : i == 3 ? 0x75bba827u : i == 4 ? 0x819caa80u : i == 5 ? 0x5301fa84u
         : i == 6 ? 0x563d4475u : 0x0dc83629u;
}

G16_HD Fr fr_c261() {
    Fr z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z.w[i] = c261_limb(i);
    return z;
}

// Standard form -> Montgomery form: x * R^2 * R^-1 = x R mod r.
G16_HD Fr fr_to_mont(const Fr& x) { return fr_mul(x, fr_r2()); }

// a^e for a 64-bit exponent (square and multiply, Montgomery domain).
G16_HD Fr fr_pow_u64(const Fr& a, uint64_t e) {
    Fr acc = fr_mont_one();
    Fr base = a;
    while (e) {
        if (e & 1u) acc = fr_mul(acc, base);
        base = fr_mul(base, base);
        e >>= 1;
    }
    return acc;
}

// a^e for a 256-bit exponent given as 8 little-endian limbs.
G16_HD Fr fr_pow(const Fr& a, const uint32_t e[8]) {
    Fr acc = fr_mont_one();
    for (int bit = 255; bit >= 0; --bit) {
        acc = fr_mul(acc, acc);
        if ((e[bit >> 5] >> (bit & 31)) & 1u) acc = fr_mul(acc, a);
    }
    return acc;
}

// a^-1 = a^(r-2) (Fermat); a must be nonzero.
G16_HD Fr fr_inv(const Fr& a) {
    uint32_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = r_limb(i);
    e[0] -= 2u;  // r0 = 0xf0000001, no borrow
    return fr_pow(a, e);
}

}  // namespace g16
