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

// ---------------------------------------------------------------- products by a table
//
// Twiddles and coset factors are fixed tables, so their products use a second
// Montgomery radix, R' = 2^261, on nine 29-bit limbs: every limb product is below 2^58
// and a column of the product holds at most nine a*b and nine m*r terms plus the carry
// from the column below, less than 2^63, so each column accumulates in one 64-bit
// register pair with v_mad_u64_u32 and no carry chain (finely integrated product
// scanning, Koc-Acar-Kaliski 1996).  A table entry is stored as w * 2^261 mod r, and
// then x (in the 2^256 Montgomery form) times it gives x w 2^256 * 2^261 / 2^261, i.e.
// x w still in the 2^256 form.

constexpr uint32_t kM29 = (1u << 29) - 1u;

struct F29 {
    uint32_t l[9];  // little-endian 29-bit limbs (limb 8 holds bits 232..255)
};

// r in nine 29-bit limbs
G16_HD constexpr uint32_t r29_limb(int k) {
    return k == 0 ? 0x10000001u : k == 1 ? 0x1f0fac9fu : k == 2 ? 0x0e5c2450u
         : k == 3 ? 0x07d090f3u : k == 4 ? 0x1585d283u : k == 5 ? 0x02db40c0u
         : k == 6 ? 0x00a6e141u : k == 7 ? 0x0e5c2634u : 0x0030644eu;
}
// -r^-1 mod 2^29
constexpr uint32_t kNPrime29 = kNPrime & kM29;
static_assert(uint32_t(0x10000001u * kNPrime29) % (1u << 29) == kM29, "kNPrime29");

// 2^261 mod r (standard form): multiplying a 2^256-form value by it gives the 2^261 form.
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

G16_HD F29 unpack29(const Fr& x) {
    F29 r;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int bit = 29 * k, w = bit >> 5, s = bit & 31;
        uint32_t v = x.w[w] >> s;
        if (s > 3 && w + 1 < 8) v |= x.w[w + 1] << (32 - s);
        r.l[k] = (k < 8) ? (v & kM29) : v;
    }
    return r;
}

// Limbs below 2^29 (limb 8 below 2^24) back to eight 32-bit words.
G16_HD Fr pack29(const F29& u) {
    Fr x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int bit = 32 * j;
        const int k = bit / 29, off = bit - 29 * k;
        uint32_t v = u.l[k] >> off;
        if (k + 1 < 9) v |= u.l[k + 1] << (29 - off);
        if (k + 2 < 9 && 58 - off < 32) v |= u.l[k + 2] << (58 - off);
        x.w[j] = v;
    }
    return x;
}

// a * b * 2^-261 mod r for any 256-bit a and canonical b (b already unpacked), NOT
// reduced: the Montgomery sum a b + m r is below 2^256 r + 2^261 r, so the result is
// below (1 + 2^-5) r < 2r.
G16_HD Fr fr_mul29_lazy(const Fr& ap, const F29& b) {
    const F29 a = unpack29(ap);
    uint32_t m[9];
    F29 u;
    uint64_t acc = 0;
#pragma unroll
    for (int i = 0; i < 9; ++i) {
#pragma unroll
        for (int j = 0; j < i; ++j) {
            acc += (uint64_t)a.l[j] * b.l[i - j];
            acc += (uint64_t)m[j] * r29_limb(i - j);
        }
        acc += (uint64_t)a.l[i] * b.l[0];
        m[i] = ((uint32_t)acc * kNPrime29) & kM29;
        acc += (uint64_t)m[i] * r29_limb(0);  // the low 29 bits become zero
        acc >>= 29;
    }
#pragma unroll
    for (int i = 9; i < 17; ++i) {
#pragma unroll
        for (int j = i - 8; j < 9; ++j) {
            acc += (uint64_t)a.l[j] * b.l[i - j];
            acc += (uint64_t)m[j] * r29_limb(i - j);
        }
        u.l[i - 9] = (uint32_t)acc & kM29;
        acc >>= 29;
    }
    u.l[8] = (uint32_t)acc;
    return pack29(u);
}

// The same product reduced to [0, r).
G16_HD Fr fr_mul29(const Fr& ap, const F29& b) { return fr_reduce_once(fr_mul29_lazy(ap, b)); }

// ---------------------------------------------------------------- lazy ranges
//
// Inside a transform kernel values may sit in [0, 2r) or [0, 4r) between passes (4r is
// below 2^256 because r < 2^254); every value a kernel stores to HBM is canonical.

G16_HD constexpr uint32_t r2_times_limb(int i) {  // 2r, little-endian 32-bit limbs
    return i == 0 ? 0xe0000002u : i == 1 ? 0x87c3eb27u : i == 2 ? 0xf372e122u
         : i == 3 ? 0x5067d090u : i == 4 ? 0x0302b0bau : i == 5 ? 0x70a08b6du
         : i == 6 ? 0xc2634053u : 0x60c89ce5u;
}

// x in [0, 4r) -> [0, 2r)
G16_HD Fr fr_reduce_2r(const Fr& x) {
    Fr d;
    uint32_t borrow = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) d.w[i] = subb(x.w[i], r2_times_limb(i), borrow);
    Fr out;
#pragma unroll
    for (int i = 0; i < 8; ++i) out.w[i] = borrow ? x.w[i] : d.w[i];
    return out;
}

// x in [0, 4r) -> canonical
G16_HD Fr fr_canon_4r(const Fr& x) { return fr_reduce_once(fr_reduce_2r(x)); }

// a + b for a + b < 2^256 (no reduction)
G16_HD Fr fr_add_lazy(const Fr& a, const Fr& b) {
    Fr s;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.w[i] = addc(a.w[i], b.w[i], c);
    return s;
}

// a + 2r - b for a < 2r, b <= 2r: in [0, 4r)
G16_HD Fr fr_sub_lazy(const Fr& a, const Fr& b) {
    Fr s;
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.w[i] = addc(a.w[i], r2_times_limb(i), c);
    uint32_t borrow = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.w[i] = subb(s.w[i], b.w[i], borrow);
    return s;
}

// x * w for a table entry w stored in the 2^261 form (see above): x w in x's form.
G16_HD Fr fr_mul_tab(const Fr& x, const Fr& w261) { return fr_mul29(x, unpack29(w261)); }

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
