// BN254 base field Fp in nine 29-bit digits for the MSM's point arithmetic.
//
// Why: a product of two variables on 8 x 32-bit limbs (fp.hpp) needs a carry chain per
// limb product, about three issue slots each on gfx950 (plus wait states after the
// add-with-carry instructions).  With 29-bit digits a digit product is below 2^58 and a
// column of 18 products stays inside a signed 64-bit accumulator, so every product is
// one v_mad_i64_i32 and carries move once per column (the same reasoning as the
// transforms' digit layer, fr29.hpp).
//
// Value of an Fp29: sum of d[k] 2^(29k) with signed 32-bit digits, held in Montgomery
// form with R' = 2^261 (a canonical 2^256-form element x R converts by x R 2^5, a shift).
// "Normalized": digits 0..7 in [-4, 2^29 + 4), digit 8 small and signed.  Every function
// here returns normalized digits.  Values are lazy.  A converted input is below 32p (the
// shift by 2^5 is not reduced); a product of inputs below Ap and Bp in magnitude lies
// below (A B 2^-7.4 + 1) p (the 2^-7.4 is p / 2^261).  Through the MSM's formulas that
// keeps an accumulator's X below 20p, Y below 7p and ZZ, ZZZ below 6p after its first
// addition; the largest value ever formed is a difference such as U2 - X1 in the first
// mixed addition onto a converted point, below 40p, inside the 64p that fp29_canon
// allows.
//
// The product is Montgomery's REDC in radix 2^29 (P. L. Montgomery, Math. Comp. 1985),
// in the product-scanning order: column k takes carry + sum a_i b_(k-i) + sum m_i p_(k-i),
// for k < 9 the digit m_k = (column * -p^-1) mod 2^29 that clears the column, for k >= 9
// the result digit.  162 digit products; a square takes 126 (the cross products once,
// against a doubled digit), and a b - c d takes 243 with one reduction.  On the device
// each column is one chain of multiply-adds from the carry (fp29_cols.hpp): 212
// instructions a product against 228 for the compiler's own reassociated columns.
#pragma once

#include "fp.hpp"
#include "fr29.hpp"  // static_for, kM29

namespace g16 {

struct Fp29 {
    int32_t d[9];
};

// p in 29-bit digits, and 64 p (fp29_canon adds it to make a lazy value positive)
G16_HD constexpr int32_t p29_digit(int k) {
    return k == 0 ? 0x187cfd47 : k == 1 ? 0x010460b6 : k == 2 ? 0x1c72a34f
         : k == 3 ? 0x02d522d0 : k == 4 ? 0x1585d978 : k == 5 ? 0x02db40c0
         : k == 6 ? 0x00a6e141 : k == 7 ? 0x0e5c2634 : 0x0030644e;
}
G16_HD constexpr int32_t p64_29_digit(int k) {
    return k == 0 ? 0x1f3f51c0 : k == 1 ? 0x01182db0 : k == 2 ? 0x1ca8d3c2
         : k == 3 ? 0x1548b438 : k == 4 ? 0x01765e05 : k == 5 ? 0x16d0302b
         : k == 6 ? 0x09b85045 : k == 7 ? 0x17098d01 : 0x0c19139c;
}
// -p^-1 mod 2^29 (Montgomery digit) and -p^-1 mod 32 (the final division by 2^5)
constexpr uint32_t kP29NInv = 0x04866389u;
constexpr uint32_t kP5NInv = 9u;
static_assert(((uint64_t)0x187cfd47u * kP29NInv + 1u) % (1u << 29) == 0u, "kP29NInv");
static_assert((0xd87cfd47u * kP5NInv + 1u) % 32u == 0u, "kP5NInv");

G16_HD Fp29 fp29_zero() {
    Fp29 z;
#pragma unroll
    for (int k = 0; k < 9; ++k) z.d[k] = 0;
    return z;
}

G16_HD bool fp29_digits_zero(const Fp29& a) {
    int32_t o = 0;
#pragma unroll
    for (int k = 0; k < 9; ++k) o |= a.d[k];
    return o == 0;
}

// canonical x (2^256 Montgomery form, < p) -> x 2^5 in digits [0, 2^29)
G16_HD Fp29 fp29_from_fp(const Fp& x) {
    Fp29 r;
    r.d[0] = (int32_t)((x.w[0] << 5) & kM29);
#pragma unroll
    for (int k = 1; k < 9; ++k) {
        const int pos = 29 * k - 5, w = pos >> 5, s = pos & 31;
        uint32_t v = x.w[w] >> s;
        if (s > 3 && w + 1 < 8) v |= x.w[w + 1] << (32 - s);
        r.d[k] = (int32_t)(v & kM29);
    }
    return r;
}

// Carry-save normalization (as fr29_normalize): digit k keeps its low 29 bits plus the
// signed carry out of digit k - 1.
G16_HD Fp29 fp29_norm(const Fp29& a) {
    Fp29 o;
    o.d[0] = a.d[0] & (int32_t)kM29;
#pragma unroll
    for (int k = 1; k < 8; ++k) o.d[k] = (a.d[k] & (int32_t)kM29) + (a.d[k - 1] >> 29);
    o.d[8] = a.d[8] + (a.d[7] >> 29);
    return o;
}

G16_HD Fp29 fp29_add(const Fp29& a, const Fp29& b) {
    Fp29 s;
#pragma unroll
    for (int k = 0; k < 9; ++k) s.d[k] = a.d[k] + b.d[k];
    return fp29_norm(s);
}

G16_HD Fp29 fp29_sub(const Fp29& a, const Fp29& b) {
    Fp29 s;
#pragma unroll
    for (int k = 0; k < 9; ++k) s.d[k] = a.d[k] - b.d[k];
    return fp29_norm(s);
}

G16_HD Fp29 fp29_neg(const Fp29& a) { return fp29_sub(fp29_zero(), a); }
G16_HD Fp29 fp29_dbl(const Fp29& a) { return fp29_add(a, a); }

}  // namespace g16

#include "fp29_cols.hpp"

namespace g16 {

// REDC in the product-scanning order over the columns that COL adds to the running sum
// (carry + the column's digit products + m_i p_(k-i) for the Montgomery digits already
// known): below column 9 the column fixes m_k = (column (-p^-1)) mod 2^29 and adds m_k p_0,
// which clears its low 29 bits; from column 9 on it gives result digit k - 9.
template <class Col>
G16_HD Fp29 fp29_redc(Col col) {
    int64_t acc = 0;
    uint32_t m[9];
    Fp29 r;
    static_for<17>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        col(k_c, acc, m);
        if constexpr (k < 9) {
            m[k] = ((uint32_t)acc * kP29NInv) & kM29;
            acc += (int64_t)m[k] * (int64_t)p29_digit(0);
        } else {
            r.d[k - 9] = (int32_t)((uint32_t)acc & kM29);
        }
        acc >>= 29;
    });
    r.d[8] = (int32_t)acc;
    return r;
}

// The host's columns: the digit products x_i y_(k-i) of column k, and its Montgomery
// terms m_i p_(k-i) for the m_i already known (i < k).
template <int k>
G16_HD int64_t fp29_col_xy(const Fp29& x, const Fp29& y) {
    int64_t col = 0;
    static_for<9>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int j = k - i;
        if constexpr (j >= 0 && j < 9) col += (int64_t)x.d[i] * (int64_t)y.d[j];
    });
    return col;
}
template <int k>
G16_HD int64_t fp29_col_mp(const uint32_t (&m)[9]) {
    int64_t col = 0;
    static_for<9>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int j = k - i;
        if constexpr (i < k && j >= 1 && j < 9) col += (int64_t)m[i] * (int64_t)p29_digit(j);
    });
    return col;
}

// a b 2^-261 mod p, lazily reduced (see the header).  Inputs normalized.  On the device
// each column is one chain of v_mad_i64_i32 from fp29_cols.hpp.
G16_HD Fp29 fp29_mul(const Fp29& a, const Fp29& b) {
    return fp29_redc([&](auto k_c, int64_t& acc, const uint32_t (&m)[9]) {
        constexpr int k = decltype(k_c)::value;
#if defined(__HIP_DEVICE_COMPILE__)
        fp29_col_mul<k>(acc, a, b, m);
#else
        acc += fp29_col_xy<k>(a, b) + fp29_col_mp<k>(m);
#endif
    });
}

// a^2 2^-261: the same columns as fp29_mul(a, a), formed on the device from (2 a_i) a_j
// for i < j and a_i^2 (45 digit products instead of 81; each column's bound is that of
// a product, as a doubled digit product counts for two).
G16_HD Fp29 fp29_sqr(const Fp29& a) {
#if defined(__HIP_DEVICE_COMPILE__)
    int32_t a2[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) a2[k] = a.d[k] + a.d[k];
    return fp29_redc([&](auto k_c, int64_t& acc, const uint32_t (&m)[9]) {
        fp29_col_sqr<decltype(k_c)::value>(acc, a, a2, m);
    });
#else
    return fp29_mul(a, a);
#endif
}

// (a b - c d) 2^-261 with one reduction: a column holds both products' digit products
// (27 terms below 2^58 with the Montgomery terms, below 2^63), and the result is below
// (|a b| + |c d|) 2^-261 + p, no more than the difference of two reduced products.
G16_HD Fp29 fp29_mul_sub(const Fp29& a, const Fp29& b, const Fp29& c, const Fp29& d) {
    Fp29 nc;
#pragma unroll
    for (int k = 0; k < 9; ++k) nc.d[k] = -c.d[k];
    return fp29_redc([&](auto k_c, int64_t& acc, const uint32_t (&m)[9]) {
        constexpr int k = decltype(k_c)::value;
#if defined(__HIP_DEVICE_COMPILE__)
        fp29_col_mulsub<k>(acc, a, b, nc, d, m);
#else
        acc += fp29_col_xy<k>(a, b) + fp29_col_xy<k>(nc, d) + fp29_col_mp<k>(m);
#endif
    });
}

// The value mod p, canonical, as eight 32-bit words (not converted out of the 2^261
// Montgomery form).  |value| < 64 p: u = value + 64 p is in (0, 128 p), below 2^261; q
// from bits 224..287 of u over the top word of p is floor(u / p) or one more or less,
// and u - q p is brought into [0, p) by one conditional addition or subtraction of p.
G16_HD Fp fp29_canon(const Fp29& a) {
    uint32_t u[10];
    {
        // u = a + 64p with full carry propagation: digits in [0, 2^29), digit 8 >= 0
        int32_t dg[9];
        int32_t c = 0;
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            const int32_t x = a.d[k] + p64_29_digit(k) + c;
            if (k < 8) {
                dg[k] = x & (int32_t)kM29;
                c = x >> 29;
            } else {
                dg[k] = x;
            }
        }
        // pack 8 x 29 + the top digit into ten 32-bit words
#pragma unroll
        for (int j = 0; j < 10; ++j) {
            const int bit = 32 * j;
            const int k = bit / 29, off = bit - 29 * k;
            uint32_t v = k < 9 ? (uint32_t)dg[k] >> off : 0u;
            if (k + 1 < 9) v |= (uint32_t)dg[k + 1] << (29 - off);
            if (k + 2 < 9 && 58 - off < 32) v |= (uint32_t)dg[k + 2] << (58 - off);
            u[j] = v;
        }
    }
    const uint64_t hi = (uint64_t)u[8] << 32 | u[7];  // bits 224..287
    const uint32_t q = (uint32_t)(hi / 0x30644e72ull);
    // t = u - q p over nine words (borrow propagated through a signed 64-bit carry)
    int64_t t[9];
    int64_t carry = 0;
#pragma unroll
    for (int j = 0; j < 9; ++j) {
        const int64_t x = (int64_t)u[j] - (int64_t)((uint64_t)q * (j < 8 ? p_limb(j) : 0u)) + carry;
        t[j] = x & 0xffffffffll;
        carry = x >> 32;
    }
    // t in [-p, 2p): sign from the top word (carry below zero means negative)
    const bool neg = carry < 0 || (int32_t)t[8] < 0;
    Fp v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v.w[j] = (uint32_t)t[j];
    if (neg) {
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) v.w[j] = addc(v.w[j], p_limb(j), c);
        return v;
    }
    // top word t[8] is 0 here (t < 2p < 2^255)
    return fp_reduce_once(v);
}

// a == 0 mod p, for |value| < 64 p.  If the value is k p, then k = v / p is the nearest
// integer to the top two digits' ratio (their relative error is below 2^-49 and |k| <= 64),
// and the value is zero mod p exactly when v - k p, carried through the digits, is zero.
// For any other value v - k p is not zero whatever k is.  About a third of fp29_canon.
G16_HD bool fp29_is_zero(const Fp29& a) {
    constexpr double kInvPTop = 1.0 / ((double)p29_digit(8) * 536870912.0 + (double)p29_digit(7));
    const double top = (double)a.d[8] * 536870912.0 + (double)a.d[7];
    const int64_t k = (int64_t)__builtin_rint(top * kInvPTop);
    int64_t carry = 0;
    int64_t nonzero = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t x = (int64_t)a.d[i] - k * (int64_t)p29_digit(i) + carry;
        nonzero |= x & (int64_t)kM29;
        carry = x >> 29;
    }
    nonzero |= (int64_t)a.d[8] - k * (int64_t)p29_digit(8) + carry;
    return nonzero == 0;
}

// a^(p-2) = a^-1 (Fermat; 0 -> 0), square and multiply in the 2^261 Montgomery form.
G16_HD Fp29 fp29_inv(const Fp29& a) {
    Fp29 acc = fp29_from_fp(fp_one());
    for (int bit = 253; bit >= 0; --bit) {
        acc = fp29_sqr(acc);
        uint32_t e = p_limb(bit >> 5);
        if ((bit >> 5) == 0) e -= 2u;  // low limb of p - 2 (p's low limb is odd and large)
        if ((e >> (bit & 31)) & 1u) acc = fp29_mul(acc, a);
    }
    return acc;
}

// -> canonical 2^256 Montgomery form: (value mod p) 2^-5 = (c + k p) / 32 with
// k = c (-p^-1) mod 32, which is below p for c < p.
G16_HD Fp fp29_to_fp(const Fp29& a) {
    const Fp c = fp29_canon(a);
    const uint32_t k = (c.w[0] * kP5NInv) & 31u;
    uint32_t t[9];
    uint64_t carry = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint64_t x = (uint64_t)k * p_limb(j) + c.w[j] + carry;
        t[j] = (uint32_t)x;
        carry = x >> 32;
    }
    t[8] = (uint32_t)carry;
    Fp r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.w[j] = (t[j] >> 5) | (t[j + 1] << 27);
    return r;
}

}  // namespace g16
