// Fr in nine signed 29-bit digits, kept in registers and LDS through the transform
// passes, and the product by a fixed table entry (Shoup's method).
//
// Why a second representation.  On gfx950 every add-with-carry that reads the carry of
// the previous VALU instruction waits two issue slots, so the 8 x 32-bit carry chains
// of fr.hpp cost about three slots per limb, and a 32-bit limb product cannot be
// accumulated without one.  With 29-bit digits a digit product is below 2^58 and a
// column of up to 18 products plus a carry stays inside a signed 64-bit accumulator,
// so every product is one v_mad_i64_i32 and nothing else propagates carries; adds and
// subtracts are digit-wise 32-bit adds with no carry at all.
//
// Value of a V29: sum of l[k] 2^(29k) with signed 32-bit digits.  "Normalized" means
// digits 0..7 in [-4, 2^29 + 3) (what fr29_normalize returns; a product output and a
// freshly split canonical value have them in [0, 2^29)).  A Cooley-Tukey butterfly
// replaces (lo, hi) by lo + t and lo - t with t = w hi a product output, so both results
// sit one pass further from lo's last normalization than lo did, and hi's own growth
// does not carry over.  (Digit 8 is never masked: it moves by less than 2^27 a pass and
// stays far inside 32 bits over the at most ten passes between a load or product and
// the next canonical store.)  After p passes from normalized a digit is below
// 2^29 + 3 + p (2^29 - 1) in magnitude, so three passes still fit in 32 bits (and any
// 32-bit digits are a valid product input).  The transforms therefore normalize, at the start of each register group of two
// passes, only the elements that are "lo" in the group's first pass: every group output
// is then exactly two passes from normalized.
//
// Product by a table entry (V. Shoup, NTL; D. Harvey, "Faster arithmetic for
// number-theoretic transforms", J. Symb. Comp. 2014): for a fixed w < r store w and
// w' = floor(w 2^261 / r).  Then q = floor(x w' / 2^261) is within one or two of
// x w / r and x w - q r is x w mod r up to a few multiples of r.  Only the top columns
// of x w' are needed for q and only the low 261 bits of x w - q r, because that
// difference is small.  This needs 45 + 45 + 45 = 135 digit products against 162 for a
// Montgomery product on nine digits.  The result keeps x's Montgomery factor (w is a
// plain integer), so data stay in the 2^256 Montgomery form of the library's
// interface.  Table digits are balanced (|digit| <= 2^28, the top digit of w' up to
// 2^29 + 1), which halves the size of every product and so doubles the input range a
// column can absorb.
#pragma once

#include <type_traits>
#include <utility>

#include "fr.hpp"

namespace g16 {

struct V29 {
    int32_t l[9];
};

// A table entry: w and w' = floor(w 2^261 / r) in balanced 29-bit digits, padded to
// 80 bytes: five 16-byte parts (w0-3, w4-7, w8 w'0-2, w'3-6, w'7-8 and padding).
struct Tw29 {
    int32_t w[9];
    int32_t wp[9];
    int32_t pad[2];
};
static_assert(sizeof(Tw29) == 80, "table entries are 80 bytes");

// A table of entries in five planes: part q of entry e at base[q * stride + e], so the
// lanes of a wave that read neighbouring entries read one contiguous run per part (a few
// cache lines per load instruction) instead of 80-byte records spread over five times
// as many lines.
struct TwTab {
    uint4* base;
    uint32_t stride;  // entries per plane
};

// -r in balanced 29-bit digits (x w - q r is formed as x w + q (-r))
G16_HD constexpr int32_t mr29_digit(int k) {
    return k == 0 ? 0x0fffffff : k == 1 ? 0x00f05360 : k == 2 ? -0x0e5c2451
         : k == 3 ? -0x07d090f3 : k == 4 ? 0x0a7a2d7d : k == 5 ? -0x02db40c1
         : k == 6 ? -0x00a6e141 : k == 7 ? -0x0e5c2634 : -0x0030644e;
}
// r^-1 mod 2^261 in unsigned 29-bit digits (exact division by r in the table builder)
G16_HD constexpr uint32_t rinv261_limb(int k) {
    return k == 0 ? 0x10000001u : k == 1 ? 0x08f05360u : k == 2 ? 0x05bb930fu
         : k == 3 ? 0x12f36967u : k == 4 ? 0x1dc6e9a7u : k == 5 ? 0x13ebb37cu
         : k == 6 ? 0x19347195u : k == 7 ? 0x1c5e4f97u : 0x0d8c07d0u;
}

// canonical 8 x 32-bit -> nine 29-bit digits (all in [0, 2^29))
G16_HD V29 fr29_from_fr(const Fr& x) {
    V29 r;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int bit = 29 * k, w = bit >> 5, s = bit & 31;
        uint32_t v = x.w[w] >> s;
        if (s > 3 && w + 1 < 8) v |= x.w[w + 1] << (32 - s);
        r.l[k] = (int32_t)((k < 8) ? (v & kM29) : v);
    }
    return r;
}

// Digits in [0, 2^29) (value below 2^256) -> eight 32-bit words.
G16_HD Fr fr29_pack(const V29& u) {
    Fr x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int bit = 32 * j;
        const int k = bit / 29, off = bit - 29 * k;
        uint32_t v = (uint32_t)u.l[k] >> off;
        if (k + 1 < 9) v |= (uint32_t)u.l[k + 1] << (29 - off);
        if (k + 2 < 9 && 58 - off < 32) v |= (uint32_t)u.l[k + 2] << (58 - off);
        x.w[j] = v;
    }
    return x;
}

G16_HD V29 fr29_add(const V29& a, const V29& b) {
    V29 s;
#pragma unroll
    for (int k = 0; k < 9; ++k) s.l[k] = a.l[k] + b.l[k];
    return s;
}

G16_HD V29 fr29_sub(const V29& a, const V29& b) {
    V29 s;
#pragma unroll
    for (int k = 0; k < 9; ++k) s.l[k] = a.l[k] - b.l[k];
    return s;
}

// Carry-save normalization: digit k keeps its low 29 bits plus the (signed) carry out of
// digit k-1, which is in [-4, 4) for digits below 2^31 in magnitude.  The value is
// unchanged; digit 8 absorbs the carry of digit 7.
G16_HD V29 fr29_normalize(const V29& a) {
    V29 o;
    o.l[0] = a.l[0] & (int32_t)kM29;
#pragma unroll
    for (int k = 1; k < 8; ++k) o.l[k] = (a.l[k] & (int32_t)kM29) + (a.l[k - 1] >> 29);
    o.l[8] = a.l[8] + (a.l[7] >> 29);
    return o;
}

// The product on the device: one asm block per column.  A column is one chain of
// v_mad_i64_i32 that starts from the carry of the column below.  Written in C, the chain
// is reassociated by the compiler into parallel partial sums with the carry added
// separately (about 40 more instructions a product); with an empty asm statement after
// each multiply-add the chain stays whole, but the compiler then inserts a wait state
// after every one of them, since it has to assume that an asm statement might be an
// instruction with a result-forwarding hazard.  One block per column leaves at most one
// wait state per column (none where another chain's block comes in between).  The
// multiply-adds write their unused carry-out to vcc, which each block clobbers.
#if defined(__HIP_DEVICE_COMPILE__)
#define G16_X(i, j) "v_mad_i64_i32 %[acc], vcc, %[x" #i "], %[b" #j "], %[acc]\n\t"
#define G16_X0(i, j) "v_mad_i64_i32 %[acc], vcc, %[x" #i "], %[b" #j "], 0\n\t"
#define G16_Q(i, j) "v_mad_i64_i32 %[acc], vcc, %[q" #i "], %[m" #j "], %[acc]\n\t"
#define G16_XOPS(v) \
    [x0] "v"(v[0]), \
    [x1] "v"(v[1]), \
    [x2] "v"(v[2]), \
    [x3] "v"(v[3]), \
    [x4] "v"(v[4]), \
    [x5] "v"(v[5]), \
    [x6] "v"(v[6]), \
    [x7] "v"(v[7]), \
    [x8] "v"(v[8])
#define G16_BOPS(v) \
    [b0] "v"(v[0]), \
    [b1] "v"(v[1]), \
    [b2] "v"(v[2]), \
    [b3] "v"(v[3]), \
    [b4] "v"(v[4]), \
    [b5] "v"(v[5]), \
    [b6] "v"(v[6]), \
    [b7] "v"(v[7]), \
    [b8] "v"(v[8])
#define G16_BOPS_S(v) \
    [b0] "s"(v[0]), \
    [b1] "s"(v[1]), \
    [b2] "s"(v[2]), \
    [b3] "s"(v[3]), \
    [b4] "s"(v[4]), \
    [b5] "s"(v[5]), \
    [b6] "s"(v[6]), \
    [b7] "s"(v[7]), \
    [b8] "s"(v[8])
#define G16_QOPS(v) \
    [q0] "v"(v[0]), \
    [q1] "v"(v[1]), \
    [q2] "v"(v[2]), \
    [q3] "v"(v[3]), \
    [q4] "v"(v[4]), \
    [q5] "v"(v[5]), \
    [q6] "v"(v[6]), \
    [q7] "v"(v[7]), \
    [q8] "v"(v[8])
#define G16_MOPS \
    [m0] "s"(mr29_digit(0)), \
    [m1] "s"(mr29_digit(1)), \
    [m2] "s"(mr29_digit(2)), \
    [m3] "s"(mr29_digit(3)), \
    [m4] "s"(mr29_digit(4)), \
    [m5] "s"(mr29_digit(5)), \
    [m6] "s"(mr29_digit(6)), \
    [m7] "s"(mr29_digit(7)), \
    [m8] "s"(mr29_digit(8))

// Column C (8..16) of x b: acc = carry + sum of x_i b_(C-i); column 8 starts from zero.
// BOPS names the constraint set of b (in VGPRs, or in SGPRs for an entry every lane of
// the wave shares).
#define G16_COL_Q(BOPS) \
    if constexpr (C == 8) { \
        asm(G16_X0(0, 8) G16_X(1, 7) G16_X(2, 6) G16_X(3, 5) G16_X(4, 4) G16_X(5, 3) \
            G16_X(6, 2) G16_X(7, 1) G16_X(8, 0) \
            : [acc] "=&v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    } else if constexpr (C == 9) { \
        asm(G16_X(1, 8) G16_X(2, 7) G16_X(3, 6) G16_X(4, 5) G16_X(5, 4) G16_X(6, 3) \
            G16_X(7, 2) G16_X(8, 1) \
            : [acc] "+v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    } else if constexpr (C == 10) { \
        asm(G16_X(2, 8) G16_X(3, 7) G16_X(4, 6) G16_X(5, 5) G16_X(6, 4) G16_X(7, 3) \
            G16_X(8, 2) \
            : [acc] "+v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    } else if constexpr (C == 11) { \
        asm(G16_X(3, 8) G16_X(4, 7) G16_X(5, 6) G16_X(6, 5) G16_X(7, 4) G16_X(8, 3) \
            : [acc] "+v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    } else if constexpr (C == 12) { \
        asm(G16_X(4, 8) G16_X(5, 7) G16_X(6, 6) G16_X(7, 5) G16_X(8, 4) \
            : [acc] "+v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    } else if constexpr (C == 13) { \
        asm(G16_X(5, 8) G16_X(6, 7) G16_X(7, 6) G16_X(8, 5) \
            : [acc] "+v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    } else if constexpr (C == 14) { \
        asm(G16_X(6, 8) G16_X(7, 7) G16_X(8, 6) \
            : [acc] "+v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    } else if constexpr (C == 15) { \
        asm(G16_X(7, 8) G16_X(8, 7) \
            : [acc] "+v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    } else if constexpr (C == 16) { \
        asm(G16_X(8, 8) \
            : [acc] "+v"(acc) : G16_XOPS(x), BOPS(b) : "vcc"); \
    }

// Column C (0..8) of x b + q (-r): acc = carry + sum of x_i b_(C-i) + q_i (-r)_(C-i);
// column 0 starts from zero.
#define G16_COL_Y(BOPS) \
    if constexpr (C == 0) { \
        asm(G16_X0(0, 0) G16_Q(0, 0) \
            : [acc] "=&v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    } else if constexpr (C == 1) { \
        asm(G16_X(0, 1) G16_Q(0, 1) G16_X(1, 0) G16_Q(1, 0) \
            : [acc] "+v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    } else if constexpr (C == 2) { \
        asm(G16_X(0, 2) G16_Q(0, 2) G16_X(1, 1) G16_Q(1, 1) G16_X(2, 0) G16_Q(2, 0) \
            : [acc] "+v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    } else if constexpr (C == 3) { \
        asm(G16_X(0, 3) G16_Q(0, 3) G16_X(1, 2) G16_Q(1, 2) G16_X(2, 1) G16_Q(2, 1) \
            G16_X(3, 0) G16_Q(3, 0) \
            : [acc] "+v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    } else if constexpr (C == 4) { \
        asm(G16_X(0, 4) G16_Q(0, 4) G16_X(1, 3) G16_Q(1, 3) G16_X(2, 2) G16_Q(2, 2) \
            G16_X(3, 1) G16_Q(3, 1) G16_X(4, 0) G16_Q(4, 0) \
            : [acc] "+v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    } else if constexpr (C == 5) { \
        asm(G16_X(0, 5) G16_Q(0, 5) G16_X(1, 4) G16_Q(1, 4) G16_X(2, 3) G16_Q(2, 3) \
            G16_X(3, 2) G16_Q(3, 2) G16_X(4, 1) G16_Q(4, 1) G16_X(5, 0) G16_Q(5, 0) \
            : [acc] "+v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    } else if constexpr (C == 6) { \
        asm(G16_X(0, 6) G16_Q(0, 6) G16_X(1, 5) G16_Q(1, 5) G16_X(2, 4) G16_Q(2, 4) \
            G16_X(3, 3) G16_Q(3, 3) G16_X(4, 2) G16_Q(4, 2) G16_X(5, 1) G16_Q(5, 1) \
            G16_X(6, 0) G16_Q(6, 0) \
            : [acc] "+v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    } else if constexpr (C == 7) { \
        asm(G16_X(0, 7) G16_Q(0, 7) G16_X(1, 6) G16_Q(1, 6) G16_X(2, 5) G16_Q(2, 5) \
            G16_X(3, 4) G16_Q(3, 4) G16_X(4, 3) G16_Q(4, 3) G16_X(5, 2) G16_Q(5, 2) \
            G16_X(6, 1) G16_Q(6, 1) G16_X(7, 0) G16_Q(7, 0) \
            : [acc] "+v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    } else if constexpr (C == 8) { \
        asm(G16_X(0, 8) G16_Q(0, 8) G16_X(1, 7) G16_Q(1, 7) G16_X(2, 6) G16_Q(2, 6) \
            G16_X(3, 5) G16_Q(3, 5) G16_X(4, 4) G16_Q(4, 4) G16_X(5, 3) G16_Q(5, 3) \
            G16_X(6, 2) G16_Q(6, 2) G16_X(7, 1) G16_Q(7, 1) G16_X(8, 0) G16_Q(8, 0) \
            : [acc] "+v"(acc) \
            : G16_XOPS(x), BOPS(b), G16_QOPS(q), G16_MOPS : "vcc"); \
    }

template <int C, bool BS>
__device__ __forceinline__ void col_q(int64_t& acc, const int32_t (&x)[9], const int32_t (&b)[9]) {
    if constexpr (BS) {
        G16_COL_Q(G16_BOPS_S)
    } else {
        G16_COL_Q(G16_BOPS)
    }
}

template <int C, bool BS>
__device__ __forceinline__ void col_y(int64_t& acc, const int32_t (&x)[9], const int32_t (&b)[9],
                                      const int32_t (&q)[9]) {
    if constexpr (BS) {
        G16_COL_Y(G16_BOPS_S)
    } else {
        G16_COL_Y(G16_BOPS)
    }
}

#undef G16_X
#undef G16_X0
#undef G16_Q
#undef G16_XOPS
#undef G16_BOPS
#undef G16_BOPS_S
#undef G16_COL_Q
#undef G16_COL_Y
#undef G16_QOPS
#undef G16_MOPS
#endif

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so that every
// register array index is a constant and arrays stay in registers.
template <typename F, int... I>
G16_HD void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
G16_HD void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// y[n] = x[n] w_n mod r up to a small multiple of r, for table entries t[n] = (w, w').
//   Any 32-bit digits are admissible: with |digit| <= 2^31 every column stays inside the
//   signed 64-bit range (ten products below 2^59 for the q columns, whose top w' digit
//   may reach 2^29 + 1; nine below 2^59 plus nine below 2^57 for the low columns; plus a
//   carry below 2^35).
//   Result: digits 0..7 in [0, 2^29), digit 8 signed; value congruent to x w, with
//   |value| < 23 r, so |digit 8| < 2^27.
// q is taken from columns 8..16 of x w' (45 products): the dropped columns 0..7 add less
// than 2^265 in magnitude, sixteen units of q (2^261), so q is within 17 of
// x w' / 2^261, and x w - q r lies within (|x|/2^261 + 19) r of zero; |x| < 2^263 keeps
// that below 23 r.  The N products run as N interleaved chains.  BS: the entries are the
// same in every lane of the wave and held in SGPRs (device builds).
template <int N, bool BS = false>
G16_HD void shoup_mul_n(const V29 (&x)[N], const Tw29 (&t)[N], V29 (&y)[N]) {
    int32_t q[N][9];
    int64_t acc[N];
#if defined(__HIP_DEVICE_COMPILE__)
    // q: columns 8..16 of x w'; its digits are taken in [0, 2^29) (q mod 2^261 is all the
    // low part needs)
    static_for<9>([&](auto c_c) {
        constexpr int c = 8 + decltype(c_c)::value;
#pragma unroll
        for (int n = 0; n < N; ++n) col_q<c, BS>(acc[n], x[n].l, t[n].wp);
#pragma unroll
        for (int n = 0; n < N; ++n) {
            if (c >= 9) q[n][c - 9] = (int32_t)((uint32_t)acc[n] & kM29);
            acc[n] >>= 29;
        }
    });
#pragma unroll
    for (int n = 0; n < N; ++n) q[n][8] = (int32_t)((uint32_t)acc[n] & kM29);
    // y: columns 0..8 of x w + q (-r) = (x w - q r) mod 2^261; the top digit is read back
    // as a signed 29-bit number, which is exact since |x w - q r| < 2^259
    static_for<9>([&](auto c_c) {
        constexpr int c = decltype(c_c)::value;
#pragma unroll
        for (int n = 0; n < N; ++n) col_y<c, BS>(acc[n], x[n].l, t[n].w, q[n]);
#pragma unroll
        for (int n = 0; n < N; ++n) {
            if (c < 8) {
                y[n].l[c] = (int32_t)((uint32_t)acc[n] & kM29);
                acc[n] >>= 29;
            } else {
                y[n].l[8] = ((int32_t)((uint32_t)acc[n] << 3)) >> 3;
            }
        }
    });
#else
    // The same columns in C (host builds).
    for (int n = 0; n < N; ++n) {
        acc[n] = 0;
        for (int c = 8; c < 17; ++c) {
            for (int i = 0; i < 9; ++i)
                if (c - i >= 0 && c - i < 9) acc[n] += (int64_t)x[n].l[i] * t[n].wp[c - i];
            if (c >= 9) q[n][c - 9] = (int32_t)((uint32_t)acc[n] & kM29);
            acc[n] >>= 29;
        }
        q[n][8] = (int32_t)((uint32_t)acc[n] & kM29);
        acc[n] = 0;
        for (int c = 0; c < 9; ++c) {
            for (int i = 0; i <= c; ++i) {
                acc[n] += (int64_t)x[n].l[i] * t[n].w[c - i];
                acc[n] += (int64_t)q[n][i] * mr29_digit(c - i);
            }
            if (c < 8) {
                y[n].l[c] = (int32_t)((uint32_t)acc[n] & kM29);
                acc[n] >>= 29;
            } else {
                y[n].l[8] = ((int32_t)((uint32_t)acc[n] << 3)) >> 3;
            }
        }
    }
#endif
}

G16_HD V29 shoup_mul(const V29& x, const Tw29& t) {
    V29 xs[1] = {x};
    Tw29 ts[1] = {t};
    V29 ys[1];
    shoup_mul_n<1>(xs, ts, ys);
    return ys[0];
}

// Any V29 with digits 0..7 below 2^31 and digit 8 below 2^30 in magnitude -> 8 x 32-bit
// words of a value in [0, 2r) congruent to it (fr29_canon without the last step; what the
// transform batches hand to one another, since fr29_from_fr and the table products take
// any value below 2^256).
//   1. q = floor(value / r) or one less, from the top two digits as they are, in double
//      precision: the digits below contribute less than 2^205 (2^-48 of r), the
//      estimate's own error is below 2^-40, the margin 2^-10;
//   2. value - q r = (value + q (-r)) mod 2^261, in [0, 2r), its digits' carries taken
//      along one multiply-add row (so the digits need no normalization first);
//   3. pack.
G16_HD Fr fr29_reduce_2r(const V29& a) {
    int32_t l[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) l[k] = a.l[k];
    // 2^232 / r and 2^203 / r
    const double c8 = 0x1.5291d18988e81p-22, c7 = 0x1.5291d18988e81p-51;
    const double qd = floor((double)l[8] * c8 + (double)l[7] * c7 - 0x1p-10);
    const int32_t q = (int32_t)qd;
    V29 y;
    int64_t acc = 0;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        acc += (int64_t)q * mr29_digit(k) + l[k];
        y.l[k] = (int32_t)((uint32_t)acc & kM29);
        acc >>= 29;
    }
    return fr29_pack(y);
}

// Any V29 with digits below 2^31 in magnitude -> canonical 8 x 32-bit: fr29_reduce_2r and
// one conditional subtraction.
G16_HD Fr fr29_canon(const V29& a) { return fr_reduce_once(fr29_reduce_2r(a)); }

// Products of two variables (the join of the H epilogue and the CSR gather).  Montgomery's
// REDC (P. L. Montgomery, Math. Comp. 1985) in radix 2^29 with R' = 2^261, in the
// product-scanning order: column k adds the digit products x_i y_(k-i) and the terms
// m_i r_(k-i) of the Montgomery digits already fixed; below column 9 the column fixes
// m_k = column (-r^-1) mod 2^29, whose m_k r_0 clears its low 29 bits, and from column 9
// on it yields result digit k - 9.  r = 1 + 2^28 mod 2^29, so -r^-1 = 2^28 - 1 mod 2^29.
// Every product is one multiply-add into a signed 64-bit column and carries move once a
// column: no add-with-carry chains (fr_mul's CIOS needs one per 32-bit limb product).
// The interface keeps R = 2^256: one factor enters shifted by 2^5 (fr29_from_fr_shl5), and
// x 2^5 y 2^-261 = x y 2^-256.

// r in 29-bit digits
G16_HD constexpr int32_t r29_digit(int k) {
    return k == 0 ? 0x10000001 : k == 1 ? 0x1f0fac9f : k == 2 ? 0x0e5c2450
         : k == 3 ? 0x07d090f3 : k == 4 ? 0x1585d283 : k == 5 ? 0x02db40c0
         : k == 6 ? 0x00a6e141 : k == 7 ? 0x0e5c2634 : 0x0030644e;
}
constexpr uint32_t kR29NInv = 0x0fffffffu;  // -r^-1 mod 2^29
static_assert((0x10000001ull * kR29NInv + 1ull) % (1ull << 29) == 0ull, "kR29NInv");

// canonical 8 x 32-bit x -> digits of x 2^5, all in [0, 2^29) (x 2^5 < 2^259)
G16_HD V29 fr29_from_fr_shl5(const Fr& x) {
    V29 r;
    r.l[0] = (int32_t)((x.w[0] << 5) & kM29);
#pragma unroll
    for (int k = 1; k < 9; ++k) {
        const int pos = 29 * k - 5, w = pos >> 5, s = pos & 31;
        uint32_t v = x.w[w] >> s;
        if (s > 3 && w + 1 < 8) v |= x.w[w + 1] << (32 - s);
        r.l[k] = (int32_t)((k < 8) ? (v & kM29) : v);
    }
    return r;
}

// REDC over the columns that XY adds (the digit products of column k, or nothing): the
// value (X + m r) / 2^261 with m < 2^261 chosen so that 2^261 divides X + m r, where X is
// the sum XY forms.  Result digits 0..7 in [0, 2^29), digit 8 the signed remainder.
template <class XY>
G16_HD V29 fr29_redc_cols(XY xy) {
    int64_t acc = 0;
    int32_t m[9];
    V29 o;
    static_for<17>([&](auto k_c) {
        constexpr int k = decltype(k_c)::value;
        xy(k_c, acc);
        static_for<9>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            constexpr int j = k - i;
            if constexpr (i < k && j >= 1 && j < 9) acc += (int64_t)m[i] * r29_digit(j);
        });
        if constexpr (k < 9) {
            m[k] = (int32_t)(((uint32_t)acc * kR29NInv) & kM29);
            acc += (int64_t)m[k] * r29_digit(0);
        } else {
            o.l[k - 9] = (int32_t)((uint32_t)acc & kM29);
        }
        acc >>= 29;
    });
    o.l[8] = (int32_t)acc;
    return o;
}

// x y 2^-261 for digits below 2^29 + 8 in magnitude: a column holds at most 18 products
// below 2^58.01 and a carry, inside 2^63.  For 0 <= x, y the result is below
// x y / 2^261 + r.
G16_HD V29 fr29_mont_mul(const V29& x, const V29& y) {
    return fr29_redc_cols([&](auto k_c, int64_t& acc) {
        constexpr int k = decltype(k_c)::value;
        static_for<9>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            constexpr int j = k - i;
            if constexpr (j >= 0 && j < 9) acc += (int64_t)x.l[i] * (int64_t)y.l[j];
        });
    });
}

// x 2^-261 for digits in [0, 2^29) (x < 2^261): below x / 2^261 + r < 2r.
G16_HD V29 fr29_redc1(const V29& x) {
    return fr29_redc_cols([&](auto k_c, int64_t& acc) {
        constexpr int k = decltype(k_c)::value;
        if constexpr (k < 9) acc += x.l[k];
    });
}

// Montgomery product of canonical a, b (R = 2^256): a b 2^-256 mod r, canonical.  The
// REDC value is below 32 a b / 2^261 + r < (32 r / 2^261 + 1) r < 2r, with digits in
// [0, 2^29), so one conditional subtraction after packing.
G16_HD Fr fr_mul29(const Fr& a, const Fr& b) {
    return fr_reduce_once(fr29_pack(fr29_mont_mul(fr29_from_fr_shl5(a), fr29_from_fr(b))));
}

// Montgomery form -> standard form of a canonical a: a 2^5 2^-261, below 2r.
G16_HD Fr fr_from_mont29(const Fr& a) {
    return fr_reduce_once(fr29_pack(fr29_redc1(fr29_from_fr_shl5(a))));
}

// Unsigned 29-bit digits (the top one below 2^29) -> balanced digits, value unchanged.
G16_HD void balance29(const uint32_t (&d)[9], int32_t (&o)[9]) {
    int32_t carry = 0;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        int32_t v = (int32_t)d[k] + carry;
        if (k < 8 && v >= (1 << 28)) {
            v -= (1 << 29);
            carry = 1;
        } else {
            carry = 0;
        }
        o[k] = v;
    }
}

// The table entry for a value given in Montgomery form: w = wm 2^-256 (plain) and
// w' = floor(w 2^261 / r).  With rem = w 2^261 mod r (fr_mul(wm, 2^261 mod r)), w 2^261
// = w' r + rem exactly, so w' = -rem r^-1 mod 2^261 (exact division by the odd r).
G16_HD Tw29 tw29_entry(const Fr& wm) {
    Tw29 t;
    const V29 w = fr29_from_fr(fr_from_mont(wm));
    const V29 rem = fr29_from_fr(fr_mul(wm, fr_c261()));
    // p = rem r^-1 mod 2^261 (low half product), then w' = 2^261 - p mod 2^261
    uint32_t p[9];
    uint64_t acc = 0;
#pragma unroll
    for (int c = 0; c < 9; ++c) {
#pragma unroll
        for (int i = 0; i <= c; ++i) acc += (uint64_t)(uint32_t)rem.l[i] * rinv261_limb(c - i);
        p[c] = (uint32_t)acc & kM29;
        acc >>= 29;
    }
    uint32_t wp[9], wd[9];
    uint32_t borrow = 0;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        uint32_t d = 0u - p[k] - borrow;  // digit of 2^261 - p, with borrow
        borrow = (p[k] + borrow) != 0u ? 1u : 0u;
        wp[k] = d & kM29;
        wd[k] = (uint32_t)w.l[k];
    }
    balance29(wd, t.w);
    balance29(wp, t.wp);
    t.pad[0] = t.pad[1] = 0;
    return t;
}

}  // namespace g16
