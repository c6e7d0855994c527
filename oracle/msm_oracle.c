/*
 * CPU oracle for the G1 multi-scalar multiplication over BN254 (the MSM_CU page:
 * sum_i k_i P_i over the curve y^2 = x^3 + 3 on the base field Fp).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests load this library.  It shares no code,
 * header, table or constant with the GPU library, and none with oracle.c either:
 * its field arithmetic is its own.
 *
 * Arithmetic is deliberately plain:
 *   - Fp elements in STANDARD form as four 64-bit little-endian limbs; a product is
 *     the schoolbook 512-bit product reduced by Barrett's method (Menezes, van
 *     Oorschot, Vanstone, Handbook of Applied Cryptography, algorithm 14.42); the
 *     inverse is a^(p-2) (Fermat).  Montgomery form (R = 2^256) only at the I/O
 *     boundary, for the conversion helpers.
 *   - Points: affine chord-and-tangent addition and doubling (the textbook group law,
 *     one field inversion each), and Jacobian coordinates (x, y) = (X/Z^2, Y/Z^3)
 *     with the textbook addition and a = 0 doubling formulas, so that a scalar
 *     multiple costs no inversion until the end.  The tests check the two against
 *     each other.
 *   - k P by left-to-right double and add over the 256 bits of k.
 *   - The MSM is its definition: sum over i of k_i P_i, each term by double and add.
 *     There is no bucketing, windowing or batching here: that is what the GPU side
 *     does and what this checks.
 *
 * Encodings.  A point crosses the boundary as 16 little-endian 32-bit words: x (8)
 * then y (8), standard form.  The point at infinity is (0, 0), which is not on the
 * curve (0 != 0 + 3).  Scalars are 8 words, any 256-bit integer.
 *
 * Constants derived here: p is given; b = 3; the generator is (1, 2); Barrett's mu is
 * computed from p at start-up.
 */
#include <stdint.h>
#include <string.h>

typedef uint64_t u64;
typedef unsigned __int128 u128;

typedef struct { u64 v[4]; } fp;

/* p = 21888242871839275222246405745257275088696311157297823662689037894645226208583 */
static const fp PMOD = {{0x3c208c16d87cfd47ULL, 0x97816a916871ca8dULL,
                         0xb85045b68181585dULL, 0x30644e72e131a029ULL}};
static u64 MU[5];   /* floor(2^512 / p) */
static int READY = 0;

/* ---------------------------------------------------------------- limb helpers */

static int ge_n(const u64* a, const u64* b, int n) {
    for (int i = n - 1; i >= 0; --i)
        if (a[i] != b[i]) return a[i] > b[i];
    return 1;
}

static u64 sub_limbs(u64* out, const u64* a, const u64* b, int n) {
    u64 borrow = 0;
    for (int i = 0; i < n; ++i) {
        u128 d = (u128)a[i] - b[i] - borrow;
        out[i] = (u64)d;
        borrow = (u64)(d >> 64) ? 1 : 0;
    }
    return borrow;
}

static u64 add_limbs(u64* out, const u64* a, const u64* b, int n) {
    u64 carry = 0;
    for (int i = 0; i < n; ++i) {
        u128 s = (u128)a[i] + b[i] + carry;
        out[i] = (u64)s;
        carry = (u64)(s >> 64);
    }
    return carry;
}

static void mul_limbs(u64* out, const u64* a, int na, const u64* b, int nb) {
    memset(out, 0, sizeof(u64) * (size_t)(na + nb));
    for (int i = 0; i < na; ++i) {
        u64 carry = 0;
        for (int j = 0; j < nb; ++j) {
            u128 t = (u128)a[i] * b[j] + out[i + j] + carry;
            out[i + j] = (u64)t;
            carry = (u64)(t >> 64);
        }
        out[i + nb] = carry;
    }
}

/* ---------------------------------------------------------------- Fp, standard form */

static fp fp_zero(void) { fp z; memset(&z, 0, sizeof z); return z; }
static fp fp_small(u64 x) { fp z = fp_zero(); z.v[0] = x; return z; }
static int fp_is_zero(fp a) { return (a.v[0] | a.v[1] | a.v[2] | a.v[3]) == 0; }
static int fp_eq(fp a, fp b) { return memcmp(a.v, b.v, sizeof a.v) == 0; }

static fp fp_add(fp a, fp b) {
    fp s;
    u64 c = add_limbs(s.v, a.v, b.v, 4);
    if (c || ge_n(s.v, PMOD.v, 4)) sub_limbs(s.v, s.v, PMOD.v, 4);
    return s;
}

static fp fp_sub(fp a, fp b) {
    fp d;
    if (sub_limbs(d.v, a.v, b.v, 4)) add_limbs(d.v, d.v, PMOD.v, 4);
    return d;
}

static fp fp_neg(fp a) { return fp_sub(fp_zero(), a); }

/* x < p 2^256 (any product of two canonical elements) -> x mod p, HAC 14.42 with
 * base 2^64 and k = 4. */
static fp barrett(const u64 x[8]) {
    u64 q2[10], q3[5], r2[10], r1[5], rr[5];
    mul_limbs(q2, x + 3, 5, MU, 5);
    memcpy(q3, q2 + 5, sizeof q3);
    memcpy(r1, x, sizeof r1);
    mul_limbs(r2, q3, 5, PMOD.v, 4);
    sub_limbs(rr, r1, r2, 5);
    u64 m5[5] = {PMOD.v[0], PMOD.v[1], PMOD.v[2], PMOD.v[3], 0};
    while (ge_n(rr, m5, 5)) sub_limbs(rr, rr, m5, 5);
    fp out;
    memcpy(out.v, rr, sizeof out.v);
    return out;
}

static fp fp_mul(fp a, fp b) {
    u64 prod[8];
    mul_limbs(prod, a.v, 4, b.v, 4);
    return barrett(prod);
}

static fp fp_pow(fp a, const u64 e[4]) {
    fp acc = fp_small(1);
    for (int bit = 255; bit >= 0; --bit) {
        acc = fp_mul(acc, acc);
        if ((e[bit >> 6] >> (bit & 63)) & 1u) acc = fp_mul(acc, a);
    }
    return acc;
}

static fp fp_inv(fp a) {   /* a^(p-2); 0 maps to 0 */
    u64 e[4];
    memcpy(e, PMOD.v, sizeof e);
    e[0] -= 2;   /* the low limb of p is odd and large: no borrow */
    return fp_pow(a, e);
}

static void init(void) {
    if (READY) return;
    /* mu = floor(2^512 / p) by binary long division of the single bit 2^512 */
    u64 rem[5] = {0, 0, 0, 0, 0};
    u64 q[9] = {0};
    u64 m5[5] = {PMOD.v[0], PMOD.v[1], PMOD.v[2], PMOD.v[3], 0};
    for (int bit = 512; bit >= 0; --bit) {
        /* rem = 2 rem + (bit == 512) */
        u64 carry = bit == 512 ? 1u : 0u;
        for (int i = 0; i < 5; ++i) {
            u64 nc = rem[i] >> 63;
            rem[i] = (rem[i] << 1) | carry;
            carry = nc;
        }
        if (ge_n(rem, m5, 5)) {
            sub_limbs(rem, rem, m5, 5);
            q[bit >> 6] |= (u64)1 << (bit & 63);
        }
    }
    memcpy(MU, q, sizeof MU);
    READY = 1;
}

/* 2^256 mod p, for the Montgomery conversions */
static fp r_mod_p(void) {
    u64 x[8] = {0, 0, 0, 0, 1, 0, 0, 0};
    return barrett(x);
}

/* ---------------------------------------------------------------- affine group law */

typedef struct { fp x, y; int inf; } aff;

static aff aff_inf(void) { aff p; p.x = fp_zero(); p.y = fp_zero(); p.inf = 1; return p; }

static int aff_on_curve(aff p) {
    if (p.inf) return 1;
    fp lhs = fp_mul(p.y, p.y);
    fp rhs = fp_add(fp_mul(fp_mul(p.x, p.x), p.x), fp_small(3));
    return fp_eq(lhs, rhs);
}

static aff aff_double(aff p) {
    if (p.inf || fp_is_zero(p.y)) return aff_inf();
    /* lambda = 3 x^2 / (2 y) */
    fp num = fp_mul(fp_small(3), fp_mul(p.x, p.x));
    fp lam = fp_mul(num, fp_inv(fp_add(p.y, p.y)));
    aff r;
    r.inf = 0;
    r.x = fp_sub(fp_mul(lam, lam), fp_add(p.x, p.x));
    r.y = fp_sub(fp_mul(lam, fp_sub(p.x, r.x)), p.y);
    return r;
}

static aff aff_add(aff p, aff q) {
    if (p.inf) return q;
    if (q.inf) return p;
    if (fp_eq(p.x, q.x)) {
        if (fp_eq(p.y, q.y)) return aff_double(p);
        return aff_inf();   /* q = -p */
    }
    /* lambda = (y2 - y1) / (x2 - x1) */
    fp lam = fp_mul(fp_sub(q.y, p.y), fp_inv(fp_sub(q.x, p.x)));
    aff r;
    r.inf = 0;
    r.x = fp_sub(fp_sub(fp_mul(lam, lam), p.x), q.x);
    r.y = fp_sub(fp_mul(lam, fp_sub(p.x, r.x)), p.y);
    return r;
}

/* ---------------------------------------------------------------- Jacobian */

typedef struct { fp X, Y, Z; } jac;   /* (X/Z^2, Y/Z^3); Z = 0 is infinity */

static jac jac_inf(void) { jac p; p.X = fp_small(1); p.Y = fp_small(1); p.Z = fp_zero(); return p; }

static jac jac_from_aff(aff a) {
    if (a.inf) return jac_inf();
    jac p;
    p.X = a.x;
    p.Y = a.y;
    p.Z = fp_small(1);
    return p;
}

static aff jac_to_aff(jac p) {
    if (fp_is_zero(p.Z)) return aff_inf();
    fp zi = fp_inv(p.Z);
    fp zi2 = fp_mul(zi, zi);
    aff a;
    a.inf = 0;
    a.x = fp_mul(p.X, zi2);
    a.y = fp_mul(p.Y, fp_mul(zi2, zi));
    return a;
}

/* a = 0: S = 4 X Y^2, M = 3 X^2, X' = M^2 - 2 S, Y' = M (S - X') - 8 Y^4, Z' = 2 Y Z */
static jac jac_double(jac p) {
    if (fp_is_zero(p.Z) || fp_is_zero(p.Y)) return jac_inf();
    fp yy = fp_mul(p.Y, p.Y);
    fp s = fp_mul(fp_small(4), fp_mul(p.X, yy));
    fp m = fp_mul(fp_small(3), fp_mul(p.X, p.X));
    jac r;
    r.X = fp_sub(fp_mul(m, m), fp_add(s, s));
    r.Y = fp_sub(fp_mul(m, fp_sub(s, r.X)), fp_mul(fp_small(8), fp_mul(yy, yy)));
    r.Z = fp_mul(fp_small(2), fp_mul(p.Y, p.Z));
    return r;
}

/* U1 = X1 Z2^2, U2 = X2 Z1^2, S1 = Y1 Z2^3, S2 = Y2 Z1^3, H = U2 - U1, R = S2 - S1,
 * X3 = R^2 - H^3 - 2 U1 H^2, Y3 = R (U1 H^2 - X3) - S1 H^3, Z3 = H Z1 Z2 */
static jac jac_add(jac p, jac q) {
    if (fp_is_zero(p.Z)) return q;
    if (fp_is_zero(q.Z)) return p;
    fp z1z1 = fp_mul(p.Z, p.Z), z2z2 = fp_mul(q.Z, q.Z);
    fp u1 = fp_mul(p.X, z2z2), u2 = fp_mul(q.X, z1z1);
    fp s1 = fp_mul(p.Y, fp_mul(z2z2, q.Z)), s2 = fp_mul(q.Y, fp_mul(z1z1, p.Z));
    fp h = fp_sub(u2, u1), rr = fp_sub(s2, s1);
    if (fp_is_zero(h)) {
        if (fp_is_zero(rr)) return jac_double(p);
        return jac_inf();
    }
    fp hh = fp_mul(h, h), hhh = fp_mul(hh, h), u1hh = fp_mul(u1, hh);
    jac r;
    r.X = fp_sub(fp_sub(fp_mul(rr, rr), hhh), fp_add(u1hh, u1hh));
    r.Y = fp_sub(fp_mul(rr, fp_sub(u1hh, r.X)), fp_mul(s1, hhh));
    r.Z = fp_mul(h, fp_mul(p.Z, q.Z));
    return r;
}

/* k P, left to right over the 256 bits of k */
static jac jac_mul(jac p, const u64 k[4]) {
    jac acc = jac_inf();
    for (int bit = 255; bit >= 0; --bit) {
        acc = jac_double(acc);
        if ((k[bit >> 6] >> (bit & 63)) & 1u) acc = jac_add(acc, p);
    }
    return acc;
}

/* ---------------------------------------------------------------- I/O */

static fp load_fp(const uint32_t* w) {
    fp a;
    for (int i = 0; i < 4; ++i) a.v[i] = (u64)w[2 * i] | ((u64)w[2 * i + 1] << 32);
    return a;
}

static void store_fp(uint32_t* w, fp a) {
    for (int i = 0; i < 4; ++i) {
        w[2 * i] = (uint32_t)a.v[i];
        w[2 * i + 1] = (uint32_t)(a.v[i] >> 32);
    }
}

static aff load_aff(const uint32_t* w) {
    aff a;
    a.x = load_fp(w);
    a.y = load_fp(w + 8);
    a.inf = fp_is_zero(a.x) && fp_is_zero(a.y);
    return a;
}

static void store_aff(uint32_t* w, aff a) {
    if (a.inf) {
        memset(w, 0, 64);
        return;
    }
    store_fp(w, a.x);
    store_fp(w + 8, a.y);
}

static int canonical(fp a) { return !ge_n(a.v, PMOD.v, 4); }

static void load_scalar(const uint32_t* w, u64 k[4]) {
    for (int i = 0; i < 4; ++i) k[i] = (u64)w[2 * i] | ((u64)w[2 * i + 1] << 32);
}

/* ---------------------------------------------------------------- entry points */

int msm_oracle_modulus(uint32_t* out8) {
    store_fp(out8, PMOD);
    return 0;
}

/* op: 0 add, 1 sub, 2 mul, 3 inv (b ignored), 4 to Montgomery, 5 from Montgomery */
int msm_oracle_fp_op(int op, size_t n, const uint32_t* a, const uint32_t* b, uint32_t* out) {
    init();
    fp rm = r_mod_p(), rinv = fp_inv(rm);
    for (size_t i = 0; i < n; ++i) {
        fp x = load_fp(a + 8 * i), y = b ? load_fp(b + 8 * i) : fp_zero(), z;
        if (!canonical(x) || !canonical(y)) return 1;
        switch (op) {
            case 0: z = fp_add(x, y); break;
            case 1: z = fp_sub(x, y); break;
            case 2: z = fp_mul(x, y); break;
            case 3: z = fp_inv(x); break;
            case 4: z = fp_mul(x, rm); break;
            case 5: z = fp_mul(x, rinv); break;
            default: return 2;
        }
        store_fp(out + 8 * i, z);
    }
    return 0;
}

/* 1 if every point is on the curve or the point at infinity (canonical coordinates) */
int msm_oracle_on_curve(size_t n, const uint32_t* pts, int* ok) {
    init();
    *ok = 1;
    for (size_t i = 0; i < n; ++i) {
        aff a = load_aff(pts + 16 * i);
        if (!canonical(a.x) || !canonical(a.y) || !aff_on_curve(a)) *ok = 0;
    }
    return 0;
}

/* Affine group law on pairs: op 0: out = a + b, op 1: out = 2 a, op 2: out = -a. */
int msm_oracle_affine_op(int op, size_t n, const uint32_t* a, const uint32_t* b, uint32_t* out) {
    init();
    for (size_t i = 0; i < n; ++i) {
        aff p = load_aff(a + 16 * i), r;
        if (op == 0) r = aff_add(p, load_aff(b + 16 * i));
        else if (op == 1) r = aff_double(p);
        else if (op == 2) { r = p; if (!p.inf) r.y = fp_neg(p.y); }
        else return 2;
        store_aff(out + 16 * i, r);
    }
    return 0;
}

/* The same additions and doublings through Jacobian coordinates. */
int msm_oracle_jacobian_op(int op, size_t n, const uint32_t* a, const uint32_t* b, uint32_t* out) {
    init();
    for (size_t i = 0; i < n; ++i) {
        jac p = jac_from_aff(load_aff(a + 16 * i)), r;
        if (op == 0) r = jac_add(p, jac_from_aff(load_aff(b + 16 * i)));
        else if (op == 1) r = jac_double(p);
        else return 2;
        store_aff(out + 16 * i, jac_to_aff(r));
    }
    return 0;
}

/* out_i = k_i P (P affine; pass the generator (1, 2) for synthetic bases) */
int msm_oracle_scalar_mul(size_t n, const uint32_t* scalars, const uint32_t* point,
                          uint32_t* out) {
    init();
    jac p = jac_from_aff(load_aff(point));
    for (size_t i = 0; i < n; ++i) {
        u64 k[4];
        load_scalar(scalars + 8 * i, k);
        store_aff(out + 16 * i, jac_to_aff(jac_mul(p, k)));
    }
    return 0;
}

/* out = sum_i k_i P_i (the definition, term by term) */
int msm_oracle_msm(size_t n, const uint32_t* scalars, const uint32_t* bases, uint32_t* out) {
    init();
    jac acc = jac_inf();
    for (size_t i = 0; i < n; ++i) {
        u64 k[4];
        load_scalar(scalars + 8 * i, k);
        acc = jac_add(acc, jac_mul(jac_from_aff(load_aff(bases + 16 * i)), k));
    }
    store_aff(out, jac_to_aff(acc));
    return 0;
}
