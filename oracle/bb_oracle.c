/*
 * CPU oracle for the BabyBear NTT (the Reed-Solomon encoding step of WHIR proving).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark load this library.  It shares no code, header, table or constant with
 * the GPU library: p is written out below, everything else is derived from it here.
 *
 * What is computed, and where the pages define it (the forum post "GPU-Accelerated
 * WHIR Proving on Apple Silicon"):
 *   - the field: BabyBear, p = 2^31 - 2^27 + 1, elements held by the prover in
 *     Montgomery form (section 2, and section 3.4 on Montgomery multiplication);
 *   - the transform: the number-theoretic transform that evaluates a polynomial on the
 *     2^L-th roots of unity, in natural order in and out (section 3.2: the NTT stages
 *     followed by the bit-reversal permutation, which that pipeline folds into its last
 *     stage);
 *   - the low-degree extension: a polynomial of 2^(L - rate) coefficients, zero-padded
 *     and evaluated on 2^L points (the "rate" of the page's benchmark grids, the inverse
 *     code rate being 2^rate);
 *   - a batch of columns: the coefficients as a row-major matrix of 2^lw columns, each
 *     column one polynomial (the page's "fold" parameter groups coefficients this way).
 *
 * Readings where the page is silent (each stated in the design notes):
 *   - the root: g = 31, the smallest generator of the multiplicative group, found here
 *     by testing (p - 1) / q for q in {2, 3, 5}; omega_{2^27} = g^((p-1)/2^27) and
 *     omega_{2^L} = omega_{2^27}^(2^(27-L));
 *   - Montgomery radix R = 2^32, elements stored as 32-bit little-endian words < p.
 *
 * Arithmetic is deliberately plain: standard-form residues in 64-bit integers, every
 * product reduced with the % operator.  The transform is the textbook radix-2
 * decimation in time: bit-reverse the input by swaps, then passes half = 1, 2, ...,
 * n/2 with butterfly j of a block using the root's power j * n / (2 half) from a
 * natural-order table built by repeated multiplication.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef uint64_t u64;
typedef uint32_t u32;

static const u64 P = 2013265921ULL;  /* 2^31 - 2^27 + 1 */

static u64 add_p(u64 a, u64 b) { return (a + b) % P; }
static u64 sub_p(u64 a, u64 b) { return (a + P - b) % P; }
static u64 mul_p(u64 a, u64 b) { return (a * b) % P; }

static u64 pow_p(u64 a, u64 e) {
    u64 r = 1 % P;
    a %= P;
    while (e) {
        if (e & 1) r = mul_p(r, a);
        a = mul_p(a, a);
        e >>= 1;
    }
    return r;
}

static u64 inv_p(u64 a) { return pow_p(a, P - 2); }   /* Fermat; a != 0 */

/* 2^32 mod p and its inverse: Montgomery conversions */
static u64 r_mod_p(void) { return ((u64)1 << 32) % P; }
static u64 R_INV = 0;  /* (2^32)^-1 mod p, set on first use */

static u64 to_mont(u64 x) { return mul_p(x, r_mod_p()); }
static u64 from_mont(u64 y) {
    if (!R_INV) R_INV = inv_p(r_mod_p());
    return mul_p(y, R_INV);
}

/* The smallest g whose order is p - 1 = 2^27 * 3 * 5. */
static u64 generator(void) {
    const u64 q[3] = {2, 3, 5};
    for (u64 g = 2;; ++g) {
        int ok = 1;
        for (int i = 0; i < 3; ++i)
            if (pow_p(g, (P - 1) / q[i]) == 1) ok = 0;
        if (ok) return g;
    }
}

/* A primitive 2^L-th root of unity (L in [0, 27]). */
static u64 root_of_unity(unsigned L) {
    u64 w = pow_p(generator(), (P - 1) >> 27);
    for (unsigned i = L; i < 27; ++i) w = mul_p(w, w);
    return w;
}

static size_t bitrev(size_t i, unsigned L) {
    size_t r = 0;
    for (unsigned b = 0; b < L; ++b) r |= ((i >> b) & 1) << (L - 1 - b);
    return r;
}

/* x_i <- sum_j x_j w^(i j), w = root (forward) in place, standard form, n = 2^L. */
static void dit(u64* x, unsigned L, u64 root) {
    size_t n = (size_t)1 << L;
    if (n == 1) return;
    size_t nt = n / 2;
    u64* tw = (u64*)malloc(sizeof(u64) * nt);
    tw[0] = 1;
    for (size_t j = 1; j < nt; ++j) tw[j] = mul_p(tw[j - 1], root);
    for (size_t i = 0; i < n; ++i) {
        size_t j = bitrev(i, L);
        if (j > i) { u64 t = x[i]; x[i] = x[j]; x[j] = t; }
    }
    for (size_t half = 1; half < n; half *= 2) {
        size_t step = n / (2 * half);
        for (size_t start = 0; start < n; start += 2 * half) {
            for (size_t j = 0; j < half; ++j) {
                u64 u = x[start + j];
                u64 v = mul_p(x[start + j + half], tw[j * step]);
                x[start + j] = add_p(u, v);
                x[start + j + half] = sub_p(u, v);
            }
        }
    }
    free(tw);
}

/* ================================================================ exported API
 * Element arrays are u32 words.  Return 0 on success, -1 on bad arguments. */

int bb_oracle_modulus(u32* out) { *out = (u32)P; return 0; }

int bb_oracle_generator(u32* out) { *out = (u32)generator(); return 0; }

/* omega (a primitive 2^L-th root) and n^-1, standard form */
int bb_oracle_roots(unsigned L, u32* omega, u32* size_inv) {
    if (L > 27) return -1;
    *omega = (u32)root_of_unity(L);
    *size_inv = (u32)inv_p((u64)1 << L);
    return 0;
}

/* op: 0 add, 1 sub, 2 mul, standard form, element-wise */
int bb_oracle_field_op(int op, size_t n, const u32* a, const u32* b, u32* out) {
    for (size_t i = 0; i < n; ++i) {
        if (a[i] >= P || b[i] >= P) return -1;
        u64 z = op == 0 ? add_p(a[i], b[i]) : op == 1 ? sub_p(a[i], b[i])
              : op == 2 ? mul_p(a[i], b[i]) : P;
        if (z >= P) return -1;
        out[i] = (u32)z;
    }
    return 0;
}

/* dir 0: standard -> Montgomery, 1: Montgomery -> standard */
int bb_oracle_convert(int dir, size_t n, const u32* in, u32* out) {
    for (size_t i = 0; i < n; ++i) {
        if (in[i] >= P) return -1;
        out[i] = (u32)(dir == 0 ? to_mont(in[i]) : from_mont(in[i]));
    }
    return 0;
}

/* The definition, for small L: y_i = sum_j x_j w^(i j) (inverse: w^-1 and the 1/n
 * factor).  One vector, standard form. */
int bb_oracle_dft_naive(unsigned L, int inverse, const u32* x, u32* y) {
    if (L > 14) return -1;
    size_t n = (size_t)1 << L;
    u64 w = root_of_unity(L);
    if (inverse) w = inv_p(w);
    for (size_t i = 0; i < n; ++i) {
        u64 wi = pow_p(w, i), acc = 0, wij = 1;
        for (size_t j = 0; j < n; ++j) {
            acc = add_p(acc, mul_p(x[j], wij));
            wij = mul_p(wij, wi);
        }
        if (inverse) acc = mul_p(acc, inv_p(n));
        y[i] = (u32)acc;
    }
    return 0;
}

/* The batched low-degree extension, Montgomery in and out.  `count` matrices one after
 * another; each input matrix has 2^log_in rows and 2^lw columns (row-major: element
 * (i, c) at i * 2^lw + c), each output matrix 2^L rows and 2^lw columns.  Column c of
 * an output matrix is the forward transform (inverse = 0) of column c of the input,
 * zero-padded from 2^log_in to 2^L rows; inverse = 1 gives the inverse transform (then
 * log_in must equal L). */
int bb_oracle_ntt(unsigned L, unsigned lw, size_t count, unsigned log_in, int inverse,
                  const u32* in_mont, u32* out_mont) {
    if (L > 27 || lw > 10 || log_in > L || (inverse && log_in != L)) return -1;
    size_t n = (size_t)1 << L, h_in = (size_t)1 << log_in, w = (size_t)1 << lw;
    u64 root = root_of_unity(L);
    if (inverse) root = inv_p(root);
    u64 scale = inverse ? inv_p(n) : 1;
    u64* col = (u64*)malloc(sizeof(u64) * n);
    if (!col) return -1;
    for (size_t v = 0; v < count; ++v) {
        const u32* src = in_mont + v * h_in * w;
        u32* dst = out_mont + v * n * w;
        for (size_t c = 0; c < w; ++c) {
            for (size_t i = 0; i < n; ++i) {
                if (i < h_in) {
                    u32 y = src[i * w + c];
                    if (y >= P) { free(col); return -1; }
                    col[i] = from_mont(y);
                } else {
                    col[i] = 0;
                }
            }
            dit(col, L, root);
            for (size_t i = 0; i < n; ++i) dst[i * w + c] = (u32)to_mont(mul_p(col[i], scale));
        }
    }
    free(col);
    return 0;
}
