/*
 * CPU oracle for the Groth16 H-polynomial pipeline over the BN254 scalar field.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  It shares no code, header, table or
 * constant with the GPU library: every constant below is derived here at start-up
 * from the modulus r and the generator 5.
 *
 * Arithmetic is deliberately plain: elements are kept in STANDARD form (the integer
 * in [0, r)) as four 64-bit little-endian limbs; a product is the schoolbook 512-bit
 * product reduced by Barrett's method (Menezes, van Oorschot, Vanstone, Handbook of
 * Applied Cryptography, algorithm 14.42).  Montgomery form (R = 2^256) appears only
 * at the I/O boundary, as a multiplication by R mod r or by its inverse.
 *
 * What is computed, and where the pages define it:
 *   - the transform: the NTT_CU page, section "THE ALGORITHM IS THE CPU BACKEND'S,
 *     EXACTLY": decimation in time, bit-reverse the input, then log n passes with
 *     half = 1, 2, ..., n/2, butterfly j of a block using twiddle j * n / (2 half)
 *     of a natural-order table of the root's powers;
 *   - the inverse transform: the same passes with the inverse root, then every
 *     output times size_inv = 1/n (same page and section, first bullet);
 *   - the coset shift x[j] *= shift^j, shift a primitive 2n-th root (second bullet);
 *   - H = A*B - C pointwise, no division by the vanishing polynomial (the
 *     POINTWISE_CU page, section "NO DIVISION BY Z(coset)");
 *   - the two encodings h_mont and h_std (same page, "TWO OUTPUT BUFFERS");
 *   - the CSR gather and C = A o B (the GATHER_CU page, kernel description and
 *     "WHY C IS COMPUTED HERE AND NOT GATHERED").
 *
 * Threads.  The transform passes, the element-wise loops and the barycentric sums run
 * over a fixed number of threads (oracle_set_threads; 1 by default): each thread takes a
 * contiguous range of the butterflies of one pass, or of the elements, and a pass ends
 * when every thread has finished it.  The butterflies of one pass are independent, so
 * every butterfly computes exactly what it computes single-threaded; only wall time
 * changes.
 *
 * Readings where the pages are silent (each stated in the design notes):
 *   - the primitive root: g = 5, omega_{2^28} = 5^((r-1)/2^28), the coset shift for
 *     a domain of 2^L points is omega_{2^28}^(2^(27-L)) and the domain root is its
 *     square;
 *   - the inverse transform uses the natural-order table of omega^{-1};
 *   - Fr elements are 32-byte little-endian integers (8 x u32 = 4 x u64 words).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef uint64_t u64;
typedef unsigned __int128 u128;

typedef struct { u64 v[4]; } fe;

/* r = 21888242871839275222246405745257275088548364400416034343698204186575808495617 */
static const fe MOD = {{0x43e1f593f0000001ULL, 0x2833e84879b97091ULL,
                        0xb85045b68181585dULL, 0x30644e72e131a029ULL}};

static u64 BARRETT_MU[5];     /* floor(2^512 / r), five limbs */
static fe R_MOD_R;            /* 2^256 mod r */
static fe R_INV;              /* (2^256)^-1 mod r */
static fe ROOT_2_28;          /* 5^((r-1)/2^28), a primitive 2^28-th root of unity */
static int INITIALISED = 0;
static int THREADS = 1;       /* oracle_set_threads */

/* ---------------------------------------------------------------- threads */

typedef void (*range_fn)(void* arg, size_t lo, size_t hi);
typedef struct { range_fn fn; void* arg; size_t lo, hi; } range_task;

static void* range_entry(void* t) {
    range_task* r = (range_task*)t;
    r->fn(r->arg, r->lo, r->hi);
    return NULL;
}

/* fn(arg, lo, hi) over [0, count) split into THREADS contiguous ranges, one per thread;
 * returns when all are done.  Small counts run on the calling thread. */
static void parallel_for(size_t count, range_fn fn, void* arg) {
    int t = THREADS;
    if (t > 256) t = 256;
    if (t <= 1 || count < 1024) { fn(arg, 0, count); return; }
    pthread_t th[256];
    range_task task[256];
    int started[256];
    size_t per = (count + (size_t)t - 1) / (size_t)t;
    for (int i = 0; i < t; ++i) {
        size_t lo = (size_t)i * per < count ? (size_t)i * per : count;
        size_t hi = lo + per < count ? lo + per : count;
        task[i].fn = fn; task[i].arg = arg; task[i].lo = lo; task[i].hi = hi;
        started[i] = 0;
        if (i > 0 && lo < hi) started[i] = pthread_create(&th[i], NULL, range_entry, &task[i]) == 0;
    }
    fn(arg, task[0].lo, task[0].hi);
    for (int i = 1; i < t; ++i) {
        if (started[i]) pthread_join(th[i], NULL);
        else if (task[i].lo < task[i].hi) fn(arg, task[i].lo, task[i].hi);
    }
}

/* ---------------------------------------------------------------- multi-limb helpers */

static int geq_n(const u64* a, const u64* b, int n) {      /* a >= b, n limbs */
    for (int i = n - 1; i >= 0; --i) {
        if (a[i] != b[i]) return a[i] > b[i];
    }
    return 1;
}

static u64 sub_n(u64* out, const u64* a, const u64* b, int n) {   /* out = a - b, returns borrow */
    u64 borrow = 0;
    for (int i = 0; i < n; ++i) {
        u128 d = (u128)a[i] - b[i] - borrow;
        out[i] = (u64)d;
        borrow = (u64)(d >> 64) ? 1 : 0;
    }
    return borrow;
}

static u64 add_n(u64* out, const u64* a, const u64* b, int n) {   /* out = a + b, returns carry */
    u64 carry = 0;
    for (int i = 0; i < n; ++i) {
        u128 s = (u128)a[i] + b[i] + carry;
        out[i] = (u64)s;
        carry = (u64)(s >> 64);
    }
    return carry;
}

/* out[0 .. na+nb) = a * b, schoolbook */
static void mul_n(u64* out, const u64* a, int na, const u64* b, int nb) {
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

/* ---------------------------------------------------------------- field, standard form */

static fe fe_zero(void) { fe z; memset(&z, 0, sizeof z); return z; }
static fe fe_small(u64 x) { fe z = fe_zero(); z.v[0] = x; return z; }

static fe fe_add(fe a, fe b) {
    fe s;
    u64 c = add_n(s.v, a.v, b.v, 4);
    if (c || geq_n(s.v, MOD.v, 4)) sub_n(s.v, s.v, MOD.v, 4);
    return s;
}

static fe fe_sub(fe a, fe b) {
    fe d;
    if (sub_n(d.v, a.v, b.v, 4)) add_n(d.v, d.v, MOD.v, 4);
    return d;
}

/* x: 8 limbs, x < 2^512 with x < r * 2^256 (true for any product of two canonical
 * elements).  Returns x mod r.  HAC 14.42 with base b = 2^64, k = 4. */
static fe barrett_reduce(const u64 x[8]) {
    u64 q2[10], q3[5], r2full[10], r1[5], rr[5];
    /* q1 = floor(x / b^(k-1)) = limbs 3..7 */
    mul_n(q2, x + 3, 5, BARRETT_MU, 5);
    /* q3 = floor(q2 / b^(k+1)) = limbs 5..9 */
    memcpy(q3, q2 + 5, sizeof q3);
    /* r1 = x mod b^(k+1); r2 = q3 * m mod b^(k+1) */
    memcpy(r1, x, sizeof r1);
    mul_n(r2full, q3, 5, MOD.v, 4);     /* 9 limbs used, 10th is zero */
    /* r = r1 - r2 (mod b^(k+1)): the wrap-around of step 3 is implicit */
    sub_n(rr, r1, r2full, 5);
    u64 m5[5] = {MOD.v[0], MOD.v[1], MOD.v[2], MOD.v[3], 0};
    while (geq_n(rr, m5, 5)) sub_n(rr, rr, m5, 5);
    fe out;
    memcpy(out.v, rr, sizeof out.v);
    return out;
}

static fe fe_mul(fe a, fe b) {
    u64 p[8];
    mul_n(p, a.v, 4, b.v, 4);
    return barrett_reduce(p);
}

static fe fe_pow(fe a, const u64 e[4]) {
    fe acc = fe_small(1);
    for (int bit = 255; bit >= 0; --bit) {
        acc = fe_mul(acc, acc);
        if ((e[bit / 64] >> (bit % 64)) & 1) acc = fe_mul(acc, a);
    }
    return acc;
}

static fe fe_inv(fe a) {       /* Fermat: a^(r-2); a must be nonzero */
    u64 e[4];
    u64 two[4] = {2, 0, 0, 0};
    sub_n(e, MOD.v, two, 4);
    return fe_pow(a, e);
}

static int fe_eq(fe a, fe b) { return memcmp(a.v, b.v, sizeof a.v) == 0; }

/* ---------------------------------------------------------------- start-up constants */

static void oracle_init(void) {
    if (INITIALISED) return;
    /* mu = floor(2^512 / r) by binary long division of the single bit 2^512. */
    u64 rem[5] = {0, 0, 0, 0, 0};
    u64 q[9] = {0};
    u64 m5[5] = {MOD.v[0], MOD.v[1], MOD.v[2], MOD.v[3], 0};
    for (int bit = 512; bit >= 0; --bit) {
        /* rem = 2 * rem + (bit == 512) */
        u64 carry = (bit == 512) ? 1 : 0;
        for (int i = 0; i < 5; ++i) {
            u64 nc = rem[i] >> 63;
            rem[i] = (rem[i] << 1) | carry;
            carry = nc;
        }
        if (geq_n(rem, m5, 5)) {
            sub_n(rem, rem, m5, 5);
            q[bit / 64] |= 1ULL << (bit % 64);
        }
    }
    memcpy(BARRETT_MU, q, sizeof BARRETT_MU);

    /* 2^256 mod r by 256 doublings of 1 */
    fe x = fe_small(1);
    for (int i = 0; i < 256; ++i) x = fe_add(x, x);
    R_MOD_R = x;
    R_INV = fe_inv(R_MOD_R);

    /* (r - 1) / 2^28 */
    u64 e[4];
    u64 one[4] = {1, 0, 0, 0};
    sub_n(e, MOD.v, one, 4);
    for (int s = 0; s < 28; ++s) {
        for (int i = 0; i < 4; ++i) e[i] = (e[i] >> 1) | (i < 3 ? (e[i + 1] << 63) : 0);
    }
    ROOT_2_28 = fe_pow(fe_small(5), e);
    INITIALISED = 1;
}

static fe from_mont(fe y) { return fe_mul(y, R_INV); }
static fe to_mont(fe x) { return fe_mul(x, R_MOD_R); }

/* Roots of a domain of 2^L points (L in [1, 27]): the coset shift s (a primitive
 * 2^(L+1)-th root), the domain root omega = s^2 and size_inv = 2^-L. */
static void domain_roots(unsigned L, fe* omega, fe* shift, fe* size_inv) {
    fe s = ROOT_2_28;
    for (unsigned i = 0; i < 27 - L; ++i) s = fe_mul(s, s);
    *shift = s;
    *omega = fe_mul(s, s);
    fe n = fe_small(1);
    for (unsigned i = 0; i < L; ++i) n = fe_add(n, n);
    *size_inv = fe_inv(n);
}

/* ---------------------------------------------------------------- transforms */

static size_t bitrev(size_t i, unsigned L) {
    size_t r = 0;
    for (unsigned b = 0; b < L; ++b) r |= ((i >> b) & 1) << (L - 1 - b);
    return r;
}

/* One pass of the DIT: butterflies b in [lo, hi) of the pass with half-size `half`;
 * butterfly b is position j = b mod half of block b / half. */
typedef struct { fe* x; const fe* tw; size_t half, step; } pass_job;

static void pass_range(void* arg, size_t lo, size_t hi) {
    const pass_job* p = (const pass_job*)arg;
    fe* x = p->x;
    const fe* tw = p->tw;
    size_t half = p->half, step = p->step;
    for (size_t b = lo; b < hi; ++b) {
        size_t start = (b / half) * 2 * half, j = b % half;
        fe u = x[start + j];
        fe v = fe_mul(x[start + j + half], tw[j * step]);
        x[start + j] = fe_add(u, v);
        x[start + j + half] = fe_sub(u, v);
    }
}

/* x[i] *= k for i in [lo, hi) */
typedef struct { fe* x; fe k; } scale_job;

static void scale_range(void* arg, size_t lo, size_t hi) {
    scale_job* p = (scale_job*)arg;
    fe* x = p->x;
    fe size_inv = p->k;
    for (size_t i = lo; i < hi; ++i) x[i] = fe_mul(x[i], size_inv);
}

/* Forward DIT with the CPU backend's order: swap pass, then half = 1, 2, ..., n/2. */
static void dit_in_place(fe* x, unsigned L, fe root) {
    size_t n = (size_t)1 << L;
    if (n == 1) return;
    size_t nt = n / 2;
    fe* tw = (fe*)malloc(sizeof(fe) * nt);
    tw[0] = fe_small(1);
    for (size_t j = 1; j < nt; ++j) tw[j] = fe_mul(tw[j - 1], root);
    for (size_t i = 0; i < n; ++i) {
        size_t j = bitrev(i, L);
        if (j > i) { fe t = x[i]; x[i] = x[j]; x[j] = t; }
    }
    for (size_t half = 1; half < n; half *= 2) {
        pass_job job = {x, tw, half, n / (2 * half)};
        parallel_for(n / 2, pass_range, &job);
    }
    free(tw);
}

static void ntt_std(fe* x, unsigned L) {
    fe omega, shift, size_inv;
    domain_roots(L, &omega, &shift, &size_inv);
    dit_in_place(x, L, omega);
}

static void intt_std(fe* x, unsigned L) {
    fe omega, shift, size_inv;
    domain_roots(L, &omega, &shift, &size_inv);
    dit_in_place(x, L, fe_inv(omega));
    size_t n = (size_t)1 << L;
    scale_job job = {x, size_inv};
    parallel_for(n, scale_range, &job);
}

/* Element-wise conversions of n Montgomery inputs to standard form (dir 1) or of
 * standard-form values to Montgomery outputs (dir 0). */
typedef struct { int dir; const u64* in; u64* out; } convert_job;

static void convert_range(void* arg, size_t lo, size_t hi) {
    convert_job* p = (convert_job*)arg;
    for (size_t i = lo; i < hi; ++i) {
        fe x; memcpy(x.v, p->in + 4 * i, 32);
        fe z = p->dir == 0 ? to_mont(x) : from_mont(x);
        memcpy(p->out + 4 * i, z.v, 32);
    }
}

static void convert_n(int dir, size_t n, const u64* in, u64* out) {
    convert_job job = {dir, in, out};
    parallel_for(n, convert_range, &job);
}

/* ================================================================ exported API
 * Arrays are n elements of 4 x u64 little-endian limbs (the same bytes as 8 x u32).
 * "mont" arguments are Montgomery form (R = 2^256), "std" standard form.  Functions
 * return 0 on success, -1 on bad arguments. */

int oracle_modulus(u64 out[4]) { memcpy(out, MOD.v, 32); return 0; }

/* Threads used by the transforms, the element-wise loops and the barycentric sums
 * (1 .. 256); returns the previous setting. */
int oracle_set_threads(int threads) {
    int prev = THREADS;
    if (threads >= 1 && threads <= 256) THREADS = threads;
    return prev;
}

int oracle_constants(u64 mu[5], u64 r_mod_r[4], u64 root_2_28[4]) {
    oracle_init();
    memcpy(mu, BARRETT_MU, 40);
    memcpy(r_mod_r, R_MOD_R.v, 32);
    memcpy(root_2_28, ROOT_2_28.v, 32);
    return 0;
}

/* op: 0 add, 1 sub, 2 mul (element-wise over n), std form */
int oracle_field_op(int op, size_t n, const u64* a, const u64* b, u64* out) {
    oracle_init();
    for (size_t i = 0; i < n; ++i) {
        fe x, y, z;
        memcpy(x.v, a + 4 * i, 32);
        memcpy(y.v, b + 4 * i, 32);
        if (op == 0) z = fe_add(x, y);
        else if (op == 1) z = fe_sub(x, y);
        else if (op == 2) z = fe_mul(x, y);
        else return -1;
        memcpy(out + 4 * i, z.v, 32);
    }
    return 0;
}

int oracle_pow(const u64 a[4], const u64 e[4], u64 out[4]) {
    oracle_init();
    fe x; memcpy(x.v, a, 32);
    fe z = fe_pow(x, e);
    memcpy(out, z.v, 32);
    return 0;
}

int oracle_inv(const u64 a[4], u64 out[4]) {
    oracle_init();
    fe x; memcpy(x.v, a, 32);
    if (fe_eq(x, fe_zero())) return -1;
    fe z = fe_inv(x);
    memcpy(out, z.v, 32);
    return 0;
}

/* dir: 0 std -> mont, 1 mont -> std */
int oracle_convert(int dir, size_t n, const u64* in, u64* out) {
    oracle_init();
    convert_n(dir, n, in, out);
    return 0;
}

int oracle_domain_roots(unsigned L, u64 omega[4], u64 shift[4], u64 size_inv[4]) {
    if (L < 1 || L > 27) return -1;
    oracle_init();
    fe w, s, si;
    domain_roots(L, &w, &s, &si);
    memcpy(omega, w.v, 32); memcpy(shift, s.v, 32); memcpy(size_inv, si.v, 32);
    return 0;
}

/* Standalone transforms, std form, in place: inverse = 0 forward, 1 inverse. */
int oracle_ntt(unsigned L, int inverse, u64* x) {
    if (L < 1 || L > 27) return -1;
    oracle_init();
    if (inverse) intt_std((fe*)x, L); else ntt_std((fe*)x, L);
    return 0;
}

/* The definition: y_i = sum_j x_j w^(i j), w = omega (forward) or omega^-1 times 1/n
 * on the result (inverse).  O(n^2); for small L only. */
int oracle_dft_naive(unsigned L, int inverse, const u64* x, u64* y) {
    if (L < 1 || L > 16) return -1;
    oracle_init();
    fe omega, shift, size_inv;
    domain_roots(L, &omega, &shift, &size_inv);
    fe w = inverse ? fe_inv(omega) : omega;
    size_t n = (size_t)1 << L;
    const fe* xs = (const fe*)x;
    fe wi = fe_small(1);                       /* w^i */
    for (size_t i = 0; i < n; ++i) {
        fe acc = fe_zero(), wij = fe_small(1); /* w^(i j) */
        for (size_t j = 0; j < n; ++j) {
            acc = fe_add(acc, fe_mul(xs[j], wij));
            wij = fe_mul(wij, wi);
        }
        if (inverse) acc = fe_mul(acc, size_inv);
        memcpy(y + 4 * i, acc.v, 32);
        wi = fe_mul(wi, w);
    }
    return 0;
}

/* The coset shift x_j *= shift^j for j in [lo, hi), the powers by repeated
 * multiplication from shift^lo. */
typedef struct { fe* x; fe shift; } shift_job;

static void shift_range(void* arg, size_t lo, size_t hi) {
    shift_job* p = (shift_job*)arg;
    fe* x = p->x;
    fe shift = p->shift;
    u64 e[4] = {lo, 0, 0, 0};
    fe sj = fe_pow(shift, e);
    for (size_t j = lo; j < hi; ++j) {
        x[j] = fe_mul(x[j], sj);
        sj = fe_mul(sj, shift);
    }
}

/* Stages 1 to 3 on one standard-form vector, in place: the inverse transform, the
 * coset shift x_j *= shift^j, the forward transform. */
static void coset_eval_std(fe* x, unsigned L) {
    size_t n = (size_t)1 << L;
    fe omega, shift, size_inv;
    domain_roots(L, &omega, &shift, &size_inv);
    intt_std(x, L);                              /* stage 1 */
    shift_job job = {x, shift};                  /* stage 2: x_j *= shift^j */
    parallel_for(n, shift_range, &job);
    ntt_std(x, L);                               /* stage 3 */
}

/* One vector's coset evaluations, Montgomery in and out. */
int oracle_coset_eval(unsigned L, const u64* in_mont, u64* out_mont) {
    if (L < 1 || L > 27) return -1;
    oracle_init();
    size_t n = (size_t)1 << L;
    fe* v = (fe*)malloc(sizeof(fe) * n);
    if (!v) return -1;
    convert_n(1, n, in_mont, (u64*)v);
    coset_eval_std(v, L);
    convert_n(0, n, (const u64*)v, out_mont);
    free(v);
    return 0;
}

/* Stage 4 for i in [lo, hi): H = A'B' - C', both encodings. */
typedef struct { fe* v[3]; u64* h_mont; u64* h_std; } join_job;

static void join_range(void* arg, size_t lo, size_t hi) {
    join_job* p = (join_job*)arg;
    fe** v = p->v;
    u64* h_mont = p->h_mont;
    u64* h_std = p->h_std;
    for (size_t i = lo; i < hi; ++i) {
        fe h = fe_sub(fe_mul(v[0][i], v[1][i]), v[2][i]);
        memcpy(h_std + 4 * i, h.v, 32);
        fe hm = to_mont(h);
        memcpy(h_mont + 4 * i, hm.v, 32);
    }
}

/* The H pipeline on Montgomery inputs: three inverse transforms, the coset shift,
 * three forward transforms, H = A'B' - C', written as h_mont and h_std. */
int oracle_h_pipeline(unsigned L, const u64* a_mont, const u64* b_mont, const u64* c_mont,
                      u64* h_mont, u64* h_std) {
    if (L < 1 || L > 27) return -1;
    oracle_init();
    size_t n = (size_t)1 << L;
    const u64* ins[3] = {a_mont, b_mont, c_mont};
    join_job job;
    for (int k = 0; k < 3; ++k) {
        job.v[k] = (fe*)malloc(sizeof(fe) * n);
        if (!job.v[k]) return -1;
        convert_n(1, n, ins[k], (u64*)job.v[k]);
        coset_eval_std(job.v[k], L);             /* stages 1 to 3 */
    }
    job.h_mont = h_mont;                         /* stage 4 */
    job.h_std = h_std;
    parallel_for(n, join_range, &job);
    for (int k = 0; k < 3; ++k) free(job.v[k]);
    return 0;
}

/* H at chosen indices by a different route: the value at x = shift * omega^i of the
 * polynomial interpolating A (and B, C) on the domain, from the barycentric form of
 * the Lagrange basis on the n-th roots of unity,
 *     a(x) = (x^n - 1) / n * sum_j A_j omega^j / (x - omega^j),
 * then H_i = a(x) b(x) - c(x).  O(n) per index.  The sums over j are split into ranges,
 * one per thread; each range inverts its own denominators with one inversion (prefix
 * products, then back substitution), and the ranges' partial sums are added at the end.
 * Inputs Montgomery, outputs both encodings for the chosen indices. */
typedef struct {
    const fe* wj;          /* omega^j, j < n */
    const u64* ins[3];     /* A, B, C, Montgomery */
    fe x;                  /* the evaluation point */
    fe* pre;               /* scratch, n elements */
    fe* part;              /* partial sums, 3 per range */
    size_t per;            /* range length */
} bary_job;

typedef struct { fe* wj; fe omega; } powers_job;

static void powers_range(void* arg, size_t lo, size_t hi) {   /* wj[j] = omega^j */
    fe* wj = ((powers_job*)arg)->wj;
    fe omega = ((powers_job*)arg)->omega;
    u64 e[4] = {lo, 0, 0, 0};
    fe w = fe_pow(omega, e);
    for (size_t j = lo; j < hi; ++j) {
        wj[j] = w;
        w = fe_mul(w, omega);
    }
}

static void bary_range(void* arg, size_t lo, size_t hi) {
    bary_job* p = (bary_job*)arg;
    const fe* wj = p->wj;
    fe* pre = p->pre;
    fe x = p->x;
    fe acc = fe_small(1);                      /* prefix products of (x - omega^j) */
    for (size_t j = lo; j < hi; ++j) {
        acc = fe_mul(acc, fe_sub(x, wj[j]));
        pre[j] = acc;
    }
    fe inv = fe_inv(acc);                      /* 1 / prod over the range */
    fe sum[3] = {fe_zero(), fe_zero(), fe_zero()};
    for (size_t jj = hi; jj-- > lo;) {
        fe inv_d = jj > lo ? fe_mul(inv, pre[jj - 1]) : inv;   /* 1 / (x - omega^j) */
        inv = fe_mul(inv, fe_sub(x, wj[jj]));
        fe weight = fe_mul(wj[jj], inv_d);
        for (int k = 0; k < 3; ++k) {
            fe y; memcpy(y.v, p->ins[k] + 4 * jj, 32);
            sum[k] = fe_add(sum[k], fe_mul(from_mont(y), weight));
        }
    }
    for (int k = 0; k < 3; ++k) p->part[3 * (lo / p->per) + (size_t)k] = sum[k];
}

int oracle_h_at(unsigned L, const u64* a_mont, const u64* b_mont, const u64* c_mont,
                size_t count, const uint32_t* idx, u64* h_mont, u64* h_std) {
    if (L < 1 || L > 27) return -1;
    oracle_init();
    size_t n = (size_t)1 << L;
    for (size_t q = 0; q < count; ++q) if (idx[q] >= n) return -1;
    fe omega, shift, size_inv;
    domain_roots(L, &omega, &shift, &size_inv);
    fe* wj = (fe*)malloc(sizeof(fe) * n);      /* omega^j */
    fe* pre = (fe*)malloc(sizeof(fe) * n);
    fe* part = (fe*)malloc(sizeof(fe) * 3 * 257);
    if (!wj || !pre || !part) { free(wj); free(pre); free(part); return -1; }
    powers_job pw = {wj, omega};
    parallel_for(n, powers_range, &pw);
    /* the same split as parallel_for makes (or one range on the calling thread) */
    size_t ranges = (THREADS > 1 && n >= 1024) ? (size_t)(THREADS > 256 ? 256 : THREADS) : 1;
    bary_job job = {wj, {a_mont, b_mont, c_mont}, fe_zero(), pre, part, (n + ranges - 1) / ranges};
    for (size_t q = 0; q < count; ++q) {
        fe x = fe_mul(shift, wj[idx[q]]);     /* shift * omega^i */
        job.x = x;
        for (size_t t = 0; t < 3 * ranges; ++t) part[t] = fe_zero();
        parallel_for(n, bary_range, &job);
        fe sum[3] = {fe_zero(), fe_zero(), fe_zero()};
        for (size_t t = 0; t < ranges; ++t)
            for (int k = 0; k < 3; ++k) sum[k] = fe_add(sum[k], part[3 * t + (size_t)k]);
        /* (x^n - 1) / n */
        u64 e[4] = {n, 0, 0, 0};
        fe scale = fe_mul(fe_sub(fe_pow(x, e), fe_small(1)), size_inv);
        fe va = fe_mul(sum[0], scale), vb = fe_mul(sum[1], scale), vc = fe_mul(sum[2], scale);
        fe h = fe_sub(fe_mul(va, vb), vc);
        memcpy(h_std + 4 * q, h.v, 32);
        fe hm = to_mont(h);
        memcpy(h_mont + 4 * q, hm.v, 32);
    }
    free(wj); free(pre); free(part);
    return 0;
}

/* Pointwise product out_i = a_i * b_i of Montgomery vectors (Montgomery out). */
typedef struct { const u64* a; const u64* b; u64* out; } product_job;

static void product_range(void* arg, size_t lo, size_t hi) {
    product_job* p = (product_job*)arg;
    for (size_t i = lo; i < hi; ++i) {
        fe x, y;
        memcpy(x.v, p->a + 4 * i, 32);
        memcpy(y.v, p->b + 4 * i, 32);
        fe z = to_mont(fe_mul(from_mont(x), from_mont(y)));
        memcpy(p->out + 4 * i, z.v, 32);
    }
}

int oracle_pointwise_mul_mont(size_t n, const u64* a_mont, const u64* b_mont, u64* out_mont) {
    oracle_init();
    product_job job = {a_mont, b_mont, out_mont};
    parallel_for(n, product_range, &job);
    return 0;
}

/* CSR gather: out_a[row] = sum over the row of value_a[k] * witness[signal_a[k]], the
 * same for B, out_c = out_a * out_b.  Montgomery in and out. */
int oracle_gather(size_t rows, const uint32_t* row_ptr_a, const uint32_t* signal_a,
                  const u64* value_a, const uint32_t* row_ptr_b, const uint32_t* signal_b,
                  const u64* value_b, const u64* witness, size_t n_witness,
                  u64* out_a, u64* out_b, u64* out_c) {
    oracle_init();
    const uint32_t* rp[2] = {row_ptr_a, row_ptr_b};
    const uint32_t* sg[2] = {signal_a, signal_b};
    const u64* vl[2] = {value_a, value_b};
    u64* out[2] = {out_a, out_b};
    for (size_t row = 0; row < rows; ++row) {
        fe acc[2];
        for (int m = 0; m < 2; ++m) {
            acc[m] = fe_zero();
            for (uint32_t k = rp[m][row]; k < rp[m][row + 1]; ++k) {
                if (sg[m][k] >= n_witness) return -1;
                fe v, w;
                memcpy(v.v, vl[m] + 4 * (size_t)k, 32);
                memcpy(w.v, witness + 4 * (size_t)sg[m][k], 32);
                acc[m] = fe_add(acc[m], fe_mul(from_mont(v), from_mont(w)));
            }
            fe am = to_mont(acc[m]);
            memcpy(out[m] + 4 * row, am.v, 32);
        }
        fe c = to_mont(fe_mul(acc[0], acc[1]));
        memcpy(out_c + 4 * row, c.v, 32);
    }
    return 0;
}
