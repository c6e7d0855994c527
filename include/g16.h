/*
 * g16.h -- C ABI of libg16.so, the MI355X (gfx950) Groth16 H-polynomial library.
 *
 * What it computes (the pages this follows are the snarkrs-gpu-kernels docs pages
 * NTT_CU, POINTWISE_CU and GATHER_CU):
 *   stage 0  A, B = CSR row dot products with the witness, C = A o B
 *            (GATHER_CU, kernel description and "WHY C IS COMPUTED HERE");
 *   stage 1  three inverse NTTs of A, B, C (evaluations on the n-th roots of unity
 *            to coefficients), normalised by 1/n (NTT_CU, "THE ALGORITHM IS THE CPU
 *            BACKEND'S, EXACTLY", first bullet);
 *   stage 2  the coset shift x_j *= s^j with s a primitive 2n-th root (same section,
 *            second bullet);
 *   stage 3  three forward NTTs (the coset evaluations A', B', C');
 *   stage 4  H = A' * B' - C' with no division by the vanishing polynomial, written
 *            in Montgomery form and in standard form (POINTWISE_CU, "NO DIVISION BY
 *            Z(coset)" and "TWO OUTPUT BUFFERS").
 *
 * Field and layout.  Fr is the BN254 scalar field, r = 0x30644e72e131a029b85045b6
 * 8181585d2833e84879b9709143e1f593f0000001.  An element is 32 bytes: a little-endian
 * 256-bit integer (eight 32-bit words, word 0 least significant; the same bytes as
 * four little-endian 64-bit limbs).  "mont" buffers hold x * 2^256 mod r, "std"
 * buffers hold x itself; both are canonical (< r).  Every vector is n contiguous
 * elements in natural order, n = 2^log_n.
 *
 * Roots (a reading of the pages, which name no element): g = 5, w28 =
 * g^((r-1)/2^28) is a primitive 2^28-th root of unity, the coset shift of a 2^L
 * domain is s = w28^(2^(27-L)) and the domain root is omega = s^2.
 *
 * Memory and streams.  Every pointer argument named *_mont, *_std, a, b, c, h_*,
 * in, out, witness, value_*, row_ptr_*, signal_* or workspace is a DEVICE pointer
 * (HIP, the current device) owned by the caller.  `stream` is a hipStream_t passed as
 * void* (NULL = the null stream).  Calls only ENQUEUE work on `stream`; none of them
 * synchronises, and the caller keeps every buffer alive until that work is done.
 * Device memory is never assumed to be zero: every output element is written.
 *
 * Errors.  Functions return G16_OK (0) or a negative code.  Argument errors are
 * detected on the host before anything is enqueued.  G16_EHIP reports a HIP launch or
 * runtime error seen after enqueueing; the outputs are then unspecified.
 * Preconditions that are NOT checked (they would cost a pass over the data): inputs
 * are canonical (< r).  Out-of-range CSR indices are caught on the device (see
 * g16_gather_abc) and never read out of bounds.
 */
#ifndef G16_H
#define G16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define G16_ABI_VERSION 1u

#define G16_OK        0
#define G16_EINVAL   (-1) /* null pointer, zero or oversized length, wrong context */
#define G16_ERANGE   (-2) /* log_n outside [1, 27] */
#define G16_ENOSPACE (-3) /* workspace smaller than g16_h_workspace_bytes(log_n) */
#define G16_EALIAS   (-4) /* buffers overlap where the call forbids it */
#define G16_EHIP     (-5) /* HIP launch or runtime error */
#define G16_ESTATE   (-6) /* context released or not prepared */

#define G16_MIN_LOG_N 1u
#define G16_MAX_LOG_N 27u /* r - 1 = 2^28 * odd: a primitive 2n-th root exists up to n = 2^27 */

typedef struct g16_ctx g16_ctx; /* opaque host object, owned by the library */

/* G16_ABI_VERSION of the loaded library. */
uint32_t g16_abi_version(void);

/* Static description of a status code (never NULL). */
const char* g16_strerror(int code);

/* Bytes of device workspace g16_h_prepare needs for a 2^log_n domain, or 0 when
 * log_n is out of range.  The workspace holds the resident tables (the powers of omega
 * and of omega^-1 stored by level, n - 1 entries each; the same levels of omega with the
 * coset shift folded into the passes on bits 2 and up, n - 1 entries; and four entries
 * that hold the rest of the shift and n^-1; each entry is 80 bytes: the plain value and
 * its companion floor(w 2^261 / r) in nine 29-bit digits) and three n-element scratch
 * vectors of 32-byte elements: 3 * n * 80 + 3 * n * 32 + 320 bytes, each of the seven
 * sections rounded up to 256 bytes. */
size_t g16_h_workspace_bytes(uint32_t log_n);

/* The pass batching the library uses for a 2^log_n transform when each workgroup
 * batches at most kmax passes: ceil(log_n / kmax) batches of near-equal size, larger
 * ones first (the NTT_CU page, "SHARED MEMORY BUDGET": 18 passes under a cap of 10
 * split 9 + 9, not 10 + 8).  kmax = 0: the library's default, which the environment
 * variable G16_MAX_K in [1, 12] overrides: the same split under a cap of 10, except
 * 2^21, 2^22, 2^23, 2^25 and 2^26, which take the measured plans 6 + 7 + 8, 8 + 6 + 8,
 * 8 + 7 + 8, 10 + 8 + 7 and 10 + 8 + 8 (mostly even batches, no odd one at the top:
 * 1-3% faster there; results do not depend on the plan).  Writes up to `cap` batch sizes, lowest bits first, and returns
 * the number of batches, or a negative code (G16_ERANGE for log_n, G16_EINVAL for
 * kmax > 12 or a NULL ks with cap > 0).  Host only; never touches the GPU. */
int g16_batch_plan(uint32_t log_n, uint32_t kmax, uint32_t* ks, uint32_t cap);

/* Prepares a context for the 2^log_n domain: computes the roots on the host and
 * enqueues on `stream` the kernels that fill the resident tables inside
 * `workspace` (the NTT_CU page: the host builds the tables once at prepare time
 * and leaves them resident).  The workspace (device memory, >= 256-byte aligned,
 * at least g16_h_workspace_bytes(log_n) bytes) stays owned by the caller and must
 * outlive the context.  Work later enqueued on another stream must be ordered after
 * this call by the caller.  On success *out_ctx receives a new context.
 * Settings read from the environment here, once, for the context's lifetime (results
 * never depend on them): G16_MAX_K (see g16_batch_plan), G16_RADIX2 (set: every batch
 * on the radix-2 kernel), G16_NARROW ("1": the register-group kernel's narrow geometry
 * for every launch, "0": never; unset: for launches of at most 3 * 2^18 elements).
 * Errors: G16_EINVAL (null out_ctx or workspace, misaligned workspace),
 * G16_ERANGE, G16_ENOSPACE, G16_EHIP. */
int g16_h_prepare(uint32_t log_n, void* workspace, size_t workspace_bytes, void* stream,
                  g16_ctx** out_ctx);

/* Frees the host context (not the workspace).  G16_EINVAL on NULL. */
int g16_release(g16_ctx* ctx);

/* log2 of the context's domain size, or 0 for NULL. */
uint32_t g16_ctx_log_n(const g16_ctx* ctx);

/* Host copies (32 bytes each, Montgomery form) of the domain root omega, the coset
 * shift s and size_inv = 1/n, so a caller can check the root convention.  Any
 * output pointer may be NULL.  Errors: G16_EINVAL. */
int g16_domain_roots(const g16_ctx* ctx, uint8_t omega_mont[32], uint8_t shift_mont[32],
                     uint8_t size_inv_mont[32]);

/* Forward transform out_i = sum_j in_j omega^(i j), natural order in and out (the
 * NTT_CU page: decimation in time, the bit-reverse permutation folded into the first
 * batch's load).  in == out is allowed; partial overlap is G16_EALIAS.  Uses the
 * context's scratch: calls on one context must not overlap in time. */
int g16_ntt_forward(g16_ctx* ctx, const void* in_mont, void* out_mont, void* stream);

/* Inverse transform out_j = n^-1 sum_i in_i omega^(-i j) (the 1/n folded into the
 * load).  Same aliasing and scratch rules as g16_ntt_forward. */
int g16_ntt_inverse(g16_ctx* ctx, const void* in_mont, void* out_mont, void* stream);

/* Stages 1 to 3 for one vector: out_i = x(s omega^i) where x interpolates `in` on the
 * domain (inverse transform, coset shift, forward transform).  The materialised coset
 * vector lets a caller finish with g16_h_join (the unfused path).  in == out allowed;
 * partial overlap is G16_EALIAS.  Uses the context's scratch. */
int g16_coset_eval(g16_ctx* ctx, const void* in_mont, void* out_mont, void* stream);

/* The whole pipeline, stages 1 to 4: h_mont and h_std receive H_i = A'_i B'_i - C'_i
 * (Montgomery and standard form).  a, b, c are only read.  h_mont and h_std must not
 * overlap each other, the inputs or the workspace (G16_EALIAS).  Uses the context's
 * scratch: calls on one context must not overlap in time. */
int g16_h_compute(g16_ctx* ctx, const void* a_mont, const void* b_mont, const void* c_mont,
                  void* h_mont, void* h_std, void* stream);

/* g16_h_compute for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same results, but the call uses
 * no workspace scratch and allocates nothing.  A' and B' are kept in h_mont and h_std
 * until the join overwrites them; C' goes to a device array of the library's own, of
 * 2^G16_NOALLOC_MAX_LOG_N * 32 bytes (128 MiB), which each device the library runs on
 * holds until the process ends.  Domains above 2^G16_NOALLOC_MAX_LOG_N are refused with
 * G16_ENOSPACE before anything is enqueued.  All calls on one device share that array
 * (it keeps the last call's contents; every element is written before it is read), so
 * calls that overlap in time on one device race, whatever their contexts and streams.
 * Arguments and the other errors as g16_h_compute; G16_EHIP also when the array's
 * device address cannot be resolved. */
#define G16_NOALLOC_MAX_LOG_N 22u
int g16_h_compute_noalloc(g16_ctx* ctx, const void* a_mont, const void* b_mont,
                          const void* c_mont, void* h_mont, void* h_std, void* stream);

/* Several proofs over one domain in one call (the same launches as g16_h_compute,
 * each covering every proof's vectors, so small domains pay the per-launch cost once
 * per batch rather than once per proof; the NTT_CU page's "BATCHING" section counts
 * that cost).  a_mont, b_mont, c_mont, h_mont and h_std each hold n_proofs vectors of
 * n elements back to back: proof q's vector starts at element q * n.  scratch is
 * caller-owned device memory of at least g16_h_batch_scratch_bytes(log_n, n_proofs)
 * bytes (n_proofs * n * 32; that function returns 0 for a log_n outside [1, 27] or a
 * batch over the limits below), whose contents are overwritten.  Results equal
 * g16_h_compute on each proof.  n_proofs == 0 enqueues nothing and returns G16_OK;
 * n_proofs > G16_MAX_PROOFS or n_proofs * n > 2^31 is G16_EINVAL.  h_mont, h_std and
 * scratch must not overlap each other, the inputs or the workspace (G16_EALIAS);
 * G16_ENOSPACE for a short scratch.  The context's own scratch is not used, so batch
 * calls on one context may overlap in time when their buffers are distinct. */
#define G16_MAX_PROOFS 16384u
size_t g16_h_batch_scratch_bytes(uint32_t log_n, uint64_t n_proofs);
int g16_h_compute_batch(g16_ctx* ctx, uint64_t n_proofs, const void* a_mont,
                        const void* b_mont, const void* c_mont, void* h_mont, void* h_std,
                        void* scratch, size_t scratch_bytes, void* stream);

/* g16_h_compute is a fixed sequence of kernel launches ("stages"): the inverse
 * transform's high batches, the fused lowest batch (end of the inverse, coset
 * multiply, start of the forward transform), the forward transform's high batches,
 * and the final batch of C with the join epilogue.  g16_h_stage_count returns their
 * number (2 * number of pass batches; one fewer on small domains, where the final batch
 * of A, B and C is one launch that joins them in LDS), or a negative code for a bad
 * context.
 * g16_h_stage enqueues stage `stage` alone, with g16_h_compute's arguments and
 * checks; enqueueing stages 0 .. count-1 in order on one stream is exactly
 * g16_h_compute.  Lets a caller time or interleave individual kernels.
 * G16_EINVAL for stage >= count. */
int g16_h_stage_count(const g16_ctx* ctx);
int g16_h_stage(g16_ctx* ctx, uint32_t stage, const void* a_mont, const void* b_mont,
                const void* c_mont, void* h_mont, void* h_std, void* stream);

/* Unfused stage 4 on materialised coset vectors: h_mont_i = a_i b_i - c_i and
 * h_std_i = h_mont_i * 2^-256 mod r (the POINTWISE_CU page's standalone join, the
 * reference the fused epilogue is checked against).  n >= 1.  h_mont and h_std must
 * not overlap each other or the inputs. */
int g16_h_join(uint64_t n, const void* a_mont, const void* b_mont, const void* c_mont,
               void* h_mont, void* h_std, void* stream);

/* Stage 0, the CSR gather (the GATHER_CU page): for each row i < n_rows,
 *   out_a[i] = sum_{k in [row_ptr_a[i], row_ptr_a[i+1])} value_a[k] * witness[signal_a[k]]
 *   out_b[i] = the same for B,   out_c[i] = out_a[i] * out_b[i]   (all Montgomery).
 * row_ptr_* hold n_rows + 1 words; signal_* / value_* hold nnz_* entries; witness
 * holds n_witness elements.  A row whose range is not within [0, nnz] or that names a
 * witness index >= n_witness is not read out of bounds: its three outputs are set to
 * the invalid value 2^256 - 1 (all words 0xffffffff), which no canonical element
 * equals.  Outputs must not overlap the inputs or each other. */
int g16_gather_abc(uint64_t n_rows,
                   const uint32_t* row_ptr_a, const uint32_t* signal_a, const void* value_a,
                   uint64_t nnz_a,
                   const uint32_t* row_ptr_b, const uint32_t* signal_b, const void* value_b,
                   uint64_t nnz_b,
                   const void* witness, uint64_t n_witness,
                   void* out_a, void* out_b, void* out_c, void* stream);

/* Element-wise conversions (in == out allowed): standard -> Montgomery, and
 * Montgomery -> standard (the latter is the POINTWISE_CU page's witness conversion
 * for the MSM). */
int g16_to_mont(uint64_t n, const void* in_std, void* out_mont, void* stream);
int g16_from_mont(uint64_t n, const void* in_mont, void* out_std, void* stream);

/* Element-wise product out_i = a_i * b_i (Montgomery in and out; out may equal a or
 * b).  Forms C = A o B for the workloads that start from A and B. */
int g16_fr_mul(uint64_t n, const void* a_mont, const void* b_mont, void* out_mont,
               void* stream);

/* ---------------------------------------------------------------- G1 MSM
 *
 * The multi-scalar multiplication that consumes h_std (the MSM_CU page): the sum over
 * i < n of k_i P_i on BN254 G1, y^2 = x^3 + 3 over the base field p =
 * 0x30644e72e131a029b85045b68181585d97816a916871ca8d3c208c16d87cfd47.  Pippenger with
 * c-bit signed windows (2^(c-1) buckets per window), a counting sort of (window,
 * bucket) entries, load-balanced bucket accumulation in XYZZ coordinates with affine
 * bases, scalars 0 skipped and scalars 1 summed apart (the page's header, sections 1-4).
 *
 * Layouts.  A scalar is an Fr element in STANDARD form (32 bytes, < r; h_std is one).
 * A base is an affine point of 64 bytes: x then y, each a 32-byte little-endian
 * Montgomery-form Fp element (x * 2^256 mod p); (0, 0) stands for the point at infinity.
 * A window sum is an XYZZ point of 128 bytes: X, Y, ZZ, ZZZ (Montgomery), with
 * (x, y) = (X/ZZ, Y/ZZZ) and ZZ = 0 for infinity.  The result is affine in STANDARD form,
 * 64 bytes, (0, 0) for infinity.
 *
 * c = 0 picks the default window width for n (g16_msm_g1_window_bits). */

/* Default window width for n scalars (from 2^10 scalars the fastest width measured at
 * that size, below it a cost model of point additions), and the number of windows
 * ceil(255 / c) (0 for c outside [1, 16]). */
uint32_t g16_msm_g1_window_bits(uint64_t n);
uint32_t g16_msm_g1_window_count(uint32_t c);

/* Device workspace for g16_msm_g1 (digit codes, counters, sorted entries, spills,
 * buckets, partial sums), or 0 when (n, c) is out of range: n >= 1, c in [1, 16] (a
 * window's signed digits take 2^c values, stored as 16-bit codes), windows * n < 2^32. */
size_t g16_msm_g1_workspace_bytes(uint64_t n, uint32_t c);

/* Enqueues the MSM and writes g16_msm_g1_window_count(c) window sums (XYZZ, device)
 * into window_sums; sum_w 2^(c w) window_sums[w] is the result.  scalars_std: n
 * scalars; bases_mont: n bases; workspace: 256-byte aligned, caller-owned, at least
 * g16_msm_g1_workspace_bytes(n, c) bytes, contents overwritten.  n == 0 sets every
 * window sum to infinity.  Errors: G16_EINVAL (null or host pointers, (n, c) out of
 * range, misaligned workspace), G16_ENOSPACE, G16_EALIAS (window_sums or the workspace
 * overlapping an input or each other), G16_EHIP.  Scalars >= 2^254 are not rejected and
 * give a wrong sum. */
int g16_msm_g1(uint64_t n, const void* scalars_std, const void* bases_mont, uint32_t c,
               void* workspace, size_t workspace_bytes, void* window_sums, void* stream);

/* HOST: combines g16_msm_g1_window_count(c) window sums, copied to host memory, by
 * Horner's rule (c doublings per window) into the affine result, standard form.  The
 * MSM_CU page leaves this serial tail to the host. */
int g16_msm_g1_finish(uint32_t c, const void* window_sums_host, void* out_affine_std);

/* out_i = k_i G for the generator G = (1, 2): affine, Montgomery form, one thread per
 * scalar.  Builds synthetic bases (multiples of G stand in for a proving key's points).
 * n >= 1; scalars any 256-bit integers. */
int g16_g1_generator_mul(uint64_t n, const void* scalars_std, void* out_affine_mont,
                         void* stream);

/* ======================================================================================
 * BabyBear transform: the Reed-Solomon encoding step of WHIR proving (the forum post
 * "GPU-Accelerated WHIR Proving on Apple Silicon", sections 2, 3.2 and 3.4).
 *
 * Field: p = 2^31 - 2^27 + 1.  An element is one 32-bit word, canonical (< p), in
 * Montgomery form with R = 2^32 ("mont") or plain ("std").  Roots (a reading; the post
 * names none): 31 generates the multiplicative group and omega_(2^L) = 31^((p-1)/2^L).
 *
 * The transform (g16_bb_lde): `count` matrices one after another, each row-major with
 * 2^log_w columns (element (i, c) at i * 2^log_w + c); an input matrix has 2^log_in rows,
 * an output matrix 2^log_n rows (log_n fixed by the context).  Output column c holds
 * y_i = sum_j x_j omega^(i j), i < 2^log_n, where x is input column c zero-padded to
 * 2^log_n rows: the values of the column's polynomial on the 2^log_n-th roots of unity,
 * natural order, i.e. the low-degree extension at rate 2^-(log_n - log_in).
 * ====================================================================================== */
typedef struct g16_bb_ctx g16_bb_ctx; /* opaque host object, owned by the library */
#define G16_BB_MAX_LOG_N 27u
#define G16_BB_MAX_LOG_W 10u

/* Bytes of device workspace for the twiddle levels of a 2^log_n domain: (2^log_n - 1)
 * entries of 8 bytes (w and its Shoup companion) and the same entries again as 4 bytes
 * (Montgomery form), each table rounded up to 256 bytes; 0 for log_n outside [1, 27]. */
size_t g16_bb_workspace_bytes(uint32_t log_n);

/* The pass batches of a 2^log_n transform (lowest bits first; at most 8 passes each,
 * near-equal, larger first; one batch of log_n for log_n <= 4).  Writes up to `cap` sizes
 * and returns the count, or G16_ERANGE / G16_EINVAL.  Host only. */
int g16_bb_batch_plan(uint32_t log_n, uint32_t* ks, uint32_t cap);

/* Enqueues the twiddle table build into `workspace` (device memory, 256-byte aligned, at
 * least g16_bb_workspace_bytes(log_n) bytes, owned by the caller and kept alive until
 * g16_bb_release) and returns a new context.  Errors: G16_EINVAL (null or misaligned),
 * G16_ERANGE, G16_ENOSPACE, G16_EHIP. */
int g16_bb_prepare(uint32_t log_n, void* workspace, size_t workspace_bytes, void* stream,
                   g16_bb_ctx** out_ctx);

/* Frees the context (not the workspace).  G16_ESTATE for a pointer that is not a live
 * context (never read), G16_EINVAL for NULL. */
int g16_bb_release(g16_bb_ctx* ctx);

/* The batched low-degree extension described above, in_mont -> out_mont (device
 * pointers, count * 2^(log_in + log_w) and count * 2^(log_n + log_w) words).  count == 0
 * enqueues nothing.  Errors: G16_ESTATE (bad context), G16_EINVAL (log_in > log_n,
 * log_w > G16_BB_MAX_LOG_W, log_n + log_w > 30, count > 2^20, null, host or short
 * buffers), G16_EALIAS (input and output overlap, or the output overlaps the
 * workspace), G16_EHIP.  Inputs must be canonical (not checked).  Calls on one context
 * may overlap in time: the context holds only the read-only table. */
int g16_bb_lde(g16_bb_ctx* ctx, uint32_t log_in, uint32_t log_w, uint64_t count,
               const void* in_mont, void* out_mont, void* stream);

/* Element-wise conversions (in == out allowed): plain -> Montgomery and back. */
int g16_bb_to_mont(uint64_t n, const void* in_std, void* out_mont, void* stream);
int g16_bb_from_mont(uint64_t n, const void* in_mont, void* out_std, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* G16_H */
