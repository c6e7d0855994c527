// gfx950 kernels of the H-polynomial pipeline.
//
// Transform structure.  A transform of 2^L points runs log n radix-2 passes; pass b
// pairs indices that differ only in bit b.  Passes [s0, s0 + k) touch only bits
// [s0, s0 + k), so they can run together on a "slice": the 2^k indices that agree on
// all other bits (the NTT_CU page, "BATCHING" section).  A workgroup loads one or
// more slices, runs the k passes with the data in registers and LDS and writes the
// slices back, so a transform costs one HBM round trip per batch of passes.
//
// Every butterfly is the Cooley-Tukey form (x_lo, x_hi) <- (x_lo + w x_hi,
// x_lo - w x_hi): the product output is small and normalized, so the only growth is the
// limb-wise add or subtract of it, which keeps the 29-bit limb representation of
// fr29.hpp within bounds for three passes between normalizations (the other butterfly,
// (x_lo + x_hi, (x_lo - x_hi) w), adds two unnormalized values and doubles the bound
// each pass).  Two pass orders are used, both exact, so any schedule gives the
// same bits:
//   forward order: bits 0, 1, ..., L-1; bit-reversed input to natural output; the pass
//       on bit b uses w = root^((i mod 2^b) 2^(L-1-b));
//   inverse order: bits L-1, ..., 1, 0; natural input to bit-reversed output; the pass
//       on bit b uses w = root^(2^b bitrev_(L-1-b)(i >> (b+1))).
// (The second splits x mod (X^(2m) - c) into x mod (X^m - sqrt c) and x mod (X^m +
// sqrt c); with the roots visited in bit-reversed order it evaluates at every power of
// the root and leaves the results in bit-reversed positions.)  Both read w from a
// natural-order table of the root's first n/2 powers, i the lower index of the pair.
//
// Pipeline mapping (per vector; the pages fold the bit reversal into the first load,
// here it disappears instead): the inverse transform runs in the inverse order on the
// natural-order input with the powers of omega^-1, leaving coefficients in bit-reversed
// order; the coset shift and 1/n (position p holds coefficient bitrev(p) and needs the
// factor n^-1 s^bitrev(p)) are split by the bits of p (the coset shift, below): the part of bits 0
// and 1, with n^-1, is one multiply by one of four constants; the part of every higher bit
// is folded into the forward twiddles of that bit's pass; the forward transform runs in
// the forward order on that
// bit-reversed vector and produces natural order.  The lowest batch of passes of both
// transforms covers the same contiguous slices, so the end of the inverse, the shift
// and the start of the forward transform share one kernel and one HBM round trip.
#pragma once

#include "fr29.hpp"

namespace g16 {

enum class Mode : int {
    HeadBitrev = 0,  // load src[bitrev(i)] (inverse: src[-bitrev(i)] x kscale), forward [0, k)
    FwdStrided = 1,  // forward-order passes [s0, s0 + k) on slices strided by 2^s0
    InvStrided = 2,  // inverse-order passes s0 + k - 1 down to s0, slices strided by 2^s0
    Fused = 3,       // contiguous slices: inverse passes k-1..0, x kappa[p mod 4], forward 0..k-1
};

struct BatchParams {
    // Vector v of a launch (0 <= v < n_vec) is kind v mod n_kind (A, B, C, or fewer) of
    // proof v / n_kind; proof q's vectors start q * vstride elements after the pointers
    // below, and so do its join inputs and outputs.
    const Fr* src[3];
    Fr* dst[3];
    TwTab tw;             // twiddles of this batch's passes (Fused: the inverse table)
    TwTab tw_fwd;         // Fused only: the forward table
    const Fr* join_a;     // store epilogue H = A' B' - x (join kernels only)
    const Fr* join_b;
    Fr* h_mont;
    Fr* h_std;
    Tw29 kscale;          // HeadBitrev, inverse transform: multiplier applied on load
    TwTab kappa;          // Fused only: four entries, the factor between the transforms
                          // of the elements at positions p = q mod 4 (coset shift below)
    uint32_t log_n;
    uint32_t s0;
    uint32_t k;
    uint32_t log_spw;     // log2 of slices per workgroup (radix-2 kernel)
    uint32_t head_inverse;  // HeadBitrev: the inverse transform (see the head load)
    uint32_t n_vec;       // register-group kernel: number of vectors (grid = groups x n_vec)
    uint32_t n_kind;      // vectors per proof in this launch, 1..3
    uint32_t lazy_out;    // register-group kernel: the output feeds only further transform
                          // batches, so it is stored in [0, 2r) (no final subtraction)
    uint64_t vstride;     // elements from one proof's vectors to the next proof's
};

// Element offset of vector v's proof, and v's kind (index into src / dst).
__device__ __forceinline__ uint64_t proof_offset(const BatchParams& p, uint32_t v,
                                                 uint32_t& kind) {
    const uint32_t q = v / p.n_kind;
    kind = v - q * p.n_kind;
    return (uint64_t)q * p.vstride;
}

__device__ __forceinline__ Fr ld_global(const Fr* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    uint4 lo = q[0];
    uint4 hi = q[1];
    Fr x;
    x.w[0] = lo.x; x.w[1] = lo.y; x.w[2] = lo.z; x.w[3] = lo.w;
    x.w[4] = hi.x; x.w[5] = hi.y; x.w[6] = hi.z; x.w[7] = hi.w;
    return x;
}

__device__ __forceinline__ void st_global(Fr* p, const Fr& x) {
    uint4* q = reinterpret_cast<uint4*>(p);
    q[0] = make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]);
    q[1] = make_uint4(x.w[4], x.w[5], x.w[6], x.w[7]);
}

__device__ __forceinline__ Fr ld_lds(const Fr* p) { return ld_global(p); }
__device__ __forceinline__ void st_lds(Fr* p, const Fr& x) { st_global(p, x); }

// Table entry e: four 16-byte and one 8-byte vector load, one per plane, each a wave-
// uniform plane base plus the lane's 32-bit offset.  The index goes through an opaque zero
// held in a VGPR: an entry every lane of a wave needs would otherwise be read with
// scalar loads into SGPRs, and the compiler lowers a signed 32 x 32-bit multiply-add
// with a sign-extended SGPR operand as four instructions instead of one
// v_mad_i64_i32.
__device__ __forceinline__ Tw29 ld_tw(const TwTab& tab, uint32_t e) {
    uint32_t z;
    asm("v_mov_b32 %0, 0" : "=v"(z));
    // a 32-bit byte offset (tables hold at most 2^27 entries) on wave-uniform plane bases:
    // one address computation per entry, the planes' bases in SGPRs
    const uint32_t off = (e + z) * 16u;
    const char* b0 = reinterpret_cast<const char*>(tab.base);
    const size_t ps = (size_t)tab.stride * 16u;
    const uint4 a = *reinterpret_cast<const uint4*>(b0 + off);
    const uint4 b = *reinterpret_cast<const uint4*>(b0 + ps + off);
    const uint4 c = *reinterpret_cast<const uint4*>(b0 + 2 * ps + off);
    const uint4 d = *reinterpret_cast<const uint4*>(b0 + 3 * ps + off);
    const uint2 e_ = *reinterpret_cast<const uint2*>(b0 + 4 * ps + off);
    Tw29 t;
    t.w[0] = a.x; t.w[1] = a.y; t.w[2] = a.z; t.w[3] = a.w;
    t.w[4] = b.x; t.w[5] = b.y; t.w[6] = b.z; t.w[7] = b.w;
    t.w[8] = c.x; t.wp[0] = c.y; t.wp[1] = c.z; t.wp[2] = c.w;
    t.wp[3] = d.x; t.wp[4] = d.y; t.wp[5] = d.z; t.wp[6] = d.w;
    t.wp[7] = e_.x; t.wp[8] = e_.y; t.pad[0] = 0u; t.pad[1] = 0u;
    return t;
}

// An entry every lane of the wave needs (idx equal in all lanes, which the caller
// guarantees): scalar loads into SGPRs, which the product takes as scalar operands and
// which leave the vector memory path to the lanes' own data.
__device__ __forceinline__ Tw29 ld_tw_uniform(const TwTab& tab, uint32_t idx) {
    typedef const __attribute__((address_space(4))) uint32_t* cptr;
    const uint32_t u = __builtin_amdgcn_readfirstlane(idx);
    uint32_t d[20];
#pragma unroll
    for (int q = 0; q < 5; ++q) {
        cptr part = (cptr)(tab.base + (size_t)q * tab.stride + u);
#pragma unroll
        for (int k = 0; k < 4; ++k) d[4 * q + k] = part[k];
    }
    Tw29 t;
#pragma unroll
    for (int k = 0; k < 9; ++k) t.w[k] = (int32_t)d[k];
#pragma unroll
    for (int k = 0; k < 9; ++k) t.wp[k] = (int32_t)d[9 + k];
    t.pad[0] = t.pad[1] = 0;
    return t;
}

__device__ __forceinline__ uint32_t bitrev_bits(uint32_t x, uint32_t bits) {
    return __builtin_bitreverse32(x) >> (32u - bits);  // bits in [1, 32]
}

// bit reversal over 0..31 bits (0 bits: 0)
__device__ __forceinline__ uint32_t bitrev_w(uint32_t x, uint32_t bits) {
    return bits ? (__builtin_bitreverse32(x) >> (32u - bits)) : 0u;
}

// Twiddle tables are stored by level: level m holds n / 2^(m+1) powers of root^(2^m) at
// offset n - n / 2^m (n - 1 entries in all), so a pass on bit b reads one level.
__device__ __forceinline__ uint32_t level_index(uint32_t log_n, uint32_t m, uint32_t j) {
    return (1u << log_n) - ((1u << log_n) >> m) + j;
}

// Forward order (table of omega): level m serves the pass on bit b = L-1-m and holds the
// 2^b powers omega^(2^m j), j < 2^b.  The pass on global bit b = s0 + t of a batch that
// starts at bit s0, for the pair whose lower element has column `low` (< 2^s0) and local
// index bits below t equal to jm, needs j = low + jm 2^s0 = i mod 2^b.  The level stores
// that entry at position jm + low 2^t (j itself when s0 = 0 or t = 0): the lanes of one
// column of a strided batch, which differ in jm, read consecutive entries.  The table
// builder therefore takes the batch plan (the bits where batches start).
__device__ __forceinline__ uint32_t fwd_tw_exp(uint32_t s0, uint32_t low, uint32_t jm) {
    return low + (jm << s0);
}
__device__ __forceinline__ uint32_t fwd_tw_index(uint32_t log_n, uint32_t s0, uint32_t t,
                                                 uint32_t low, uint32_t jm) {
    return level_index(log_n, log_n - 1u - s0 - t, jm + (low << t));
}

// Inverse order (table of omega^-1, bit-reversed within each level: entry X of level m is
// omega^-(2^m bitrev_(L-1-m)(X))).  The pass on global bit b = s0 + t of a batch of k
// passes needs omega^-(2^b bitrev_(L-1-b)(i >> (b+1))): level b, entry X = i >> (b+1) =
// a + h 2^(k-t-1), for the pair whose lower element has local bits above t equal to a
// and slice row (global bits above the batch) h.  Neighbouring lanes again read
// neighbouring entries.
__device__ __forceinline__ uint32_t inv_tw_exp(uint32_t k, uint32_t t, uint32_t a, uint32_t h) {
    return a + (h << (k - t - 1u));
}
__device__ __forceinline__ uint32_t inv_tw_index(uint32_t log_n, uint32_t s0, uint32_t k,
                                                 uint32_t t, uint32_t a, uint32_t h) {
    return level_index(log_n, s0 + t, inv_tw_exp(k, t, a, h));
}

// Source index of the head's load: bitrev(i) for the forward transform.  The inverse
// transform runs the same forward passes on x[-k mod n]: sum_k x[-k] omega^(jk) =
// sum_k x[k] omega^(-jk).
__device__ __forceinline__ uint32_t head_index(uint64_t i, uint32_t log_n, uint32_t inverse) {
    const uint32_t br = bitrev_bits((uint32_t)i, log_n);
    return inverse ? ((0u - br) & ((1u << log_n) - 1u)) : br;
}

// The coset shift of the H pipeline.  Position p of the bit-reversed coefficient vector
// holds coefficient j = bitrev_L(p), which the shift multiplies by s^j / n; bit b of p
// contributes s^(2^(L-1-b)) to s^j.  A forward-order pass on bit b pairs p (bit b clear)
// with p + 2^b, whose factors differ by sigma_b = s^(2^(L-1-b)) alone, so with every
// element still owing the factor of its bits above the passes done so far,
//   F(p) x_lo + w F(p) sigma_b x_hi  and  F(p) x_lo - w F(p) sigma_b x_hi
// are F(p) times a butterfly with twiddle w sigma_b, and both outputs owe F(p), the factor
// without bit b.  So the shifted forward table holds w sigma_b for the passes on bits
// b >= 2 (after the last pass nothing is owed), and the elements are multiplied before the
// forward transform only by kappa[p mod 4] = n^-1 s^(2^(L-1) p_0 + 2^(L-2) p_1), the part of
// bits 0 and 1 (whose passes keep their twiddles of 1).  One product per element, like a
// table S[p] = n^-1 s^bitrev(p), whose n entries would have to be read from HBM; the four
// kappa entries stay in the caches.

// The H epilogue: h_mont[i] = A'[i] B'[i] - x, h_std[i] = the same without the factor R.
// i counts from the join pointers, proof offset included.  A' and B' may be stored in
// h_mont and h_std themselves: element i is read here before it is written, by this
// thread alone.  The product and the conversion to standard form are radix-2^29 REDCs
// (fr29.hpp); xn has normalized digits (any value fr29_canon takes).
__device__ __forceinline__ void store_h_digits(const BatchParams& p, uint64_t i, const V29& xn) {
    const V29 ab = fr29_mont_mul(fr29_from_fr_shl5(ld_global(p.join_a + i)),
                                 fr29_from_fr(ld_global(p.join_b + i)));
    const Fr h = fr29_canon(fr29_sub(ab, xn));
    st_global(p.h_mont + i, h);
    st_global(p.h_std + i, fr_from_mont29(h));
}
// x canonical
__device__ __forceinline__ void store_h(const BatchParams& p, uint64_t i, const Fr& x) {
    store_h_digits(p, i, fr29_from_fr(x));
}
// x a transform's lazy digits
__device__ __forceinline__ void store_h(const BatchParams& p, uint64_t i, const V29& x) {
    store_h_digits(p, i, fr29_normalize(x));
}

// The same with A' and B' at hand (canonical).
__device__ __forceinline__ void store_h3(const BatchParams& p, uint64_t i, const Fr& a,
                                         const Fr& b, const Fr& x) {
    const V29 ab = fr29_mont_mul(fr29_from_fr_shl5(a), fr29_from_fr(b));
    const Fr h = fr29_canon(fr29_sub(ab, fr29_from_fr(x)));
    st_global(p.h_mont + i, h);
    st_global(p.h_std + i, fr_from_mont29(h));
}

// x w mod r, canonical, for a canonical x and a table entry (radix-2 kernel and
// element-wise use).
__device__ __forceinline__ Fr fr_mul_entry(const Fr& x, const Tw29& t) {
    return fr29_canon(shoup_mul(fr29_from_fr(x), t));
}

// One radix-2 pass over the workgroup's slices in LDS (values canonical).
//   bit t of the local index is flipped; the global bit is s0 + t; slice g0 + sl has
//   column low = (g0 + sl) mod 2^s0 and row h = (g0 + sl) >> s0.
template <bool INV>
__device__ __forceinline__ void lds_pass(Fr* sh, const TwTab& tw, uint32_t log_n, uint32_t s0,
                                         uint32_t k, uint32_t t, uint32_t n_bfly,
                                         uint32_t g0) {
    const uint32_t half_k = 1u << (k - 1u);
    for (uint32_t f = threadIdx.x; f < n_bfly; f += blockDim.x) {
        uint32_t sl = f >> (k - 1u);
        uint32_t bf = f & (half_k - 1u);
        uint32_t jm = bf & ((1u << t) - 1u);
        uint32_t lo = ((bf >> t) << (t + 1u)) | jm;
        uint32_t hi = lo + (1u << t);
        Fr* base = sh + ((size_t)sl << k);
        Fr u = ld_lds(base + lo);
        Fr v = ld_lds(base + hi);
        const uint32_t g = g0 + sl;
        const uint32_t low = g & ((1u << s0) - 1u);
        const uint32_t ex = INV ? inv_tw_exp(k, t, bf >> t, g >> s0) : fwd_tw_exp(s0, low, jm);
        const uint32_t idx = INV ? inv_tw_index(log_n, s0, k, t, bf >> t, g >> s0)
                                 : fwd_tw_index(log_n, s0, t, low, jm);
        // exponent 0 is the twiddle 1, except in the forward passes on bits 2 and up,
        // whose entries may carry the coset shift's factor (sigma_b above)
        Fr vw = (ex == 0u && (INV || s0 + t < 2u)) ? v : fr_mul_entry(v, ld_tw(tw, idx));
        st_lds(base + lo, fr_add(u, vw));
        st_lds(base + hi, fr_sub(u, vw));
    }
    __syncthreads();
}

// Grid: x = number of slice groups (2^(L-k) / spw), y = number of vectors.
// Block: any width; dynamic LDS = spw * 2^k * 32 bytes.
template <Mode M, bool JOIN>
__global__ void __launch_bounds__(256) ntt_batch_kernel(BatchParams p) {
    extern __shared__ uint4 lds_raw[];
    Fr* sh = reinterpret_cast<Fr*>(lds_raw);

    const uint32_t k = p.k;
    const uint32_t s0 = p.s0;
    const uint32_t spw = 1u << p.log_spw;
    const uint32_t slice_len = 1u << k;
    const uint32_t total = spw << k;
    uint32_t kind;
    const uint64_t off = proof_offset(p, blockIdx.y, kind);
    const Fr* src = p.src[kind] + off;
    Fr* dst = p.dst[kind] + off;
    const uint32_t g0 = blockIdx.x << p.log_spw;  // first slice of this workgroup
    const bool strided = (M == Mode::FwdStrided || M == Mode::InvStrided);

    // Global index of local element (sl, m).
    auto gindex = [&](uint32_t sl, uint32_t m) -> uint64_t {
        uint32_t g = g0 + sl;
        uint64_t low = g & ((1u << s0) - 1u);
        uint64_t high = g >> s0;
        return low + (high << (s0 + k)) + ((uint64_t)m << s0);
    };

    // ---- load: adjacent lanes take adjacent columns (strided) or elements (contiguous)
    for (uint32_t e = threadIdx.x; e < total; e += blockDim.x) {
        uint32_t sl, m;
        if (strided) { sl = e & (spw - 1u); m = e >> p.log_spw; }
        else { sl = e >> k; m = e & (slice_len - 1u); }
        uint64_t i = gindex(sl, m);
        Fr x;
        if (M == Mode::HeadBitrev) {
            x = ld_global(src + head_index(i, p.log_n, p.head_inverse));  // caller's, canonical
            if (p.head_inverse) x = fr_mul_entry(x, p.kscale);
        } else {
            x = fr_reduce_once(ld_global(src + i));  // another batch's output: [0, 2r)
        }
        st_lds(sh + ((size_t)sl << k) + m, x);
    }
    __syncthreads();

    const uint32_t n_bfly = spw << (k - 1u);
    if (M == Mode::HeadBitrev || M == Mode::FwdStrided) {
        for (uint32_t t = 0; t < k; ++t) lds_pass<false>(sh, p.tw, p.log_n, s0, k, t, n_bfly, g0);
    } else if (M == Mode::InvStrided) {
        for (uint32_t t = k; t-- > 0;) lds_pass<true>(sh, p.tw, p.log_n, s0, k, t, n_bfly, g0);
    } else {  // Fused
        for (uint32_t t = k; t-- > 0;) lds_pass<true>(sh, p.tw, p.log_n, 0u, k, t, n_bfly, g0);
        for (uint32_t e = threadIdx.x; e < total; e += blockDim.x) {
            uint32_t sl = e >> k, m = e & (slice_len - 1u);
            Fr* q = sh + ((size_t)sl << k) + m;
            st_lds(q, fr_mul_entry(ld_lds(q), ld_tw(p.kappa, (uint32_t)gindex(sl, m) & 3u)));
        }
        __syncthreads();
        for (uint32_t t = 0; t < k; ++t)
            lds_pass<false>(sh, p.tw_fwd, p.log_n, 0u, k, t, n_bfly, g0);
    }

    // ---- store
    for (uint32_t e = threadIdx.x; e < total; e += blockDim.x) {
        uint32_t sl, m;
        if (strided) { sl = e & (spw - 1u); m = e >> p.log_spw; }
        else { sl = e >> k; m = e & (slice_len - 1u); }
        uint64_t i = gindex(sl, m);
        Fr x = ld_lds(sh + ((size_t)sl << k) + m);
        if (JOIN) store_h(p, off + i, x);
        else st_global(dst + i, x);
    }
}

}  // namespace g16

#include "ntt_groups.hpp"
