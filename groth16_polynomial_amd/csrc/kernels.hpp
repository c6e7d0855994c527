// gfx950 kernels of the H-polynomial pipeline.
//
// Transform structure.  A transform of 2^L points runs log n radix-2 passes; pass b
// pairs indices that differ only in bit b.  Passes [s0, s0 + k) touch only bits
// [s0, s0 + k), so they can run together on a "slice": the 2^k indices that agree on
// all other bits (the NTT_CU page, "BATCHING" section).  A workgroup loads one or
// more slices into LDS, runs the k passes with a barrier between them and writes the
// slices back, so a transform costs one HBM round trip per batch of passes.
//
// Two butterfly forms are used (both exact, so any schedule gives identical bits):
//   DIT (Cooley-Tukey): (x_lo, x_hi) <- (x_lo + w x_hi, x_lo - w x_hi), passes in
//       increasing bit order, bit-reversed input to natural output;
//   DIF (Gentleman-Sande): (x_lo, x_hi) <- (x_lo + x_hi, (x_lo - x_hi) w), passes in
//       decreasing bit order, natural input to bit-reversed output.
// In both, the pass on bit b uses w = root^(j n / 2^(b+1)) with j = index mod 2^b, read
// from a natural-order table of the root's first n/2 powers.
//
// Pipeline mapping (per vector; the pages fold the bit reversal into the first load,
// here it disappears instead): the inverse transform runs as DIF on the natural-order
// input, leaving coefficients in bit-reversed order; the coset shift and 1/n become one
// multiply by a table S[p] = n^-1 s^bitrev(p) stored in bit-reversed order; the forward
// transform runs as DIT on that bit-reversed vector and produces natural order.  The
// lowest batch of passes of both transforms covers the same contiguous slices, so the
// end of the inverse, the shift and the start of the forward transform share one
// kernel and one HBM round trip.
#pragma once

#include "fr.hpp"

namespace g16 {

enum class Mode : int {
    HeadBitrev = 0,  // load src[bitrev(i)] (optionally x kscale), DIT passes [0, k)
    DitStrided = 1,  // DIT passes [s0, s0 + k) on slices strided by 2^s0
    DifStrided = 2,  // DIF passes [s0 + k) down to s0 on slices strided by 2^s0
    Fused = 3,       // contiguous slices: DIF passes k-1..0, x S[p], DIT passes 0..k-1
};

struct BatchParams {
    const Fr* src[3];    // per vector (blockIdx.y)
    Fr* dst[3];
    const Fr* tw;        // twiddles of this batch's passes (Fused: the DIF table)
    const Fr* tw_fwd;    // Fused only: the DIT table
    const Fr* scale;     // Fused only: S[p]
    const Fr* join_a;    // store epilogue H = A' B' - x (join kernels only)
    const Fr* join_b;
    Fr* h_mont;
    Fr* h_std;
    Fr kscale;           // HeadBitrev: multiplier applied on load (inverse transform)
    uint32_t log_n;
    uint32_t s0;
    uint32_t k;
    uint32_t log_spw;    // log2 of slices per workgroup
    uint32_t use_kscale;
};

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

__device__ __forceinline__ Fr ld_lds(const Fr* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    uint4 lo = q[0];
    uint4 hi = q[1];
    Fr x;
    x.w[0] = lo.x; x.w[1] = lo.y; x.w[2] = lo.z; x.w[3] = lo.w;
    x.w[4] = hi.x; x.w[5] = hi.y; x.w[6] = hi.z; x.w[7] = hi.w;
    return x;
}

__device__ __forceinline__ void st_lds(Fr* p, const Fr& x) {
    uint4* q = reinterpret_cast<uint4*>(p);
    q[0] = make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]);
    q[1] = make_uint4(x.w[4], x.w[5], x.w[6], x.w[7]);
}

__device__ __forceinline__ uint32_t bitrev_bits(uint32_t x, uint32_t bits) {
    return __builtin_bitreverse32(x) >> (32u - bits);  // bits in [1, 32]
}

// The H epilogue: h_mont[i] = A'[i] B'[i] - x, h_std[i] = the same without the factor R.
__device__ __forceinline__ void store_h(const BatchParams& p, uint64_t i, const Fr& x) {
    Fr h = fr_sub(fr_mul(ld_global(p.join_a + i), ld_global(p.join_b + i)), x);
    st_global(p.h_mont + i, h);
    st_global(p.h_std + i, fr_from_mont(h));
}

// One radix-2 pass over the workgroup's slices in LDS.
//   bit t of the local index is flipped; the global bit is b = s0 + t;
//   slice sl has low part low(sl) (global index bits below s0).
template <bool DIF>
__device__ __forceinline__ void lds_pass(Fr* sh, const Fr* tw, uint32_t log_n, uint32_t s0,
                                         uint32_t k, uint32_t t, uint32_t n_bfly,
                                         uint32_t low_base, uint32_t strided) {
    const uint32_t half_k = 1u << (k - 1u);
    const uint32_t b = s0 + t;
    const uint32_t twshift = log_n - b - 1u;
    for (uint32_t f = threadIdx.x; f < n_bfly; f += blockDim.x) {
        uint32_t sl = f >> (k - 1u);
        uint32_t bf = f & (half_k - 1u);
        uint32_t jm = bf & ((1u << t) - 1u);
        uint32_t lo = ((bf >> t) << (t + 1u)) | jm;
        uint32_t hi = lo + (1u << t);
        Fr* base = sh + ((size_t)sl << k);
        Fr u = ld_lds(base + lo);
        Fr v = ld_lds(base + hi);
        // j = global index mod 2^b: the slice's low bits plus the local bits below t
        uint32_t low = strided ? (low_base + sl) & ((1u << s0) - 1u) : 0u;
        if (b == 0u) {
            // the root^0 = 1 twiddle: no multiply
            st_lds(base + lo, fr_add(u, v));
            st_lds(base + hi, fr_sub(u, v));
        } else {
            Fr w = ld_global(tw + ((size_t)(low + (jm << s0)) << twshift));
            if (DIF) {
                st_lds(base + lo, fr_add(u, v));
                st_lds(base + hi, fr_mul_tab(fr_sub(u, v), w));
            } else {
                Fr vw = fr_mul_tab(v, w);
                st_lds(base + lo, fr_add(u, vw));
                st_lds(base + hi, fr_sub(u, vw));
            }
        }
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
    const Fr* src = p.src[blockIdx.y];
    Fr* dst = p.dst[blockIdx.y];
    // Workgroups are dispatched to the eight XCDs round-robin (workgroup i to XCD i mod 8),
    // and each XCD has its own L2.  Renumber them so that each XCD takes one contiguous
    // run of slice groups: neighbouring slices (strided batches: neighbouring columns,
    // which share 128-byte lines of data and twiddles) and the same slice of all
    // vectors (grid.y) then meet in one L2.
    uint32_t wg = blockIdx.x;
    if ((gridDim.x & 7u) == 0u) wg = (wg & 7u) * (gridDim.x >> 3) + (wg >> 3);
    const uint32_t g0 = wg << p.log_spw;  // first slice of this workgroup
    const bool strided = (M == Mode::DitStrided || M == Mode::DifStrided);

    // Global index of local element (sl, m).
    auto gindex = [&](uint32_t sl, uint32_t m) -> uint64_t {
        if (strided) {
            uint32_t g = g0 + sl;
            uint64_t low = g & ((1u << s0) - 1u);
            uint64_t high = g >> s0;
            return low + (high << (s0 + k)) + ((uint64_t)m << s0);
        }
        return ((uint64_t)(g0 + sl) << k) + m;
    };

    // ---- load: adjacent lanes take adjacent columns (strided) or elements (contiguous)
    for (uint32_t e = threadIdx.x; e < total; e += blockDim.x) {
        uint32_t sl, m;
        if (strided) { sl = e & (spw - 1u); m = e >> p.log_spw; }
        else { sl = e >> k; m = e & (slice_len - 1u); }
        uint64_t i = gindex(sl, m);
        Fr x;
        if (M == Mode::HeadBitrev) {
            x = ld_global(src + bitrev_bits((uint32_t)i, p.log_n));
            if (p.use_kscale) x = fr_mul(x, p.kscale);
        } else {
            x = ld_global(src + i);
        }
        st_lds(sh + ((size_t)sl << k) + m, x);
    }
    __syncthreads();

    const uint32_t n_bfly = spw << (k - 1u);
    if (M == Mode::HeadBitrev || M == Mode::DitStrided) {
        for (uint32_t t = 0; t < k; ++t)
            lds_pass<false>(sh, p.tw, p.log_n, s0, k, t, n_bfly, g0, strided);
    } else if (M == Mode::DifStrided) {
        for (uint32_t t = k; t-- > 0;)
            lds_pass<true>(sh, p.tw, p.log_n, s0, k, t, n_bfly, g0, strided);
    } else {  // Fused
        for (uint32_t t = k; t-- > 0;)
            lds_pass<true>(sh, p.tw, p.log_n, 0u, k, t, n_bfly, 0u, 0u);
        for (uint32_t e = threadIdx.x; e < total; e += blockDim.x) {
            uint32_t sl = e >> k, m = e & (slice_len - 1u);
            Fr* q = sh + ((size_t)sl << k) + m;
            st_lds(q, fr_mul_tab(ld_lds(q), ld_global(p.scale + gindex(sl, m))));
        }
        __syncthreads();
        for (uint32_t t = 0; t < k; ++t)
            lds_pass<false>(sh, p.tw_fwd, p.log_n, 0u, k, t, n_bfly, 0u, 0u);
    }

    // ---- store
    for (uint32_t e = threadIdx.x; e < total; e += blockDim.x) {
        uint32_t sl, m;
        if (strided) { sl = e & (spw - 1u); m = e >> p.log_spw; }
        else { sl = e >> k; m = e & (slice_len - 1u); }
        uint64_t i = gindex(sl, m);
        Fr x = ld_lds(sh + ((size_t)sl << k) + m);
        if (JOIN) store_h(p, i, x);
        else st_global(dst + i, x);
    }
}

}  // namespace g16

#include "ntt_r8.hpp"

namespace g16 {

}  // namespace g16
