// The BabyBear transform of the Reed-Solomon encoding (the WHIR forum post, section 3.2):
// for each column of a row-major matrix (2^lw columns), the values at the 2^L-th roots of
// unity of the polynomial whose coefficients are the column, zero-padded from 2^log_in to
// 2^L rows.  Natural order in and out.
//
// Index algebra.  A matrix is a flat array: element (row i, column c) at i 2^lw + c.  The
// transform runs radix-2 Cooley-Tukey passes on the row bits 0 .. L-1 (flat bits lw ..
// lw + L - 1) after a bit reversal of the row index: the pass on row bit b pairs rows i
// and i + 2^b (bit b of i clear) as (y_i + t, y_i - t), t = w^(i mod 2^b) y_(i + 2^b),
// w a primitive 2^(b+1)-th root.  Passes [s0, s0 + K) touch only those row bits, so they
// run together on a "slice": the 2^K elements that agree on every other flat bit (the
// column and the row bits outside the batch) - the same (s0, k) algebra as the BN254
// transforms, with the column bits below the row bits.
//
// Geometry.  An element is one 32-bit register, so a thread holds 16 elements of one
// slice and runs four passes on them in registers before exchanging through LDS (radix
// 16; the post's Metal kernels use radix 16 and 32 stages, here they are register groups
// inside an LDS batch of up to 8 passes).  A workgroup holds SPW slices (32 when there
// are enough), and neighbouring lanes take neighbouring slices: in the later batches
// those are neighbouring flat addresses (the slice coordinate below the batch is the
// column plus the lower row bits), so every global access of a wave covers whole 128-byte
// lines.  The first batch reads its input through the bit reversal; its workgroup takes
// its columns (up to 32) times the 32 / columns row blocks whose reversed indices are
// consecutive, so for each element the workgroup's loads are one run of addresses and go
// straight into registers.  Its stores are one run per row block: at 8 or more columns
// they go straight out of registers too, with fewer they are staged through LDS into
// whole rows.  Rows at or past 2^log_in read as zero (the extension's padding) and are
// never loaded.
//
// Twiddles: level b of the table holds w_(2^(b+1))^j for j < 2^b at offset 2^b - 1 (the
// same entries for every domain size), each as (w, floor(w 2^32 / p)), and a second table
// holds the same entries as w 2^32 mod p (4 bytes, a Montgomery product: two more
// instructions, half the bytes; the later batches of matrices of one or two columns read
// this one, since there each entry serves one or two rows' elements only); in a batch at s0
// the pass on row bit b = s0 + t of the pair whose lower element is slice element m needs
// j = (the slice's row bits below s0) + (m mod 2^t) 2^s0, so neighbouring slices read
// neighbouring entries.
#pragma once

#include <type_traits>
#include <utility>

#include "bb_field.hpp"

namespace g16 {

template <typename F, int... I>
__device__ __forceinline__ void bb_static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void bb_static_for(F&& f) {
    bb_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Word i of an array by a 32-bit byte offset on a wave-uniform base (a matrix holds at most
// 2^30 words): one address computation per access, the base in SGPRs.
template <typename T>
__device__ __forceinline__ T& bb_at(T* base, uint32_t i) {
    return *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + i * (uint32_t)sizeof(T));
}
template <typename T>
__device__ __forceinline__ const T& bb_at(const T* base, uint32_t i) {
    return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + i * (uint32_t)sizeof(T));
}

struct BbParams {
    const uint32_t* src;  // input matrices (first batch), else == dst
    uint32_t* dst;
    const uint2* tw;      // levels of (w, w')
    const uint32_t* twm;  // the same levels as w 2^32 mod p
    uint64_t in_stride;   // elements from one input matrix to the next
    uint64_t out_stride;  // elements from one output matrix to the next
    uint32_t log_n;       // L: rows of an output matrix, log2
    uint32_t log_w;       // columns, log2
    uint32_t log_in;      // rows of an input matrix, log2 (<= L)
    uint32_t s0;          // first row bit of the batch
    uint32_t k;           // passes in the batch (4..8; the kernel's K)
    uint32_t log_spw;     // slices per workgroup, log2 (<= 5)
    uint32_t groups;      // workgroups per matrix
};

constexpr int kBbE = 16;  // elements per thread
constexpr int kBbMaxSpw = 32;

__device__ __forceinline__ uint32_t bb_bitrev(uint32_t x, uint32_t bits) {
    return bits ? (__builtin_bitreverse32(x) >> (32u - bits)) : 0u;
}

// c with the r bits of q inserted at bit b0
__device__ __forceinline__ uint32_t bb_insert(uint32_t c, uint32_t q, uint32_t b0, uint32_t r) {
    return (c & ((1u << b0) - 1u)) | (q << b0) | ((c >> b0) << (b0 + r));
}

// Grid: groups * matrices workgroups of (SPW 2^K / 16) threads; LDS (SPW + 1) 2^K words.
// HEAD: the first batch (s0 = 0), staged load through the bit reversal and staged store.
// MONT: products by the 4-byte Montgomery-form table (later batches only).
template <int K, bool HEAD, bool MONT>
__global__ void __launch_bounds__(512) bb_batch_kernel(BbParams p) {
    extern __shared__ uint32_t lds[];
    constexpr uint32_t SLICE = 1u << K;
    constexpr uint32_t U = SLICE / kBbE;  // threads per slice
    const uint32_t spw = 1u << p.log_spw;
    const uint32_t pitch = spw + 1u;       // LDS words per slice element (one spare bank)
    const uint32_t tid = threadIdx.x;
    const uint32_t nthreads = spw * U;
    const uint32_t vec = blockIdx.x / p.groups;
    const uint32_t wg = blockIdx.x - vec * p.groups;
    const uint32_t sl = tid & (spw - 1u);
    const uint32_t u = tid >> p.log_spw;
    const uint32_t L = p.log_n, lw = p.log_w, s0 = p.s0;
    uint32_t* out = p.dst + vec * p.out_stride;

    // ---- the workgroup's slices
    //   later batches: slice index wg * spw + sl; its bits below lw + s0 are `low` (the
    //   column and the row bits below s0), the rest `high` (row bits above the batch)
    //   first batch: columns cb * wc + ci (wc = min(2^lw, spw)) and row blocks
    //   h0 + gi 2^(L - K - lg) (g = spw / wc of them), whose reversed indices are
    //   bitrev(h0) + bitrev_lg(gi)
    uint32_t low_row, base_flat;  // the slice's row bits below s0; flat index of element 0
    uint32_t wc = 0, lg = 0, cb = 0, h0 = 0;
    if constexpr (HEAD) {
        const uint32_t lwc = lw < p.log_spw ? lw : p.log_spw;
        wc = 1u << lwc;
        lg = p.log_spw - lwc;
        const uint32_t col_blocks = 1u << (lw - lwc);
        cb = wg % col_blocks;
        h0 = wg / col_blocks;
        const uint32_t gi = sl >> lwc, ci = sl & (wc - 1u);
        const uint32_t high = h0 + (gi << (L - K - lg));
        low_row = 0u;
        base_flat = ((high << K) << lw) + cb * wc + ci;
    } else {
        const uint32_t s = wg * spw + sl;
        const uint32_t lowbits = lw + s0;
        const uint32_t low = s & ((1u << lowbits) - 1u);
        const uint32_t high = s >> lowbits;
        low_row = low >> lw;
        base_flat = low + ((high << (s0 + K)) << lw);
    }
    const uint32_t mstride = 1u << (lw + s0);  // flat distance of consecutive slice elements

    uint32_t x[kBbE];

    // ---- the first batch's source: slice sl = (gi, ci) (row block gi, column ci of the
    // workgroup's wc) holds at element m the input row bitrev_K(m) 2^(L-K) + bitrev(h0) 2^lg
    // + bitrev_lg(gi): for one m the workgroup's slices read 2^lg consecutive rows (in
    // reversed order) of wc consecutive columns, one run of addresses, so group 0 loads
    // its elements straight into registers.
    const uint32_t* head_in = nullptr;
    uint32_t head_row0 = 0u, head_col = 0u;
    // The first batch's output: slice (gi, ci) writes rows (h0 + gi 2^(L-K-lg)) 2^K + m, so
    // for one m the workgroup writes 2^lg runs of wc words.  At 8 or more columns (runs of
    // 32 bytes and up) the last group stores them directly; with fewer, the runs are
    // staged through LDS into whole rows of the row blocks (measured: direct stores were
    // 5% faster at 8 columns, 36-43% slower at 1 or 2).
    const bool head_direct_store = HEAD && wc >= 8u;
    if constexpr (HEAD) {
        const uint32_t lwc = lw < p.log_spw ? lw : p.log_spw;
        head_in = p.src + vec * p.in_stride;
        head_row0 = (bb_bitrev(h0, L - K - lg) << lg) + bb_bitrev(sl >> lwc, lg);
        head_col = cb * wc + (sl & (wc - 1u));
    }

    // ---- passes, in groups of four row bits (the last group may be shorter)
    constexpr int NG = (K + 3) / 4;
    auto group = [&](auto g_c) __attribute__((always_inline)) {
        constexpr int g = decltype(g_c)::value;
        constexpr uint32_t b0 = 4u * g;
        constexpr uint32_t r = (K - 4 * g) < 4 ? (K - 4 * g) : 4;
        constexpr uint32_t nsets = 16u >> r;
        // element e of the thread: set e >> r, position q = e & (2^r - 1)
        auto m_of = [&](uint32_t e) { return bb_insert(u * nsets + (e >> r), e & ((1u << r) - 1u), b0, r); };
        if (g == 0 && HEAD) {
            const uint32_t h_in = 1u << p.log_in;
#pragma unroll
            for (uint32_t e = 0; e < 16; ++e) {
                const uint32_t row = (bb_bitrev(m_of(e), K) << (L - K)) + head_row0;
                x[e] = row < h_in ? bb_at(head_in, (row << lw) + head_col) : 0u;  // padding: 0
            }
        } else if (g == 0) {
#pragma unroll
            for (uint32_t e = 0; e < 16; ++e) x[e] = bb_at(out, base_flat + m_of(e) * mstride);
        } else {
#pragma unroll
            for (uint32_t e = 0; e < 16; ++e) x[e] = lds[m_of(e) * pitch + sl];
        }
#pragma unroll
        for (uint32_t t = 0; t < r; ++t) {
            const uint32_t b = s0 + b0 + t;  // row bit of this pass
            const uint2* level = p.tw + ((1u << b) - 1u);
            const uint32_t* mlevel = p.twm + ((1u << b) - 1u);
#pragma unroll
            for (uint32_t e = 0; e < 16; ++e) {
                if ((e >> t) & 1u) continue;  // e is the upper element of its pair
                const uint32_t hi = e + (1u << t);
                const uint32_t m = m_of(e);
                const uint32_t j = low_row + ((m & ((1u << (b0 + t)) - 1u)) << s0);
                uint32_t tt;
                if constexpr (MONT) {
                    tt = bb_mont_mul(x[hi], bb_at(mlevel, j));
                } else {
                    const uint2 wv = bb_at(level, j);
                    tt = bb_shoup(x[hi], wv.x, wv.y);
                }
                x[hi] = bb_sub(x[e], tt);
                x[e] = bb_add(x[e], tt);
            }
        }
        if (g == NG - 1 && (!HEAD || head_direct_store)) {
#pragma unroll
            for (uint32_t e = 0; e < 16; ++e) bb_at(out, base_flat + m_of(e) * mstride) = x[e];
        } else {
            // a thread writes back exactly the slots it read for this group, so only the
            // next group's reads (or the staged store) wait for the barrier
#pragma unroll
            for (uint32_t e = 0; e < 16; ++e) lds[m_of(e) * pitch + sl] = x[e];
            __syncthreads();
        }
    };
    bb_static_for<NG>(group);

    // ---- staged store of the first batch (fewer than 8 columns): per row block, lanes
    // over consecutive addresses (element m, column ci of block gi at
    // ((high 2^K + m) << lw) + cb wc + ci)
    if (HEAD && !head_direct_store) {
        const uint32_t lwc = lw < p.log_spw ? lw : p.log_spw;
        const uint32_t g = 1u << lg;
        for (uint32_t gi = 0; gi < g; ++gi) {
            const uint32_t high = h0 + (gi << (L - K - lg));
            const uint64_t row0 = (uint64_t)high << K;
            for (uint32_t q = tid; q < SLICE * wc; q += nthreads) {
                const uint32_t m = q >> lwc, ci = q & (wc - 1u);
                bb_at(out, (((uint32_t)row0 + m) << lw) + cb * wc + ci) = lds[m * pitch + (gi << lwc) + ci];
            }
        }
    }
}

// Table entries: level b (0 <= b < L) at offset 2^b - 1 holds (w^j, floor(w^j 2^32 / p))
// in tw and w^j 2^32 mod p in twm, for j < 2^b, w a primitive 2^(b+1)-th root.  One thread
// per entry.
__global__ void bb_table_kernel(uint2* tw, uint32_t* twm, uint32_t log_n) {
    const uint64_t total = (1ull << log_n) - 1u;
    for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t b = 63u - (uint32_t)__builtin_clzll(e + 1u);  // level: 2^b - 1 <= e
        const uint32_t j = (uint32_t)(e + 1u - (1ull << b));
        const uint32_t w = bb_pow_plain(bb_root(b + 1u), j);
        tw[e] = make_uint2(w, bb_shoup_companion(w));
        twm[e] = (uint32_t)(((uint64_t)w << 32) % kBbP);
    }
}

// Element-wise x * m mod p for a fixed multiplier (m, floor(m 2^32 / p)): the conversions
// to Montgomery form (m = 2^32 mod p) and back (m = 2^-32 mod p).
__global__ void bb_scale_kernel(const uint32_t* in, uint32_t* out, uint64_t n, uint32_t m,
                                uint32_t mp) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        out[i] = bb_shoup(in[i], m, mp);
}

// Domains of up to 2^4 points, or fewer than 16 elements per slice: one thread per column
// runs the whole transform (bit-reversed load, radix-2 passes) in registers.
__global__ void bb_small_kernel(BbParams p, uint64_t columns) {
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= columns) return;
    const uint32_t L = p.log_n, lw = p.log_w;
    const uint64_t vec = t >> lw;
    const uint32_t c = (uint32_t)(t & ((1u << lw) - 1u));
    const uint32_t* in = p.src + vec * p.in_stride;
    uint32_t* out = p.dst + vec * p.out_stride;
    const uint32_t n = 1u << L, h_in = 1u << p.log_in;
    uint32_t x[16];
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i) {
        if (i < n) {
            const uint32_t row = bb_bitrev(i, L);
            x[i] = row < h_in ? in[((uint64_t)row << lw) + c] : 0u;
        }
    }
#pragma unroll
    for (uint32_t b = 0; b < 4; ++b) {
        if (b >= L) break;
#pragma unroll
        for (uint32_t i = 0; i < 16; ++i) {
            if (i >= n || ((i >> b) & 1u)) continue;
            const uint2 wv = p.tw[((1u << b) - 1u) + (i & ((1u << b) - 1u))];
            const uint32_t tt = bb_shoup(x[i + (1u << b)], wv.x, wv.y);
            x[i + (1u << b)] = bb_sub(x[i], tt);
            x[i] = bb_add(x[i], tt);
        }
    }
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i)
        if (i < n) out[((uint64_t)i << lw) + c] = x[i];
}

}  // namespace g16
