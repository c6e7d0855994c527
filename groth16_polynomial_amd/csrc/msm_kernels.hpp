// Pippenger multi-scalar multiplication over BN254 G1: sum_i k_i P_i.
//
// The method is the MSM_CU page's (its header sections 1-4 and the kernels' comments):
//   * windows of c bits with signed digits, so a window has 2^(c-1) buckets, one per
//     digit magnitude, and a negative digit adds the negated base;
//   * scalars 0 and 1 never reach a bucket: zeros are skipped and ones are summed by a
//     separate pass, one mixed addition each;
//   * a counting sort by bucket (count, prefix-sum per window, scatter point indices
//     through a cursor), so that no atomic ever touches a point;
//   * load-balanced accumulation: fixed-length slices of the sorted entries, one thread
//     each; a run strictly inside a slice is written to its bucket directly, the first
//     and last run of a slice go to two spill slots, and a merge pass adds each bucket's
//     spills; XYZZ accumulators with affine bases, the arithmetic of every point kernel
//     in nine 29-bit digits (fp29.hpp), which is also the form the point kernels pass
//     to one another (only the bases and the final window sums are canonical);
//   * each window reduced to sum_m m B_m on the device; the host combines the windows
//     by Horner's rule (the page's "THE WINDOW REDUCTION ENDS ON THE HOST").
//
// Differences from the page (see the notes at each kernel): the digits are computed once,
// for all windows of a scalar in one thread (a signed recoding with carries), and stored
// as 16-bit codes; the counting sort runs in two levels (coarse bins of rows, then rows
// within a bin) with all its counters in LDS, so its atomics are LDS atomics and none is
// global; a bucket never written
// is recognised from its count and from the run geometry instead of being cleared first;
// the window reduction is spread over many threads (one per short segment of buckets)
// rather than one block per window; the ones' partial sums are added into window 0.
#pragma once

#include <type_traits>

#include "g1.hpp"
#include "msm_digit.hpp"

namespace g16 {

struct MsmParams {
    uint32_t n;          // scalars and bases
    uint32_t c;          // window width in bits
    uint32_t windows;    // ceil(255 / c)
    uint32_t buckets;    // 2^(c - 1) per window
    uint32_t slice_len;  // sorted entries per accumulation thread
    uint32_t slices;     // ceil(n / slice_len) accumulation threads per window
    uint32_t seg_len;    // buckets per reduction thread
    uint32_t segs;       // buckets / seg_len reduction threads per window
    uint32_t ones_groups;  // workgroups of the ones pass
    uint32_t n_pad;      // n rounded up to a multiple of 8 (a window's codes in 16-byte words)
    uint32_t bins;       // coarse sorting bins per window, a power of two up to buckets
    uint32_t bin_shift;  // log2(buckets / bins): rows per bin
    uint32_t chunk;      // codes per coarse-sorting workgroup, a multiple of 8
    uint32_t chunks;     // ceil(n_pad / chunk) coarse-sorting workgroups per window
    uint32_t stage;      // entries of a bin the row sort keeps in LDS
};

constexpr uint32_t kMsmNoRow = 0xffffffffu;
// A bucket whose run spans more slices than this is merged by a workgroup of its own.
constexpr uint32_t kMsmFatSlices = 8;
constexpr uint32_t kMsmThreads = 256;
constexpr uint32_t kMsmSortThreads = 1024;

__device__ __forceinline__ void msm_load_scalar(const uint32_t* s, uint32_t i, uint32_t k[8]) {
    const uint4* q = reinterpret_cast<const uint4*>(s + 8 * (size_t)i);
    const uint4 a = q[0], b = q[1];
    k[0] = a.x; k[1] = a.y; k[2] = a.z; k[3] = a.w;
    k[4] = b.x; k[5] = b.y; k[6] = b.z; k[7] = b.w;
}

// 0: zero, 1: one, 2: anything else
__device__ __forceinline__ uint32_t msm_scalar_kind(const uint32_t k[8]) {
    uint32_t hi = k[1] | k[2] | k[3] | k[4] | k[5] | k[6] | k[7];
    if (hi) return 2u;
    return k[0] == 0u ? 0u : k[0] == 1u ? 1u : 2u;
}

__device__ __forceinline__ Fp msm_ld_fp(const Fp* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    const uint4 a = q[0], b = q[1];
    Fp x;
    x.w[0] = a.x; x.w[1] = a.y; x.w[2] = a.z; x.w[3] = a.w;
    x.w[4] = b.x; x.w[5] = b.y; x.w[6] = b.z; x.w[7] = b.w;
    return x;
}

__device__ __forceinline__ void msm_st_fp(Fp* p, const Fp& x) {
    uint4* q = reinterpret_cast<uint4*>(p);
    q[0] = make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]);
    q[1] = make_uint4(x.w[4], x.w[5], x.w[6], x.w[7]);
}

__device__ __forceinline__ G1Aff msm_ld_aff(const G1Aff* p) {
    G1Aff a;
    a.x = msm_ld_fp(&p->x);
    a.y = msm_ld_fp(&p->y);
    return a;
}

__device__ __forceinline__ G1Xyzz msm_ld_xyzz(const G1Xyzz* p) {
    G1Xyzz a;
    a.x = msm_ld_fp(&p->x);
    a.y = msm_ld_fp(&p->y);
    a.zz = msm_ld_fp(&p->zz);
    a.zzz = msm_ld_fp(&p->zzz);
    return a;
}

__device__ __forceinline__ void msm_st_xyzz(G1Xyzz* p, const G1Xyzz& a) {
    msm_st_fp(&p->x, a.x);
    msm_st_fp(&p->y, a.y);
    msm_st_fp(&p->zz, a.zz);
    msm_st_fp(&p->zzz, a.zzz);
}

// A point as the point kernels pass it to one another (bucket partials, spills, segment and
// group sums): the nine-digit form itself, 144 bytes (nine 16-byte words), lazily reduced
// (bounds in fp29.hpp: a sum of two such points forms smaller values than a converted
// base does), so neither side converts; infinity stays all-zero digits.  Only the window
// sums handed to the host are canonical.
using P29 = XyzzT<Fp29>;
static_assert(sizeof(P29) == 144, "P29 is nine 16-byte words");

__device__ __forceinline__ P29 msm_ld_p29(const P29* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    P29 a;
    int32_t* o = reinterpret_cast<int32_t*>(&a);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        const uint4 v = q[i];
        o[4 * i] = (int32_t)v.x;
        o[4 * i + 1] = (int32_t)v.y;
        o[4 * i + 2] = (int32_t)v.z;
        o[4 * i + 3] = (int32_t)v.w;
    }
    return a;
}

__device__ __forceinline__ void msm_st_p29(P29* p, const P29& a) {
    uint4* q = reinterpret_cast<uint4*>(p);
    const int32_t* o = reinterpret_cast<const int32_t*>(&a);
#pragma unroll
    for (int i = 0; i < 9; ++i)
        q[i] = make_uint4((uint32_t)o[4 * i], (uint32_t)o[4 * i + 1], (uint32_t)o[4 * i + 2],
                          (uint32_t)o[4 * i + 3]);
}

// Fills a u32 array (the counters start at zero: device memory is never assumed clear).
__global__ void msm_fill_u32(uint32_t* p, uint32_t len, uint32_t v) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < len) p[i] = v;
}

// Counting sort by (window, bucket) in two levels, every counter in LDS: a coarse pass
// moves the entries into bins of consecutive rows (few bins, so each workgroup writes long
// runs), then one workgroup per bin sorts its entries by row within the bin's part of the
// array (small, so its scattered writes stay in the cache).
//
// Pass 1: the digits of every window, one thread per scalar, as 16-bit codes
// codes[w n_pad + i] (msm_digit.hpp); scalars 0 and 1 and the padding indices n .. n_pad - 1
// (whole 16-byte words per window) get the zero digit in every window.
__global__ void __launch_bounds__(kMsmThreads) msm_digits(const uint32_t* scalars, MsmParams mp,
                                                          uint16_t* codes) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= mp.n_pad) return;
    uint32_t k[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (i < mp.n) {
        msm_load_scalar(scalars, i, k);
        if (msm_scalar_kind(k) != 2u)
            for (int j = 0; j < 8; ++j) k[j] = 0u;
    }
    if (mp.c == 16u) {  // msm_recode for c = 16, whose 16 windows are the halves of the words
        uint32_t carry = 0;
#pragma unroll
        for (uint32_t w = 0; w < 16u; ++w) {
            const uint32_t v = ((k[w >> 1] >> (16u * (w & 1u))) & 0xffffu) + carry;
            carry = v > 32768u ? 1u : 0u;
            codes[(size_t)w * mp.n_pad + i] =
                (uint16_t)msm_code((int32_t)v - (int32_t)(carry << 16), 16u);
        }
        return;
    }
    msm_recode(k, mp.c, [&](uint32_t w, int32_t d) {
        codes[(size_t)w * mp.n_pad + i] = (uint16_t)msm_code(d, mp.c);
    });
}

// The coarse order: bin = row >> bin_shift, bins of 2^bin_shift rows, mp.bins per window.
// Passes 2 and 4 run one workgroup per (window, chunk of scalars) over the chunk's codes,
// eight per 16-byte load, in rounds of kMsmRound codes.
constexpr uint32_t kMsmBinThreads = 256;
constexpr uint32_t kMsmRound = 8192;

template <class F>
__device__ __forceinline__ void msm_round_codes(const uint16_t* codes, const MsmParams& mp,
                                                uint32_t w, uint32_t r0, uint32_t r1, F&& f) {
    const uint4* cw = reinterpret_cast<const uint4*>(codes + (size_t)w * mp.n_pad);
    for (uint32_t q = r0 + threadIdx.x; q < r1; q += kMsmBinThreads) {
        const uint4 v = cw[q];
        const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j) {
            uint32_t row, neg;
            if (msm_decode((h[j >> 1] >> (16u * (j & 1u))) & 0xffffu, mp.c, row, neg))
                f(row, 8u * q + j, neg);
        }
    }
}

// The chunk's range of 16-byte code words.
__device__ __forceinline__ void msm_chunk_words(const MsmParams& mp, uint32_t ch, uint32_t& q0,
                                                uint32_t& q1) {
    q0 = ch * (mp.chunk / 8u);
    q1 = q0 + mp.chunk / 8u < mp.n_pad / 8u ? q0 + mp.chunk / 8u : mp.n_pad / 8u;
}

// Index of the count of (window w, bin, chunk): a window's counts run bin by bin, then
// chunk by chunk, the order in which pass 4 fills a window's part of the array.
__device__ __forceinline__ size_t msm_bin_index(const MsmParams& mp, uint32_t w, uint32_t bin,
                                                uint32_t ch) {
    return ((size_t)w * mp.bins + bin) * mp.chunks + ch;
}

// Exclusive scan of x[0 .. len) in LDS by the workgroup's first wave: each lane takes a
// contiguous range, and the range sums are scanned by cross-lane shifts (no barrier
// inside).  f(r, count) sees each element before it is overwritten.  Every thread of the
// workgroup must call it (it ends with a barrier); returns the total to all of them.
template <class F>
__device__ __forceinline__ uint32_t msm_wave_scan(uint32_t* x, uint32_t len, uint32_t base,
                                                  uint32_t* total, F&& f) {
    const uint32_t t = threadIdx.x;
    if (t < 64u) {
        const uint32_t per = (len + 63u) / 64u;
        const uint32_t r0 = t * per < len ? t * per : len;
        const uint32_t r1 = r0 + per < len ? r0 + per : len;
        uint32_t local = 0;
        for (uint32_t r = r0; r < r1; ++r) local += x[r];
        uint32_t inc = local;
#pragma unroll
        for (uint32_t d = 1; d < 64u; d <<= 1) {
            const uint32_t y = __shfl_up(inc, d, 64);
            if (t >= d) inc += y;
        }
        uint32_t run = base + inc - local;
        for (uint32_t r = r0; r < r1; ++r) {
            const uint32_t c = x[r];
            f(r, c);
            x[r] = run;
            run += c;
        }
        if (t == 63u) *total = inc;
    }
    __syncthreads();
    return *total;
}

// Pass 2: the chunk's count of entries in each bin (per-wave counters in LDS, added up).
__global__ void __launch_bounds__(kMsmBinThreads) msm_bin_count(const uint16_t* codes,
                                                                MsmParams mp,
                                                                uint32_t* bin_counts) {
    extern __shared__ uint32_t hist[];  // [wave][bin]
    const uint32_t w = blockIdx.x / mp.chunks, ch = blockIdx.x - w * mp.chunks;
    const uint32_t t = threadIdx.x;
    for (uint32_t b = t; b < 4u * mp.bins; b += kMsmBinThreads) hist[b] = 0u;
    __syncthreads();
    uint32_t* mine = hist + (t >> 6) * mp.bins;
    uint32_t q0, q1;
    msm_chunk_words(mp, ch, q0, q1);
    msm_round_codes(codes, mp, w, q0, q1, [&](uint32_t row, uint32_t, uint32_t) {
        atomicAdd(&mine[row >> mp.bin_shift], 1u);
    });
    __syncthreads();
    for (uint32_t b = t; b < mp.bins; b += kMsmBinThreads)
        bin_counts[msm_bin_index(mp, w, b, ch)] =
            hist[b] + hist[mp.bins + b] + hist[2u * mp.bins + b] + hist[3u * mp.bins + b];
}

// Pass 3: exclusive prefix sum of each window's len counts (the bins' per-wave counts, bin
// by bin), from the window's region start w n in the entry array.  One workgroup per
// window: each thread sums a contiguous range, the range sums are scanned in LDS, then
// each thread writes its range's starts.
__global__ void __launch_bounds__(kMsmSortThreads) msm_scan(const uint32_t* counts, uint32_t len,
                                                            MsmParams mp, uint32_t* cursor,
                                                            uint32_t* fat_count) {
    __shared__ uint32_t sums[kMsmSortThreads];
    const uint32_t w = blockIdx.x, t = threadIdx.x;
    if (w == 0 && t == 0) *fat_count = 0u;  // the merge pass appends to the list again
    const uint32_t per = (len + kMsmSortThreads - 1u) / kMsmSortThreads;
    const uint32_t b0 = t * per;
    const uint32_t b1 = b0 + per < len ? b0 + per : len;
    const uint32_t* cw = counts + (size_t)w * len;
    // When every range is whole 16-byte words (4 | per and len = 1024 per; a window's counts
    // start 16-byte aligned as 4 | len): vector loads, all issued before the sum.
    const bool vec = (per & 3u) == 0u && len == per * kMsmSortThreads;
    uint32_t local = 0;
    if (vec) {
        const uint4* v = (const uint4*)(cw + b0);
        uint4 q[8];
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j)
            if (j < per / 4u) q[j] = v[j];
#pragma unroll
        for (uint32_t j = 0; j < 8; ++j)
            if (j < per / 4u) local += q[j].x + q[j].y + q[j].z + q[j].w;
        for (uint32_t j = 8; j < per / 4u; ++j) {
            const uint4 r = v[j];
            local += r.x + r.y + r.z + r.w;
        }
    } else {
        for (uint32_t b = b0; b < b1; ++b) local += cw[b];
    }
    sums[t] = local;
    __syncthreads();
    // Hillis-Steele inclusive scan; every thread reaches every barrier
    for (uint32_t d = 1; d < kMsmSortThreads; d <<= 1) {
        const uint32_t add = t >= d ? sums[t - d] : 0u;
        __syncthreads();
        sums[t] += add;
        __syncthreads();
    }
    uint32_t run = w * mp.n + sums[t] - local;
    uint32_t* out = cursor + (size_t)w * len;
    if (vec) {
        const uint4* v = (const uint4*)(cw + b0);
        uint4* o = (uint4*)(out + b0);
        for (uint32_t j = 0; j < per / 4u; ++j) {
            const uint4 c = v[j];
            uint4 r;
            r.x = run;
            r.y = r.x + c.x;
            r.z = r.y + c.y;
            r.w = r.z + c.z;
            run = r.w + c.w;
            o[j] = r;
        }
    } else {
        for (uint32_t b = b0; b < b1; ++b) {
            out[b] = run;
            run += cw[b];
        }
    }
}

// Pass 4: the same workgroups move each entry (row, index << 1 | negative) to its bin, a
// round of the chunk at a time: the round's entries are counted per bin, ranked by LDS
// atomics into a buffer in bin order, and written out bin by bin at the bin's next
// global slots, so that consecutive threads write consecutive slots.
__global__ void __launch_bounds__(kMsmBinThreads) msm_bin_place(const uint16_t* codes,
                                                                MsmParams mp,
                                                                const uint32_t* bin_offs,
                                                                uint2* binned) {
    constexpr uint32_t T = kMsmBinThreads;
    extern __shared__ uint2 buf[];  // kMsmRound entries, then three counters per bin
    uint32_t* gcur = reinterpret_cast<uint32_t*>(buf + kMsmRound);  // next global slot
    uint32_t* cur = gcur + mp.bins;                                  // the round's cursor
    uint32_t* lst = cur + mp.bins;                                   // the round's start
    __shared__ uint32_t total_sh;
    const uint32_t w = blockIdx.x / mp.chunks, ch = blockIdx.x - w * mp.chunks;
    const uint32_t t = threadIdx.x;
    const uint32_t base = w * mp.buckets;
    for (uint32_t b = t; b < mp.bins; b += T) gcur[b] = bin_offs[msm_bin_index(mp, w, b, ch)];
    uint32_t q0, q1;
    msm_chunk_words(mp, ch, q0, q1);
    for (uint32_t r0 = q0; r0 < q1; r0 += kMsmRound / 8u) {  // the same rounds in every thread
        const uint32_t r1 = r0 + kMsmRound / 8u < q1 ? r0 + kMsmRound / 8u : q1;
        for (uint32_t b = t; b < mp.bins; b += T) lst[b] = 0u;
        __syncthreads();
        msm_round_codes(codes, mp, w, r0, r1, [&](uint32_t row, uint32_t, uint32_t) {
            atomicAdd(&lst[row >> mp.bin_shift], 1u);
        });
        __syncthreads();
        const uint32_t total =
            msm_wave_scan(lst, mp.bins, 0u, &total_sh, [](uint32_t, uint32_t) {});
        for (uint32_t b = t; b < mp.bins; b += T) cur[b] = lst[b];
        __syncthreads();
        msm_round_codes(codes, mp, w, r0, r1, [&](uint32_t row, uint32_t i, uint32_t neg) {
            buf[atomicAdd(&cur[row >> mp.bin_shift], 1u)] = make_uint2(base + row, (i << 1) | neg);
        });
        __syncthreads();
        for (uint32_t p = t; p < total; p += T) {
            const uint2 x = buf[p];
            const uint32_t b = (x.x - base) >> mp.bin_shift;
            binned[gcur[b] + p - lst[b]] = x;
        }
        __syncthreads();
        for (uint32_t b = t; b < mp.bins; b += T) gcur[b] += cur[b] - lst[b];
        __syncthreads();
    }
}

// Pass 5: one workgroup per (window, bin) sorts the bin's entries by row, from their
// contiguous part of binned into the same part of entries: a count per row in LDS, an
// exclusive scan, then each entry to its row's next slot.  Writes counts[row] and
// cursor[row] (the row's run end) for the bin's rows.  A bin of at most mp.stage entries
// (every bin of uniform scalars) is sorted in LDS: loaded once, ranked into a second
// buffer, and written out in order, so the global writes are contiguous.  A larger bin (as
// equal scalars make) keeps its first mp.stage entries in LDS, reads the rest again and
// writes each entry to its slot.  Each thread loads kMsmSortBatch entries before it uses
// any, so that their loads overlap.
constexpr uint32_t kMsmSortBatch = 8;

__global__ void __launch_bounds__(kMsmSortThreads) msm_bin_sort(const uint2* binned,
                                                                const uint32_t* bin_counts,
                                                                const uint32_t* bin_offs,
                                                                MsmParams mp, uint32_t* counts,
                                                                uint32_t* cursor, uint2* entries) {
    constexpr uint32_t T = kMsmSortThreads, NB = kMsmSortBatch;
    // mp.stage entries as loaded, mp.stage entries in row order, a counter per row
    extern __shared__ uint2 stage[];
    uint2* sorted = stage + mp.stage;
    uint32_t* cnt = reinterpret_cast<uint32_t*>(sorted + mp.stage);
    __shared__ uint32_t total_sh;
    const uint32_t w = blockIdx.x / mp.bins, bin = blockIdx.x - w * mp.bins;
    const uint32_t t = threadIdx.x;
    const uint32_t rows = 1u << mp.bin_shift;
    // the bin's part: from its first chunk's offset to the next bin's (or the window's
    // last entry, the last offset plus the last count)
    const uint32_t start = bin_offs[msm_bin_index(mp, w, bin, 0u)];
    const size_t last = msm_bin_index(mp, w, mp.bins - 1u, mp.chunks - 1u);
    const uint32_t end = bin + 1u < mp.bins ? bin_offs[msm_bin_index(mp, w, bin + 1u, 0u)]
                                            : bin_offs[last] + bin_counts[last];
    const bool in_lds = end - start <= mp.stage;  // the same in every thread
    const uint32_t row0 = w * mp.buckets + bin * rows;
    for (uint32_t r = t; r < rows; r += T) cnt[r] = 0u;
    __syncthreads();
    for (uint32_t e0 = start + t; e0 < end; e0 += NB * T) {
        uint2 x[NB];
#pragma unroll
        for (uint32_t j = 0; j < NB; ++j)
            x[j] = j * T < end - e0 ? binned[e0 + j * T] : make_uint2(kMsmNoRow, 0u);
#pragma unroll
        for (uint32_t j = 0; j < NB; ++j) {
            if (x[j].x == kMsmNoRow) continue;
            atomicAdd(&cnt[x[j].x - row0], 1u);
            const uint32_t k = e0 + j * T - start;
            if (k < mp.stage) stage[k] = x[j];
        }
    }
    __syncthreads();
    // the rows' run starts: relative to the bin in LDS, absolute otherwise
    msm_wave_scan(cnt, rows, in_lds ? 0u : start, &total_sh,
                  [&](uint32_t r, uint32_t c) { counts[row0 + r] = c; });
    if (in_lds) {
        for (uint32_t k = t; k < end - start; k += T) {
            const uint2 x = stage[k];
            sorted[atomicAdd(&cnt[x.x - row0], 1u)] = x;
        }
        __syncthreads();
        for (uint32_t k = t; k < end - start; k += T) entries[start + k] = sorted[k];
        for (uint32_t r = t; r < rows; r += T) cursor[row0 + r] = start + cnt[r];
        return;
    }
    for (uint32_t e0 = start + t; e0 < end; e0 += NB * T) {
        uint2 x[NB];
#pragma unroll
        for (uint32_t j = 0; j < NB; ++j) {
            const uint32_t k = e0 + j * T - start;
            x[j] = j * T >= end - e0 ? make_uint2(kMsmNoRow, 0u)
                   : k < mp.stage   ? stage[k]
                                    : binned[e0 + j * T];
        }
#pragma unroll
        for (uint32_t j = 0; j < NB; ++j)
            if (x[j].x != kMsmNoRow) entries[atomicAdd(&cnt[x[j].x - row0], 1u)] = x[j];
    }
    __syncthreads();
    for (uint32_t r = t; r < rows; r += T) cursor[row0 + r] = cnt[r];
}

// The entries of window w occupy [w n, cursor[last row of w]).
__device__ __forceinline__ uint32_t msm_used(const uint32_t* cursor, const MsmParams& mp,
                                             uint32_t w) {
    return cursor[(size_t)w * mp.buckets + mp.buckets - 1u] - w * mp.n;
}

// Pass 5: one thread per slice of slice_len sorted entries of one window.  A run that
// neither contains the slice's first entry nor reaches its end is complete here and is
// written to its bucket; the first run goes to the head spill slot and the run still
// open at the slice's end to the tail slot (a slice holding one run spills once).
__global__ void __launch_bounds__(kMsmThreads) msm_accumulate(const uint2* entries,
                                                              const G1Aff* bases,
                                                              const uint32_t* cursor, MsmParams mp,
                                                              P29* buckets, P29* spill_pts,
                                                              uint32_t* spill_rows) {
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t w = gid / mp.slices;
    if (w >= mp.windows) return;
    const uint32_t s = gid - w * mp.slices;
    const uint32_t head = 2u * gid, tail = head + 1u;
    spill_rows[head] = kMsmNoRow;
    spill_rows[tail] = kMsmNoRow;
    const uint32_t used = msm_used(cursor, mp, w);
    const uint32_t lo = s * mp.slice_len;
    if (lo >= used) return;
    const uint32_t hi = lo + mp.slice_len < used ? lo + mp.slice_len : used;
    const uint2* ew = entries + (size_t)w * mp.n;
    uint32_t cur = ew[lo].x;
    bool first = true;
    XyzzT<Fp29> acc = xyzz_zero<Fp29>();
    for (uint32_t e = lo; e < hi; ++e) {
        const uint2 ent = ew[e];
        if (ent.x != cur) {
            if (first) {
                spill_rows[head] = cur;
                msm_st_p29(spill_pts + head, acc);
                first = false;
            } else {
                msm_st_p29(buckets + cur, acc);
            }
            acc = xyzz_zero<Fp29>();
            cur = ent.x;
        }
        AffT<Fp29> b = aff_to29(msm_ld_aff(bases + (ent.y >> 1)));
        if (ent.y & 1u) b.y = fp29_neg(b.y);
        acc = xyzz_madd(acc, b);
    }
    const uint32_t slot = first ? head : tail;
    spill_rows[slot] = cur;
    msm_st_p29(spill_pts + slot, acc);
}

// Pass 6: one thread per bucket row with entries.  Starts from the direct write when
// the run lies strictly inside one slice (the accumulation wrote it), else from
// infinity, and adds the spills of the slices the run overlaps.  A run over more than
// kMsmFatSlices slices (many equal digits: repeated scalars, or the few buckets of a
// narrow top window) is appended to a list for msm_merge_fat instead, so that no thread
// adds thousands of spills one after another.
__global__ void __launch_bounds__(kMsmThreads) msm_merge(const uint32_t* counts,
                                                         const uint32_t* cursor,
                                                         const P29* spill_pts,
                                                         const uint32_t* spill_rows, MsmParams mp,
                                                         P29* buckets, uint32_t* fat_count,
                                                         uint32_t* fat_rows) {
    const uint32_t row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= mp.windows * mp.buckets) return;
    const uint32_t cnt = counts[row];
    if (cnt == 0u) return;
    const uint32_t w = row / mp.buckets;
    const uint32_t used = msm_used(cursor, mp, w);
    const uint32_t end = cursor[row] - w * mp.n;
    const uint32_t start = end - cnt;
    const uint32_t k_lo = start / mp.slice_len, k_hi = (end - 1u) / mp.slice_len;
    if (k_hi - k_lo >= kMsmFatSlices) {
        fat_rows[atomicAdd(fat_count, 1u)] = row;
        return;
    }
    const uint32_t slice_lo = k_lo * mp.slice_len;
    const uint32_t slice_hi = slice_lo + mp.slice_len < used ? slice_lo + mp.slice_len : used;
    const bool direct = k_lo == k_hi && start > slice_lo && end < slice_hi;
    XyzzT<Fp29> acc = direct ? msm_ld_p29(buckets + row) : xyzz_zero<Fp29>();
    for (uint32_t k = k_lo; k <= k_hi; ++k) {
        const uint32_t slot = 2u * (w * mp.slices + k);
        if (spill_rows[slot] == row) acc = xyzz_add(acc, msm_ld_p29(spill_pts + slot));
        if (spill_rows[slot + 1u] == row)
            acc = xyzz_add(acc, msm_ld_p29(spill_pts + slot + 1u));
    }
    msm_st_p29(buckets + row, acc);
}

// Pass 6b: the listed rows, one workgroup at a time (a grid-stride loop over the list,
// whose length every thread reads once before the loop, so all reach every barrier):
// the threads take the run's slices in turn, each adding the spills that carry the row,
// then a tree in LDS over the threads that took one.  Such a run spans at least two
// slices, so the accumulation never wrote its bucket directly.
__global__ void __launch_bounds__(kMsmThreads) msm_merge_fat(const uint32_t* counts,
                                                             const uint32_t* cursor,
                                                             const P29* spill_pts,
                                                             const uint32_t* spill_rows,
                                                             MsmParams mp,
                                                             const uint32_t* fat_count,
                                                             const uint32_t* fat_rows,
                                                             P29* buckets) {
    __shared__ XyzzT<Fp29> sh[kMsmThreads];
    const uint32_t t = threadIdx.x;
    const uint32_t listed = *fat_count;
    for (uint32_t i = blockIdx.x; i < listed; i += gridDim.x) {
        const uint32_t row = fat_rows[i];
        const uint32_t w = row / mp.buckets;
        const uint32_t end = cursor[row] - w * mp.n;
        const uint32_t start = end - counts[row];
        const uint32_t k_lo = start / mp.slice_len, k_hi = (end - 1u) / mp.slice_len;
        XyzzT<Fp29> acc = xyzz_zero<Fp29>();
        for (uint32_t k = k_lo + t; k <= k_hi; k += kMsmThreads) {
            const uint32_t slot = 2u * (w * mp.slices + k);
            if (spill_rows[slot] == row) acc = xyzz_add(acc, msm_ld_p29(spill_pts + slot));
            if (spill_rows[slot + 1u] == row)
                acc = xyzz_add(acc, msm_ld_p29(spill_pts + slot + 1u));
        }
        sh[t] = acc;
        // the tree spans the threads that took a slice (the same bound in every thread)
        const uint32_t used = k_hi - k_lo + 1u < kMsmThreads ? k_hi - k_lo + 1u : kMsmThreads;
        uint32_t top = 1;
        while (top < used) top *= 2;
        for (uint32_t s = top / 2; s > 0; s >>= 1) {
            __syncthreads();
            if (t < s) sh[t] = xyzz_add(sh[t], sh[t + s]);
        }
        __syncthreads();
        if (t == 0) msm_st_p29(buckets + row, sh[0]);
        __syncthreads();  // sh is reused by the next listed row
    }
}

// Pass 7: the window sum sum_m m B_m, bucket j holding magnitude m = j + 1.  One thread
// per segment [lo, lo + seg_len) of a window's buckets: the running sum from the top
// gives T = sum_j (j - lo + 1) B_j and Q = sum_j B_j, and the segment contributes
// T + lo Q.  Buckets with no entries are infinity (never read).
__global__ void __launch_bounds__(kMsmThreads) msm_reduce_segments(const uint32_t* counts,
                                                                   const P29* buckets,
                                                                   MsmParams mp, P29* seg_out) {
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t w = gid / mp.segs;
    if (w >= mp.windows) return;
    const uint32_t lo = (gid - w * mp.segs) * mp.seg_len;
    const size_t base = (size_t)w * mp.buckets;
    XyzzT<Fp29> run = xyzz_zero<Fp29>(), tot = xyzz_zero<Fp29>();
    for (uint32_t j = lo + mp.seg_len; j-- > lo;) {
        if (counts[base + j]) run = xyzz_add(run, msm_ld_p29(buckets + base + j));
        tot = xyzz_add(tot, run);
    }
    if (lo) tot = xyzz_add(tot, xyzz_mul_small(run, lo));
    msm_st_p29(seg_out + gid, tot);
}

// The scalar-one pass: sum of the bases whose scalar is exactly 1, strided over the
// scalars, then a tree in LDS; one partial sum per workgroup.
__global__ void __launch_bounds__(kMsmThreads) msm_ones(const uint32_t* scalars,
                                                        const G1Aff* bases, MsmParams mp,
                                                        P29* out) {
    __shared__ XyzzT<Fp29> sh[kMsmThreads];
    const uint32_t t = threadIdx.x;
    XyzzT<Fp29> acc = xyzz_zero<Fp29>();
    for (uint32_t i = blockIdx.x * kMsmThreads + t; i < mp.n; i += mp.ones_groups * kMsmThreads) {
        uint32_t k[8];
        msm_load_scalar(scalars, i, k);
        if (msm_scalar_kind(k) == 1u) acc = xyzz_madd(acc, aff_to29(msm_ld_aff(bases + i)));
    }
    sh[t] = acc;
    for (uint32_t s = kMsmThreads / 2; s > 0; s >>= 1) {
        __syncthreads();
        if (t < s) sh[t] = xyzz_add(sh[t], sh[t + s]);
    }
    if (t == 0) msm_st_p29(out + blockIdx.x, sh[0]);
}

// Pass 8: group sums.  Workgroup g adds in[g per, (g + 1) per) (and, for g = 0, the
// n_extra points of extra) into out[g], a tree in LDS after a strided serial sum.  Run
// twice: the segments' contributions into a few partials per window, then the partials
// (and the ones' sums, into window 0) into the window sums.
template <class Out>
__global__ void __launch_bounds__(kMsmThreads) msm_sum_groups(const P29* in, uint32_t per,
                                                              const P29* extra, uint32_t n_extra,
                                                              Out* out) {
    __shared__ XyzzT<Fp29> sh[kMsmThreads];
    const uint32_t g = blockIdx.x, t = threadIdx.x;
    XyzzT<Fp29> acc = xyzz_zero<Fp29>();
    for (uint32_t s = t; s < per; s += kMsmThreads)
        acc = xyzz_add(acc, msm_ld_p29(in + (size_t)g * per + s));
    if (g == 0)
        for (uint32_t e = t; e < n_extra; e += kMsmThreads)
            acc = xyzz_add(acc, msm_ld_p29(extra + e));
    sh[t] = acc;
    for (uint32_t s = kMsmThreads / 2; s > 0; s >>= 1) {
        __syncthreads();
        if (t < s) sh[t] = xyzz_add(sh[t], sh[t + s]);
    }
    if (t == 0) {
        if constexpr (std::is_same<Out, G1Xyzz>::value)  // the window sums: canonical
            msm_st_xyzz(out + g, xyzz_from29(sh[0]));
        else
            msm_st_p29(out + g, sh[0]);
    }
}

// Synthetic bases and fixed-base multiples: out_i = k_i G in affine Montgomery form, one
// thread each (left-to-right double and add over the 256 bits, one inversion at the end).
__global__ void __launch_bounds__(kMsmThreads) g1_generator_mul(const uint32_t* scalars,
                                                                uint32_t n, G1Aff* out) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    uint32_t k[8];
    msm_load_scalar(scalars, i, k);
    const AffT<Fp29> g = aff_to29(g1_generator());
    XyzzT<Fp29> acc = xyzz_zero<Fp29>();
    for (int bit = 255; bit >= 0; --bit) {
        acc = xyzz_dbl(acc);
        if ((k[bit >> 5] >> (bit & 31)) & 1u) acc = xyzz_madd(acc, g);
    }
    const G1Aff a = xyzz_to_aff(acc);
    msm_st_fp(&out[i].x, a.x);
    msm_st_fp(&out[i].y, a.y);
}

}  // namespace g16
