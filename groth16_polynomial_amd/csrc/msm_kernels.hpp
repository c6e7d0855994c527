// Pippenger multi-scalar multiplication over BN254 G1: sum_i k_i P_i.
//
// The method is the MSM_CU page's (its header sections 1-4 and the kernels' comments):
//   * windows of c bits with signed digits, so a window has 2^(c-1) buckets, one per
//     digit magnitude, and a negative digit adds the negated base;
//   * scalars 0 and 1 never reach a bucket: zeros are skipped and ones are summed by a
//     separate pass, one mixed addition each;
//   * a counting sort by bucket (count, prefix-sum per window, scatter point indices
//     through a cursor), so that no atomic ever touches a point;
//   * load-balanced accumulation: fixed-length runs of the sorted entries per thread, so
//     that a bucket with many entries is shared by several threads and its parts are
//     added afterwards; XYZZ accumulators with affine bases, the arithmetic of every point
//     kernel in nine 29-bit digits (fp29.hpp), which is also the form the point kernels
//     pass to one another (only the bases and the final window sums are canonical);
//   * each window reduced to sum_m m B_m on the device; the host combines the windows
//     by Horner's rule (the page's "THE WINDOW REDUCTION ENDS ON THE HOST").
//
// Differences from the page (see the notes at each kernel): the parts of a bucket shared by
// several threads are joined inside the wave by shuffles and, across waves, by the same
// kernel run again on each wave's two boundary parts (a segmented reduction in levels),
// so there is no per-thread spill and no separate merge pass; the digits are computed once,
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
    uint32_t slice_len;  // sorted entries per lane of the bucket sums' first level
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

// A point as the point kernels pass it to one another (bucket partials, level items, segment and
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
                                                            MsmParams mp, uint32_t* cursor) {
    __shared__ uint32_t sums[kMsmSortThreads];
    const uint32_t w = blockIdx.x, t = threadIdx.x;
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

// Pass 6: the bucket sums, as a segmented reduction over each window's row-sorted items
// (an item is a row and a point: an entry and its signed base at level 0, a partial
// bucket sum at the levels above), in tiles of one wave each.
//
// A tile is 64 lane_len consecutive items of one window; lane l takes lane_len of them
// and adds up each run of equal rows it sees.  A run that begins and ends inside the
// lane's items is a whole bucket and is stored right away.  What is left per lane is
// its first run (which may have begun in lanes to its left) and its last run (which may
// go on in lanes to its right), or one run when all its items share a row.  The wave
// then joins those pieces across lanes by shuffles:
//   * a lane whose items are all one row takes over the sum of the run from the lanes to
//     its left whenever their last row is its row: a segmented inclusive scan over the
//     lanes (steps of 1, 2, 4, ...; the wave stops as soon as no lane still waits), so a
//     run over m lanes costs log2 m additions, and none when no lane is covered by a
//     single run;
//   * every other lane adds its left neighbour's running sum to its first run when the
//     rows match, which completes that run.
// Each completed run is stored to its bucket, except the tile's first and last runs,
// which may continue in the neighbouring tiles: those two go up as the tile's two items
// of the next level (a tile that is one run sends one item and a blank), and the next
// level runs this same kernel on them, with fewer tiles, until a window's items fit in
// one tile and nothing goes up.  Every row with entries is thus stored exactly once, by
// the level and lane where its run is complete; buckets without entries are never
// written (the window sums read the counts).
//
// Items of the levels above the first come two per tile of the level below: the tile's
// first run at index 2t + 1 and its last at 2t + 2 of the window's stride (index 0 and
// the last index are blanks), so that the pair most likely to be one bucket, the last
// run of tile t and the first of tile t + 1, falls on one even-aligned pair and, with an
// even lane_len, inside one lane.  A blank (kMsmNoRow) is skipped by the lanes; blanks
// come from single-run tiles (their second item) and from empty tiles past a window's
// entries, so a lane without any row is never followed by one with rows.
struct MsmLevel {
    uint32_t lane_len;  // items per lane (even above the first level)
    uint32_t tiles;     // tiles per window
    uint32_t stride;    // items per window in the item arrays (level 0: n)
    uint32_t last;      // 1: each window's items fit in one tile; nothing goes up
};

__device__ __forceinline__ P29 msm_shfl_up(const P29& a, uint32_t d) {
    P29 r;
    const int32_t* s = reinterpret_cast<const int32_t*>(&a);
    int32_t* o = reinterpret_cast<int32_t*>(&r);
#pragma unroll
    for (int i = 0; i < 36; ++i) o[i] = __shfl_up(s[i], d, 64);
    return r;
}

template <bool BASES>
__global__ void __launch_bounds__(kMsmThreads, 4) msm_tile_sums(const uint2* entries,
                                                             const G1Aff* bases,
                                                             const uint32_t* in_rows,
                                                             const P29* in_pts,
                                                             const uint32_t* cursor,
                                                             MsmParams mp, MsmLevel lv,
                                                             P29* buckets, uint32_t* out_rows,
                                                             P29* out_pts) {
    __shared__ P29 first_run[kMsmThreads];  // each lane's first run, until the joins
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = (blockIdx.x * kMsmThreads + threadIdx.x) >> 6;
    const uint32_t w = wave / lv.tiles;
    if (w >= mp.windows) return;  // whole waves: the grid is a whole number of waves
    const uint32_t t = wave - w * lv.tiles;
    const uint32_t count = BASES ? msm_used(cursor, mp, w) : lv.stride;
    const uint32_t start = (t * 64u + lane) * lv.lane_len;
    const uint32_t lo = start < count ? start : count;
    const uint32_t hi = lo + lv.lane_len < count ? lo + lv.lane_len : count;
    const size_t base = (size_t)w * lv.stride;

    // ---- the lane's items: runs inside the lane are stored, the first one is kept
    uint32_t first = kMsmNoRow, cur = kMsmNoRow;
    XyzzT<Fp29> acc = xyzz_zero<Fp29>();
    for (uint32_t e = lo; e < hi; ++e) {
        uint32_t row;
        uint2 ent;
        if constexpr (BASES) {
            ent = entries[base + e];
            row = ent.x;
        } else {
            row = in_rows[base + e];
            if (row == kMsmNoRow) continue;
        }
        if (row != cur) {
            if (cur == first && cur != kMsmNoRow) first_run[threadIdx.x] = acc;
            else if (cur != kMsmNoRow) msm_st_p29(buckets + cur, acc);
            if (first == kMsmNoRow) first = row;
            acc = xyzz_zero<Fp29>();
            cur = row;
        }
        if constexpr (BASES) {
            AffT<Fp29> b = aff_to29(msm_ld_aff(bases + (ent.y >> 1)));
            if (ent.y & 1u) b.y = fp29_neg(b.y);
            acc = xyzz_madd(acc, b);
        } else {
            acc = xyzz_add(acc, msm_ld_p29(in_pts + base + e));
        }
    }
    const uint32_t last = cur;  // acc: the lane's last run (its only one when single)
    const bool active = first != kMsmNoRow;
    const bool single = active && first == last;

    // ---- the tile's rows at both ends, the neighbours' rows
    const uint64_t act = __ballot(active);
    const size_t slot = (size_t)w * (2u * lv.tiles + 2u) + 2u * t;  // next level's items
    if (act == 0u) {  // an empty tile (past the window's entries): blanks go up
        if (!lv.last && lane == 0) {
            out_rows[slot + 1u] = kMsmNoRow;
            out_rows[slot + 2u] = kMsmNoRow;
            if (t == 0) out_rows[slot] = kMsmNoRow;
            if (t + 1u == lv.tiles) out_rows[slot + 3u] = kMsmNoRow;
        }
        return;
    }
    const uint32_t head_lane = (uint32_t)__builtin_ctzll(act);
    const uint32_t tail_lane = 63u - (uint32_t)__builtin_clzll(act);
    const uint32_t head_row = __shfl(first, head_lane, 64);
    const uint32_t prev_last = __shfl_up(last, 1u, 64);
    const uint32_t next_first = __shfl_down(first, 1u, 64);
    if (!lv.last && lane == 0) {  // the blanks at both ends of the window's item list
        if (t == 0) out_rows[slot] = kMsmNoRow;
        if (t + 1u == lv.tiles) out_rows[slot + 3u] = kMsmNoRow;
    }

    // ---- single lanes take over the running sum from their left
    bool wait = single && lane > 0 && prev_last == first;
    for (uint32_t d = 1; d < 64u && __any(wait); d <<= 1) {
        const XyzzT<Fp29> left = msm_shfl_up(acc, d);
        const bool left_wait = __shfl_up((int)wait, d, 64) != 0;
        if (wait && lane >= d) {
            acc = xyzz_add(left, acc);
            wait = left_wait;
        }
    }
    const XyzzT<Fp29> carry = msm_shfl_up(acc, 1u);  // the left lane's running sum

    // ---- completed runs: to the bucket, or up as the tile's first or last item
    auto put = [&](uint32_t row, const XyzzT<Fp29>& p, bool tail_run) {
        if (lv.last) {
            msm_st_p29(buckets + row, p);
        } else if (row == head_row) {
            out_rows[slot + 1u] = row;
            msm_st_p29(out_pts + slot + 1u, p);
            if (tail_run) out_rows[slot + 2u] = kMsmNoRow;  // the whole tile was one run
        } else if (tail_run) {
            out_rows[slot + 2u] = row;
            msm_st_p29(out_pts + slot + 2u, p);
        } else {
            msm_st_p29(buckets + row, p);
        }
    };
    // the last run, unless the next lane goes on with it
    if (active && !(lane < tail_lane && next_first == last)) put(last, acc, lane == tail_lane);
    // the first run of a lane with more than one run, with the left lane's sum when the
    // rows match
    if (active && !single) {
        XyzzT<Fp29> f = first_run[threadIdx.x];
        if (lane > 0 && prev_last == first) f = xyzz_add(carry, f);
        put(first, f, false);
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
