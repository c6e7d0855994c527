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
//     in nine 29-bit digits (fp29.hpp) between loads and stores of canonical values;
//   * each window reduced to sum_m m B_m on the device; the host combines the windows
//     by Horner's rule (the page's "THE WINDOW REDUCTION ENDS ON THE HOST").
//
// Differences from the page (see the notes at each kernel): the digit recoding is
// computed per window from the window's bits and the bit below it (so count and scatter
// need no sequential carry); the counting sort keeps each window's counters in LDS, one
// workgroup per (window, chunk of scalars), so its atomics are LDS atomics and none is
// global; a bucket never written is recognised from its count and from the run geometry
// instead of being cleared first; the window reduction is spread over many threads (one
// per short segment of buckets) rather than one block per window; the ones' partial
// sums are added into window 0.
#pragma once

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
    uint32_t chunk;      // scalars per sorting workgroup
    uint32_t chunks;     // ceil(n / chunk) sorting workgroups per window
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

// Fills a u32 array (the counters start at zero: device memory is never assumed clear).
__global__ void msm_fill_u32(uint32_t* p, uint32_t len, uint32_t v) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < len) p[i] = v;
}

// Counting sort by (window, bucket), with the counters in LDS: one workgroup per (window,
// chunk of scalars) keeps the window's 2^(c-1) counters in LDS (c <= 16: at most
// 128 KiB), so the only atomics are LDS ones and nothing global is contended.
//
// Pass 1: each (window, chunk) workgroup's histogram, written to
// chunk_counts[(w chunks + chunk) B + bucket].
__global__ void __launch_bounds__(kMsmSortThreads) msm_hist(const uint32_t* scalars, MsmParams mp,
                                                            uint32_t* chunk_counts) {
    extern __shared__ uint32_t hist[];
    const uint32_t w = blockIdx.x / mp.chunks, ch = blockIdx.x - w * mp.chunks;
    const uint32_t t = threadIdx.x;
    for (uint32_t b = t; b < mp.buckets; b += kMsmSortThreads) hist[b] = 0u;
    __syncthreads();
    const uint32_t i0 = ch * mp.chunk;
    const uint32_t i1 = i0 + mp.chunk < mp.n ? i0 + mp.chunk : mp.n;
    for (uint32_t i = i0 + t; i < i1; i += kMsmSortThreads) {
        uint32_t k[8];
        msm_load_scalar(scalars, i, k);
        if (msm_scalar_kind(k) != 2u) continue;
        const int32_t d = msm_digit(k, w, mp.c);
        if (d != 0) atomicAdd(&hist[(uint32_t)(d < 0 ? -d : d) - 1u], 1u);
    }
    __syncthreads();
    uint32_t* out = chunk_counts + (size_t)blockIdx.x * mp.buckets;
    for (uint32_t b = t; b < mp.buckets; b += kMsmSortThreads) out[b] = hist[b];
}

// Pass 2a: one thread per bucket row: counts[row] = the row's total over the chunks.
__global__ void __launch_bounds__(kMsmThreads) msm_totals(const uint32_t* chunk_counts,
                                                          MsmParams mp, uint32_t* counts) {
    const uint32_t row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= mp.windows * mp.buckets) return;
    const uint32_t w = row / mp.buckets, b = row - w * mp.buckets;
    const uint32_t* cw = chunk_counts + (size_t)w * mp.chunks * mp.buckets + b;
    uint32_t tot = 0;
    for (uint32_t ch = 0; ch < mp.chunks; ++ch) tot += cw[(size_t)ch * mp.buckets];
    counts[row] = tot;
}

// Pass 2b: exclusive prefix sum of one window's totals, from the window's region start
// w n in the entry array, into cursor[row] (the run's start).  One workgroup per window:
// each thread sums a contiguous range of buckets, the range sums are scanned in LDS, then
// each thread writes its range's starts.
__global__ void __launch_bounds__(kMsmSortThreads) msm_scan(const uint32_t* counts, MsmParams mp,
                                                            uint32_t* cursor, uint32_t* fat_count) {
    __shared__ uint32_t sums[kMsmSortThreads];
    const uint32_t w = blockIdx.x, t = threadIdx.x;
    if (w == 0 && t == 0) *fat_count = 0u;  // the merge pass appends to the list again
    const uint32_t per = (mp.buckets + kMsmSortThreads - 1u) / kMsmSortThreads;
    const uint32_t b0 = t * per;
    const uint32_t b1 = b0 + per < mp.buckets ? b0 + per : mp.buckets;
    const uint32_t* cw = counts + (size_t)w * mp.buckets;
    uint32_t local = 0;
    for (uint32_t b = b0; b < b1; ++b) local += cw[b];
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
    uint32_t* out = cursor + (size_t)w * mp.buckets;
    for (uint32_t b = b0; b < b1; ++b) {
        out[b] = run;
        run += cw[b];
    }
}

// Pass 2c: one thread per bucket row: each chunk's histogram entry becomes the chunk's
// first slot in the row's run, and cursor[row] moves to the run's end.
__global__ void __launch_bounds__(kMsmThreads) msm_chunk_offsets(uint32_t* chunk_counts,
                                                                 MsmParams mp, uint32_t* cursor) {
    const uint32_t row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= mp.windows * mp.buckets) return;
    const uint32_t w = row / mp.buckets, b = row - w * mp.buckets;
    uint32_t* cw = chunk_counts + (size_t)w * mp.chunks * mp.buckets + b;
    uint32_t run = cursor[row];
    for (uint32_t ch = 0; ch < mp.chunks; ++ch) {
        uint32_t* q = cw + (size_t)ch * mp.buckets;
        const uint32_t c = *q;
        *q = run;
        run += c;
    }
    cursor[row] = run;
}

// Pass 3: the same (window, chunk) workgroups place each entry (row, index << 1 |
// negative) at its chunk's next slot in the bucket's run, the slots handed out by LDS
// atomics on the chunk's offsets.
__global__ void __launch_bounds__(kMsmSortThreads) msm_place(const uint32_t* scalars, MsmParams mp,
                                                             const uint32_t* chunk_offsets,
                                                             uint2* entries) {
    extern __shared__ uint32_t next[];
    const uint32_t w = blockIdx.x / mp.chunks, ch = blockIdx.x - w * mp.chunks;
    const uint32_t t = threadIdx.x;
    const uint32_t* in = chunk_offsets + (size_t)blockIdx.x * mp.buckets;
    for (uint32_t b = t; b < mp.buckets; b += kMsmSortThreads) next[b] = in[b];
    __syncthreads();
    const uint32_t i0 = ch * mp.chunk;
    const uint32_t i1 = i0 + mp.chunk < mp.n ? i0 + mp.chunk : mp.n;
    const uint32_t row0 = w * mp.buckets;
    for (uint32_t i = i0 + t; i < i1; i += kMsmSortThreads) {
        uint32_t k[8];
        msm_load_scalar(scalars, i, k);
        if (msm_scalar_kind(k) != 2u) continue;
        const int32_t d = msm_digit(k, w, mp.c);
        if (d == 0) continue;
        const uint32_t b = (uint32_t)(d < 0 ? -d : d) - 1u;
        const uint32_t slot = atomicAdd(&next[b], 1u);
        entries[slot] = make_uint2(row0 + b, (i << 1) | (d < 0 ? 1u : 0u));
    }
}

// The entries of window w occupy [w n, cursor[last row of w]).
__device__ __forceinline__ uint32_t msm_used(const uint32_t* cursor, const MsmParams& mp,
                                             uint32_t w) {
    return cursor[(size_t)w * mp.buckets + mp.buckets - 1u] - w * mp.n;
}

// Pass 4: one thread per slice of slice_len sorted entries of one window.  A run that
// neither contains the slice's first entry nor reaches its end is complete here and is
// written to its bucket; the first run goes to the head spill slot and the run still
// open at the slice's end to the tail slot (a slice holding one run spills once).
__global__ void __launch_bounds__(kMsmThreads) msm_accumulate(const uint2* entries,
                                                              const G1Aff* bases,
                                                              const uint32_t* cursor, MsmParams mp,
                                                              G1Xyzz* buckets, G1Xyzz* spill_pts,
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
                msm_st_xyzz(spill_pts + head, xyzz_from29(acc));
                first = false;
            } else {
                msm_st_xyzz(buckets + cur, xyzz_from29(acc));
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
    msm_st_xyzz(spill_pts + slot, xyzz_from29(acc));
}

// Pass 5: one thread per bucket row with entries.  Starts from the direct write when
// the run lies strictly inside one slice (the accumulation wrote it), else from
// infinity, and adds the spills of the slices the run overlaps.  A run over more than
// kMsmFatSlices slices (many equal digits: repeated scalars, or the few buckets of a
// narrow top window) is appended to a list for msm_merge_fat instead, so that no thread
// adds thousands of spills one after another.
__global__ void __launch_bounds__(kMsmThreads) msm_merge(const uint32_t* counts,
                                                         const uint32_t* cursor,
                                                         const G1Xyzz* spill_pts,
                                                         const uint32_t* spill_rows, MsmParams mp,
                                                         G1Xyzz* buckets, uint32_t* fat_count,
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
    XyzzT<Fp29> acc = direct ? xyzz_to29(msm_ld_xyzz(buckets + row)) : xyzz_zero<Fp29>();
    for (uint32_t k = k_lo; k <= k_hi; ++k) {
        const uint32_t slot = 2u * (w * mp.slices + k);
        if (spill_rows[slot] == row) acc = xyzz_add(acc, xyzz_to29(msm_ld_xyzz(spill_pts + slot)));
        if (spill_rows[slot + 1u] == row)
            acc = xyzz_add(acc, xyzz_to29(msm_ld_xyzz(spill_pts + slot + 1u)));
    }
    msm_st_xyzz(buckets + row, xyzz_from29(acc));
}

// Pass 5b: the listed rows, one workgroup at a time (a grid-stride loop over the list,
// whose length every thread reads once before the loop, so all reach every barrier):
// the threads take the run's slices in turn, each adding the spills that carry the row,
// then a tree in LDS.  Such a run spans at least two slices, so the accumulation never
// wrote its bucket directly.
__global__ void __launch_bounds__(kMsmThreads) msm_merge_fat(const uint32_t* counts,
                                                             const uint32_t* cursor,
                                                             const G1Xyzz* spill_pts,
                                                             const uint32_t* spill_rows,
                                                             MsmParams mp,
                                                             const uint32_t* fat_count,
                                                             const uint32_t* fat_rows,
                                                             G1Xyzz* buckets) {
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
            if (spill_rows[slot] == row) acc = xyzz_add(acc, xyzz_to29(msm_ld_xyzz(spill_pts + slot)));
            if (spill_rows[slot + 1u] == row)
                acc = xyzz_add(acc, xyzz_to29(msm_ld_xyzz(spill_pts + slot + 1u)));
        }
        sh[t] = acc;
        for (uint32_t s = kMsmThreads / 2; s > 0; s >>= 1) {
            __syncthreads();
            if (t < s) sh[t] = xyzz_add(sh[t], sh[t + s]);
        }
        if (t == 0) msm_st_xyzz(buckets + row, xyzz_from29(sh[0]));
        __syncthreads();  // sh is reused by the next listed row
    }
}

// Pass 6: the window sum sum_m m B_m, bucket j holding magnitude m = j + 1.  One thread
// per segment [lo, lo + seg_len) of a window's buckets: the running sum from the top
// gives T = sum_j (j - lo + 1) B_j and Q = sum_j B_j, and the segment contributes
// T + lo Q.  Buckets with no entries are infinity (never read).
__global__ void __launch_bounds__(kMsmThreads) msm_reduce_segments(const uint32_t* counts,
                                                                   const G1Xyzz* buckets,
                                                                   MsmParams mp, G1Xyzz* seg_out) {
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t w = gid / mp.segs;
    if (w >= mp.windows) return;
    const uint32_t lo = (gid - w * mp.segs) * mp.seg_len;
    const size_t base = (size_t)w * mp.buckets;
    XyzzT<Fp29> run = xyzz_zero<Fp29>(), tot = xyzz_zero<Fp29>();
    for (uint32_t j = lo + mp.seg_len; j-- > lo;) {
        if (counts[base + j]) run = xyzz_add(run, xyzz_to29(msm_ld_xyzz(buckets + base + j)));
        tot = xyzz_add(tot, run);
    }
    if (lo) tot = xyzz_add(tot, xyzz_mul_small(run, lo));
    msm_st_xyzz(seg_out + gid, xyzz_from29(tot));
}

// The scalar-one pass: sum of the bases whose scalar is exactly 1, strided over the
// scalars, then a tree in LDS; one partial sum per workgroup.
__global__ void __launch_bounds__(kMsmThreads) msm_ones(const uint32_t* scalars,
                                                        const G1Aff* bases, MsmParams mp,
                                                        G1Xyzz* out) {
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
    if (t == 0) msm_st_xyzz(out + blockIdx.x, xyzz_from29(sh[0]));
}

// Pass 7: group sums.  Workgroup g adds in[g per, (g + 1) per) (and, for g = 0, the
// n_extra points of extra) into out[g], a tree in LDS after a strided serial sum.  Run
// twice: the segments' contributions into a few partials per window, then the partials
// (and the ones' sums, into window 0) into the window sums.
__global__ void __launch_bounds__(kMsmThreads) msm_sum_groups(const G1Xyzz* in, uint32_t per,
                                                              const G1Xyzz* extra,
                                                              uint32_t n_extra, G1Xyzz* out) {
    __shared__ XyzzT<Fp29> sh[kMsmThreads];
    const uint32_t g = blockIdx.x, t = threadIdx.x;
    XyzzT<Fp29> acc = xyzz_zero<Fp29>();
    for (uint32_t s = t; s < per; s += kMsmThreads)
        acc = xyzz_add(acc, xyzz_to29(msm_ld_xyzz(in + (size_t)g * per + s)));
    if (g == 0)
        for (uint32_t e = t; e < n_extra; e += kMsmThreads)
            acc = xyzz_add(acc, xyzz_to29(msm_ld_xyzz(extra + e)));
    sh[t] = acc;
    for (uint32_t s = kMsmThreads / 2; s > 0; s >>= 1) {
        __syncthreads();
        if (t < s) sh[t] = xyzz_add(sh[t], sh[t + s]);
    }
    if (t == 0) msm_st_xyzz(out + g, xyzz_from29(sh[0]));
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
