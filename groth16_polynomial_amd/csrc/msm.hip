// libg16.so: host side of the G1 multi-scalar multiplication (include/g16.h, "G1 MSM").
//
// g16_msm_g1 only enqueues (counting sort, bucket sums, window reduction) and
// leaves one XYZZ point per window in the caller's buffer; g16_msm_g1_finish combines
// them on the host by Horner's rule, as the MSM_CU page does ("THE WINDOW REDUCTION
// ENDS ON THE HOST").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "g16.h"
#include "host_util.hpp"
#include "msm_kernels.hpp"

using g16::G1Aff;
using g16::G1Xyzz;
using g16::MsmParams;

namespace {

constexpr size_t kAlign = 256;
constexpr uint32_t kMaxC = 16;  // a window's counters fit in LDS (2^15 x 4 bytes)
constexpr uint32_t kSegLen = 8;
constexpr uint32_t kMaxOnesGroups = 1024;  // workgroups of the scalar-one pass, at most
constexpr uint32_t kBinEntries = 8192;   // entries per coarse bin, about (at most 1024 bins)
constexpr uint32_t kStage = 9216;        // entries of a bin staged in LDS by the row sort (its
                                         // bins hold ~8192 on average)
constexpr uint32_t kMinChunk = 8192;     // codes per coarse-sorting workgroup, at least
constexpr uint32_t kMaxLevels = 8;      // levels of the bucket sums (a few suffice)

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

uint32_t windows_for(uint32_t c) { return (255u + c - 1u) / c; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

using g16::device_range;

// Entries per lane at the bucket sums' first level.  Lanes whose entries all belong to
// one bucket make the wave join them by a scan of log2 steps, so the lane length grows
// from 32 toward twice a bucket's mean run n / 2^(c-1), where such lanes become rare, up
// to 64 and while the windows still give 4096 waves (16 per CU); and it shrinks, down to
// 2, while they give fewer than 1024 waves, since at small n the time is the chain of
// dependent additions in a lane.  Measured at c = 16: 2^20 (mean run 32) 32 / 64 / 128
// entries: 1.77 / 1.67 / 1.74 ms; 2^22 (mean run 128) 64 / 128 / 256 / 512: 6.13 / 6.10 /
// 6.29 / 6.47 ms.
uint32_t slice_len_for(uint64_t n, uint32_t c) {
    const uint64_t mean = n >> (c - 1);
    const uint64_t entries = (uint64_t)windows_for(c) * n;
    uint32_t len = 32;
    while (len < 2 * mean && len < 64u && entries / (64u * 2u * len) >= 4096u) len *= 2;
    while (len > 2u && entries / (64u * len) < 1024u) len /= 2;
    return len;
}

// Buckets per window-sum thread: kSegLen, halved, down to 1, while the windows give fewer
// than 2^16 threads (the same reason).
uint32_t seg_len_for(uint32_t W, uint32_t buckets) {
    uint32_t len = buckets < kSegLen ? buckets : kSegLen;
    while (len > 1u && (uint64_t)W * (buckets / len) < (1u << 16)) len /= 2;
    return len;
}

// Window width minimising a cost in point additions: n per window for the bucket sums and
// about one per bucket for the joins and the weighted window sum (much of that work
// overlaps: measured widths at 2^12 .. 2^22 fit this weight, not three).
uint32_t model_c(uint64_t n) {
    uint32_t best = 1;
    double best_cost = 0.0;
    for (uint32_t c = 1; c <= kMaxC; ++c) {
        const uint32_t W = windows_for(c);
        const double cost = (double)W * ((double)n + (double)(1u << (c - 1)));
        if (c == 1 || cost < best_cost) {
            best = c;
            best_cost = cost;
        }
    }
    return best;
}

// The default width: from 2^10 terms, the fastest width measured on MI355X at each size
// (every width timed at 2^10, 2^12, 2^14 .. 2^21; sizes between take the entry below).
// Up to 2^15 the MSM is bound by the latency of its serial chains (a slice's additions,
// a segment's double-and-add, the tree passes) and narrower windows win; from 2^16 the
// accumulation's n W additions dominate and 16 wins.  Below 2^10 the cost model, at most
// 5.
uint32_t default_c(uint64_t n) {
    if (n < (1u << 10)) return std::min<uint32_t>(model_c(n), 5u);
    uint32_t lg = 0;
    while ((n >> (lg + 1)) != 0) ++lg;
    if (lg >= 16) return 16;
    static const uint8_t kBest[6] = {8, 8, 6, 6, 10, 10};  // 2^10 .. 2^15
    return kBest[lg - 10];
}

struct Layout {
    MsmParams mp;
    uint32_t per_group, groups;  // segment sums per partial, partials per window
    uint32_t n_levels;
    g16::MsmLevel levels[kMaxLevels];
    size_t item_cap;  // items per ping-pong buffer of the levels above the first
    size_t counts, cursor, codes, bin_counts, bin_offs, entries, items, buckets, seg_out,
        partials, ones_out, total;
};

bool make_layout(uint64_t n, uint32_t c, Layout* L) {
    if (c < 1 || c > kMaxC) return false;
    const uint32_t W = windows_for(c);
    if (n == 0 || (uint64_t)W * n >= (1ull << 32) || n >= (1ull << 31)) return false;
    MsmParams& mp = L->mp;
    std::memset(&mp, 0, sizeof mp);
    mp.n = (uint32_t)n;
    mp.c = c;
    mp.windows = W;
    mp.buckets = 1u << (c - 1);
    mp.slice_len = slice_len_for(n, c);
    // the bucket sums' levels: the first over each window's n entries (at most), each
    // next one over two items per tile of the one below, two items per lane
    {
        uint32_t items = (uint32_t)n, len = mp.slice_len, stride = (uint32_t)n;
        L->n_levels = 0;
        L->item_cap = 0;
        for (;;) {
            if (L->n_levels == kMaxLevels) return false;
            g16::MsmLevel& lv = L->levels[L->n_levels++];
            lv.lane_len = len;
            lv.tiles = (uint32_t)((items + 64ull * len - 1) / (64ull * len));
            lv.stride = stride;
            lv.last = lv.tiles == 1u ? 1u : 0u;
            if (lv.last) break;
            items = 2u * lv.tiles + 2u;
            stride = items;
            len = 2u;
            L->item_cap = std::max<size_t>(L->item_cap, (size_t)W * items);
        }
    }
    mp.seg_len = seg_len_for(W, mp.buckets);
    mp.segs = mp.buckets / mp.seg_len;
    const uint64_t groups = (n + g16::kMsmThreads - 1) / g16::kMsmThreads;
    mp.ones_groups = (uint32_t)(groups < kMaxOnesGroups ? groups : kMaxOnesGroups);
    mp.n_pad = (uint32_t)((n + 7) / 8 * 8);
    // Bins: a power of two up to the bucket count (and 1024), enough for about
    // kBinEntries entries each and for 256 bin-sorting workgroups over the windows.
    mp.bins = 1;
    while (mp.bins < mp.buckets && mp.bins < 1024 &&
           (n / mp.bins > kBinEntries || W * mp.bins < 256))
        mp.bins *= 2;
    for (mp.bin_shift = 0; (mp.bins << mp.bin_shift) < mp.buckets; ++mp.bin_shift) {
    }
    // Chunks: at most about 128 per window, whole multiples of 2048 codes (eight per
    // thread of a 256-thread workgroup).
    uint64_t chunk = (mp.n_pad + 127) / 128;
    chunk = (chunk + 2047) / 2048 * 2048;
    if (chunk < kMinChunk) chunk = kMinChunk;
    mp.chunk = (uint32_t)chunk;
    mp.chunks = (uint32_t)((mp.n_pad + chunk - 1) / chunk);
    // LDS of the row sort: two buffers of staged entries and a counter per row, within
    // 144 KiB
    const uint64_t row_bytes = ((uint64_t)1 << mp.bin_shift) * 4;
    mp.stage = row_bytes >= 144 * 1024 ? 0u
               : (uint32_t)std::min<uint64_t>(kStage, (144 * 1024 - row_bytes) / 16);
    L->per_group = mp.segs < g16::kMsmThreads ? mp.segs : g16::kMsmThreads;
    L->groups = mp.segs / L->per_group;
    const size_t rows = (size_t)W * mp.buckets;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round_up(bytes);
        return at;
    };
    L->counts = take(rows * 4);
    L->cursor = take(rows * 4);
    L->codes = take((size_t)W * mp.n_pad * 2);
    L->bin_counts = take((size_t)W * mp.bins * mp.chunks * 4);
    L->bin_offs = take((size_t)W * mp.bins * mp.chunks * 4);
    L->entries = take((size_t)W * n * 8);
    // the coarse-sorted entries, then (once the row sort has read them) two buffers of
    // the upper levels' items, rows then points
    const size_t item_bytes = 2 * L->item_cap * (4 + sizeof(g16::P29)) + 1024;
    L->items = take(std::max(item_bytes, (size_t)W * n * 8));
    L->buckets = take(rows * sizeof(g16::P29));
    L->seg_out = take((size_t)W * mp.segs * sizeof(g16::P29));
    L->partials = take((size_t)W * L->groups * sizeof(g16::P29));
    L->ones_out = take((size_t)mp.ones_groups * sizeof(g16::P29));
    L->total = off;
    return true;
}

uint32_t blocks_for(uint64_t threads) {
    return (uint32_t)((threads + g16::kMsmThreads - 1) / g16::kMsmThreads);
}

}  // namespace

extern "C" {

uint32_t g16_msm_g1_window_bits(uint64_t n) { return n ? default_c(n) : 1u; }

uint32_t g16_msm_g1_window_count(uint32_t c) {
    return (c >= 1 && c <= kMaxC) ? windows_for(c) : 0u;
}

size_t g16_msm_g1_workspace_bytes(uint64_t n, uint32_t c) {
    if (c == 0) c = g16_msm_g1_window_bits(n);
    Layout L;
    if (n == 0) return 0;
    return make_layout(n, c, &L) ? L.total : 0;
}

int g16_msm_g1(uint64_t n, const void* scalars_std, const void* bases_mont, uint32_t c,
               void* workspace, size_t workspace_bytes, void* window_sums, void* stream) {
    if (c == 0) c = g16_msm_g1_window_bits(n);
    if (c > kMaxC || !window_sums) return G16_EINVAL;
    const uint32_t W = windows_for(c);
    const size_t sums_bytes = (size_t)W * sizeof(G1Xyzz);
    if (!device_range(window_sums, sums_bytes)) return G16_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (n == 0) {  // the empty sum: every window at infinity
        const uint32_t words = (uint32_t)(sums_bytes / 4);
        hipLaunchKernelGGL(g16::msm_fill_u32, dim3(blocks_for(words)), dim3(g16::kMsmThreads), 0,
                           s, (uint32_t*)window_sums, words, 0u);
        return hipGetLastError() == hipSuccess ? G16_OK : G16_EHIP;
    }
    Layout L;
    if (!make_layout(n, c, &L)) return G16_EINVAL;
    if (!scalars_std || !bases_mont || !workspace) return G16_EINVAL;
    if ((uintptr_t)workspace % kAlign) return G16_EINVAL;
    if (workspace_bytes < L.total) return G16_ENOSPACE;
    const size_t sb = n * 32, bb = n * sizeof(G1Aff);
    if (overlaps(workspace, L.total, scalars_std, sb) || overlaps(workspace, L.total, bases_mont, bb) ||
        overlaps(window_sums, sums_bytes, scalars_std, sb) ||
        overlaps(window_sums, sums_bytes, bases_mont, bb) ||
        overlaps(window_sums, sums_bytes, workspace, L.total))
        return G16_EALIAS;
    if (!device_range(scalars_std, sb) || !device_range(bases_mont, bb) ||
        !device_range(workspace, L.total))
        return G16_EINVAL;

    uint8_t* ws = (uint8_t*)workspace;
    const MsmParams mp = L.mp;
    uint32_t* counts = (uint32_t*)(ws + L.counts);
    uint32_t* cursor = (uint32_t*)(ws + L.cursor);
    uint16_t* codes = (uint16_t*)(ws + L.codes);
    uint32_t* bin_counts = (uint32_t*)(ws + L.bin_counts);
    uint32_t* bin_offs = (uint32_t*)(ws + L.bin_offs);
    uint2* entries = (uint2*)(ws + L.entries);
    g16::P29* buckets = (g16::P29*)(ws + L.buckets);
    g16::P29* seg_out = (g16::P29*)(ws + L.seg_out);
    g16::P29* partials = (g16::P29*)(ws + L.partials);
    g16::P29* ones_out = (g16::P29*)(ws + L.ones_out);
    const uint32_t* sc = (const uint32_t*)scalars_std;
    const G1Aff* bases = (const G1Aff*)bases_mont;
    const dim3 blk(g16::kMsmThreads), sort_blk(g16::kMsmSortThreads);
    // The coarse-sorted entries live in the items area until the row sort has read them
    // (the area holds W n entries of 8 bytes); then the levels' items take it over.
    uint2* binned = (uint2*)(ws + L.items);
    uint32_t* item_rows[2] = {(uint32_t*)(ws + L.items),
                              (uint32_t*)(ws + L.items) + L.item_cap};
    g16::P29* item_pts[2];
    {
        const size_t pts_at = round_up(2 * L.item_cap * 4);
        item_pts[0] = (g16::P29*)(ws + L.items + pts_at);
        item_pts[1] = item_pts[0] + L.item_cap;
    }
    const size_t count_lds = (size_t)mp.bins * 16;
    const size_t place_lds = (size_t)g16::kMsmRound * 8 + (size_t)mp.bins * 12;
    const size_t row_lds = (size_t)mp.stage * 16 + ((size_t)1 << mp.bin_shift) * 4;
    // LDS beyond the default 64 KiB is allowed per kernel
    if (g16::allow_lds((const void*)g16::msm_bin_place, place_lds) != hipSuccess ||
        g16::allow_lds((const void*)g16::msm_bin_sort, row_lds) != hipSuccess)
        return G16_EHIP;
    const dim3 bin_blk(g16::kMsmBinThreads);

    hipLaunchKernelGGL(g16::msm_digits, dim3(blocks_for(mp.n_pad)), blk, 0, s, sc, mp, codes);
    hipLaunchKernelGGL(g16::msm_bin_count, dim3(W * mp.chunks), bin_blk, count_lds, s,
                       (const uint16_t*)codes, mp, bin_counts);
    hipLaunchKernelGGL(g16::msm_scan, dim3(W), sort_blk, 0, s, (const uint32_t*)bin_counts,
                       mp.bins * mp.chunks, mp, bin_offs);
    hipLaunchKernelGGL(g16::msm_bin_place, dim3(W * mp.chunks), bin_blk, place_lds, s,
                       (const uint16_t*)codes, mp, (const uint32_t*)bin_offs, binned);
    hipLaunchKernelGGL(g16::msm_bin_sort, dim3(W * mp.bins), sort_blk, row_lds, s,
                       (const uint2*)binned, (const uint32_t*)bin_counts,
                       (const uint32_t*)bin_offs, mp, counts, cursor, entries);
    // the bucket sums, level by level (each level's items go to the other buffer)
    for (uint32_t k = 0; k < L.n_levels; ++k) {
        const g16::MsmLevel& lv = L.levels[k];
        const uint32_t blocks = blocks_for((uint64_t)W * lv.tiles * 64u);
        uint32_t* out_r = item_rows[k & 1u];
        g16::P29* out_p = item_pts[k & 1u];
        if (k == 0)
            hipLaunchKernelGGL(g16::msm_tile_sums<true>, dim3(blocks), blk, 0, s,
                               (const uint2*)entries, bases, (const uint32_t*)nullptr,
                               (const g16::P29*)nullptr, (const uint32_t*)cursor, mp, lv,
                               buckets, out_r, out_p);
        else
            hipLaunchKernelGGL(g16::msm_tile_sums<false>, dim3(blocks), blk, 0, s,
                               (const uint2*)nullptr, bases,
                               (const uint32_t*)item_rows[(k - 1) & 1u],
                               (const g16::P29*)item_pts[(k - 1) & 1u], (const uint32_t*)cursor,
                               mp, lv, buckets, out_r, out_p);
    }
    hipLaunchKernelGGL(g16::msm_reduce_segments, dim3(blocks_for((uint64_t)W * mp.segs)), blk, 0,
                       s, counts, buckets, mp, seg_out);
    hipLaunchKernelGGL(g16::msm_ones, dim3(mp.ones_groups), blk, 0, s, sc, bases, mp, ones_out);
    hipLaunchKernelGGL(g16::msm_sum_groups<g16::P29>, dim3(W * L.groups), blk, 0, s,
                       (const g16::P29*)seg_out, L.per_group, (const g16::P29*)nullptr, 0u,
                       partials);
    hipLaunchKernelGGL(g16::msm_sum_groups<G1Xyzz>, dim3(W), blk, 0, s, (const g16::P29*)partials,
                       L.groups, (const g16::P29*)ones_out, mp.ones_groups, (G1Xyzz*)window_sums);
    return hipGetLastError() == hipSuccess ? G16_OK : G16_EHIP;
}

int g16_msm_g1_finish(uint32_t c, const void* window_sums_host, void* out_affine_std) {
    if (c < 1 || c > kMaxC || !window_sums_host || !out_affine_std) return G16_EINVAL;
    const uint32_t W = windows_for(c);
    const G1Xyzz* ws = (const G1Xyzz*)window_sums_host;
    // in the 29-bit digit form: on the host its digit products are native 64-bit
    // multiplies, about half the time of the 32-bit-limb products
    g16::XyzzT<g16::Fp29> acc = g16::xyzz_to29(ws[W - 1]);
    for (uint32_t w = W - 1; w-- > 0;) {
        for (uint32_t i = 0; i < c; ++i) acc = g16::xyzz_dbl(acc);
        acc = g16::xyzz_add(acc, g16::xyzz_to29(ws[w]));
    }
    const G1Aff a = g16::xyzz_to_aff(acc);
    const g16::Fp x = g16::fp_from_mont(a.x), y = g16::fp_from_mont(a.y);
    std::memcpy(out_affine_std, x.w, 32);
    std::memcpy((uint8_t*)out_affine_std + 32, y.w, 32);
    return G16_OK;
}

int g16_g1_generator_mul(uint64_t n, const void* scalars_std, void* out_affine_mont,
                         void* stream) {
    if (n == 0 || n >= (1ull << 31) || !scalars_std || !out_affine_mont) return G16_EINVAL;
    if (overlaps(scalars_std, n * 32, out_affine_mont, n * sizeof(G1Aff))) return G16_EALIAS;
    if (!device_range(scalars_std, n * 32) || !device_range(out_affine_mont, n * sizeof(G1Aff)))
        return G16_EINVAL;
    hipLaunchKernelGGL(g16::g1_generator_mul, dim3(blocks_for(n)), dim3(g16::kMsmThreads), 0,
                       (hipStream_t)stream, (const uint32_t*)scalars_std, (uint32_t)n,
                       (G1Aff*)out_affine_mont);
    return hipGetLastError() == hipSuccess ? G16_OK : G16_EHIP;
}

}  // extern "C"
