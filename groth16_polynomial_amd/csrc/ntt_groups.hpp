// Register-group batch kernel: the k passes of a batch run in groups of up to GR
// passes, each group entirely in registers, on the 29-bit limb representation.  Two
// geometries: radix-4 groups (GR = 2, four elements a thread) for large launches, and the
// narrow one (GR = 1, two elements a thread, one- or two-wave workgroups, each group's
// table entry loaded one group ahead) for launches too small to fill the chip, where
// each thread's chain of dependent products sets the time.
//
// A thread owns 2^GR elements of its slice for a group covering local index bits
// [b0, b0 + r): the elements whose local index has the thread's value in every other
// bit, r bits varying (for r < GR, 2^(GR-r) such sets).  It runs the group's r passes
// on them in registers and exchanges elements with the other threads through LDS
// before the next group.  A group that starts from LDS first normalizes the elements
// that are "lo" in its first pass, which keeps every value within two passes of
// normalized (fr29.hpp).  The first group reads HBM directly and the last
// writes HBM directly, so a batch of k passes costs ceil(k/GR) - 1 LDS exchanges.
//
// LDS layout: five planes (limb pairs 0-1, 2-3, 4-5, 6-7 as 64-bit words, limb 8 as a
// 32-bit word).  Element e of slice sl sits at slot sl * 2^K + swz(e) (contiguous
// batches) or swz(e) * spw + sl (strided batches and the head batch, where adjacent lanes
// hold adjacent slices), with a bank-conflict-free remapping swz of the element's low
// bits (no padding; lds_swz_contig, lds_swz_strided).
#pragma once

#include <type_traits>
#include <utility>

#include "fr29.hpp"

namespace g16 {

// Slices per workgroup.  Contiguous batches: 2^(10-K) slices (36 KiB of LDS).
// Strided batches and the head batch: at least kStridedCols slices whose data sit in
// adjacent columns, so that the lanes reading one
// row of a workgroup's columns read 64 contiguous bytes of the vector instead of 32; at
// K = 10 that is 72 KiB of LDS and 512 threads, two workgroups per CU (four columns, a
// whole 128-byte line per row in one 1024-thread workgroup, measured no faster).
#ifndef G16_STRIDED_COLS
#define G16_STRIDED_COLS 2
#endif
constexpr int kStridedCols = G16_STRIDED_COLS;

#ifndef G16_NARROW_PREFETCH
#define G16_NARROW_PREFETCH 1
#endif

constexpr bool strided_mode(Mode m) { return m == Mode::FwdStrided || m == Mode::InvStrided; }

// The head batch (bit-reversed load) pairs its slices the same way: slice g reads input
// column bitrev(g), so slices g and g + 2^(L-K-1) read adjacent columns.
constexpr bool interleaved_mode(Mode m) { return strided_mode(m) || m == Mode::HeadBitrev; }

constexpr int slices_per_wg(int k, Mode m) {
    const int base = k >= 10 ? 1 : (1 << (10 - k));
    return interleaved_mode(m) && base < kStridedCols ? kStridedCols : base;
}

// K passes per batch in groups of GR (the last group may be shorter); each thread
// holds 2^GR elements; SPW slices per workgroup.
template <int K, int GR, int SPW>
struct GroupGeom {
    static constexpr int kE = 1 << GR;
    static constexpr int kThreadsPerSlice = 1 << (K - GR);
    static constexpr int kSpw = SPW;
    static constexpr int kThreads = kThreadsPerSlice * kSpw;
    static constexpr int kPlane = kSpw << K;                    // slots per plane
    static constexpr int kLdsBytes = kPlane * 36;
    static constexpr int kGroups = (K + GR - 1) / GR;
    static constexpr int group_b0(int g) { return GR * g; }
    static constexpr int group_r(int g) { return (K - GR * g) < GR ? (K - GR * g) : GR; }
};

template <int K, int GR, Mode M>
using GroupGeomFor = GroupGeom<K, GR, slices_per_wg(K, M)>;

// Narrow geometry, for launches too small to fill the chip, where each thread's chain of
// dependent products sets the time: one pass per group (two elements and one butterfly per
// thread and pass, half the products of the radix-4 groups in each chain, twice the
// threads) and the fewest slices a workgroup may hold (a workgroup is one or two waves),
// so the slices spread over as many CUs as there are.
constexpr int narrow_slices_per_wg(int k, Mode m) {
    return interleaved_mode(m) ? kStridedCols : (k >= 7 ? 1 : (64 >> (k - 1)));
}
template <int K, Mode M>
using NarrowGeomFor = GroupGeom<K, 1, narrow_slices_per_wg(K, M)>;

// Threads of a workgroup that takes three kinds in the narrow geometry (NK = 3 below).
template <int K, Mode M>
constexpr bool narrow_join3_fits() { return 3 * NarrowGeomFor<K, M>::kThreads <= 1024; }

// Whether the exchange from group GA to group GB stays inside every wave: the lanes of a
// wave (64 consecutive threads) hold the elements whose index has the wave's value in the
// bits that thread-index bits above the lane bits land on, and the exchange needs no
// workgroup barrier when those bits are the same in both groups (each wave then reads
// back only elements it wrote; LDS operations of one wave complete in issue order).
// Thread t's element for set s and group member q is e = insert_bits(t 2^(GR-r) + s, q,
// b0, r).  The wave bits of t: contiguous layout (tid = slice * threads-per-slice + t) the
// bits from 6 up, or none when a wave holds whole slices; interleaved (tid = t SPW + slice)
// the bits from 6 - log2(SPW) up.
template <int K, int GR, int SPW, bool INTERLEAVED>
constexpr bool exchange_in_wave(int ga, int gb) {
    using G = GroupGeom<K, GR, SPW>;
    int tbits = 0;
    while ((1 << tbits) < G::kThreadsPerSlice) ++tbits;
    int sbits = 0;
    while ((1 << sbits) < SPW) ++sbits;
    const int w0 = INTERLEAVED ? (6 - sbits > 0 ? 6 - sbits : 0) : 6;
    if (!INTERLEAVED && tbits <= 6) return true;  // a wave holds whole slices
    auto pos = [](int g, int j) {  // element bit that bit j of t lands on in group g
        const int r = G::group_r(g), b0 = G::group_b0(g);
        const int cj = j + (GR - r);
        return cj < b0 ? cj : cj + r;
    };
    for (int j = w0; j < tbits; ++j)
        if (pos(ga, j) != pos(gb, j)) return false;
    return true;
}

// The same by enumeration (checked against exchange_in_wave at compile time): every
// element that a wave writes after group GA is read before group GB by a thread of the
// same wave.
template <int K, int GR, int SPW, bool INTERLEAVED>
constexpr bool exchange_in_wave_enum(int ga, int gb) {
    using G = GroupGeom<K, GR, SPW>;
    constexpr int kElems = SPW << K;
    int wave_of[kElems] = {};
    for (int pass = 0; pass < 2; ++pass) {
        const int g = pass == 0 ? ga : gb;
        const int r = G::group_r(g), b0 = G::group_b0(g);
        const int nsets = 1 << (GR - r);
        for (int tid = 0; tid < G::kThreads; ++tid) {
            const int sl = INTERLEAVED ? tid % SPW : tid / G::kThreadsPerSlice;
            const int t = INTERLEAVED ? tid / SPW : tid % G::kThreadsPerSlice;
            for (int st = 0; st < nsets; ++st)
                for (int q = 0; q < (1 << r); ++q) {
                    const int c = t * nsets + st;
                    const int e = (c & ((1 << b0) - 1)) | (q << b0) | ((c >> b0) << (b0 + r));
                    const int id = sl * (1 << K) + e;
                    if (pass == 0) wave_of[id] = tid / 64;
                    else if (wave_of[id] != tid / 64) return false;
                }
        }
    }
    return true;
}

// c with the r bits of q inserted at bit b0
__device__ __forceinline__ uint32_t insert_bits(uint32_t c, uint32_t q, int b0, int r) {
    return (c & ((1u << b0) - 1u)) | (q << b0) | ((c >> b0) << (b0 + r));
}

// LDS slot of element e within its slice: e with its low bits remapped by a GF(2)-linear
// map (a bijection on every batch size of 6..10 passes).  The lanes served in one LDS cycle
// (the first 16, 32 or 64 of a wave, for 8- and 4-byte accesses on 32 or 64 banks) differ
// in element bits that depend on the group; the maps are chosen so that for every group of
// a 10-pass batch those lanes land on distinct banks.  Contiguous batches: low six bits
// of the slot from element bits 0..7; strided batches (two columns interleaved, the
// column is slot bit 0): low five bits of swz(e) from element bits 0..6.
__device__ __forceinline__ uint32_t lds_swz_contig(uint32_t e) {
    return e ^ (((e >> 4) & 3u) * 5u) ^ (((e >> 6) & 3u) << 4);
}
__device__ __forceinline__ uint32_t lds_swz_strided(uint32_t e) {
    return e ^ ((e >> 2) & 0x1cu) ^ ((e >> 1) & 2u) ^ ((e >> 3) & 1u);
}

__device__ __forceinline__ void lds_put(uint2* lds, uint32_t plane, uint32_t slot, const V29& x) {
    lds[slot] = make_uint2(x.l[0], x.l[1]);
    lds[plane + slot] = make_uint2(x.l[2], x.l[3]);
    lds[2 * plane + slot] = make_uint2(x.l[4], x.l[5]);
    lds[3 * plane + slot] = make_uint2(x.l[6], x.l[7]);
    reinterpret_cast<uint32_t*>(lds + 4 * plane)[slot] = x.l[8];
}

__device__ __forceinline__ V29 lds_get(const uint2* lds, uint32_t plane, uint32_t slot) {
    uint2 a = lds[slot], b = lds[plane + slot], c = lds[2 * plane + slot],
          d = lds[3 * plane + slot];
    V29 x;
    x.l[0] = a.x; x.l[1] = a.y; x.l[2] = b.x; x.l[3] = b.y;
    x.l[4] = c.x; x.l[5] = c.y; x.l[6] = d.x; x.l[7] = d.y;
    x.l[8] = reinterpret_cast<const uint32_t*>(lds + 4 * plane)[slot];
    return x;
}

// Products computed together (interleaved multiply-add chains, shoup_mul_n).  One chain
// issues as fast as two at four waves per SIMD now that a column is one asm block, and
// it leaves the registers for loading table entries ahead.
constexpr int chains_for(Mode) { return 1; }

// Table loads one product ahead (two_passes) where the registers allow it without
// spills: the forward batches, whose top passes read one table entry per butterfly.
constexpr bool prefetch_for(Mode m) { return m == Mode::FwdStrided || m == Mode::HeadBitrev; }

// Butterflies of a pass whose twiddle is 1: bit b of the mask for butterfly b.
template <unsigned MASK>
constexpr int count_nontrivial(int nb) {
    int c = 0;
    for (int b = 0; b < nb; ++b) c += ((MASK >> b) & 1u) ? 0 : 1;
    return c;
}
template <unsigned MASK>
constexpr int nth_nontrivial(int nb, int k) {
    for (int b = 0; b < nb; ++b)
        if (!((MASK >> b) & 1u)) {
            if (k == 0) return b;
            --k;
        }
    return 0;
}

// One pass of a group on x[OFF .. OFF + 2^R): the 2^(R-1) butterflies x_lo, x_hi <-
// x_lo + t, x_lo - t with t = w x_hi, the products computed CH at a time
// (shoup_mul_n).  Butterfly b has lower element q(b) (b with a zero inserted at bit U)
// and its entry in pw[j] for the j-th butterfly not in TRIV (LAZY: loaded here, from
// tw[idx(b)], just before its product; UNI: with scalar loads, the index being the same in
// every lane of the wave).  Butterflies in TRIV have twiddle 1 and take t = x_hi; they
// occur only where x_hi is fresh (canonical, a product output, or the sum or difference
// of two such in the second pass of a batch's first group), which keeps every digit
// inside 32 bits.
template <int OFF, int R, int U, unsigned TRIV, int CH, bool LAZY, bool UNI, int E, typename IdxF>
__device__ __forceinline__ void ct_pass(V29 (&x)[E], const Tw29 (&pw)[1 << (R - 1)],
                                        const TwTab& tw, IdxF&& idx) {
    constexpr int NB = 1 << (R - 1);
    constexpr int NT = count_nontrivial<TRIV>(NB);
    auto lower = [](int b) { return ((b >> U) << (U + 1)) | (b & ((1 << U) - 1)); };
    V29 t[NB];
    static_for<NB>([&](auto b_c) {
        constexpr int b = decltype(b_c)::value;
        if constexpr ((TRIV >> b) & 1u) t[b] = x[OFF + lower(b) + (1 << U)];
    });
    constexpr int NC = NT < CH ? (NT > 0 ? NT : 1) : CH;
    static_for<(NT + NC - 1) / NC>([&](auto ch_c) {
        constexpr int c0 = decltype(ch_c)::value * NC;
        constexpr int nc = (NT - c0) < NC ? (NT - c0) : NC;
        V29 h[nc], y[nc];
        Tw29 w[nc];
        static_for<nc>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            constexpr int b = nth_nontrivial<TRIV>(NB, c0 + j);
            h[j] = x[OFF + lower(b) + (1 << U)];
            if constexpr (LAZY && UNI) w[j] = ld_tw_uniform(tw, idx(std::integral_constant<int, b>{}));
            else if constexpr (LAZY) w[j] = ld_tw(tw, idx(std::integral_constant<int, b>{}));
            else w[j] = pw[c0 + j];
        });
        shoup_mul_n<nc, LAZY && UNI>(h, w, y);
        static_for<nc>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            t[nth_nontrivial<TRIV>(NB, c0 + j)] = y[j];
        });
    });
    static_for<NB>([&](auto b_c) {
        constexpr int b = decltype(b_c)::value;
        constexpr int q = ((b >> U) << (U + 1)) | (b & ((1 << U) - 1));
        x[OFF + q + (1 << U)] = fr29_sub(x[OFF + q], t[b]);
        x[OFF + q] = fr29_add(x[OFF + q], t[b]);
    });
}

// The R passes of a group, in the order u = 0 .. R-1 (forward) or R-1 .. 0 (INV);
// bit b of TM[u] marks the butterflies of pass u with twiddle 1.  PF: table loads one
// product ahead: before each pass the rest of its entries and the first entry of the next
// pass are loaded (the first pass's butterflies share one entry in both orders), behind
// scheduling barriers that keep the compiler from sinking the loads to their uses.
// Without PF each entry is loaded just before its product, which needs fewer registers.
// NORM: the elements that are "lo" in the first pass are normalized first.  UNI: every
// entry of the group is the same in all lanes of the wave (scalar loads; only without PF).
// PRE: a one-pass group whose entry the caller loaded earlier (pre).
template <int OFF, int R, bool INV, bool NORM, int CH, bool PF, bool UNI, unsigned TM0,
          unsigned TM1, unsigned TM2, bool PRE, int E, typename IdxFor>
__device__ __forceinline__ void run_passes(V29 (&x)[E], const TwTab& tw, IdxFor&& idx_for,
                                           const Tw29& pre) {
    static_assert(!PRE || (R == 1 && !PF), "a preloaded entry serves one-pass groups");
    constexpr int NB = 1 << (R - 1);
    constexpr unsigned tm[3] = {TM0, TM1, TM2};
    Tw29 ent[R][NB];
    if constexpr (PRE) ent[0][0] = pre;
    auto fetch = [&](auto s_c, auto j0_c, auto j1_c) {
        constexpr int s = decltype(s_c)::value;
        if constexpr (s < R) {
            constexpr int u = INV ? R - 1 - s : s;
            constexpr int nt = count_nontrivial<tm[u]>(NB);
            constexpr int j0 = decltype(j0_c)::value;
            constexpr int j1 = decltype(j1_c)::value < nt ? decltype(j1_c)::value : nt;
            if constexpr (j0 < j1) {
                auto idx = idx_for(std::integral_constant<int, u>{});
                static_for<j1 - j0>([&](auto j_c) {
                    constexpr int j = j0 + decltype(j_c)::value;
                    constexpr int b = nth_nontrivial<tm[u]>(NB, j);
                    ent[s][j] = ld_tw(tw, idx(std::integral_constant<int, b>{}));
                });
            }
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using INB = std::integral_constant<int, NB>;
    if constexpr (PF) {
        fetch(I0{}, I0{}, INB{});
        fetch(I1{}, I0{}, I1{});
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NORM) {
        // lo elements of the first pass: bit u0 of q clear
        constexpr int u0 = INV ? R - 1 : 0;
        static_for<(1 << R)>([&](auto q_c) {
            constexpr int q = decltype(q_c)::value;
            if constexpr (((q >> u0) & 1) == 0) x[OFF + q] = fr29_normalize(x[OFF + q]);
        });
    }
    static_for<R>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        constexpr int u = INV ? R - 1 - s : s;
        if constexpr (PF && s > 0) {
            fetch(s_c, I1{}, INB{});
            fetch(std::integral_constant<int, s + 1>{}, I0{}, I1{});
            __builtin_amdgcn_sched_barrier(0);
        }
        ct_pass<OFF, R, u, tm[u], CH, !PF && !PRE, UNI && !PF && !PRE>(
            x, ent[s], tw, idx_for(std::integral_constant<int, u>{}));
    });
}

// The R forward-order passes of one group on x[OFF .. OFF + 2^R): pass u flips local
// bit B0 + u (global bit s0 + B0 + u); the pair (q, q + 2^u) has local index bits below
// the pass equal to (c mod 2^B0) + (q mod 2^u) 2^B0.  Global bit 0 has twiddle 1.
template <int OFF, int R, int B0, bool NORM, bool CONTIG, int CH, bool PF, int E, bool PRE>
__device__ __forceinline__ void group_fwd(V29 (&x)[E], uint32_t c, uint32_t low, uint32_t s0,
                                          uint32_t log_n, const TwTab& tw, const Tw29& pre) {
    const uint32_t cl = c & ((1u << B0) - 1u);
    auto idx_for = [&](auto u_c) {
        return [&](auto b_c) {  // u from the type alone: the lambda outlives this call
            constexpr int u = decltype(u_c)::value;
            constexpr int m = decltype(b_c)::value & ((1 << u) - 1);
            return fwd_tw_index(log_n, s0, (uint32_t)(B0 + u), low, cl + ((uint32_t)m << B0));
        };
    };
    // First group of a contiguous batch (s0 = 0): bit 0 has twiddle 1 throughout, bit 1
    // for the pairs with m = 0 (even b); the latter only in a two-pass group, the growth
    // of a third pass would no longer fit in 32 bits.
    constexpr unsigned all = (1u << (1 << (R - 1))) - 1u;
    constexpr unsigned t0 = (CONTIG && B0 == 0) ? all : 0u;
    constexpr unsigned t1 = (CONTIG && B0 == 0 && R == 2) ? (0x55555555u & all) : 0u;
    // in the first group of a contiguous batch (B0 = 0, column 0) the entry index depends
    // on the butterfly only: the same in every lane
    run_passes<OFF, R, false, NORM, CH, PF, (CONTIG && B0 == 0), t0, t1, 0u, PRE>(x, tw, idx_for,
                                                                                pre);
}

// The R inverse-order passes of one group, u = R-1 down to 0: the pair (q, q + 2^u) has
// local bits above the pass a = (q >> (u+1)) + (c >> B0) 2^(R-1-u) and slice row h.
// The pass on the transform's top bit (only in the top batch) has twiddle 1 throughout.
// LB: the bits of c that differ between the lanes of a wave are bits 0 .. LB-1 (and h is
// the same in all of them), so for B0 >= LB every entry of the group is wave-uniform.
template <int OFF, int R, int B0, int K, bool NORM, int CH, bool PF, int LB, int E, bool PRE>
__device__ __forceinline__ void group_inv(V29 (&x)[E], uint32_t c, uint32_t h, uint32_t s0,
                                          uint32_t log_n, const TwTab& tw, const Tw29& pre) {
    const uint32_t ch = c >> B0;
    auto idx_for = [&](auto u_c) {
        return [&](auto b_c) {  // u from the type alone: the lambda outlives this call
            constexpr int u = decltype(u_c)::value;
            constexpr int m = decltype(b_c)::value >> u;  // = q >> (u + 1)
            const uint32_t a = (uint32_t)m + (ch << (R - 1 - u));
            return inv_tw_index(log_n, s0, (uint32_t)K, (uint32_t)(B0 + u), a, h);
        };
    };
    // Top group of the top batch (ch = 0 and h = 0 there): the transform's top bit has
    // twiddle 1 throughout, the next bit for the pairs with q >> (u + 1) = 0 (only in a
    // two-pass group, as in group_fwd).
    constexpr unsigned all = (1u << (1 << (R - 1))) - 1u;
    constexpr bool top_group = B0 + R == K;
    auto run = [&](auto triv_c) {
        constexpr bool tv = decltype(triv_c)::value;
        constexpr unsigned t_top = tv ? all : 0u;                // pass u = R - 1
        constexpr unsigned t_0 = (tv && R == 2) ? 1u : 0u;       // pass u = 0 of two
        run_passes<OFF, R, true, NORM, CH, PF, (B0 >= LB), (R == 1 ? t_top : t_0),
                   (R == 2 ? t_top : 0u), (R == 3 ? t_top : 0u), PRE>(x, tw, idx_for, pre);
    };
    if constexpr (top_group) {
        if (s0 + (uint32_t)K == log_n) run(std::true_type{});
        else run(std::false_type{});
    } else {
        run(std::false_type{});
    }
}

// Grid: (2^(L-K) / SPW) slice groups x n_vec vectors, one-dimensional;
// block = NK x GroupGeom<K, GR, SPW>::kThreads; dynamic LDS = NK x GroupGeom<K, GR, SPW>::
// kLdsBytes.  Launch bounds: at least four waves per SIMD (the second argument is the
// minimum waves per execution unit), i.e. at most 128 VGPRs, whatever the workgroup size.
//
// NK = 3 (with JOIN, the last batch of the pipeline): a workgroup takes the same slices of
// a proof's three vectors, kind = thread / kThreads, each kind in an LDS region of its
// own, and the grid's vectors are proofs.  After the last group the three kinds meet in
// LDS and the A and B threads form H = A' B' - C' (one element each), so A' and B' never
// go back to HBM and the join needs no launch of its own.
template <int K, int GR, Mode M, bool JOIN, int SPW, int NK>
__global__ void __launch_bounds__((GroupGeom<K, GR, SPW>::kThreads * NK), 4)
ntt_group_kernel(BatchParams p) {
    using G = GroupGeom<K, GR, SPW>;
    static_assert(NK == 1 || (NK == 3 && JOIN), "three kinds per workgroup only with the join");
    extern __shared__ uint2 lds_all[];
    constexpr bool kStrided = strided_mode(M);
    // lanes interleave the workgroup's slices (strided batches and the head batch)
    constexpr bool kInterleaved = interleaved_mode(M);
    constexpr int NG = G::kGroups;

    const uint32_t s0 = p.s0;
    const uint32_t L = p.log_n;
    // Workgroups are dispatched to the eight XCDs round-robin in linear order and each XCD
    // has its own L2.  The grid is one-dimensional (slice groups x vectors); renumber it so
    // that each XCD takes one contiguous run of slice groups and, within it, the vectors
    // of a slice group one after another: they use the same twiddle and coset entries,
    // which the later ones then find in that XCD's L2.
    const uint32_t nv = p.n_vec;
    uint32_t lin = blockIdx.x;
    if ((gridDim.x & 7u) == 0u) lin = (lin & 7u) * (gridDim.x >> 3) + (lin >> 3);
    const uint32_t wg = lin / nv;
    uint32_t kind;
    uint64_t off;
    uint32_t tid = threadIdx.x;
    if constexpr (NK == 1) {
        off = proof_offset(p, lin - wg * nv, kind);
    } else {
        kind = tid / G::kThreads;
        tid -= kind * G::kThreads;
        off = (uint64_t)(lin - wg * nv) * p.vstride;
    }
    constexpr uint32_t kRegion = G::kLdsBytes / sizeof(uint2);  // one kind's LDS, in uint2
    uint2* lds = lds_all + (NK == 1 ? 0u : kind * kRegion);
    const Fr* src = p.src[kind] + off;
    Fr* dst = p.dst[kind] + off;
    // strided and head: adjacent lanes take adjacent columns; contiguous: one slice per run
    // of lanes
    const uint32_t sl = kInterleaved ? tid % G::kSpw : tid / G::kThreadsPerSlice;
    const uint32_t t = kInterleaved ? tid / G::kSpw : tid % G::kThreadsPerSlice;
    // global slice number; the head's slices wg + j 2^(L-K) / spw read adjacent input
    // columns bitrev(slice) (the top bits of the slice are the low bits of its column)
    const uint32_t g = M == Mode::HeadBitrev ? wg + sl * ((1u << (L - K)) / G::kSpw)
                                             : wg * G::kSpw + sl;
    const uint32_t low = g & ((1u << s0) - 1u);
    const uint32_t row = g >> s0;
    const uint64_t slice_base = (uint64_t)low + ((uint64_t)row << (s0 + K));
    // Bits of t that differ between the lanes of one wave, where all lanes of a wave work
    // on slices of one row (32: never).  Strided: t = tid / spw, so the low 6 - log2(spw)
    // bits; the spw columns of a workgroup are adjacent and, as 2^s0 >= 64 >= spw in every
    // strided batch this kernel takes (s0 is at least the first batch's k >= 6), share the
    // row.  Contiguous: the low 6 bits when a wave holds one slice.
    constexpr int kLaneBits = kStrided ? 6 - __builtin_ctz(G::kSpw)
                              : kInterleaved ? 32 : (G::kThreadsPerSlice >= 64 ? 6 : 32);

    // narrow geometry: each group's table entry loaded one group ahead (entry below)
    constexpr bool kPre = GR == 1 && G16_NARROW_PREFETCH;

    auto gidx = [&](uint32_t e) -> uint64_t { return slice_base + ((uint64_t)e << s0); };
    auto slot = [&](uint32_t e) -> uint32_t {
        return kInterleaved ? lds_swz_strided(e) * G::kSpw + sl : sl * (1u << K) + lds_swz_contig(e);
    };

    V29 x[G::kE];

    // After the LDS writes of group GA, before the reads of group GB.  Three kinds per
    // workgroup: always the barrier (a wave may hold threads of two kinds).
    auto exchange = [&](auto ga_c, auto gb_c) {
        constexpr int ga = decltype(ga_c)::value, gb = decltype(gb_c)::value;
        static_assert(!exchange_in_wave<K, GR, SPW, kInterleaved>(ga, gb) ||
                          exchange_in_wave_enum<K, GR, SPW, kInterleaved>(ga, gb),
                      "an exchange taken as inside every wave crosses waves");
        if constexpr (NK == 1 && exchange_in_wave<K, GR, SPW, kInterleaved>(ga, gb))
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // order for the compiler
        else
            __syncthreads();
    };

    // Visits the elements of group GI: f(index into x, local element index e).
    auto for_group = [&](auto gi_c, auto&& f) {
        constexpr int gi = decltype(gi_c)::value;
        constexpr int b0 = G::group_b0(gi), r = G::group_r(gi);
        constexpr int nsets = 1 << (GR - r);
        static_for<nsets>([&](auto s_c) {
            constexpr int s = decltype(s_c)::value;
            const uint32_t c = t * nsets + s;
            static_for<(1 << r)>([&](auto q_c) {
                constexpr int q = decltype(q_c)::value;
                f(std::integral_constant<int, s * (1 << r) + q>{}, insert_bits(c, q, b0, r));
            });
        });
    };
    auto load_global = [&](auto gi_c) {
        for_group(gi_c, [&](auto xi_c, uint32_t e) {
            constexpr int xi = decltype(xi_c)::value;
            const uint64_t i = gidx(e);
            if constexpr (M == Mode::HeadBitrev) {
                V29 v = fr29_from_fr(ld_global(src + head_index(i, L, p.head_inverse)));
                x[xi] = p.head_inverse ? shoup_mul(v, p.kscale) : v;
            } else {
                x[xi] = fr29_from_fr(ld_global(src + i));
            }
        });
    };
    auto store_global = [&](auto gi_c) {
        if constexpr (NK == 3) {
            // Every thread holds two elements (one pass per group).  The A thread joins its
            // first element and the B thread its second, so each does one join; each kind
            // leaves in its own slots what the other two need, and C's threads are done.
            static_assert(G::kE == 2, "three kinds per workgroup only in the narrow geometry");
            for_group(gi_c, [&](auto xi_c, uint32_t e) {
                constexpr uint32_t xi = decltype(xi_c)::value;
                if (kind == 2u || xi != kind) lds_put(lds, G::kPlane, slot(e), x[xi]);
            });
            __syncthreads();
            if (kind < 2u) {
                for_group(gi_c, [&](auto xi_c, uint32_t e) {
                    constexpr uint32_t xi = decltype(xi_c)::value;
                    if (xi != kind) return;
                    const uint32_t se = slot(e);
                    const Fr other = fr29_canon(lds_get(lds_all + (1u - kind) * kRegion,
                                                        G::kPlane, se));
                    const Fr cv = fr29_canon(lds_get(lds_all + 2u * kRegion, G::kPlane, se));
                    store_h3(p, off + gidx(e), fr29_canon(x[xi]), other, cv);
                });
            }
            return;
        }
        for_group(gi_c, [&](auto xi_c, uint32_t e) {
            constexpr int xi = decltype(xi_c)::value;
            const uint64_t i = gidx(e);
            if constexpr (JOIN) {
                store_h(p, off + i, x[xi]);
            } else {
                const Fr v = fr29_reduce_2r(x[xi]);
                st_global(dst + i, p.lazy_out ? v : fr_reduce_once(v));
            }
        });
    };
    auto lds_write = [&](auto gi_c) {
        for_group(gi_c, [&](auto xi_c, uint32_t e) {
            constexpr int xi = decltype(xi_c)::value;
            lds_put(lds, G::kPlane, slot(e), x[xi]);
        });
    };
    auto lds_read = [&](auto gi_c) {
        for_group(gi_c, [&](auto xi_c, uint32_t e) {
            constexpr int xi = decltype(xi_c)::value;
            x[xi] = lds_get(lds, G::kPlane, slot(e));
        });
    };
    // passes of group GI in the forward or inverse order; FRESH: the elements come
    // straight from HBM or from a product (no normalization needed); pre: the group's
    // entry, loaded ahead (narrow geometry)
    auto passes = [&](auto gi_c, auto inv_c, auto fresh_c, const TwTab& tw, uint32_t ls0,
                      uint32_t llow, uint32_t lrow, const Tw29& pre) {
        constexpr int gi = decltype(gi_c)::value;
        constexpr bool inv = decltype(inv_c)::value;
        constexpr bool norm = !decltype(fresh_c)::value;
        constexpr int b0 = G::group_b0(gi), r = G::group_r(gi);
        constexpr int nsets = 1 << (GR - r);
        static_for<nsets>([&](auto s_c) {
            constexpr int s = decltype(s_c)::value;
            if constexpr (inv)
                group_inv<s * (1 << r), r, b0, K, norm, chains_for(M), prefetch_for(M) && !kPre,
                          kLaneBits, G::kE, kPre>(x, t * nsets + s, lrow, ls0, L, tw, pre);
            else
                group_fwd<s * (1 << r), r, b0, norm, !kStrided, chains_for(M),
                          prefetch_for(M) && !kPre, G::kE, kPre>(x, t * nsets + s, llow, ls0, L,
                                                                 tw, pre);
        });
    };
    // Narrow geometry (one pass per group, one product per thread and group): the table
    // entry of the next group is loaded while this one runs (its index depends only on
    // the thread's position), so no product waits for its entry.  entry(GI): group GI's
    // entry (group_fwd / group_inv with R = 1, c = t).
    auto entry = [&](auto gi_c, auto inv_c, const TwTab& tw, uint32_t ls0, uint32_t llow,
                     uint32_t lrow) -> Tw29 {
        constexpr uint32_t b0 = decltype(gi_c)::value;
        if constexpr (decltype(inv_c)::value)
            return ld_tw(tw, inv_tw_index(L, ls0, K, b0, t >> b0, lrow));
        else
            return ld_tw(tw, fwd_tw_index(L, ls0, b0, llow, t & ((1u << b0) - 1u)));
    };
    using FWD = std::false_type;
    using INV = std::true_type;
    using FRESH = std::true_type;
    using OLD = std::false_type;
    Tw29 nxt{};  // kPre: the next group's entry

    // One synchronization after every LDS write (exchange): a group reads and rewrites the
    // same slots, all owned by the one thread, so the only ordering needed is that a
    // group's writes land before the next group's reads.
    if constexpr (M == Mode::FwdStrided || M == Mode::HeadBitrev) {
        if constexpr (kPre) nxt = entry(std::integral_constant<int, 0>{}, FWD{}, p.tw, s0, low, row);
        static_for<NG>([&](auto gi_c) {
            constexpr int gi = decltype(gi_c)::value;
            const Tw29 cur = nxt;
            if constexpr (kPre && gi + 1 < NG)
                nxt = entry(std::integral_constant<int, gi + 1>{}, FWD{}, p.tw, s0, low, row);
            if constexpr (gi == 0) {
                load_global(gi_c);
                passes(gi_c, FWD{}, FRESH{}, p.tw, s0, low, row, cur);
            } else {
                lds_read(gi_c);
                passes(gi_c, FWD{}, OLD{}, p.tw, s0, low, row, cur);
            }
            if constexpr (gi == NG - 1) {
                store_global(gi_c);
            } else {
                lds_write(gi_c);
                exchange(gi_c, std::integral_constant<int, gi + 1>{});
            }
        });
    } else if constexpr (M == Mode::InvStrided) {
        if constexpr (kPre)
            nxt = entry(std::integral_constant<int, NG - 1>{}, INV{}, p.tw, s0, low, row);
        static_for<NG>([&](auto step_c) {
            constexpr int gi = NG - 1 - decltype(step_c)::value;
            using GI = std::integral_constant<int, gi>;
            const Tw29 cur = nxt;
            if constexpr (kPre && gi > 0)
                nxt = entry(std::integral_constant<int, gi - 1>{}, INV{}, p.tw, s0, low, row);
            if constexpr (gi == NG - 1) {
                load_global(GI{});
                passes(GI{}, INV{}, FRESH{}, p.tw, s0, low, row, cur);
            } else {
                lds_read(GI{});
                passes(GI{}, INV{}, OLD{}, p.tw, s0, low, row, cur);
            }
            if constexpr (gi == 0) {
                store_global(GI{});
            } else {
                lds_write(GI{});
                exchange(GI{}, std::integral_constant<int, gi - 1>{});
            }
        });
    } else {  // Fused: inverse groups high to low, coset multiply, forward groups low to high
        if constexpr (kPre)
            nxt = entry(std::integral_constant<int, NG - 1>{}, INV{}, p.tw, 0u, 0u, g);
        static_for<NG>([&](auto step_c) {
            constexpr int gi = NG - 1 - decltype(step_c)::value;
            using GI = std::integral_constant<int, gi>;
            const Tw29 cur = nxt;
            // after the last inverse group: the second forward group's (the first
            // forward group, local bit 0, has twiddle 1)
            if constexpr (kPre && gi > 0)
                nxt = entry(std::integral_constant<int, gi - 1>{}, INV{}, p.tw, 0u, 0u, g);
            else if constexpr (kPre && NG > 1)
                nxt = entry(std::integral_constant<int, 1>{}, FWD{}, p.tw_fwd, 0u, 0u, g);
            if constexpr (gi == NG - 1) {
                load_global(GI{});
                passes(GI{}, INV{}, FRESH{}, p.tw, 0u, 0u, g, cur);
            } else {
                lds_read(GI{});
                passes(GI{}, INV{}, OLD{}, p.tw, 0u, 0u, g, cur);
            }
            if constexpr (gi > 0) {
                lds_write(GI{});
                exchange(GI{}, std::integral_constant<int, gi - 1>{});
            }
        });
        // group 0 stays in registers: the coset multiply between the two transforms, by
        // kappa[p mod 4] (the coset shift, kernels.hpp).  With four elements a thread and
        // at least two passes, element xi of group 0 sits at p = xi mod 4, the same in
        // every lane: scalar loads and scalar operands; otherwise p mod 4 varies by lane.
        constexpr bool kUniKappa = G::kE == 4 && K >= 2;
        uint32_t cq[G::kE];
        for_group(std::integral_constant<int, 0>{}, [&](auto xi_c, uint32_t e) {
            cq[decltype(xi_c)::value] = (uint32_t)gidx(e) & 3u;
        });
        constexpr int NC = G::kE < chains_for(M) ? G::kE : chains_for(M);
        static_for<G::kE / NC>([&](auto ch_c) {
            constexpr int i0 = NC * decltype(ch_c)::value;
            V29 h[NC], y[NC];
            Tw29 w[NC];
            static_for<NC>([&](auto j_c) {
                constexpr int j = decltype(j_c)::value;
                h[j] = x[i0 + j];
                if constexpr (kUniKappa) w[j] = ld_tw_uniform(p.kappa, (uint32_t)(i0 + j));
                else w[j] = ld_tw(p.kappa, cq[i0 + j]);
            });
            shoup_mul_n<NC, kUniKappa>(h, w, y);
            static_for<NC>([&](auto j_c) {
                constexpr int j = decltype(j_c)::value;
                x[i0 + j] = y[j];
            });
        });
        static_for<NG>([&](auto gi_c) {
            constexpr int gi = decltype(gi_c)::value;
            const Tw29 cur = nxt;  // group 0: unused (twiddle 1); group 1: loaded above
            if constexpr (kPre && gi >= 1 && gi + 1 < NG)
                nxt = entry(std::integral_constant<int, gi + 1>{}, FWD{}, p.tw_fwd, 0u, 0u, g);
            if constexpr (gi == 0) {
                passes(gi_c, FWD{}, FRESH{}, p.tw_fwd, 0u, 0u, g, cur);  // coset products
            } else {
                lds_read(gi_c);
                passes(gi_c, FWD{}, OLD{}, p.tw_fwd, 0u, 0u, g, cur);
            }
            if constexpr (gi == NG - 1) {
                store_global(gi_c);
            } else {
                lds_write(gi_c);
                exchange(gi_c, std::integral_constant<int, gi + 1>{});
            }
        });
    }
}

}  // namespace g16
