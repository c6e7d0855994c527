// Radix-8 batch kernel: the k passes of a batch run in groups of up to three, each
// group entirely in registers.
//
// A thread owns eight elements of its slice for a group covering local index bits
// [b0, b0 + r): the elements whose local index has the thread's value in every other
// bit, r bits varying (for r < 3, 2^(3-r) such sets).  It runs the group's r passes on
// them in registers and exchanges elements with the other threads through LDS between
// groups.  The first group reads HBM directly and the last writes HBM directly, so a
// batch of k passes costs ceil(k/3) - 1 LDS exchanges instead of k.
//
// LDS layout: four planes of 64-bit limb pairs (limbs 2p, 2p+1 of every element in
// plane p), element e of slice sl at slot sl * SP + e + e/8.  The padding spreads the
// stride-8 and block patterns of the low groups over the banks.
#pragma once

#include <type_traits>
#include <utility>

#include "fr.hpp"

namespace g16 {

// K passes per batch in groups of GR (the last group may be shorter); each thread
// holds E = 2^GR elements.
template <int K, int GR>
struct R8Geom {
    static constexpr int kE = 1 << GR;
    static constexpr int kThreadsPerSlice = 1 << (K - GR);
    static constexpr int kSpw = (256 >> (K - GR)) > 0 ? (256 >> (K - GR)) : 1;  // slices / WG
    static constexpr int kThreads = kThreadsPerSlice * kSpw;
    static constexpr int kSlotsPerSlice = (1 << K) + (1 << (K - 3)) + 4;
    static constexpr int kPlane = kSlotsPerSlice * kSpw;                   // uint2 per plane
    static constexpr int kLdsBytes = 4 * kPlane * 8;
    static constexpr int kGroups = (K + GR - 1) / GR;
    static constexpr int group_b0(int g) { return GR * g; }
    static constexpr int group_r(int g) { return (K - GR * g) < GR ? (K - GR * g) : GR; }
};

// c with the r bits of q inserted at bit b0
__device__ __forceinline__ uint32_t insert_bits(uint32_t c, uint32_t q, int b0, int r) {
    return (c & ((1u << b0) - 1u)) | (q << b0) | ((c >> b0) << (b0 + r));
}

__device__ __forceinline__ uint32_t lds_slot(uint32_t e) { return e + (e >> 3); }

__device__ __forceinline__ void lds_put(uint2* lds, uint32_t plane, uint32_t slot, const Fr& x) {
    lds[slot] = make_uint2(x.w[0], x.w[1]);
    lds[plane + slot] = make_uint2(x.w[2], x.w[3]);
    lds[2 * plane + slot] = make_uint2(x.w[4], x.w[5]);
    lds[3 * plane + slot] = make_uint2(x.w[6], x.w[7]);
}

__device__ __forceinline__ Fr lds_get(const uint2* lds, uint32_t plane, uint32_t slot) {
    uint2 a = lds[slot], b = lds[plane + slot], c = lds[2 * plane + slot],
          d = lds[3 * plane + slot];
    Fr x;
    x.w[0] = a.x; x.w[1] = a.y; x.w[2] = b.x; x.w[3] = b.y;
    x.w[4] = c.x; x.w[5] = c.y; x.w[6] = d.x; x.w[7] = d.y;
    return x;
}

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so that every
// register array index below is a constant and the element arrays stay in VGPRs.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The R passes of one group on the set x[OFF .. OFF + 2^R) held in registers.
//   DIT: passes u = 0 .. R-1 (increasing bit order); DIF: u = R-1 .. 0.
//   Pass u flips local bit B0 + u (global bit B = s0 + B0 + u).  The butterfly of the
//   pair (q, q + 2^u) uses root^(j n / 2^(B+1)), j = the lower element's global index
//   mod 2^B = low + (((c mod 2^B0) + (q mod 2^u) 2^B0) << s0).
template <int OFF, int R, int B0, bool DIF, bool CONTIG, int E>
__device__ __forceinline__ void group_passes(Fr (&x)[E], uint32_t c, uint32_t low, uint32_t s0,
                                             uint32_t log_n, const Fr* tw) {
    const uint32_t cl = c & ((1u << B0) - 1u);
    static_for<R>([&](auto uu_c) {
        constexpr int uu = decltype(uu_c)::value;
        constexpr int u = DIF ? (R - 1 - uu) : uu;
        const uint32_t B = s0 + (uint32_t)(B0 + u);
        F29 w[1 << u];
        static_for<(1 << u)>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            const bool trivial = (B == 0u) || (CONTIG && B0 == 0 && u == 1 && m == 0);
            if (!trivial) {
                uint32_t j = low + ((cl + ((uint32_t)m << B0)) << s0);
                w[m] = unpack29(ld_global(tw + ((size_t)j << (log_n - B - 1u))));
            }
        });
        static_for<(1 << R)>([&](auto q_c) {
            constexpr int q = decltype(q_c)::value;
            if constexpr ((q & (1 << u)) == 0) {
                constexpr int q2 = q + (1 << u);
                constexpr int wi = q & ((1 << u) - 1);
                // twiddle 1: bit 0 always; bit 1 of a contiguous slice for its first pair
                const bool trivial = (B == 0u) || (CONTIG && B0 == 0 && u == 1 && wi == 0);
                if (DIF) {
                    // values in [0, 2r) before and after the pass
                    Fr a = fr_reduce_2r(fr_add_lazy(x[OFF + q], x[OFF + q2]));
                    Fr d = fr_sub_lazy(x[OFF + q], x[OFF + q2]);
                    x[OFF + q2] = trivial ? fr_reduce_2r(d) : fr_mul29_lazy(d, w[wi]);
                    x[OFF + q] = a;
                } else {
                    // values in [0, 4r) before and after the pass
                    Fr uu0 = fr_reduce_2r(x[OFF + q]);
                    Fr v = trivial ? fr_reduce_2r(x[OFF + q2]) : fr_mul29_lazy(x[OFF + q2], w[wi]);
                    x[OFF + q2] = fr_sub_lazy(uu0, v);
                    x[OFF + q] = fr_add_lazy(uu0, v);
                }
            }
        });
    });
}

// Grid: x = slice groups (2^(L-K) / kSpw), y = vectors; block = R8Geom<K, GR>::kThreads;
// dynamic LDS = R8Geom<K, GR>::kLdsBytes.
template <int K, int GR, Mode M, bool JOIN>
__global__ void __launch_bounds__(256, 4) ntt_r8_kernel(BatchParams p) {
    using G = R8Geom<K, GR>;
    extern __shared__ uint2 lds[];
    constexpr bool kStrided = (M == Mode::DitStrided || M == Mode::DifStrided);
    constexpr int NG = G::kGroups;

    const uint32_t s0 = p.s0;
    const uint32_t L = p.log_n;
    const Fr* src = p.src[blockIdx.y];
    Fr* dst = p.dst[blockIdx.y];

    // XCD-aware renumbering (see ntt_batch_kernel)
    uint32_t wg = blockIdx.x;
    if ((gridDim.x & 7u) == 0u) wg = (wg & 7u) * (gridDim.x >> 3) + (wg >> 3);
    const uint32_t tid = threadIdx.x;
    // strided: adjacent lanes take adjacent columns; contiguous: one slice per run of lanes
    const uint32_t sl = kStrided ? tid % G::kSpw : tid / G::kThreadsPerSlice;
    const uint32_t t = kStrided ? tid / G::kSpw : tid % G::kThreadsPerSlice;
    const uint32_t g = wg * G::kSpw + sl;  // global slice number
    const uint32_t low = kStrided ? (g & ((1u << s0) - 1u)) : 0u;
    const uint64_t slice_base =
        kStrided ? (uint64_t)low + ((uint64_t)(g >> s0) << (s0 + K)) : ((uint64_t)g << K);
    const uint32_t estride_log = kStrided ? s0 : 0u;
    const uint32_t lds_base = sl * G::kSlotsPerSlice;

    auto gidx = [&](uint32_t e) -> uint64_t {
        return slice_base + ((uint64_t)e << estride_log);
    };

    Fr x[G::kE];

    // Visits the elements of group GI: f(index into x, local element index e, set c).
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
                Fr v = ld_global(src + bitrev_bits((uint32_t)i, L));
                x[xi] = p.use_kscale ? fr_mul(v, p.kscale) : v;
            } else {
                x[xi] = ld_global(src + i);
            }
        });
    };
    auto store_global = [&](auto gi_c) {
        for_group(gi_c, [&](auto xi_c, uint32_t e) {
            constexpr int xi = decltype(xi_c)::value;
            const uint64_t i = gidx(e);
            const Fr v = fr_canon_4r(x[xi]);
            if constexpr (JOIN) store_h(p, i, v);
            else st_global(dst + i, v);
        });
    };
    auto lds_write = [&](auto gi_c) {
        for_group(gi_c, [&](auto xi_c, uint32_t e) {
            constexpr int xi = decltype(xi_c)::value;
            lds_put(lds, G::kPlane, lds_base + lds_slot(e), x[xi]);
        });
    };
    auto lds_read = [&](auto gi_c) {
        for_group(gi_c, [&](auto xi_c, uint32_t e) {
            constexpr int xi = decltype(xi_c)::value;
            x[xi] = lds_get(lds, G::kPlane, lds_base + lds_slot(e));
        });
    };
    auto passes = [&](auto gi_c, auto dif_c, const Fr* tw, uint32_t ls0, uint32_t llow) {
        constexpr int gi = decltype(gi_c)::value;
        constexpr bool dif = decltype(dif_c)::value;
        constexpr int b0 = G::group_b0(gi), r = G::group_r(gi);
        constexpr int nsets = 1 << (GR - r);
        static_for<nsets>([&](auto s_c) {
            constexpr int s = decltype(s_c)::value;
            group_passes<s * (1 << r), r, b0, dif, !kStrided, G::kE>(x, t * nsets + s, llow,
                                                                     ls0, L, tw);
        });
    };
    using DIT = std::false_type;
    using DIF = std::true_type;

    // One barrier after every LDS write: in each group every slot is read and then
    // rewritten by the one thread that owns it, so the only ordering needed is that a
    // group's writes land before the next group's reads.
    if constexpr (M == Mode::DitStrided || M == Mode::HeadBitrev) {
        static_for<NG>([&](auto gi_c) {
            constexpr int gi = decltype(gi_c)::value;
            if constexpr (gi == 0) load_global(gi_c);
            else lds_read(gi_c);
            passes(gi_c, DIT{}, p.tw, s0, low);
            if constexpr (gi == NG - 1) {
                store_global(gi_c);
            } else {
                lds_write(gi_c);
                __syncthreads();
            }
        });
    } else if constexpr (M == Mode::DifStrided) {
        static_for<NG>([&](auto step_c) {
            constexpr int gi = NG - 1 - decltype(step_c)::value;
            using GI = std::integral_constant<int, gi>;
            if constexpr (gi == NG - 1) load_global(GI{});
            else lds_read(GI{});
            passes(GI{}, DIF{}, p.tw, s0, low);
            if constexpr (gi == 0) {
                store_global(GI{});
            } else {
                lds_write(GI{});
                __syncthreads();
            }
        });
    } else {  // Fused: DIF groups high to low, coset multiply, DIT groups low to high
        static_for<NG>([&](auto step_c) {
            constexpr int gi = NG - 1 - decltype(step_c)::value;
            using GI = std::integral_constant<int, gi>;
            if constexpr (gi == NG - 1) load_global(GI{});
            else lds_read(GI{});
            passes(GI{}, DIF{}, p.tw, 0u, 0u);
            if constexpr (gi > 0) {
                lds_write(GI{});
                __syncthreads();
            }
        });
        // group 0 stays in registers: the coset multiply between the two transforms
        for_group(std::integral_constant<int, 0>{}, [&](auto xi_c, uint32_t e) {
            constexpr int xi = decltype(xi_c)::value;
            x[xi] = fr_mul29_lazy(x[xi], unpack29(ld_global(p.scale + gidx(e))));
        });
        static_for<NG>([&](auto gi_c) {
            constexpr int gi = decltype(gi_c)::value;
            if constexpr (gi > 0) lds_read(gi_c);
            passes(gi_c, DIT{}, p.tw_fwd, 0u, 0u);
            if constexpr (gi == NG - 1) {
                store_global(gi_c);
            } else {
                lds_write(gi_c);
                __syncthreads();
            }
        });
    }
}

}  // namespace g16
