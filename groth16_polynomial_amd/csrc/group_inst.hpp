// Defines and instantiates the launchers of the register-group batch kernel for one
// batch size G16_GROUP_K.
#pragma once

#include "host_util.hpp"
#include "group_launch.hpp"

namespace g16 {

template <int K, int GR, int SPW, Mode M, bool JOIN, int NK = 1>
hipError_t launch_geom(const BatchParams& p, uint32_t n_vec, hipStream_t stream) {
    using G = GroupGeom<K, GR, SPW>;
    constexpr size_t lds = size_t(NK) * G::kLdsBytes;
    // LDS beyond the default 64 KiB has to be allowed per kernel (on the current device)
    if constexpr (lds > 65536) {
        hipError_t e = allow_lds((const void*)ntt_group_kernel<K, GR, M, JOIN, SPW, NK>, lds);
        if (e != hipSuccess) return e;
    }
    const uint64_t groups = (1ull << (p.log_n - K)) / G::kSpw;
    BatchParams q = p;
    q.n_vec = n_vec;
    hipLaunchKernelGGL((ntt_group_kernel<K, GR, M, JOIN, SPW, NK>),
                       dim3((uint32_t)(groups * n_vec)), dim3(G::kThreads * NK), lds, stream, q);
    return hipGetLastError();
}

#ifndef G16_GROUP_NARROW
template <int K, Mode M, bool JOIN>
hipError_t launch_groups_wide(const BatchParams& p, uint32_t n_vec, hipStream_t stream) {
    return launch_geom<K, kGroupPasses, slices_per_wg(K, M), M, JOIN>(p, n_vec, stream);
}

#define G16_INST(M, J)                                                                   \
    template hipError_t launch_groups_wide<G16_GROUP_K, M, J>(const BatchParams&, uint32_t, \
                                                              hipStream_t);
#else
template <int K, Mode M, bool JOIN>
hipError_t launch_groups_narrow(const BatchParams& p, uint32_t n_vec, hipStream_t stream) {
    return launch_geom<K, 1, narrow_slices_per_wg(K, M), M, JOIN>(p, n_vec, stream);
}

template <int K, Mode M>
hipError_t launch_groups_join3(const BatchParams& p, uint32_t n_proof, hipStream_t stream) {
    if constexpr (!narrow_join3_fits<K, M>()) {
        return hipErrorInvalidValue;
    } else {
        return launch_geom<K, 1, narrow_slices_per_wg(K, M), M, true, 3>(p, n_proof, stream);
    }
}

template hipError_t launch_groups_join3<G16_GROUP_K, Mode::FwdStrided>(const BatchParams&,
                                                                      uint32_t, hipStream_t);
template hipError_t launch_groups_join3<G16_GROUP_K, Mode::Fused>(const BatchParams&, uint32_t,
                                                                 hipStream_t);

#define G16_INST(M, J)                                                                     \
    template hipError_t launch_groups_narrow<G16_GROUP_K, M, J>(const BatchParams&, uint32_t, \
                                                                hipStream_t);
#endif

G16_INST(Mode::HeadBitrev, false)
G16_INST(Mode::FwdStrided, false)
G16_INST(Mode::FwdStrided, true)
G16_INST(Mode::InvStrided, false)
G16_INST(Mode::Fused, false)
G16_INST(Mode::Fused, true)
#undef G16_INST

}  // namespace g16
