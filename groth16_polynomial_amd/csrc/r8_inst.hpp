// Defines and instantiates the launchers of the register-group batch kernel for one
// batch size G16_R8_K.
#pragma once

#include "host_util.hpp"
#include "r8_launch.hpp"

namespace g16 {

template <int K, Mode M, bool JOIN>
hipError_t launch_r8(const BatchParams& p, uint32_t n_vec, hipStream_t stream) {
    using G = R8GeomFor<K, kR8Group, M>;
    // LDS beyond the default 64 KiB has to be allowed per kernel (on the current device)
    if constexpr (G::kLdsBytes > 65536) {
        hipError_t e = allow_lds((const void*)ntt_r8_kernel<K, kR8Group, M, JOIN>, G::kLdsBytes);
        if (e != hipSuccess) return e;
    }
    const uint64_t groups = (1ull << (p.log_n - K)) / G::kSpw;
    BatchParams q = p;
    q.n_vec = n_vec;
    hipLaunchKernelGGL((ntt_r8_kernel<K, kR8Group, M, JOIN>), dim3((uint32_t)(groups * n_vec)),
                       dim3(G::kThreads), G::kLdsBytes, stream, q);
    return hipGetLastError();
}

template hipError_t launch_r8<G16_R8_K, Mode::HeadBitrev, false>(const BatchParams&, uint32_t,
                                                                 hipStream_t);
template hipError_t launch_r8<G16_R8_K, Mode::FwdStrided, false>(const BatchParams&, uint32_t,
                                                                 hipStream_t);
template hipError_t launch_r8<G16_R8_K, Mode::FwdStrided, true>(const BatchParams&, uint32_t,
                                                                hipStream_t);
template hipError_t launch_r8<G16_R8_K, Mode::InvStrided, false>(const BatchParams&, uint32_t,
                                                                 hipStream_t);
template hipError_t launch_r8<G16_R8_K, Mode::Fused, false>(const BatchParams&, uint32_t,
                                                            hipStream_t);
template hipError_t launch_r8<G16_R8_K, Mode::Fused, true>(const BatchParams&, uint32_t,
                                                           hipStream_t);

}  // namespace g16
