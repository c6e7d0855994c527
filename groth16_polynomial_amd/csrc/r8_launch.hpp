// Launchers of the register-group batch kernel (ntt_r8.hpp), one translation unit per
// batch size k (r8_k<k>.hip) so the large unrolled kernels compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace g16 {

constexpr int kR8MinK = 6;
constexpr int kR8MaxK = 10;
// Passes per register group (each thread holds 2^kR8Group elements).
#ifndef G16_R8_GROUP
#define G16_R8_GROUP 2
#endif
constexpr int kR8Group = G16_R8_GROUP;

// Enqueues ntt_r8_kernel<K, kR8Group, M, JOIN> over 2^(log_n - K) slices, n_vec vectors.
template <int K, Mode M, bool JOIN>
hipError_t launch_r8(const BatchParams& p, uint32_t n_vec, hipStream_t stream);

}  // namespace g16
