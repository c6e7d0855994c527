// Launchers of the register-group batch kernel (ntt_groups.hpp), one translation unit per
// batch size k (group_k<k>.hip) so the large unrolled kernels compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace g16 {

constexpr int kGroupMinK = 6;
constexpr int kGroupMaxK = 10;
// Passes per register group (each thread holds 2^kGroupPasses elements).
#ifndef G16_GROUP_PASSES
#define G16_GROUP_PASSES 2
#endif
constexpr int kGroupPasses = G16_GROUP_PASSES;

// Enqueues ntt_group_kernel for batch size K over 2^(log_n - K) slices, n_vec vectors: the
// radix-4 groups (GroupGeomFor<K, kGroupPasses, M>) or, with narrow, one pass per group
// (NarrowGeomFor<K, M>).  2^(log_n - K) must be at least the geometry's slices per
// workgroup.
// The two geometries are instantiated in separate units (group_kK.hip and
// group_kK_narrow.hip), which the build compiles with different scheduling.
template <int K, Mode M, bool JOIN>
hipError_t launch_groups_wide(const BatchParams& p, uint32_t n_vec, hipStream_t stream);
template <int K, Mode M, bool JOIN>
hipError_t launch_groups_narrow(const BatchParams& p, uint32_t n_vec, hipStream_t stream);

template <int K, Mode M, bool JOIN>
inline hipError_t launch_groups(const BatchParams& p, uint32_t n_vec, bool narrow,
                                hipStream_t stream) {
    return narrow ? launch_groups_narrow<K, M, JOIN>(p, n_vec, stream)
                  : launch_groups_wide<K, M, JOIN>(p, n_vec, stream);
}

// The last launch of the pipeline (M = FwdStrided or Fused, with the join) in the narrow
// geometry with the three kinds of a proof in one workgroup, over n_proof proofs
// (ntt_group_kernel with NK = 3); hipErrorInvalidValue where three kinds exceed a
// workgroup (narrow_join3_fits).
template <int K, Mode M>
hipError_t launch_groups_join3(const BatchParams& p, uint32_t n_proof, hipStream_t stream);

}  // namespace g16
