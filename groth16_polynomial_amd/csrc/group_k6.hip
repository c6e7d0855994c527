// Register-group batch kernels in the radix-4 geometry (groups of two passes) for
// k = 6 passes per batch.
#define G16_GROUP_K 6
#include "group_inst.hpp"
