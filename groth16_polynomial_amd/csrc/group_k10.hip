// Register-group batch kernels (radix-4 groups of two passes, or one pass in the narrow
// geometry) for k = 10 passes per batch.
#define G16_GROUP_K 10
#include "group_inst.hpp"
