// Register-group batch kernels in the narrow geometry (one pass per group) for k = 8
// passes per batch, with the three-kind last batch of small launches.
#define G16_GROUP_K 8
#define G16_GROUP_NARROW 1
#include "group_inst.hpp"
