// Radix-8 batch kernels for k = 6 passes per batch.
#define G16_R8_K 6
#include "r8_inst.hpp"
