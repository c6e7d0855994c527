// Radix-8 batch kernels for k = 9 passes per batch.
#define G16_R8_K 9
#include "r8_inst.hpp"
