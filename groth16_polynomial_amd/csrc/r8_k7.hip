// Radix-8 batch kernels for k = 7 passes per batch.
#define G16_R8_K 7
#include "r8_inst.hpp"
