// Radix-8 batch kernels for k = 8 passes per batch.
#define G16_R8_K 8
#include "r8_inst.hpp"
