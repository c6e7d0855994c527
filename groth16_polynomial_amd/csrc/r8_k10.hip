// Radix-8 batch kernels for k = 10 passes per batch.
#define G16_R8_K 10
#include "r8_inst.hpp"
