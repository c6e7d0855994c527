/*
 * g16_probe.h -- C ABI of libg16_probe.so, an instruction issue-rate microbenchmark.
 *
 * Not part of the H pipeline: it measures, on the device, how fast the instructions the
 * field arithmetic is built from issue, because the integer rates of the chip are not
 * published (the forum post on GPU WHIR proving, section 5, makes the same complaint
 * about Apple's GPUs) and the benchmark's ALU roofline needs them.
 */
#ifndef G16_PROBE_H
#define G16_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues on `stream` (hipStream_t as void*) `blocks` workgroups of 256 lanes; each lane
 * runs `iters` rounds of eight independent chains of instruction `op`:
 *   0 v_mad_u64_u32  a = x * y + a (64-bit accumulator)
 *   1 v_mad_i64_i32  the same, signed operands
 *   2 v_add_u32      a = x + a
 *   3 v_mul_lo_u32   a = x * a (low 32 bits)
 *   4 v_ashrrev_i64  a = a >> (x & 63) (64-bit accumulator, arithmetic shift)
 *   5 v_alignbit_b32 a = low 32 bits of ((a << 32 | x) >> 29)
 * with x = (lane id * 2654435761) ^ seed and y = seed | 1 (a lane's chain k starts from
 * (lane id + k) * 0x9e3779b97f4a7c15 for the 64-bit ops, (lane id + k) * 0x9e3779b9 | 1 for
 * the 32-bit ones; op 4 starts as ops 0 and 1).  Writes the xor of the lane's eight chains to out[lane] (u64, device,
 * blocks * 256 entries) and, per wave w, the elapsed s_memtime and s_memrealtime counts to
 * clocks[2w], clocks[2w + 1] (u64, device, blocks * 8 entries).  Returns 0, -1 for a bad op,
 * a null pointer or zero blocks, -5 for a launch error. */
int g16_probe_rate(uint32_t op, uint32_t blocks, uint32_t iters, uint32_t seed, void* out,
                   void* clocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* G16_PROBE_H */
