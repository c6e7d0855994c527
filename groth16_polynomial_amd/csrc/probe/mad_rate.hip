// libg16_probe.so: issue-rate microbenchmark of the integer instructions the field
// arithmetic is built from (a measurement aid for the roofline, not part of the H
// pipeline's API).
//
// Every lane runs `iters` rounds of eight independent chains of one instruction
// (v_mad_u64_u32, v_mad_i64_i32, v_add_u32, v_mul_lo_u32, v_ashrrev_i64 or
// v_alignbit_b32), written in one asm block per
// round so the compiler neither reorders nor splits them; with eight chains a result is
// reused eight instructions later, and with several waves per SIMD the pipeline latency is
// covered, so the count of instructions over the kernel time is the issue rate.  Each
// lane writes the xor of its chains (checked against a host computation, so the work is
// really done) and each wave its elapsed shader-clock count (s_memtime) and real-time count
// (s_memrealtime, 100 MHz), from which the host estimates the clock the chip ran at.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

#define G16_MAD8(OP)                                                                   \
    OP " %0, vcc, %8, %9, %0\n\t" OP " %1, vcc, %8, %9, %1\n\t" OP " %2, vcc, %8, %9, %2\n\t" \
    OP " %3, vcc, %8, %9, %3\n\t" OP " %4, vcc, %8, %9, %4\n\t" OP " %5, vcc, %8, %9, %5\n\t" \
    OP " %6, vcc, %8, %9, %6\n\t" OP " %7, vcc, %8, %9, %7\n\t"
#define G16_OP32_8(OP)                                                                  \
    OP " %0, %8, %0\n\t" OP " %1, %8, %1\n\t" OP " %2, %8, %2\n\t" OP " %3, %8, %3\n\t"     \
    OP " %4, %8, %4\n\t" OP " %5, %8, %5\n\t" OP " %6, %8, %6\n\t" OP " %7, %8, %7\n\t"

// OP 0: v_mad_u64_u32 a = x y + a; 1: v_mad_i64_i32 (signed); 2: v_add_u32 a = x + a;
// 3: v_mul_lo_u32 a = x a; 4: v_ashrrev_i64 a = a >> (x & 63) (64-bit, arithmetic);
// 5: v_alignbit_b32 a = low 32 bits of (a:x) >> 29.
template <int OP>
__global__ void __launch_bounds__(256) rate_kernel(uint32_t iters, uint32_t seed,
                                                   uint64_t* out, uint64_t* clocks) {
    const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
    const uint32_t x = (gid * 2654435761u) ^ seed;
    const uint32_t y = seed | 1u;
    uint64_t r = 0;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t u0 = __builtin_amdgcn_s_memrealtime();
    if constexpr (OP == 4) {
        uint64_t a[8];
        for (int k = 0; k < 8; ++k) a[k] = (uint64_t)(gid + k) * 0x9e3779b97f4a7c15ull;
        for (uint32_t i = 0; i < iters; ++i)
            asm volatile(
                "v_ashrrev_i64 %0, %8, %0\n\tv_ashrrev_i64 %1, %8, %1\n\t"
                "v_ashrrev_i64 %2, %8, %2\n\tv_ashrrev_i64 %3, %8, %3\n\t"
                "v_ashrrev_i64 %4, %8, %4\n\tv_ashrrev_i64 %5, %8, %5\n\t"
                "v_ashrrev_i64 %6, %8, %6\n\tv_ashrrev_i64 %7, %8, %7\n\t"
                : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                  "+v"(a[6]), "+v"(a[7])
                : "v"(x & 63u));
        for (int k = 0; k < 8; ++k) r ^= a[k];
    } else if constexpr (OP == 5) {
        uint32_t a[8];
        for (int k = 0; k < 8; ++k) a[k] = (gid + k) * 0x9e3779b9u | 1u;
        for (uint32_t i = 0; i < iters; ++i)
            asm volatile(
                "v_alignbit_b32 %0, %0, %8, 29\n\tv_alignbit_b32 %1, %1, %8, 29\n\t"
                "v_alignbit_b32 %2, %2, %8, 29\n\tv_alignbit_b32 %3, %3, %8, 29\n\t"
                "v_alignbit_b32 %4, %4, %8, 29\n\tv_alignbit_b32 %5, %5, %8, 29\n\t"
                "v_alignbit_b32 %6, %6, %8, 29\n\tv_alignbit_b32 %7, %7, %8, 29\n\t"
                : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                  "+v"(a[6]), "+v"(a[7])
                : "v"(x));
        for (int k = 0; k < 8; ++k) r ^= a[k];
    } else if constexpr (OP <= 1) {
        uint64_t a[8];
        for (int k = 0; k < 8; ++k) a[k] = (uint64_t)(gid + k) * 0x9e3779b97f4a7c15ull;
        for (uint32_t i = 0; i < iters; ++i) {
            if constexpr (OP == 0)
                asm volatile(G16_MAD8("v_mad_u64_u32")
                             : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]),
                               "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
                             : "v"(x), "v"(y)
                             : "vcc");
            else
                asm volatile(G16_MAD8("v_mad_i64_i32")
                             : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]),
                               "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
                             : "v"(x), "v"(y)
                             : "vcc");
        }
        for (int k = 0; k < 8; ++k) r ^= a[k];
    } else {
        uint32_t a[8];
        for (int k = 0; k < 8; ++k) a[k] = (gid + k) * 0x9e3779b9u | 1u;
        for (uint32_t i = 0; i < iters; ++i) {
            if constexpr (OP == 2)
                asm volatile(G16_OP32_8("v_add_u32")
                             : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]),
                               "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
                             : "v"(x));
            else
                asm volatile(G16_OP32_8("v_mul_lo_u32")
                             : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]),
                               "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
                             : "v"(x));
        }
        for (int k = 0; k < 8; ++k) r ^= a[k];
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t u1 = __builtin_amdgcn_s_memrealtime();
    out[gid] = r;
    if ((threadIdx.x & 63u) == 0u) {
        const uint32_t wave = gid >> 6;
        clocks[2 * (size_t)wave] = t1 - t0;
        clocks[2 * (size_t)wave + 1] = u1 - u0;
    }
}

#undef G16_MAD8
#undef G16_OP32_8

}  // namespace

extern "C" {

// Enqueues `blocks` workgroups of 256 lanes running the chains of instruction `op` (0..3,
// as above) for `iters` rounds of eight on `stream`.  out: one u64 per lane (blocks * 256);
// clocks: two u64 per wave (blocks * 4 * 2): elapsed s_memtime and s_memrealtime counts.
// Device pointers.  Returns 0, or -1 for a bad op or null pointer, -5 for a launch error.
int g16_probe_rate(uint32_t op, uint32_t blocks, uint32_t iters, uint32_t seed, void* out,
                   void* clocks, void* stream) {
    if (!out || !clocks || blocks == 0) return -1;
    hipStream_t s = (hipStream_t)stream;
    uint64_t* o = (uint64_t*)out;
    uint64_t* c = (uint64_t*)clocks;
    switch (op) {
        case 0: hipLaunchKernelGGL(rate_kernel<0>, dim3(blocks), dim3(256), 0, s, iters, seed, o, c); break;
        case 1: hipLaunchKernelGGL(rate_kernel<1>, dim3(blocks), dim3(256), 0, s, iters, seed, o, c); break;
        case 2: hipLaunchKernelGGL(rate_kernel<2>, dim3(blocks), dim3(256), 0, s, iters, seed, o, c); break;
        case 3: hipLaunchKernelGGL(rate_kernel<3>, dim3(blocks), dim3(256), 0, s, iters, seed, o, c); break;
        case 4: hipLaunchKernelGGL(rate_kernel<4>, dim3(blocks), dim3(256), 0, s, iters, seed, o, c); break;
        case 5: hipLaunchKernelGGL(rate_kernel<5>, dim3(blocks), dim3(256), 0, s, iters, seed, o, c); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
