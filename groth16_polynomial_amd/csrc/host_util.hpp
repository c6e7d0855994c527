// Host-side helpers shared by the entry points of libg16.so: the check that a caller's
// buffer is device memory, and the per-kernel LDS limit.  Both sit on the launch path of
// every call, so each remembers what it has already established instead of asking the
// HIP runtime again (a single-proof 2^12 pipeline is four launches of a few microseconds
// each, where the runtime queries were a visible share of the host time).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

namespace g16 {

// True when [p, p + bytes) is device (or managed) memory of one allocation.  A miss asks
// the runtime for the pointer's memory type and its allocation's range; the ranges found
// to be device memory are remembered per thread (16 of them, oldest replaced first), so a
// caller that reuses its buffers pays the runtime query once per allocation.  A range
// stays trusted after the caller frees it: the check guards against host pointers and
// buffers shorter than the call needs, not against use after free.
inline bool device_range(const void* p, size_t bytes) {
    if (!p) return false;
    struct Range {
        uintptr_t base, end;
    };
    thread_local Range seen[16] = {};
    thread_local unsigned next = 0;
    const uintptr_t a = (uintptr_t)p;
    const uintptr_t e = a + bytes;
    if (e < a) return false;
    for (const Range& r : seen)
        if (r.end && a >= r.base && e <= r.end) return true;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged &&
        attr.type != hipMemoryTypeUnified)
        return false;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess || !base ||
        !size) {
        // no range known for this kind of memory: the type check alone, nothing remembered
        (void)hipGetLastError();
        return true;
    }
    const uintptr_t b = (uintptr_t)base;
    if (a < b || e > b + size) return false;  // the buffer runs past its allocation
    seen[next++ % 16] = Range{b, b + size};
    return true;
}

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device (needed above
// 64 KiB), once per kernel, device and limit: later calls find it in a short list.
inline hipError_t allow_lds(const void* kernel, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    struct Entry {
        const void* kernel;
        int device;
        size_t bytes;
    };
    static std::mutex mu;
    static Entry done[256];
    static unsigned count = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    for (unsigned i = 0; i < count; ++i)
        if (done[i].kernel == kernel && done[i].device == dev && done[i].bytes >= bytes)
            return hipSuccess;
    const hipError_t e =
        hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && count < 256) done[count++] = Entry{kernel, dev, bytes};
    return e;
}

}  // namespace g16
