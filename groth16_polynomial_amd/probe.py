"""Instruction issue rates on the device (libg16_probe.so), for the roofline's peak.

The field arithmetic of the transforms is built from 64-bit integer multiply-adds
(v_mad_i64_i32 / v_mad_u64_u32) and 32-bit adds, shifts and masks.  MI355X's integer
rates are not published, so the benchmark measures them: eight independent chains of one
instruction per lane over many waves, the instruction count over the kernel time.  Each
lane's result is checked against the same chains computed here, so the timed work is
known to have run.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(_PKG, "libg16_probe.so")

OPS = {0: "v_mad_u64_u32", 1: "v_mad_i64_i32", 2: "v_add_u32", 3: "v_mul_lo_u32",
       4: "v_ashrrev_i64", 5: "v_alignbit_b32"}
CHAINS = 8
LANES = 256           # per workgroup
WAVES_PER_GROUP = 4
M64 = (1 << 64) - 1
M32 = (1 << 32) - 1
REALTIME_HZ = 100e6   # s_memrealtime counts at 100 MHz

_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError("libg16_probe.so is not built (%s); run __graft_entry__.build()"
                               % PROBE_PATH)
        lib = ctypes.CDLL(PROBE_PATH)
        lib.g16_probe_rate.restype = ctypes.c_int
        lib.g16_probe_rate.argtypes = [ctypes.c_uint32] * 4 + [ctypes.c_void_p] * 3
        _lib = lib
    return _lib


def expected(op: int, blocks: int, iters: int, seed: int) -> np.ndarray:
    """Each lane's xor of its chains after `iters` rounds, computed on the host."""
    gid = np.arange(blocks * LANES, dtype=np.uint64)
    x = ((gid * np.uint64(2654435761)) & np.uint64(M32)) ^ np.uint64(seed)
    y = np.uint64(seed | 1)
    out = np.zeros(len(gid), dtype=np.uint64)
    with np.errstate(over="ignore"):
        for k in range(CHAINS):
            if op in (0, 1):
                a = (gid + np.uint64(k)) * np.uint64(0x9E3779B97F4A7C15)
                if op == 0:
                    prod = x * y
                else:  # signed 32 x 32 -> 64, reduced mod 2^64
                    xs = x.astype(np.uint32).astype(np.int32).astype(np.int64)
                    ys = np.int64(np.uint32(seed | 1).astype(np.int32))
                    prod = (xs * ys).astype(np.uint64)
                a = a + np.uint64(iters) * prod
            elif op == 4:  # arithmetic shift right by x & 63, iters times: by the sum,
                # capped at 63 (the sign fills everything from there on)
                a = ((gid + np.uint64(k)) * np.uint64(0x9E3779B97F4A7C15)).view(np.int64)
                sh = np.minimum((x & np.uint64(63)) * np.uint64(iters), np.uint64(63))
                a = (a >> sh.astype(np.int64)).view(np.uint64)
            elif op == 5:  # a = low 32 bits of (a:x) >> 29 = (a << 3) | (x >> 29); after
                # 11 rounds every starting bit has left and a repeats x's top three bits
                a = (((gid + np.uint64(k)) * np.uint64(0x9E3779B9)) | np.uint64(1)) & np.uint64(M32)
                for _ in range(min(iters, 11)):
                    a = ((a << np.uint64(3)) | (x >> np.uint64(29))) & np.uint64(M32)
            elif op == 2:
                a = (((gid + np.uint64(k)) * np.uint64(0x9E3779B9)) | np.uint64(1)) & np.uint64(M32)
                a = (a + np.uint64(iters) * x) & np.uint64(M32)
            else:
                a = (((gid + np.uint64(k)) * np.uint64(0x9E3779B9)) | np.uint64(1)) & np.uint64(M32)
                p = np.ones_like(x)
                base, e = x.copy(), iters
                while e:
                    if e & 1:
                        p = (p * base) & np.uint64(M32)
                    base = (base * base) & np.uint64(M32)
                    e >>= 1
                a = (a * p) & np.uint64(M32)
            out ^= a
    return out


def run(op: int, blocks: int, iters: int, seed: int = 12345, reps: int = 3):
    """Times the chains of instruction `op`; returns a dict with the best rate (lane
    instructions per second over the kernel time, HIP events), the clock estimated from
    the waves' s_memtime / s_memrealtime counts, and whether every lane's result matched."""
    import torch
    lib = load()
    out = torch.empty(blocks * LANES, dtype=torch.int64, device="cuda")
    clocks = torch.empty(blocks * WAVES_PER_GROUP * 2, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def launch():
        rc = lib.g16_probe_rate(op, blocks, iters, seed, out.data_ptr(), clocks.data_ptr(),
                                stream.cuda_stream)
        if rc:
            raise RuntimeError("g16_probe_rate failed (%d)" % rc)

    launch()  # warm-up
    best_ms = None
    for _ in range(reps):
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best_ms = ms if best_ms is None else min(best_ms, ms)
    got = out.cpu().numpy().view(np.uint64)
    ok = bool(np.array_equal(got, expected(op, blocks, iters, seed)))
    c = clocks.cpu().numpy().view(np.uint64).reshape(-1, 2).astype(np.float64)
    ghz = float(np.median(c[:, 0] / np.maximum(c[:, 1], 1.0)) * REALTIME_HZ / 1e9)
    lane_ops = float(blocks) * LANES * iters * CHAINS
    rate = lane_ops / (best_ms / 1e3)
    return {"op": OPS[op], "lane_ops_per_s_t": rate / 1e12, "kernel_ms": best_ms,
            "clock_ghz_est": ghz, "results_match": ok}
