#!/usr/bin/env python3
"""Benchmark of the Groth16 H-polynomial pipeline on one MI355X.

One step = one g16_h_compute over device-resident inputs at n = 2^20 (A, B seeded
uniform Fr, C = A o B, tables prepared beforehand): three inverse NTTs, the coset
shift, three forward NTTs and H = A'B' - C' in both encodings.  Prints one JSON line.
The K timed steps follow --settle-ms of untimed pipelines (the chip reaches its working
clock only after some tens of ms of sustained load) and the W warmup steps.

Also measured (same run, reported inside the line):
  * each kernel (stage) of the pipeline alone, with HIP events on the stream it is
    launched on; the slowest is the dominant kernel and carries the roofline;
  * the instruction issue rates of the arithmetic's building blocks (the probe
    library), which give the measured multiply-add rate beside the nominal peak;
  * the other workloads: the 2^12 pipeline (median per call and launch count), the
    standalone forward and inverse NTT at 2^18 and 2^20, the CSR gather and the gather
    plus pipeline at 2^18, the 2^22 pipeline, several proofs per call, the H MSM;
  * the CPU oracle on the host, one thread and all threads, median of three, on the
    same 2^20 workload.

Units.  Work is counted in 32 x 32-bit limb products of the textbook 8-limb CIOS
Montgomery product: 136 per field product, 72 per reduction.  A transform of n points
has n/2 log n butterflies of one product each (twiddle-1 butterflies included); the H
pipeline adds n products for the 1/n scaling, n for the coset shift (both per vector)
and n for the join, plus n reductions: 70.25 M products and 9.63 G limb products at
2^20.  Algorithmic bytes count every transform as two HBM round trips of 32-byte
elements, the shift table and the join's extra reads and second output: 960 bytes per
element.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

NOMINAL_PEAK_T = 256 * 64 * 2.4e9 / 1e12  # 256 CUs x 64 lanes x 2.4 GHz, one op a lane a clock
HBM_PEAK_GBS = 8000.0
MADS_PER_MUL = 136                      # 8-limb CIOS Montgomery product: 2 s^2 + s
MADS_PER_REDC = 72                      # Montgomery reduction alone: s^2 + s
FR_BYTES = 32
ALG_BYTES_PER_ELEMENT = 960             # six transforms x two round trips x 64 + 96 + 96
# (log n, proofs) of the several-proofs-per-call measurements: small domains, where one
# call per proof is launch-bound
BATCH_SHAPES = ((12, 64), (16, 16))


def parse():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed pipelines run before the warmup steps, in ms of wall time")
    ap.add_argument("--log-n", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="only the timed 2^log_n pipeline and its stages (for profiling)")
    ap.add_argument("--part", choices=("all", "h", "msm", "bb", "probe"), default="all",
                    help="h: only the timed pipeline and its stages (as --no-side, no CPU "
                         "baseline); msm: only the G1 MSM legs; bb: only the BabyBear "
                         "encoding legs; probe: only the instruction-rate probe (for "
                         "profiling)")
    ap.add_argument("--stage-reps", type=int, default=10)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (a known-size "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def stage_work(kind: str, join: bool, n_vec: int, k: int, n: int):
    """Algorithmic (field products, reductions, bytes) of one pipeline stage.

    Strided batch of k passes on n_vec vectors: n_vec k n/2 butterflies, one product
    each; one read and one write per element.  Fused lowest batch: the last k passes of
    the inverse and the first k of the forward transform (2k n/2 butterflies), the 1/n
    scaling and the coset shift (two products per element, performed here as one product
    by one of four resident constants), and, as the pipeline's algorithmic byte count
    (960 bytes per element) has it, one read of a shift table per element.  Join: A'B' (one product),
    h_std (one reduction); writes h_mont and h_std instead of the vectors, and reads A'
    and B' when C runs alone (n_vec = 1; with all three kinds in the launch they meet in
    LDS).
    """
    if kind == "fused":
        muls = n_vec * (2 * k * n // 2 + 2 * n)
    else:
        muls = n_vec * k * n // 2
    reads = n_vec + (2 if join and n_vec == 1 else 0)
    writes = 2 if join else n_vec
    byts = (reads + writes) * n * FR_BYTES
    if kind == "fused":
        byts += n_vec * n * FR_BYTES    # a shift table (counted; the kernel reads none)
    redc = 0
    if join:
        muls += n
        redc = n
    return muls, redc, byts


def mads(muls: int, redc: int) -> int:
    return muls * MADS_PER_MUL + redc * MADS_PER_REDC


def stage_list(plan, count, n_vec=3):
    """(kind, join, n_vec, k) of each stage of g16_h_compute, in launch order; `count` is
    the library's stage count, which tells whether the last forward batch runs A, B and C
    in one launch (with the join) or C in a launch of its own."""
    nb = len(plan)
    out = []
    if nb == 1:
        if count == 1:
            return [("fused", True, n_vec, plan[0])]
        return [("fused", False, n_vec - 1, plan[0]), ("fused", True, 1, plan[0])]
    merged = count == 2 * (nb - 1) + 1
    for b in range(nb - 1, 0, -1):
        out.append(("inv", False, n_vec, plan[b]))
    out.append(("fused", False, n_vec, plan[0]))
    for b in range(1, nb):
        if b == nb - 1 and merged:
            out.append(("fwd", True, n_vec, plan[b]))
        elif b == nb - 1:
            out.append(("fwd", False, n_vec - 1, plan[b]))
            out.append(("fwd", True, 1, plan[b]))
        else:
            out.append(("fwd", False, n_vec, plan[b]))
    return out


def pipeline_work(log_n: int):
    """(products, reductions, algorithmic bytes) of one H pipeline at 2^log_n."""
    n = 1 << log_n
    muls = 6 * (n // 2) * log_n + 7 * n
    return muls, n, ALG_BYTES_PER_ELEMENT * n


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace (what the compiler sees of it, up to
    string literals, which the kernel sources use only for asm text without '//')."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


# Sources of the G1 MSM only; the H pipeline's kernels are built from the others.
MSM_SOURCES = {"fp.hpp", "fp29.hpp", "fp29_cols.hpp", "fp29_cols_gen.py", "g1.hpp", "msm.hip",
               "msm_digit.hpp", "msm_kernels.hpp"}


# Sources of the BabyBear transform only.
BB_SOURCES = {"bb.hip", "bb_field.hpp", "bb_ntt.hpp"}


def kernel_source_hash() -> str:
    """Hash of the H pipeline's kernel sources' code (comments and whitespace ignored),
    which ties a committed counter summary to the kernels it was measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "groth16_polynomial_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f in MSM_SOURCES or f in BB_SOURCES or not os.path.isfile(os.path.join(csrc, f)):
            continue
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(stage_name: str, src_hash: str):
    """HBM bytes per dispatch of the dominant kernel, from the committed counter
    summary, if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != src_hash:
        return None
    return d.get("stages", {}).get(stage_name, {}).get("hbm_bytes_per_dispatch")


class Timer:
    """HIP events on torch's current stream, which is the stream the library launches on.

    From idle the chip needs some tens of milliseconds of sustained load to reach its
    working clock (2^20 pipelines back to back after 2 s idle: 0.68 ms a step for the
    first 20, 0.48-0.50 ms from about 60 ms on), and the host work between legs lets it
    fall back, so every measurement first runs its call untimed for settle_ms."""

    def __init__(self, torch, settle_ms=50.0):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)
        self.settle_ms = settle_ms

    def settle(self, fn, ms=None, warm=3):
        """Runs fn untimed at least `warm` times and for at least `ms` milliseconds of
        wall time (in chunks, each waited for); returns the number of calls."""
        ms = self.settle_ms if ms is None else ms
        end = time.perf_counter() + ms / 1e3
        calls = 0
        while calls < warm or time.perf_counter() < end:
            for _ in range(max(1, warm)):
                fn()
            calls += max(1, warm)
            self.torch.cuda.synchronize()
        return calls

    def mean_ms(self, fn, reps, warm=3):
        self.settle(fn, warm=warm)
        self.e0.record(self.stream)
        for _ in range(reps):
            fn()
        self.e1.record(self.stream)
        self.torch.cuda.synchronize()
        return self.e0.elapsed_time(self.e1) / reps

    def median_ms(self, fn, reps, warm=3):
        """Median over reps calls, each between its own pair of events."""
        torch = self.torch
        self.settle(fn, warm=warm)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(self.stream)
            fn()
            b.record(self.stream)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in evs)


def gbfly(log_n, transforms, ms):
    return transforms * ((1 << log_n) // 2) * log_n / (ms / 1e3) / 1e9


def probe_rates(log):
    """The issue rate of the arithmetic's instructions: v_mad_i64_i32 (the transforms'
    digit products), v_mad_u64_u32, v_add_u32, v_mul_lo_u32, v_ashrrev_i64 (the digit
    products' carries) and v_alignbit_b32; 2048 workgroups of 256 lanes (eight per CU),
    4096 (1024 for the multiply and the shift) rounds of eight chains each."""
    from groth16_polynomial_amd import probe
    out = {}
    for op in (1, 0, 2, 3, 4, 5):
        r = probe.run(op, blocks=2048, iters=4096 if op not in (3, 4) else 1024)
        if not r["results_match"]:
            raise RuntimeError("probe %s: lane results differ from the host's" % r["op"])
        out[r["op"]] = {"t_lane_ops_s": round(r["lane_ops_per_s_t"], 3),
                        "clock_ghz_est": round(r["clock_ghz_est"], 3),
                        "kernel_ms": round(r["kernel_ms"], 4)}
    log("probe: %s" % out)
    return out


# The BabyBear Reed-Solomon encodings (the WHIR forum post's NTT): (label, log_n rows out,
# log_w columns, rate): the n = 24 cells of the post's grids with fold 3 and fold 1 at
# rate 1, the n = 22 fold-3 cell, and one unfolded polynomial of 2^23 coefficients.
BB_SHAPES = (("n=24 fold=3 rate=1", 22, 3, 1), ("n=24 fold=1 rate=1", 24, 1, 1),
             ("n=22 fold=3 rate=1", 20, 3, 1), ("2^23 coefficients rate=1", 24, 0, 1))


def bb_leg(g, synth, torch, tm, steps, log):
    """Times g16_bb_lde on the BB_SHAPES: output words per second; bytes the batches move
    (the first reads the input and writes the output, each later one reads and writes the
    output) and the minimum (input once, output once) per second; butterflies per
    second."""
    out = {}
    for label, log_n, log_w, rate in BB_SHAPES:
        log_in = log_n - rate
        ctx = g.BbContext(log_n)
        x = g.bb_to_mont(g.bb_to_device(synth.bb_lde_input(40, log_in, log_w)))
        y = torch.empty(1 << (log_n + log_w), dtype=torch.int32, device="cuda")
        ms = tm.mean_ms(lambda: ctx.lde(x, log_in=log_in, log_w=log_w, out=y), steps)
        n_out = 1 << (log_n + log_w)
        n_in = 1 << (log_in + log_w)
        plan = g.bb_batch_plan(log_n)
        moved = 4 * (n_in + n_out) + (len(plan) - 1) * 8 * n_out
        minimum = 4 * (n_in + n_out)
        bfly = (n_out // 2) * log_n
        out[label] = {
            "log_n": log_n, "log_w": log_w, "rate": rate, "pass_batches": plan,
            "ms": round(ms, 5),
            "g_words_out_s": round(n_out / (ms / 1e3) / 1e9, 3),
            "gbutterfly_s": round(bfly / (ms / 1e3) / 1e9, 3),
            "hbm_gbs_batches": round(moved / (ms / 1e3) / 1e9, 1),
            "hbm_gbs_minimum": round(minimum / (ms / 1e3) / 1e9, 1),
            "hbm_frac_batches": round(moved / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        ctx.release()
        del x, y
    log("bb: %s" % out)
    return out


def hs_of(ctx, ad, bd, cd, hm, hs):
    """h_std of the timed pipeline (the MSM's input in a prover)."""
    ctx.h_compute(ad, bd, cd, hm, hs)
    return hs


def msm_leg(g, synth, torch, tm, hs, log_n, steps, log):
    """The H MSM: sum_i h_i P_i over G1 on the pipeline's own h_std, with synthetic bases
    (multiples s_i G of the generator stand in for the proving key's points); then the
    same call at 2^12, 2^16 and 2^22 on uniform scalars k_i over bases k_i G."""
    n = 1 << log_n
    bases = g.g1_generator_mul(g.to_device(synth.uniform_fr(7, n)))
    mctx = g.MsmG1(n)
    msm_reps = max(1, steps // 4)
    msm_ms = tm.mean_ms(lambda: mctx.window_sums(hs, bases), msm_reps, warm=2)
    sums_host = g.to_host(mctx.sums).reshape(mctx.windows, 32)
    t_fin = time.perf_counter()
    for _ in range(10):
        mctx.finish(sums_host)
    finish_ms = (time.perf_counter() - t_fin) / 10 * 1e3
    line = {
        "workload": "G1 MSM of h_std at n=2^%d, bases s_i G (synthetic)" % log_n,
        "window_bits": mctx.c,
        "windows": mctx.windows,
        "device_ms": round(msm_ms, 4),
        "host_finish_ms": round(finish_ms, 4),
        "bucket_adds_per_s_g": round(n * mctx.windows / (msm_ms / 1e3) / 1e9, 3),
    }
    del bases, mctx
    if log_n == 20:
        sizes = {}
        for lg in (12, 16, 22):
            m = 1 << lg
            ks = g.to_device(synth.uniform_fr(8, m))
            mb = g.g1_generator_mul(ks)
            mc = g.MsmG1(m)
            t_ms = tm.mean_ms(lambda: mc.window_sums(ks, mb), 5, warm=2)
            sizes["2^%d" % lg] = {"window_bits": mc.c, "device_ms": round(t_ms, 4),
                                  "bucket_adds_per_s_g":
                                      round(m * mc.windows / (t_ms / 1e3) / 1e9, 3)}
            del ks, mb, mc
        torch.cuda.empty_cache()
        line["other_sizes"] = sizes
    log("msm: %s" % line)
    return line


def copy_calibration(torch, mib):
    """A plain device copy of mib MiB, three times: a kernel of known traffic that scales
    rocprofv3's FETCH_SIZE and WRITE_SIZE of the same run."""
    if not mib:
        return None
    nbytes = mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    return nbytes


def main():
    args = parse()
    if args.part == "h":
        args.no_side = True
        args.no_cpu_baseline = True
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU (--gpus %d requested); sharding "
              "across GPUs is designed but not implemented"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from groth16_polynomial_amd import binding as g
    from groth16_polynomial_amd import synth

    def log(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    log_n = args.log_n
    n = 1 << log_n
    log("preparing 2^%d inputs" % log_n)

    a, b = synth.h_inputs(3, log_n)
    ad, bd = g.to_mont(g.to_device(a)), g.to_mont(g.to_device(b))
    cd = g.fr_mul(ad, bd)
    ctx = g.HContext(log_n)
    hm, hs = g.empty_fr(n), g.empty_fr(n)
    stream = torch.cuda.current_stream()
    tm = Timer(torch, settle_ms=min(50.0, args.settle_ms))
    torch.cuda.synchronize()
    line_extra = {}
    if args.part == "probe":
        print(json.dumps({"instruction_rates": probe_rates(log)}), flush=True)
        ctx.release()
        return
    if args.part == "bb":
        out = {"bb_lde": bb_leg(g, synth, torch, tm, args.steps, log),
               "copy_calibration_bytes": copy_calibration(torch, args.copy_calibration_mib)}
        print(json.dumps(out), flush=True)
        ctx.release()
        return
    if args.part == "msm":
        out = {"msm_g1": msm_leg(g, synth, torch, tm, hs_of(ctx, ad, bd, cd, hm, hs), log_n,
                                 args.steps, log),
               "copy_calibration_bytes": copy_calibration(torch, args.copy_calibration_mib)}
        print(json.dumps(out), flush=True)
        ctx.release()
        return

    # The side measurements run first: they also bring the chip to its steady clock,
    # which the first ~20 ms of sustained load does not run at.
    if not args.no_side:
        rates = probe_rates(log)
        line_extra["instruction_rates"] = rates

        # ---- standalone transforms: 2^18 (its own workload) and 2^log_n, both directions
        ntt = {}
        for lg in sorted({18, log_n}):
            nctx = ctx if lg == log_n else g.HContext(lg)
            x = g.to_mont(g.to_device(synth.ntt_input(2, lg)))
            y = g.empty_fr(1 << lg)
            fwd = tm.mean_ms(lambda: nctx.ntt_forward(x, y), args.steps)
            inv = tm.mean_ms(lambda: nctx.ntt_inverse(x, y), args.steps)
            ntt["2^%d" % lg] = {"forward_ms": round(fwd, 5),
                                "forward_gbutterfly_s": round(gbfly(lg, 1, fwd), 3),
                                "inverse_ms": round(inv, 5),
                                "inverse_gbutterfly_s": round(gbfly(lg, 1, inv), 3),
                                "pass_batches": g.batch_plan(lg)}
            if nctx is not ctx:
                nctx.release()
            del x, y
        line_extra["ntt"] = ntt
        log("ntt: %s" % ntt)

        # ---- the CSR gather front end on the 2^18 proving-key shape (the GATHER_CU
        # page's largest key, synthetic rows with its statistics), alone and followed by
        # the 2^18 H pipeline
        ma, mb, wit = synth.gather_inputs(4)

        def idx(v):
            return torch.from_numpy(np.ascontiguousarray(v, np.uint32).view(np.int32)).cuda()

        ga = (idx(ma.row_ptr), idx(ma.signal), g.to_mont(g.to_device(ma.value)))
        gb = (idx(mb.row_ptr), idx(mb.signal), g.to_mont(g.to_device(mb.value)))
        gw = g.to_mont(g.to_device(wit))
        grows = len(ma.row_ptr) - 1
        gouts = [g.empty_fr(grows) for _ in range(3)]
        gctx = g.HContext(18)
        ghm, ghs = g.empty_fr(grows), g.empty_fr(grows)
        gather_ms = tm.mean_ms(lambda: g.gather_abc(*ga, *gb, gw, *gouts), args.steps)

        def gather_h():
            g.gather_abc(*ga, *gb, gw, *gouts)
            gctx.h_compute(*gouts, ghm, ghs)

        gather_h_ms = tm.mean_ms(gather_h, args.steps)
        h18_ms = tm.mean_ms(lambda: gctx.h_compute(*gouts, ghm, ghs), args.steps)
        gctx.release()
        nnz = ma.nnz + mb.nnz
        # algorithmic bytes: row pointers, column indices and coefficients of both matrices,
        # one 32-byte witness read per non-zero, three 32-byte outputs per row
        gather_bytes = 2 * 4 * (grows + 1) + nnz * (4 + 32 + 32) + 3 * 32 * grows
        line_extra["gather_2_18"] = {
            "gather_ms": round(gather_ms, 5),
            "gather_gnnz_s": round(nnz / (gather_ms / 1e3) / 1e9, 3),
            "gather_hbm_gbs_algorithmic": round(gather_bytes / (gather_ms / 1e3) / 1e9, 2),
            "gather_plus_h_ms": round(gather_h_ms, 5),
            "h_only_ms": round(h18_ms, 5),
            "nnz": nnz, "rows": grows,
        }
        del ga, gb, gw, gouts, ghm, ghs
        log("gather: %s" % line_extra["gather_2_18"])

        # ---- several proofs per call at small domains, against one call per proof
        proof_batches = {}
        for blog, proofs in BATCH_SHAPES:
            bn = 1 << blog
            bctx = g.HContext(blog)
            pa = torch.cat([g.to_mont(g.to_device(synth.h_inputs(2000 + q, blog)[0]))
                            for q in range(proofs)])
            pb = torch.cat([g.to_mont(g.to_device(synth.h_inputs(2000 + q, blog)[1]))
                            for q in range(proofs)])
            pc = g.fr_mul(pa, pb)
            phm, phs = torch.empty_like(pa), torch.empty_like(pa)
            pscr = g.empty_fr(proofs * bn)
            batched = tm.mean_ms(lambda: bctx.h_compute_batch(pa, pb, pc, phm, phs, pscr),
                                 args.steps)

            def one_by_one():
                for q in range(proofs):
                    sl = slice(q * bn, (q + 1) * bn)
                    bctx.h_compute(pa[sl], pb[sl], pc[sl], phm[sl], phs[sl])

            single = tm.mean_ms(one_by_one, max(1, args.steps // 4))
            proof_batches["2^%d_x%d" % (blog, proofs)] = {
                "batch_ms": round(batched, 5),
                "batch_gbutterfly_s": round(proofs * gbfly(blog, 6, batched), 3),
                "one_call_per_proof_ms": round(single, 5),
                "one_call_per_proof_gbutterfly_s": round(proofs * gbfly(blog, 6, single), 3),
            }
            bctx.release()
            del pa, pb, pc, phm, phs, pscr
        line_extra["proof_batches"] = proof_batches
        log("proof batches: %s" % proof_batches)

        # ---- the other single-proof workloads of the H pipeline: 2^12 (latency: median
        # of 50 calls, each between its own events, the launch count, and the host's
        # enqueue time per call) and 2^22
        other_sizes = {}
        for olog in (12, 22):
            on = 1 << olog
            octx = g.HContext(olog)
            oa, ob = (g.to_mont(g.to_device(v)) for v in synth.h_inputs(3, olog))
            oc = g.fr_mul(oa, ob)
            ohm, ohs = g.empty_fr(on), g.empty_fr(on)

            def call():
                octx.h_compute(oa, ob, oc, ohm, ohs)

            entry = {"pass_batches": g.batch_plan(olog), "launches": octx.stage_count()}
            if olog == 12:
                med = tm.median_ms(call, 50)
                entry["h_pipeline_median_us"] = round(med * 1e3, 2)
                mean = tm.mean_ms(call, max(args.steps, 200))
                # back to back, as the 2^22 figure and the main step are timed
                entry["h_pipeline_ms"] = round(mean, 5)
                entry["h_pipeline_mean_ms"] = round(mean, 5)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(200):
                    call()
                host_us = (time.perf_counter() - t0) / 200 * 1e6
                torch.cuda.synchronize()
                entry["host_enqueue_us_per_call"] = round(host_us, 2)
                ms = med
            else:
                ms = tm.mean_ms(call, max(2, args.steps // 2))
                entry["h_pipeline_ms"] = round(ms, 5)
            entry["gbutterfly_s"] = round(gbfly(olog, 6, ms), 3)
            other_sizes["2^%d" % olog] = entry
            octx.release()
            del oa, ob, oc, ohm, ohs
        line_extra["other_sizes"] = other_sizes
        log("other sizes: %s" % other_sizes)

        line_extra["bb_lde"] = bb_leg(g, synth, torch, tm, args.steps, log)

    # ---- the timed region: K whole pipelines, after args.settle_ms of untimed pipelines
    # (the chip at its working clock, see Timer) and the W warmup steps
    settle_calls = tm.settle(lambda: ctx.h_compute(ad, bd, cd, hm, hs), args.settle_ms, warm=8)
    for _ in range(args.warmup):
        ctx.h_compute(ad, bd, cd, hm, hs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        ctx.h_compute(ad, bd, cd, hm, hs)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    log("h_compute 2^%d: %.4f ms/step (wall %.3f s)" % (log_n, ms_per_step, wall))

    plan = g.batch_plan(log_n)
    butterflies = 6 * (n // 2) * log_n
    p_muls, p_redc, p_bytes = pipeline_work(log_n)
    p_mads = mads(p_muls, p_redc)
    count = ctx.stage_count()
    stages = stage_list(plan, count)
    assert count == len(stages)
    assert sum(stage_work(*st, n)[0] for st in stages) == p_muls

    # ---- each stage alone, HIP events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(count)]
    acc = [0.0] * count
    for _ in range(args.stage_reps):
        for i in range(count):
            evs[i][0].record(stream)
            ctx.h_stage(i, ad, bd, cd, hm, hs)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        for i in range(count):
            acc[i] += evs[i][0].elapsed_time(evs[i][1])
    stage_ms = [x / args.stage_reps for x in acc]

    def stage_name(st):
        kind, join, nv, k = st
        return "%s_k%d_v%d%s" % (kind, k, nv, "_join" if join else "")

    stage_report = []
    for st, ms in zip(stages, stage_ms):
        m, r, by = stage_work(*st, n)
        t = mads(m, r) / (ms / 1e3) / 1e12
        stage_report.append({"kernel": stage_name(st), "ms": round(ms, 5),
                             "t_limb_products_s": round(t, 3),
                             "alu_frac": round(t / NOMINAL_PEAK_T, 4)})

    msm_line = None
    if not args.no_side:
        msm_line = msm_leg(g, synth, torch, tm, hs, log_n, args.steps, log)

    dom = int(np.argmax(stage_ms))
    d_muls, d_redc, d_bytes = stage_work(*stages[dom], n)
    dom_mads = mads(d_muls, d_redc)
    dom_name = stage_name(stages[dom])
    achieved_t = dom_mads / (stage_ms[dom] / 1e3) / 1e12
    src_hash = kernel_source_hash()
    traffic = traffic_from_profiles(dom_name, src_hash)
    measured_peak = None
    if "instruction_rates" in line_extra:
        measured_peak = line_extra["instruction_rates"]["v_mad_i64_i32"]["t_lane_ops_s"]

    value = butterflies / (ms_per_step / 1e3) / 1e9
    pipe_t = p_mads / (ms_per_step / 1e3) / 1e12
    line = {
        "metric": "Groth16 H-pipeline ms & Fr NTT Gbutterfly/s at n=2^20; achieved HBM GB/s",
        "value": round(value, 3),
        "unit": "Gbutterfly/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"ms": args.settle_ms, "untimed_pipelines": settle_calls},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": "H pipeline over BN254 Fr, n=2^%d: A,B seeded uniform, C=A*B, "
                        "3 iNTT + coset shift + 3 NTT + H=A'B'-C' (h_mont, h_std)" % log_n,
            "log_n": log_n,
            "pass_batches": plan,
            "stages": count,
        },
        "h_pipeline_ms": round(ms_per_step, 5),
        "hbm_gbs_algorithmic": round(p_bytes / (ms_per_step / 1e3) / 1e9, 2),
        "hbm_frac_algorithmic": round(p_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "pipeline_limb_products": p_mads,
        "pipeline_t_limb_products_s": round(pipe_t, 3),
        "pipeline_alu_frac": round(pipe_t / NOMINAL_PEAK_T, 4),
        "pipeline_alu_frac_of_measured_rate": (round(pipe_t / measured_peak, 4)
                                               if measured_peak else None),
        "stages": stage_report,
        "roofline": {
            "bound": "alu",
            "kernel": dom_name,
            "achieved": round(achieved_t, 3),
            "peak": round(NOMINAL_PEAK_T, 3),
            "unit": "T limb-products/s",
            "frac": round(achieved_t / NOMINAL_PEAK_T, 4),
            "traffic": traffic,
            "peak_measured": measured_peak,
            "algorithmic_bytes": d_bytes,
            "algorithmic_mads": dom_mads,
            "avg_launch_ms": round(stage_ms[dom], 5),
            "kernel_source_sha256_16": src_hash,
        },
        "cpu_baseline": None,
    }
    line.update(line_extra)
    if msm_line:
        line["msm_g1"] = msm_line

    if args.copy_calibration_mib:
        line["copy_calibration_bytes"] = copy_calibration(torch, args.copy_calibration_mib)

    if not args.no_cpu_baseline:
        import oracle
        am, bm = oracle.to_mont(a), oracle.to_mont(b)
        cm = oracle.pointwise_mul_mont(am, bm)
        nproc = os.cpu_count() or 1
        all_threads = oracle.default_threads()
        runs = {}
        for threads in (1, all_threads):
            oracle.set_threads(threads)
            times = []
            for _ in range(3):
                c0 = time.perf_counter()
                oracle.h_pipeline(log_n, am, bm, cm)
                times.append(time.perf_counter() - c0)
            runs[threads] = statistics.median(times)
            log("oracle (CPU, %d threads): median %.2f s of %s" % (threads, runs[threads],
                                                                   times))
        line["cpu_baseline"] = {
            "value": round(butterflies / runs[all_threads] / 1e9, 6),
            "unit": "Gbutterfly/s",
            "cores": all_threads,
            "kind": "oracle",
            "sample": "the whole 2^%d H pipeline, median of 3 runs: %.2f s on %d threads, "
                      "%.2f s on one" % (log_n, runs[all_threads], all_threads, runs[1]),
            "one_core": {"value": round(butterflies / runs[1] / 1e9, 6), "seconds": round(runs[1], 3)},
            "all_cores_seconds": round(runs[all_threads], 3),
            "nproc": nproc,
            "cpu_model": cpu_model(),
        }
    ctx.release()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
