#!/usr/bin/env python3
"""Benchmark of the Groth16 H-polynomial pipeline on one MI355X.

One step = one g16_h_compute over device-resident inputs at n = 2^20 (A, B seeded
uniform Fr, C = A o B, tables prepared beforehand): three inverse NTTs, the coset
shift, three forward NTTs and H = A'B' - C' in both encodings.  Prints one JSON line.

Also measured (same run, reported inside the line):
  * each kernel (stage) of the pipeline alone, with HIP events on the stream it is
    launched on; the slowest is the dominant kernel and carries the roofline;
  * the standalone forward NTT at 2^20 (Gbutterfly/s);
  * the CPU oracle on the host, single-threaded, on the same 2^20 workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MAD_PEAK_T = 256 * 64 * 2.4e9 / 1e12   # v_mad_u64_u32: 256 CUs x 64 lanes x 2.4 GHz, T/s
HBM_PEAK_GBS = 8000.0
MADS_PER_MUL = 136                      # 8-limb CIOS Montgomery product: 2 s^2 + s
MADS_PER_REDC = 72                      # Montgomery reduction alone: s^2 + s
FR_BYTES = 32
# (log n, proofs) of the several-proofs-per-call measurements: small domains, where one
# call per proof is launch-bound
BATCH_SHAPES = ((12, 64), (16, 16))
# the H pipeline's other single-proof workloads (timed beside the headline 2^20 one)
OTHER_SIZES = (12, 22)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--log-n", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=10)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (a known-size "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def stage_work(kind: str, join: bool, n_vec: int, k: int, n: int):
    """Algorithmic (limb products, bytes) of one pipeline stage.

    Strided batch of k passes on n_vec vectors: n_vec k n/2 butterflies, each one
    twiddle product; reads and writes each element once.  Fused lowest batch: the last
    k passes of the inverse and the first k of the forward transform (the pass on bit 0
    of each needs no product) plus the coset multiply, and one read of the coset table
    per vector.  Join: A'B' (one product), h_std (one reduction), reads A' and B',
    writes h_mont and h_std instead of the vector.
    """
    if kind == "fused":
        muls = n_vec * ((2 * k - 2) * n // 2 + n)
        byts = n_vec * 3 * n * FR_BYTES
    else:
        muls = n_vec * k * n // 2
        byts = n_vec * 2 * n * FR_BYTES
    mads = muls * MADS_PER_MUL
    if join:
        mads += n * (MADS_PER_MUL + MADS_PER_REDC)
        byts += 3 * n * FR_BYTES        # + A', B' reads, + the second output
    return mads, byts


def stage_list(plan, n_vec=3):
    """(kind, join, n_vec, k) of each stage of g16_h_compute, in launch order."""
    nb = len(plan)
    out = []
    if nb == 1:
        return [("fused", False, 2, plan[0]), ("fused", True, 1, plan[0])]
    for b in range(nb - 1, 0, -1):
        out.append(("inv", False, n_vec, plan[b]))
    out.append(("fused", False, n_vec, plan[0]))
    for b in range(1, nb):
        if b == nb - 1:
            out.append(("fwd", False, n_vec - 1, plan[b]))
            out.append(("fwd", True, 1, plan[b]))
        else:
            out.append(("fwd", False, n_vec, plan[b]))
    return out


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace (what the compiler sees of it, up to
    string literals, which the kernel sources use only for asm text without '//')."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", "", text)


# Sources of the G1 MSM only; the H pipeline's kernels are built from the others.
MSM_SOURCES = {"fp.hpp", "fp29.hpp", "fp29_cols.hpp", "fp29_cols_gen.py", "g1.hpp", "msm.hip",
               "msm_digit.hpp", "msm_kernels.hpp"}


def kernel_source_hash() -> str:
    """Hash of the H pipeline's kernel sources' code (comments and whitespace ignored),
    which ties a committed counter summary to the kernels it was measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "groth16_polynomial_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f in MSM_SOURCES:
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


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU (--gpus %d requested); sharding "
              "across GPUs is designed but not implemented"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from groth16_polynomial_amd import binding as g
    from groth16_polynomial_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    log_n = args.log_n
    n = 1 << log_n
    print("[bench] preparing 2^%d inputs" % log_n, file=sys.stderr, flush=True)

    a, b = synth.h_inputs(3, log_n)
    ad, bd = g.to_mont(g.to_device(a)), g.to_mont(g.to_device(b))
    cd = g.fr_mul(ad, bd)
    ctx = g.HContext(log_n)
    hm, hs = g.empty_fr(n), g.empty_fr(n)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # The side measurements run first: they also bring the chip to its steady clock,
    # which the first ~20 ms of sustained load does not run at.
    # ---- standalone forward NTT at the same size
    x = g.to_mont(g.to_device(synth.ntt_input(2, log_n)))
    y = g.empty_fr(n)
    for _ in range(3):
        ctx.ntt_forward(x, y)
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(args.steps):
        ctx.ntt_forward(x, y)
    f1.record(stream)
    torch.cuda.synchronize()
    ntt_ms = f0.elapsed_time(f1) / args.steps
    ntt_gbfly = (n // 2) * log_n / (ntt_ms / 1e3) / 1e9

    # ---- the CSR gather front end on the 2^18 proving-key shape (its own workload: the
    # GATHER_CU page's largest key, synthetic rows with its statistics)
    ma, mb, wit = synth.gather_inputs(4)

    def idx(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).cuda()

    ga = (idx(ma.row_ptr), idx(ma.signal), g.to_mont(g.to_device(ma.value)))
    gb = (idx(mb.row_ptr), idx(mb.signal), g.to_mont(g.to_device(mb.value)))
    gw = g.to_mont(g.to_device(wit))
    grows = len(ma.row_ptr) - 1
    gouts = [g.empty_fr(grows) for _ in range(3)]
    for _ in range(3):
        g.gather_abc(*ga, *gb, gw, *gouts)
    torch.cuda.synchronize()
    f0.record(stream)
    for _ in range(args.steps):
        g.gather_abc(*ga, *gb, gw, *gouts)
    f1.record(stream)
    torch.cuda.synchronize()
    gather_ms = f0.elapsed_time(f1) / args.steps
    nnz = ma.nnz + mb.nnz
    # algorithmic bytes: row pointers, column indices and coefficients of both matrices,
    # one 32-byte witness read per non-zero, three 32-byte outputs per row
    gather_bytes = 2 * 4 * (grows + 1) + nnz * (4 + 32 + 32) + 3 * 32 * grows

    # ---- several proofs per call at small domains, against one call per proof
    def time_ms(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        f0.record(stream)
        for _ in range(reps):
            fn()
        f1.record(stream)
        torch.cuda.synchronize()
        return f0.elapsed_time(f1) / reps

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
        batched = time_ms(lambda: bctx.h_compute_batch(pa, pb, pc, phm, phs, pscr),
                          args.steps)

        def one_by_one():
            for q in range(proofs):
                sl = slice(q * bn, (q + 1) * bn)
                bctx.h_compute(pa[sl], pb[sl], pc[sl], phm[sl], phs[sl])

        single = time_ms(one_by_one, max(1, args.steps // 4))
        bfly = proofs * 6 * (bn // 2) * blog
        proof_batches["2^%d_x%d" % (blog, proofs)] = {
            "batch_ms": round(batched, 5),
            "batch_gbutterfly_s": round(bfly / (batched / 1e3) / 1e9, 3),
            "one_call_per_proof_ms": round(single, 5),
            "one_call_per_proof_gbutterfly_s": round(bfly / (single / 1e3) / 1e9, 3),
        }
        bctx.release()
        del pa, pb, pc, phm, phs, pscr
    print("[bench] proof batches: %s" % proof_batches, file=sys.stderr, flush=True)

    # ---- the other single-proof workloads of the H pipeline (2^12 and 2^22), same call
    other_sizes = {}
    for olog in OTHER_SIZES:
        on = 1 << olog
        octx = g.HContext(olog)
        oa, ob = (g.to_mont(g.to_device(v)) for v in synth.h_inputs(3, olog))
        oc = g.fr_mul(oa, ob)
        ohm, ohs = g.empty_fr(on), g.empty_fr(on)
        oms = time_ms(lambda: octx.h_compute(oa, ob, oc, ohm, ohs), args.steps)
        other_sizes["2^%d" % olog] = {
            "h_pipeline_ms": round(oms, 5),
            "gbutterfly_s": round(6 * (on // 2) * olog / (oms / 1e3) / 1e9, 3),
            "pass_batches": g.batch_plan(olog),
        }
        octx.release()
        del oa, ob, oc, ohm, ohs
    print("[bench] other sizes: %s" % other_sizes, file=sys.stderr, flush=True)

    # ---- the timed region: K whole pipelines
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
    print("[bench] h_compute 2^%d: %.4f ms/step (wall %.3f s)" % (log_n, ms_per_step, wall),
          file=sys.stderr, flush=True)

    plan = g.batch_plan(log_n)
    butterflies = 6 * (n // 2) * log_n
    total_muls = 0
    total_bytes = 0
    stages = stage_list(plan)
    for kind, join, nv, k in stages:
        m, by = stage_work(kind, join, nv, k, n)
        total_muls += m
        total_bytes += by

    # ---- each stage alone, HIP events on the launch stream
    count = ctx.stage_count()
    assert count == len(stages)
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

    # ---- the H MSM: sum_i h_i P_i over G1 on the pipeline's own h_std, with synthetic
    # bases (multiples s_i G of the generator stand in for the proving key's points)
    bases = g.g1_generator_mul(g.to_device(synth.uniform_fr(7, n)))
    mctx = g.MsmG1(n)
    for _ in range(2):
        mctx.window_sums(hs, bases)
    torch.cuda.synchronize()
    f0.record(stream)
    msm_reps = max(1, args.steps // 4)
    for _ in range(msm_reps):
        mctx.window_sums(hs, bases)
    f1.record(stream)
    torch.cuda.synchronize()
    msm_ms = f0.elapsed_time(f1) / msm_reps
    sums_host = g.to_host(mctx.sums).reshape(mctx.windows, 32)
    t_fin = time.perf_counter()
    for _ in range(10):
        mctx.finish(sums_host)
    finish_ms = (time.perf_counter() - t_fin) / 10 * 1e3
    msm_line = {
        "workload": "G1 MSM of h_std at n=2^%d, bases s_i G (synthetic)" % log_n,
        "window_bits": mctx.c,
        "windows": mctx.windows,
        "device_ms": round(msm_ms, 4),
        "host_finish_ms": round(finish_ms, 4),
        "bucket_adds_per_s_g": round(n * mctx.windows / (msm_ms / 1e3) / 1e9, 3),
    }
    del bases, mctx
    # the same MSM at other sizes (default widths), uniform scalars k_i over bases k_i G
    if log_n == 20:
        sizes = {}
        for lg in (12, 16, 22):
            m = 1 << lg
            ks = g.to_device(synth.uniform_fr(8, m))
            mb = g.g1_generator_mul(ks)
            mc = g.MsmG1(m)
            for _ in range(2):
                mc.window_sums(ks, mb)
            torch.cuda.synchronize()
            f0.record(stream)
            for _ in range(5):
                mc.window_sums(ks, mb)
            f1.record(stream)
            torch.cuda.synchronize()
            t_ms = f0.elapsed_time(f1) / 5
            sizes["2^%d" % lg] = {"window_bits": mc.c, "device_ms": round(t_ms, 4),
                                  "bucket_adds_per_s_g":
                                      round(m * mc.windows / (t_ms / 1e3) / 1e9, 3)}
            del ks, mb, mc
        torch.cuda.empty_cache()
        msm_line["other_sizes"] = sizes
    print("[bench] msm: %s" % msm_line, file=sys.stderr, flush=True)
    dom = int(np.argmax(stage_ms))
    kind, join, nv, k = stages[dom]
    dom_mads, dom_bytes = stage_work(kind, join, nv, k, n)
    dom_s = stage_ms[dom] / 1e3
    dom_name = "%s_k%d_v%d%s" % (kind, k, nv, "_join" if join else "")
    achieved_t = dom_mads / dom_s / 1e12
    src_hash = kernel_source_hash()
    traffic = traffic_from_profiles(dom_name, src_hash)

    value = butterflies / (ms_per_step / 1e3) / 1e9
    line = {
        "metric": "Groth16 H-pipeline ms & Fr NTT Gbutterfly/s at n=2^20; achieved HBM GB/s",
        "value": round(value, 3),
        "unit": "Gbutterfly/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
        "ntt_forward_ms": round(ntt_ms, 5),
        "ntt_gbutterfly_s": round(ntt_gbfly, 3),
        "gather_2_18_ms": round(gather_ms, 5),
        "gather_gnnz_s": round(nnz / (gather_ms / 1e3) / 1e9, 3),
        "gather_hbm_gbs_algorithmic": round(gather_bytes / (gather_ms / 1e3) / 1e9, 2),
        "proof_batches": proof_batches,
        "other_sizes": other_sizes,
        "msm_g1": msm_line,
        "hbm_gbs_algorithmic": round(total_bytes / (ms_per_step / 1e3) / 1e9, 2),
        "pipeline_tmad_s": round(total_muls / (ms_per_step / 1e3) / 1e12, 3),
        "pipeline_alu_frac": round(total_muls / (ms_per_step / 1e3) / 1e12 / MAD_PEAK_T, 4),
        "stage_ms": [round(v, 5) for v in stage_ms],
        "roofline": {
            "bound": "alu",
            "kernel": dom_name,
            "achieved": round(achieved_t, 3),
            "peak": round(MAD_PEAK_T, 3),
            "unit": "Tmad/s",
            "frac": round(achieved_t / MAD_PEAK_T, 4),
            "traffic": traffic,
            "algorithmic_bytes": dom_bytes,
            "algorithmic_mads": dom_mads,
            "avg_launch_ms": round(stage_ms[dom], 5),
            "kernel_source_sha256_16": src_hash,
        },
        "cpu_baseline": None,
    }

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = nbytes
        del src, dst

    if not args.no_cpu_baseline:
        import oracle
        print("[bench] oracle (CPU, 1 thread) on the same 2^%d pipeline" % log_n,
              file=sys.stderr, flush=True)
        am, bm = oracle.to_mont(a), oracle.to_mont(b)
        cm = oracle.pointwise_mul_mont(am, bm)
        c0 = time.perf_counter()
        oracle.h_pipeline(log_n, am, bm, cm)
        cpu_s = time.perf_counter() - c0
        line["cpu_baseline"] = {
            "value": round(butterflies / cpu_s / 1e9, 6),
            "unit": "Gbutterfly/s",
            "cores": 1,
            "kind": "oracle",
            "sample": "the whole 2^%d H pipeline once (%.1f s), single-threaded C oracle"
                      % (log_n, cpu_s),
        }
    ctx.release()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
