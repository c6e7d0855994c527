"""The G1 MSM of the HIP library (through the C ABI) against the MSM oracle.

Small cases compare with the oracle's MSM by definition on bases the oracle made
(multiples of the generator, in Montgomery form); large cases use bases s_i G made on
the GPU and compare with one scalar multiple (sum_i k_i s_i mod r) G from the oracle,
which holds at any size.  Edge cases: zero and one scalars, repeated bases (a bucket
adding a point to itself), opposite points, the point at infinity among the bases, the
empty MSM, every window width class."""
import random
import sys

import numpy as np
import pytest

from groth16_polynomial_amd import binding as g
from groth16_polynomial_amd import synth
from oracle import msm

pytestmark = pytest.mark.gpu

R = synth.R_MODULUS


def say(*a):
    print("[gpu-msm]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "the GPU tests need a HIP device"
    g.load()
    yield torch
    torch.cuda.synchronize()


def dev(words):
    import torch
    a = np.ascontiguousarray(words, dtype=np.uint32)
    return torch.from_numpy(a.view(np.int32).copy()).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def scalars_from(seed, n, zeros=0, ones=0):
    """n scalars below r from the seeded generator, the first `zeros` set to 0 and the
    next `ones` set to 1."""
    k = synth.uniform_fr(seed, n)
    k[:zeros] = 0
    k[zeros:zeros + ones] = 0
    k[zeros:zeros + ones, 0] = 1
    return k


def oracle_bases(seed, n):
    """Affine bases s_i G by the oracle (standard form), and their discrete logs s_i."""
    s = synth.uniform_fr(seed, n)
    return msm.scalar_mul(s), s


def ints(words):
    return synth.fr_to_ints(words)


@pytest.mark.parametrize("n", [1, 300, 2049])
def test_generator_multiples(n):
    say("g1_generator_mul n=%d" % n)
    k = synth.uniform_fr(60 + n, n)
    edge = msm.to_words([0, 1, 2, R - 1, R, (1 << 256) - 1])
    k[:min(n, len(edge))] = edge[:min(n, len(edge))]
    got = host(g.g1_generator_mul(dev(k))).reshape(n, 16)
    want = msm.points_to_mont(msm.scalar_mul(k))
    assert np.array_equal(got, want)


def _msm_case(n, c, seed, zeros=0, ones=0, mutate=None):
    say("msm n=%d c=%s seed=%d" % (n, c, seed))
    bases_std, _ = oracle_bases(seed, n)
    k = scalars_from(seed + 1, n, zeros, ones)
    if mutate:
        mutate(bases_std, k)
    want = msm.msm(k, bases_std)
    ctx = g.MsmG1(n, c)
    got = ctx(dev(k), dev(msm.points_to_mont(bases_std)))
    assert np.array_equal(got, want), "n=%d c=%d" % (n, ctx.c)
    return ctx


@pytest.mark.parametrize("n,c", [(1, 0), (2, 0), (31, 0), (100, 1), (100, 3), (257, 5),
                                 (1000, 0), (1000, 8), (2049, 13), (4097, 0), (4097, 16)])
def test_msm_against_definition(n, c):
    _msm_case(n, c, seed=7 * n + c, zeros=n // 10, ones=n // 7)


def test_msm_repeated_and_opposite_points():
    """Many copies of one base with one scalar pile into one bucket per window (the
    accumulation adds a point to itself, and runs span several slices); a base and its
    negation with equal scalars cancel; the point at infinity as a base adds nothing."""
    def mutate(bases, k):
        bases[10:300] = bases[9]
        k[10:300] = k[9]
        bases[400] = msm.affine_op("neg", bases[401:402])[0]
        k[400] = k[401]
        bases[500:520] = 0
    _msm_case(1500, 0, seed=99, mutate=mutate)
    _msm_case(1500, 10, seed=98, mutate=mutate)


def test_msm_all_zero_all_one_and_empty():
    n = 700
    bases_std, _ = oracle_bases(5, n)
    bm = dev(msm.points_to_mont(bases_std))
    ctx = g.MsmG1(n)
    assert not ctx(dev(np.zeros((n, 8), np.uint32)), bm).any()
    ones = np.zeros((n, 8), np.uint32)
    ones[:, 0] = 1
    assert np.array_equal(ctx(dev(ones), bm), msm.msm(ones, bases_std))
    empty = g.MsmG1(0)
    import torch
    e = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    eb = torch.empty((0, 16), dtype=torch.int32, device="cuda")
    assert not empty(e, eb).any()


def test_msm_top_scalars():
    """Scalars just below r (the top windows' digits and the recoding's last carry)."""
    def mutate(bases, k):
        k[:50] = msm.to_words([R - 1 - i for i in range(50)])
        k[50:60] = msm.to_words([(1 << 253) + i for i in range(10)])
    for c in (0, 7, 15, 16):
        _msm_case(600, c, seed=31 + c, mutate=mutate)


@pytest.mark.parametrize("log_n,c", [(16, 0), (18, 0), (20, 0), (22, 0), (20, 15), (22, 15)])
def test_msm_large_by_linearity(log_n, c):
    """Bases s_i G made on the GPU, scalars k_i: the result is (sum k_i s_i mod r) G.  The
    default widths, and c = 15, whose buckets' mean runs (64 and 256 entries) take longer
    accumulation slices."""
    n = 1 << log_n
    say("msm linearity n=2^%d c=%d" % (log_n, c))
    s = synth.uniform_fr(200 + log_n, n)
    k = scalars_from(300 + log_n, n, zeros=n // 50, ones=n // 60)
    bases = g.g1_generator_mul(dev(s))
    ctx = g.MsmG1(n, c)
    got = ctx(dev(k), bases)
    total = sum(a * b for a, b in zip(ints(k), ints(s))) % R
    want = msm.scalar_mul(msm.to_words([total]))[0]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("case", ["all_equal", "mixed", "narrow_windows", "all_equal_large",
                                  "two_values_large"])
def test_msm_long_runs(case):
    """Buckets whose runs cover many lanes and many tiles (joined by the in-wave scan and
    by the upper levels of the bucket sums): every scalar equal, a third of them equal to
    one value and a fifth to another, uniform scalars with 6-bit windows (32 buckets of
    ~1000 entries per window), and at 2^18 every scalar equal (each window one run over
    every tile, three levels) or one of two values."""
    n = {"all_equal": 1 << 14, "all_equal_large": 1 << 18,
         "two_values_large": 1 << 18}.get(case, 1 << 15)
    say("msm long runs: %s n=%d" % (case, n))
    s = synth.uniform_fr(400, n)
    k = synth.uniform_fr(401, n)
    if case in ("all_equal", "all_equal_large"):
        k[:] = k[0]
    elif case == "two_values_large":
        k[0::2] = k[0]
        k[1::2] = k[1]
    elif case == "mixed":
        k[: n // 3] = k[0]
        k[n // 3: n // 3 + n // 5] = k[1]
    c = 6 if case == "narrow_windows" else 0
    bases = g.g1_generator_mul(dev(s))
    got = g.MsmG1(n, c)(dev(k), bases)
    total = sum(a * b for a, b in zip(ints(k), ints(s))) % R
    assert np.array_equal(got, msm.scalar_mul(msm.to_words([total]))[0])


def test_msm_of_h_std():
    """The MSM's input in a prover: h_std of the H pipeline (2^12 here), compared with
    the oracle's MSM of the oracle's own h_std."""
    import oracle
    log_n, n = 12, 1 << 12
    say("msm of h_std 2^12")
    a, b = synth.h_inputs(41, log_n)
    am, bm = oracle.to_mont(a), oracle.to_mont(b)
    cm = oracle.pointwise_mul_mont(am, bm)
    _, hs_want = oracle.h_pipeline(log_n, am, bm, cm)
    ctx_h = g.HContext(log_n)
    ad, bd = g.to_device(am), g.to_device(bm)
    hm, hs = ctx_h.h_compute(ad, bd, g.fr_mul(ad, bd))
    assert np.array_equal(g.to_host(hs), hs_want)
    bases_std, _ = oracle_bases(42, n)
    got = g.MsmG1(n)(hs, dev(msm.points_to_mont(bases_std)))
    assert np.array_equal(got, msm.msm(hs_want, bases_std))
    ctx_h.release()


def test_msm_errors():
    import torch
    n = 64
    k = dev(synth.uniform_fr(3, n))
    b = g.g1_generator_mul(k)
    ctx = g.MsmG1(n)
    lib = g.load()
    ws = ctx.workspace
    s = ctx.sums
    need = g.msm_workspace_bytes(n, ctx.c)
    assert lib.g16_msm_g1(n, k.data_ptr(), b.data_ptr(), ctx.c, ws.data_ptr(), need - 1,
                          s.data_ptr(), None) == g.G16_ENOSPACE
    assert lib.g16_msm_g1(n, k.data_ptr(), b.data_ptr(), 25, ws.data_ptr(), need,
                          s.data_ptr(), None) == g.G16_EINVAL
    assert lib.g16_msm_g1(n, k.data_ptr(), b.data_ptr(), ctx.c, ws.data_ptr(), need,
                          k.data_ptr(), None) == g.G16_EALIAS
    host_buf = np.zeros(1 << 20, np.uint8)
    assert lib.g16_msm_g1(n, k.data_ptr(), b.data_ptr(), ctx.c, host_buf.ctypes.data,
                          host_buf.size, s.data_ptr(), None) == g.G16_EINVAL
    assert lib.g16_g1_generator_mul(0, k.data_ptr(), b.data_ptr(), None) == g.G16_EINVAL
    torch.cuda.synchronize()
