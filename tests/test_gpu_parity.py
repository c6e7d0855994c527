"""Parity of the HIP library (through the C ABI) with the CPU oracle, bit for bit.

Every case prints what it runs before touching the GPU.  Inputs come from the seeded
generator in standard form; the GPU side converts them with its own kernel
(g16_to_mont) and the oracle with its own arithmetic, and the two conversions are
compared too.  Sizes: small domains cover every code path (one batch, several
batches, multi-slice workgroups); the workloads' full sizes run in the launch
configuration the benchmark uses (the library's default batching).
"""
import os
import sys

import numpy as np
import pytest

import oracle
from groth16_polynomial_amd import binding as g
from groth16_polynomial_amd import synth

pytestmark = pytest.mark.gpu

R = synth.R_MODULUS
EDGE_INTS = [0, 1, 2, R - 1, R - 2, (1 << 256) % R, (R - 1) // 2, 2**253, 2**64 - 1]


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "the GPU tests need a HIP device"
    g.load()
    yield torch
    torch.cuda.synchronize()


def sync():
    import torch
    torch.cuda.synchronize()


def host(t):
    sync()
    return g.to_host(t)


def same(got, want, what):
    got = np.asarray(got, dtype=np.uint32).reshape(-1, 8)
    want = np.asarray(want, dtype=np.uint32).reshape(-1, 8)
    assert got.shape == want.shape, what
    bad = np.flatnonzero((got != want).any(axis=1))
    assert len(bad) == 0, "%s: %d of %d elements differ, first at %s" % (
        what, len(bad), len(got), bad[:8].tolist())


def gpu_mont(words_std):
    """Standard-form words -> Montgomery on the GPU with the library's own kernel."""
    return g.to_mont(g.to_device(words_std))


class Env:
    """Run a block with library settings read at prepare time: the batching cap
    (G16_MAX_K) and the register-group geometry (G16_NARROW: 1 narrow, 0 radix-4 groups,
    unset: by launch size)."""

    def __init__(self, **values):
        self.values = {k: v for k, v in values.items() if v is not None}

    def __enter__(self):
        self.prev = {k: os.environ.get(k) for k in self.values}
        for k, v in self.values.items():
            os.environ[k] = str(v)
        return self

    def __exit__(self, *exc):
        for k, v in self.prev.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        return False


def KMax(kmax, narrow=None):
    return Env(G16_MAX_K=kmax, G16_NARROW=narrow)


def h_inputs(workload, log_n, c_is_product=True):
    a, b = synth.h_inputs(workload, log_n)
    ad, bd = gpu_mont(a), gpu_mont(b)
    am, bm = oracle.to_mont(a), oracle.to_mont(b)
    if c_is_product:
        cd = g.fr_mul(ad, bd)
        cm = oracle.pointwise_mul_mont(am, bm)
    else:
        c = synth.random_c(workload, log_n)
        cd, cm = gpu_mont(c), oracle.to_mont(c)
    return (ad, bd, cd), (am, bm, cm)


# ------------------------------------------------------------------ element-wise

@pytest.mark.parametrize("n", [1, 255, 4097])
def test_elementwise(n):
    say("elementwise n=%d" % n)
    x = synth.uniform_fr(41, n)
    y = synth.uniform_fr(42, n)
    if n > len(EDGE_INTS):
        x[:len(EDGE_INTS)] = synth.ints_to_fr(EDGE_INTS)
        y[:len(EDGE_INTS)] = synth.ints_to_fr(list(reversed(EDGE_INTS)))
    xm = gpu_mont(x)
    same(host(xm), oracle.to_mont(x), "to_mont")
    same(host(g.from_mont(xm)), x, "from_mont")
    ym = gpu_mont(y)
    same(host(g.fr_mul(xm, ym)),
         oracle.pointwise_mul_mont(oracle.to_mont(x), oracle.to_mont(y)), "fr_mul")
    # in place
    g.fr_mul(xm, ym, out=xm)
    same(host(xm), oracle.pointwise_mul_mont(oracle.to_mont(x), oracle.to_mont(y)),
         "fr_mul in place")


@pytest.mark.parametrize("n", [1, 1000, 65536])
def test_h_join(n):
    say("h_join n=%d" % n)
    a, b, c = (synth.uniform_fr(50 + i, n) for i in range(3))
    am, bm, cm = (oracle.to_mont(v) for v in (a, b, c))
    hm, hs = g.h_join(*(g.to_device(v) for v in (am, bm, cm)))
    want_std = oracle.field_op("sub", oracle.field_op("mul", a, b), c)
    same(host(hs), want_std, "h_std")
    same(host(hm), oracle.to_mont(want_std), "h_mont")


# ------------------------------------------------------------------ transforms

def _ntt_case(log_n, kmax=None, workload=2, narrow=None):
    say("ntt log_n=%d kmax=%s narrow=%s" % (log_n, kmax, narrow))
    x = synth.ntt_input(workload, log_n)
    xm = oracle.to_mont(x)
    with KMax(kmax, narrow):
        ctx = g.HContext(log_n)
    xd = g.to_device(xm)
    fwd = ctx.ntt_forward(xd)
    inv = ctx.ntt_inverse(xd)
    same(host(fwd), oracle.ntt_mont(xm, log_n), "forward 2^%d" % log_n)
    same(host(inv), oracle.ntt_mont(xm, log_n, inverse=True), "inverse 2^%d" % log_n)
    back = ctx.ntt_inverse(fwd)
    same(host(back), xm, "round trip 2^%d" % log_n)
    # in place
    ctx.ntt_forward(xd, out=xd)
    same(host(xd), host(fwd), "in-place forward 2^%d" % log_n)
    ctx.release()


@pytest.mark.parametrize("log_n", list(range(1, 23)))
def test_ntt_default_batching(log_n):
    _ntt_case(log_n)


@pytest.mark.parametrize("log_n,kmax", [(5, 2), (7, 3), (9, 4), (12, 4), (12, 5), (13, 6),
                                        (12, 11), (12, 12), (16, 11), (16, 12), (18, 12),
                                        (23, 12), (24, 12)])
def test_ntt_other_batchings(log_n, kmax):
    _ntt_case(log_n, kmax)


@pytest.mark.parametrize("log_n,kmax,narrow", [
    (7, None, 1), (12, None, 1), (13, None, 1), (17, None, 1), (18, None, 1), (20, None, 1),
    (12, None, 0), (14, None, 0)])
def test_ntt_geometries(log_n, kmax, narrow):
    """The register-group kernel's two geometries forced on domains where the size rule
    would pick the other one (narrow: one pass per group; 0: radix-4 groups)."""
    _ntt_case(log_n, kmax, narrow=narrow)


def test_domain_roots_match_oracle():
    for log_n in (1, 12, 20, 27 - 5):
        ctx = g.HContext(log_n)
        om, sm, im = ctx.domain_roots()
        w, s, si = oracle.domain_roots(log_n)
        rr = 1 << 256
        assert (om, sm, im) == (w * rr % R, s * rr % R, si * rr % R)
        ctx.release()


# ------------------------------------------------------------------ H pipeline

def _h_case(log_n, kmax=None, workload=1, c_is_product=True, narrow=None, radix2=None):
    say("h_compute log_n=%d kmax=%s workload=%d c=A*B:%s narrow=%s radix2=%s" % (
        log_n, kmax, workload, c_is_product, narrow, radix2))
    (ad, bd, cd), (am, bm, cm) = h_inputs(workload, log_n, c_is_product)
    same(host(ad), am, "A to Montgomery")
    same(host(cd), cm, "C = A o B")
    with KMax(kmax, narrow), Env(G16_RADIX2=radix2):
        ctx = g.HContext(log_n)
    hm, hs = ctx.h_compute(ad, bd, cd)
    want_m, want_s = oracle.h_pipeline(log_n, am, bm, cm)
    same(host(hm), want_m, "h_mont 2^%d" % log_n)
    same(host(hs), want_s, "h_std 2^%d" % log_n)
    return ctx, (ad, bd, cd), (hm, hs)


# every domain from 2^1 to 2^21 (2^20 is the workload test below), whole outputs
@pytest.mark.parametrize("log_n", [L for L in range(1, 22) if L != 20])
def test_h_compute_default_batching(log_n):
    ctx, _, _ = _h_case(log_n)
    ctx.release()


@pytest.mark.parametrize("log_n,kmax", [(4, 2), (8, 3), (10, 4), (12, 5), (13, 4), (14, 12),
                                        (12, 12), (17, 6)])
def test_h_compute_other_batchings(log_n, kmax):
    ctx, _, _ = _h_case(log_n, kmax)
    ctx.release()


# Both geometries of the register-group kernel on every batch size it takes (6..10) in
# each of its modes (inverse strided, fused, forward strided, forward strided with the
# join): narrow forced on larger domains, radix-4 groups forced on small ones.
@pytest.mark.parametrize("log_n,kmax,narrow", [
    (6, None, 1), (9, None, 1), (10, None, 1), (12, None, 1), (13, None, 1), (15, None, 1),
    (16, None, 1), (18, None, 1), (20, None, 1), (12, 12, 1), (19, 7, 1),
    (10, None, 0), (12, None, 0), (13, None, 0), (14, None, 0)])
def test_h_compute_geometries(log_n, kmax, narrow):
    ctx, _, _ = _h_case(log_n, kmax, workload=9, narrow=narrow)
    ctx.release()


# Every batch on the radix-2 kernel (G16_RADIX2): one batch, two, and the 2^20 plan, with
# the coset shift's four constants and the shifted forward twiddles on that kernel too.
@pytest.mark.parametrize("log_n", [3, 10, 14, 20])
def test_h_compute_radix2_kernel(log_n):
    ctx, _, _ = _h_case(log_n, workload=10, radix2=1)
    ctx.release()


def test_h_stages_compose_to_h_compute():
    import torch
    for log_n, kmax in ((10, None), (16, None), (12, 4), (12, None), (9, None)):
        say("h stages log_n=%d kmax=%s" % (log_n, kmax))
        (ad, bd, cd), _ = h_inputs(8, log_n)
        with KMax(kmax):
            ctx = g.HContext(log_n)
        hm, hs = ctx.h_compute(ad, bd, cd)
        count = ctx.stage_count()
        nb = len(g.batch_plan(log_n, kmax or 0))
        assert count in (2 * nb, 2 * nb - 1)
        sm, ss = g.empty_fr(1 << log_n), g.empty_fr(1 << log_n)
        for i in range(count):
            ctx.h_stage(i, ad, bd, cd, sm, ss)
        same(host(sm), host(hm), "staged h_mont")
        same(host(ss), host(hs), "staged h_std")
        with pytest.raises(g.G16Error):
            ctx.h_stage(count, ad, bd, cd, sm, ss)
        ctx.release()


def test_h_compute_c_not_product():
    ctx, _, _ = _h_case(11, c_is_product=False, workload=7)
    ctx.release()


def test_h_compute_workload_2_12():
    """The 2^12 workload (A, B uniform, C = A o B), whole output."""
    ctx, _, _ = _h_case(12, workload=1)
    ctx.release()


def test_h_compute_workload_2_20():
    """The 2^20 workload in the benchmark's launch configuration, whole output."""
    ctx, _, _ = _h_case(20, workload=3)
    ctx.release()


def test_h_compute_workload_2_22():
    """The 2^22 workload in the benchmark's launch configuration (the default plan,
    8 + 6 + 8) and under the pages' near-equal split (8 + 7 + 7): every output of both
    encodings against the oracle's pipeline."""
    log_n = 22
    assert g.batch_plan(log_n) == [8, 6, 8]
    assert g.batch_plan(log_n, 10) == [8, 7, 7]
    (ad, bd, cd), (am, bm, cm) = h_inputs(5, log_n)
    want_m, want_s = oracle.h_pipeline(log_n, am, bm, cm)
    for kmax in (None, 10):
        say("h_compute log_n=22 kmax=%s" % kmax)
        with KMax(kmax):
            ctx = g.HContext(log_n)
        hm, hs = ctx.h_compute(ad, bd, cd)
        same(host(hm), want_m, "h_mont 2^22 kmax=%s" % kmax)
        same(host(hs), want_s, "h_std 2^22 kmax=%s" % kmax)
        ctx.release()


@pytest.mark.parametrize("log_n,plan", [(23, [8, 7, 8]), (24, [8, 8, 8])])
def test_ntt_large(log_n, plan):
    """Standalone transforms at 2^23 and 2^24 (three batches): forward and inverse against
    the oracle's whole output, and the round trip."""
    import torch
    say("ntt 2^%d" % log_n)
    x = synth.ntt_input(6, log_n)
    xm = oracle.to_mont(x)
    ctx = g.HContext(log_n)
    assert g.batch_plan(log_n) == plan
    xd = g.to_device(xm)
    fwd = ctx.ntt_forward(xd)
    same(host(fwd), oracle.ntt_mont(xm, log_n), "forward 2^%d" % log_n)
    inv = ctx.ntt_inverse(xd)
    same(host(inv), oracle.ntt_mont(xm, log_n, inverse=True), "inverse 2^%d" % log_n)
    assert torch.equal(ctx.ntt_inverse(fwd), xd), "round trip 2^%d" % log_n
    ctx.release()


def _gpu_canonical(n, seed):
    """n canonical values drawn on the GPU (torch generator, fixed seed; every 32-bit word
    uniform, the top word below 2^29, so every value is below 2^253 < r), in Montgomery
    form.  For the property-only tests at large domains, which compare with no oracle."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    w = torch.randint(-2**31, 2**31, (n, 8), dtype=torch.int32, device="cuda", generator=gen)
    w[:, 7] &= (1 << 29) - 1
    return g.to_mont(w)


def _h_large(log_n, inputs, samples):
    """H pipeline at a large domain: outputs at `samples` indices by the oracle's
    barycentric route (0: properties only), then on every output the quotient-degree
    property (top coefficient of the inverse transform of H is zero) and, on a prefix,
    the agreement of the two encodings.  inputs: (A, B) in Montgomery form on the GPU."""
    n = 1 << log_n
    say("h_compute 2^%d (%d sampled outputs)" % (log_n, samples))
    ad, bd = inputs
    cd = g.fr_mul(ad, bd)
    ctx = g.HContext(log_n)
    plan = g.batch_plan(log_n)
    assert len(plan) == 3 and sum(plan) == log_n and 6 <= min(plan) and max(plan) <= 10
    hm, hs = ctx.h_compute(ad, bd, cd)
    if samples:
        am, bm = host(ad), host(bd)
        cm = oracle.pointwise_mul_mont(am, bm)
        rng = np.random.default_rng(log_n)
        idx = np.array([n - 1] + sorted(rng.integers(0, n, samples - 1).tolist()), np.uint32)
        want_m, want_s = oracle.h_at(log_n, am, bm, cm, idx)
        same(host(hm)[idx], want_m, "h_mont 2^%d sampled" % log_n)
        same(host(hs)[idx], want_s, "h_std 2^%d sampled" % log_n)
    same(oracle.to_mont(host(hs[:65536])), host(hm[:65536]), "dual encoding (prefix)")
    coeffs = ctx.ntt_inverse(hm)
    assert not host(coeffs[n - 1:]).any(), "quotient degree 2^%d" % log_n
    ctx.release()


def test_h_compute_2_23_full():
    """2^23 (8 + 7 + 8), every output of both encodings against the oracle's pipeline."""
    ctx, _, _ = _h_case(23, workload=6)
    ctx.release()


def test_h_compute_2_24_sampled():
    a, b = synth.h_inputs(7, 24)
    _h_large(24, (gpu_mont(a), gpu_mont(b)), 4)


@pytest.mark.parametrize("log_n", [25, 26])
def test_large_domains(log_n):
    """2^25 and 2^26 (default plans 10 + 8 + 7 and 10 + 8 + 8): H at sampled outputs (the last
    one among them) against the oracle's barycentric route, the quotient-degree property
    on every output, the encodings on a prefix, and the transforms' round trip."""
    import torch
    n = 1 << log_n
    _h_large(log_n, (_gpu_canonical(n, log_n), _gpu_canonical(n, 100 + log_n)), 3)
    ctx = g.HContext(log_n)
    x = _gpu_canonical(n, 200 + log_n)
    assert torch.equal(ctx.ntt_inverse(ctx.ntt_forward(x)), x), "round trip 2^%d" % log_n
    ctx.release()


def _batch_case(log_n, proofs, kmax=None, seed=300, narrow=None):
    """proofs independent proofs stacked back to back through g16_h_compute_batch; every
    output of every proof against the oracle.  Even proofs use C = A o B, odd ones an
    independent C."""
    import torch
    say("h_compute_batch 2^%d x %d proofs kmax=%s narrow=%s" % (log_n, proofs, kmax, narrow))
    dev, want = ([], [], []), []
    for q in range(proofs):
        (ad, bd, cd), (am, bm, cm) = h_inputs(seed + q, log_n, c_is_product=(q % 2 == 0))
        for lst, t in zip(dev, (ad, bd, cd)):
            lst.append(t)
        want.append(oracle.h_pipeline(log_n, am, bm, cm))
    a, b, c = (torch.cat(lst) for lst in dev)
    with KMax(kmax, narrow):
        ctx = g.HContext(log_n)
    hm, hs = ctx.h_compute_batch(a, b, c)
    n = 1 << log_n
    hm_h, hs_h = host(hm), host(hs)
    for q, (want_m, want_s) in enumerate(want):
        same(hm_h[q * n:(q + 1) * n], want_m, "h_mont 2^%d proof %d" % (log_n, q))
        same(hs_h[q * n:(q + 1) * n], want_s, "h_std 2^%d proof %d" % (log_n, q))
    return ctx, (a, b, c), (hm, hs)


@pytest.mark.parametrize("log_n,proofs,kmax,narrow", [
    (1, 3, None, None), (5, 4, None, None), (9, 2, 4, None), (10, 3, None, None),
    (12, 5, None, None), (13, 3, 4, None), (16, 3, None, None), (18, 2, None, None),
    (8, 3, None, 1), (12, 3, None, 1), (14, 2, None, 1), (16, 2, None, 1), (12, 2, None, 0),
    (21, 2, None, None)])
def test_h_compute_batch(log_n, proofs, kmax, narrow):
    """(21, 2): three batches of the measured default plan (6 + 7 + 8) over two proofs."""
    ctx, _, _ = _batch_case(log_n, proofs, kmax, narrow=narrow)
    ctx.release()


def test_h_compute_batch_workloads():
    """The batch shapes the benchmark times: 64 proofs at 2^12 and 16 at 2^16, whole
    outputs."""
    for log_n, proofs in ((12, 64), (16, 16)):
        ctx, _, _ = _batch_case(log_n, proofs, seed=1000 + log_n)
        ctx.release()


def test_h_compute_batch_edges():
    """An empty batch, a smaller batch after a larger one on the same context and
    scratch, a batch of one equal to g16_h_compute, and the host-side errors."""
    import torch
    log_n, n = 12, 1 << 12
    ctx, (a, b, c), (hm, hs) = _batch_case(log_n, 4, seed=500)
    scratch = g.empty_fr(4 * n)
    # smaller batch (proofs 1 and 2) reusing the scratch the larger one left dirty
    sm, ss = ctx.h_compute_batch(a[n:3 * n], b[n:3 * n], c[n:3 * n], scratch=scratch)
    same(host(sm), host(hm[n:3 * n]), "second call, fewer proofs (mont)")
    same(host(ss), host(hs[n:3 * n]), "second call, fewer proofs (std)")
    # a batch of one is g16_h_compute
    om, os_ = ctx.h_compute(a[:n], b[:n], c[:n])
    bm, bs = ctx.h_compute_batch(a[:n], b[:n], c[:n], scratch=scratch)
    same(host(bm), host(om), "batch of one (mont)")
    same(host(bs), host(os_), "batch of one (std)")
    # empty batch: nothing enqueued, no error
    e = g.empty_fr(0)
    em, es = ctx.h_compute_batch(e, e, e)
    assert em.numel() == 0 and es.numel() == 0
    # short scratch, overlapping buffers, a length that is not whole vectors
    with pytest.raises(g.G16Error) as ex:
        ctx.h_compute_batch(a, b, c, scratch=g.empty_fr(4 * n - 1))
    assert ex.value.code == g.G16_ENOSPACE
    with pytest.raises(g.G16Error) as ex:
        ctx.h_compute_batch(a, b, c, h_mont=g.empty_fr(4 * n), h_std=g.empty_fr(4 * n),
                            scratch=a)
    assert ex.value.code == g.G16_EALIAS
    with pytest.raises(ValueError):
        ctx.h_compute_batch(a[:n + 1], b[:n + 1], c[:n + 1])
    sync()
    ctx.release()


def test_fused_equals_unfused():
    """The fused join equals coset evaluations materialised one by one and joined by the
    standalone join (the POINTWISE_CU page keeps the unfused join for this check)."""
    for log_n, kmax in ((9, None), (12, None), (12, 4), (18, None)):
        say("fused vs unfused log_n=%d kmax=%s" % (log_n, kmax))
        (ad, bd, cd), (am, bm, cm) = h_inputs(4, log_n)
        with KMax(kmax):
            ctx = g.HContext(log_n)
        hm, hs = ctx.h_compute(ad, bd, cd)
        ca, cb, cc = (ctx.coset_eval(v) for v in (ad, bd, cd))
        if log_n <= 12:
            same(host(ca), oracle.coset_eval(log_n, am), "coset_eval A")
        um, us = g.h_join(ca, cb, cc)
        same(host(um), host(hm), "fused vs unfused h_mont")
        same(host(us), host(hs), "fused vs unfused h_std")
        # in place coset evaluation
        ctx.coset_eval(ad, out=ad)
        same(host(ad), host(ca), "in-place coset_eval")
        ctx.release()


def test_degenerate_inputs():
    import torch
    for log_n in (1, 2, 10):
        n = 1 << log_n
        say("degenerate inputs log_n=%d" % log_n)
        ctx = g.HContext(log_n)
        z = torch.zeros((n, 8), dtype=torch.int32, device="cuda")
        one = gpu_mont(synth.ints_to_fr([1] * n))
        hm, hs = ctx.h_compute(z, z, z)
        assert not host(hm).any() and not host(hs).any()
        hm, hs = ctx.h_compute(one, one, z)
        assert synth.fr_to_ints(host(hs)) == [1] * n
        hm, hs = ctx.h_compute(one, one, one)
        assert not host(hs).any()
        ctx.release()


def _extreme_values(n, phase):
    """Canonical inputs at the edges of the range: r - 1, r - 2^k, 2^k - 1 and 0/1, laid out so
    that the first butterflies add and subtract the largest values (the digit and value
    bounds of the transform passes are worst-case over canonical inputs)."""
    big = [R - 1, R - 2, R - (1 << 29), R - (1 << 232), (1 << 253) - 1, (1 << 232) - 1,
           (1 << 29) - 1, 1, 0]
    return [big[(i * 7 + phase) % len(big)] if (i >> 1) % 3 else R - 1 for i in range(n)]


def test_extreme_values():
    """Transforms and the H pipeline on inputs at the edges of the canonical range, as
    standard-form values converted on the device, against the oracle."""
    # 2^12 and 2^16: narrow geometry; 2^20: radix-4 groups (the 2^20 plan's launches);
    # 2^22: three batches, the middle one strided from bit 8
    for log_n in (12, 16, 20, 22):
        n = 1 << log_n
        say("extreme values log_n=%d" % log_n)
        a = synth.ints_to_fr(_extreme_values(n, 0))
        b = synth.ints_to_fr(_extreme_values(n, 3))
        ad, bd = gpu_mont(a), gpu_mont(b)
        am, bm = oracle.to_mont(a), oracle.to_mont(b)
        same(host(ad), am, "to Montgomery")
        ctx = g.HContext(log_n)
        same(host(ctx.ntt_forward(ad)), oracle.ntt_mont(am, log_n), "forward 2^%d" % log_n)
        same(host(ctx.ntt_inverse(ad)), oracle.ntt_mont(am, log_n, inverse=True),
             "inverse 2^%d" % log_n)
        # C = A o B, and C independent of A and B (C not a product: H is then no quotient)
        for c_is_product in (True, False):
            if c_is_product:
                cd = g.fr_mul(ad, bd)
                cm = oracle.pointwise_mul_mont(am, bm)
            else:
                c = synth.ints_to_fr(_extreme_values(n, 5))
                cd, cm = gpu_mont(c), oracle.to_mont(c)
            hm, hs = ctx.h_compute(ad, bd, cd)
            want_m, want_s = oracle.h_pipeline(log_n, am, bm, cm)
            same(host(hm), want_m, "h_mont 2^%d" % log_n)
            same(host(hs), want_s, "h_std 2^%d" % log_n)
        ctx.release()


def _const(v, n):
    return np.tile(synth.ints_to_fr([v]), (n, 1))


MONT_EXTREMES = [0, 1, 2, R - 1, R - 2, R - (1 << 29), 2**253, (1 << 232) - 1, (1 << 29) - 1]


@pytest.mark.parametrize("log_n,radix2", [(12, None), (14, None), (20, None), (10, 1)])
def test_join_operands_at_extremes(log_n, radix2):
    """The join's product and conversion on extreme Montgomery words.  Constant evaluation
    vectors have constant coset evaluations (the polynomial is a constant), so A' = A,
    B' = B and C' = C reach the join as given, and H = A B - C holds element by element in
    plain integers.  Covers the join of three kinds in one workgroup (2^12), the joins
    after the register groups (2^14, 2^20) and after the radix-2 passes (2^10)."""
    n = 1 << log_n
    rinv = pow(1 << 256, -1, R)
    triples = [(R - 1, R - 1, 0), (R - 1, R - 2, R - 1), (2**253, (1 << 232) - 1, 1),
               (R - (1 << 29), R - 1, 2**253), (0, R - 1, R - 1), (1, 1, 2),
               ((1 << 29) - 1, 2, R - 2)]
    with Env(G16_RADIX2=radix2):
        ctx = g.HContext(log_n)
    for ea, eb, ec in triples:
        say("join extremes log_n=%d radix2=%s (%x, %x, %x)" % (log_n, radix2, ea, eb, ec))
        a, b, c = (g.to_device(_const(e, n)) for e in (ea, eb, ec))
        hm, hs = ctx.h_compute(a, b, c)
        h_std = (ea * rinv * eb * rinv - ec * rinv) % R
        same(host(hs), _const(h_std, n), "h_std")
        same(host(hm), _const(h_std * (1 << 256) % R, n), "h_mont")
    ctx.release()


def test_gather_extreme_values():
    """Gather products on extreme coefficients and witness values (canonical standard
    values at the edges of the range, and values whose Montgomery words are extreme)."""
    say("gather extreme values")
    ma, mb, w = synth.gather_inputs(8, rows=700, n_witness=64, a_mean=3.0, b_mean=3.0)
    rinv = pow(1 << 256, -1, R)
    ext = EDGE_INTS + [e * rinv % R for e in MONT_EXTREMES]
    ma.value = synth.ints_to_fr([ext[i % len(ext)] for i in range(ma.nnz)])
    mb.value = synth.ints_to_fr([ext[(3 * i + 1) % len(ext)] for i in range(mb.nnz)])
    w = synth.ints_to_fr([ext[(5 * i + 2) % len(ext)] for i in range(64)])
    oa, ob, oc = _gather_device(ma, mb, w)
    want = oracle.gather(ma.row_ptr, ma.signal, oracle.to_mont(ma.value), mb.row_ptr,
                         mb.signal, oracle.to_mont(mb.value), oracle.to_mont(w))
    for got, exp, name in zip((oa, ob, oc), want, "abc"):
        same(host(got), exp, "gather extreme out_" + name)


def test_closed_forms_at_2_20():
    """Closed forms, no oracle: the forward transform of the unit vector at 0 is all ones and
    that of the all-ones vector is n at index 0; the inverse undoes both; the coset
    evaluations of a constant polynomial equal that constant; H of A = B = 1, C = 0 is one
    everywhere."""
    import torch
    log_n = 20
    n = 1 << log_n
    say("closed forms log_n=%d" % log_n)
    ctx = g.HContext(log_n)
    delta = [1] + [0] * (n - 1)
    ones = [1] * n
    dd, od = gpu_mont(synth.ints_to_fr(delta)), gpu_mont(synth.ints_to_fr(ones))
    assert synth.fr_to_ints(host(g.from_mont(ctx.ntt_forward(dd)))) == ones
    assert synth.fr_to_ints(host(g.from_mont(ctx.ntt_forward(od)))) == [n] + [0] * (n - 1)
    assert synth.fr_to_ints(host(g.from_mont(ctx.ntt_inverse(od)))) == delta
    seven = gpu_mont(synth.ints_to_fr([7] * n))  # evaluations of the constant 7
    assert synth.fr_to_ints(host(g.from_mont(ctx.coset_eval(seven)))) == [7] * n
    z = torch.zeros((n, 8), dtype=torch.int32, device="cuda")
    hm, hs = ctx.h_compute(od, od, z)
    assert synth.fr_to_ints(host(hs)) == ones
    ctx.release()


def test_aliasing_and_bad_pointers():
    import torch
    log_n = 8
    ctx = g.HContext(log_n)
    (ad, bd, cd), _ = h_inputs(3, log_n)
    with pytest.raises(g.G16Error) as e:
        ctx.h_compute(ad, bd, cd, h_mont=ad)
    assert e.value.code == g.G16_EALIAS
    h = g.empty_fr(1 << log_n)
    with pytest.raises(g.G16Error) as e:
        ctx.h_compute(ad, bd, cd, h_mont=h, h_std=h)
    assert e.value.code == g.G16_EALIAS
    # a host pointer is refused before any launch
    lib = g.load()
    host_buf = np.zeros((1 << log_n, 8), np.uint32)
    rc = lib.g16_ntt_forward(ctx.handle, host_buf.ctypes.data, ad.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert rc == g.G16_EINVAL
    # the workspace is not a valid output
    rc = lib.g16_ntt_forward(ctx.handle, ad.data_ptr(), ctx.workspace.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert rc == g.G16_EALIAS
    ctx.release()
    with pytest.raises(RuntimeError):
        ctx.ntt_forward(ad)


# ------------------------------------------------------------------ gather front end

def _gather_device(ma, mb, w):
    import torch

    def idx(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).cuda()

    vd_a = gpu_mont(ma.value) if ma.nnz else torch.zeros((0, 8), dtype=torch.int32,
                                                         device="cuda")
    vd_b = gpu_mont(mb.value) if mb.nnz else torch.zeros((0, 8), dtype=torch.int32,
                                                         device="cuda")
    return g.gather_abc(idx(ma.row_ptr), idx(ma.signal), vd_a, idx(mb.row_ptr),
                        idx(mb.signal), vd_b, gpu_mont(w))


@pytest.mark.parametrize("rows,n_witness", [(1000, 777), (4096, 3000)])
def test_gather_small(rows, n_witness):
    say("gather rows=%d" % rows)
    ma, mb, w = synth.gather_inputs(4, rows=rows, n_witness=n_witness)
    oa, ob, oc = _gather_device(ma, mb, w)
    want = oracle.gather(ma.row_ptr, ma.signal, oracle.to_mont(ma.value), mb.row_ptr,
                         mb.signal, oracle.to_mont(mb.value), oracle.to_mont(w))
    for got, exp, name in zip((oa, ob, oc), want, "abc"):
        same(host(got), exp, "gather out_" + name)


@pytest.mark.parametrize("rows,a_ne,b_ne,a_mean,b_mean", [
    (1000, None, 0, 1.13, 1.70),   # B has no terms at all (nnz_b = 0)
    (1000, 0, None, 1.13, 1.70),   # A has no terms at all
    (777, 700, 650, 30.0, 50.0),   # long rows: a wave's terms span many 64-term rounds
    (130, 130, 3, 95.0, 1.001),    # every A row at the cap, B nearly empty; ragged tail
    (65, 1, 65, 1.001, 95.0),      # one A term, then every B row at the cap
])
def test_gather_row_mixes(rows, a_ne, b_ne, a_mean, b_mean):
    """A's and B's terms of a wave are gathered as one list: shapes where one matrix is
    empty, rows cross 64-term rounds, or the split between A and B falls anywhere."""
    say("gather mix rows=%d a=%s/%g b=%s/%g" % (rows, a_ne, a_mean, b_ne, b_mean))
    ma, mb, w = synth.gather_inputs(6, rows=rows, n_witness=500, a_nonempty=a_ne,
                                    b_nonempty=b_ne, a_mean=a_mean, b_mean=b_mean)
    oa, ob, oc = _gather_device(ma, mb, w)
    want = oracle.gather(ma.row_ptr, ma.signal, oracle.to_mont(ma.value), mb.row_ptr,
                         mb.signal, oracle.to_mont(mb.value), oracle.to_mont(w))
    for got, exp, name in zip((oa, ob, oc), want, "abc"):
        same(host(got), exp, "gather out_" + name)


@pytest.mark.parametrize("rows,n_witness", [(1, 1), (70, 1), (64, 2)])
def test_gather_tiny(rows, n_witness):
    """One row; a one-slot witness (every signal 0); exactly one wave of rows."""
    say("gather tiny rows=%d n_witness=%d" % (rows, n_witness))
    ma, mb, w = synth.gather_inputs(9, rows=rows, n_witness=n_witness, a_nonempty=rows,
                                    b_nonempty=rows, a_mean=2.0, b_mean=3.0)
    oa, ob, oc = _gather_device(ma, mb, w)
    want = oracle.gather(ma.row_ptr, ma.signal, oracle.to_mont(ma.value), mb.row_ptr,
                         mb.signal, oracle.to_mont(mb.value), oracle.to_mont(w))
    for got, exp, name in zip((oa, ob, oc), want, "abc"):
        same(host(got), exp, "gather out_" + name)


def test_gather_bad_b_range_spares_the_wave():
    """A malformed B row (first index past its end) is flagged; the other rows of its
    wave, whose terms share the wave's flattened list, are still exact."""
    say("gather bad B range")
    ma, mb, w = synth.gather_inputs(7, rows=200, n_witness=300, a_nonempty=200,
                                    b_nonempty=200, a_mean=3.0, b_mean=4.0)
    bad_row = 70
    want = oracle.gather(ma.row_ptr, ma.signal, oracle.to_mont(ma.value), mb.row_ptr,
                         mb.signal, oracle.to_mont(mb.value), oracle.to_mont(w))
    rp = mb.row_ptr
    mb.row_ptr = rp.copy()
    mb.row_ptr[bad_row] = rp[bad_row + 1] + 1   # row 70: lo > hi; row 69 ends later
    assert mb.row_ptr[bad_row] <= mb.nnz
    oa, ob, oc = _gather_device(ma, mb, w)
    ha, hb, hc = host(oa), host(ob), host(oc)
    for hx in (ha, hb, hc):
        assert (hx[bad_row] == 0xffffffff).all()
    good = np.ones(200, bool)
    good[bad_row - 1:bad_row + 1] = False   # the two rows whose ranges changed
    for hx, exp, name in zip((ha, hb, hc), want, "abc"):
        same(hx[good], exp[good], "gather out_%s, good rows" % name)


def test_gather_bad_indices_are_flagged():
    say("gather bad indices")
    ma, mb, w = synth.gather_inputs(4, rows=300, n_witness=100)
    rows_with_terms = np.flatnonzero(np.diff(ma.row_ptr.astype(np.int64)) > 0)
    bad_row = int(rows_with_terms[3])
    ma.signal = ma.signal.copy()
    ma.signal[ma.row_ptr[bad_row]] = 100          # == n_witness: out of range
    oa, ob, oc = _gather_device(ma, mb, w)
    ha, hb, hc = host(oa), host(ob), host(oc)
    assert (ha[bad_row] == 0xffffffff).all() and (hc[bad_row] == 0xffffffff).all()
    good = np.ones(300, bool)
    good[bad_row] = False
    ma.signal[ma.row_ptr[bad_row]] = 0
    want = oracle.gather(ma.row_ptr, ma.signal, oracle.to_mont(ma.value), mb.row_ptr,
                         mb.signal, oracle.to_mont(mb.value), oracle.to_mont(w))
    same(ha[good], want[0][good], "rows without bad indices")
    # a row range past nnz is flagged too
    ma.row_ptr = ma.row_ptr.copy()
    ma.row_ptr[-1] = ma.nnz + 5
    oa, _, _ = _gather_device(ma, mb, w)
    assert (host(oa)[-1] == 0xffffffff).all()


def test_gather_pipeline_2_18():
    """The 2^18 gather workload end to end: gather, then the H pipeline."""
    log_n = 18
    say("gather + h_compute 2^18")
    ma, mb, w = synth.gather_inputs(4)
    oa, ob, oc = _gather_device(ma, mb, w)
    want = oracle.gather(ma.row_ptr, ma.signal, oracle.to_mont(ma.value), mb.row_ptr,
                         mb.signal, oracle.to_mont(mb.value), oracle.to_mont(w))
    for got, exp, name in zip((oa, ob, oc), want, "abc"):
        same(host(got), exp, "gather 2^18 out_" + name)
    ctx = g.HContext(log_n)
    hm, hs = ctx.h_compute(oa, ob, oc)
    want_m, want_s = oracle.h_pipeline(log_n, *want)
    same(host(hm), want_m, "gather pipeline h_mont")
    same(host(hs), want_s, "gather pipeline h_std")
    ctx.release()
