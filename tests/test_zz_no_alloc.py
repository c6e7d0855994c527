"""g16_h_compute_noalloc (the entry point for callers that cannot allocate) against
g16_h_compute, bit for bit, through the C ABI: calls in a row on one device share the
library's scratch array, so each later call, smaller or larger than the one before,
must not depend on what the earlier one left there."""
import sys

import numpy as np
import pytest

from groth16_polynomial_amd import binding as g
from groth16_polynomial_amd import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)
    sys.stdout.flush()


def _inputs(workload, log_n):
    a, b = synth.h_inputs(workload, log_n)
    ad, bd = g.to_mont(g.to_device(a)), g.to_mont(g.to_device(b))
    return ad, bd, g.fr_mul(ad, bd)


def _same(x, y, what):
    import torch
    torch.cuda.synchronize()
    hx, hy = g.to_host(x), g.to_host(y)
    bad = np.flatnonzero((hx != hy).any(axis=1))
    assert len(bad) == 0, "%s: %d elements differ, first at %s" % (what, len(bad), bad[:8])


def test_noalloc_matches_h_compute_in_a_row():
    import torch
    assert torch.cuda.is_available()
    g.load()
    # larger, then smaller (the array keeps the larger call's contents), then a one-batch
    # domain (no scratch needed), then larger again
    for step, (log_n, workload) in enumerate(((20, 3), (14, 21), (9, 22), (22, 5))):
        say("call %d: 2^%d" % (step, log_n))
        n = 1 << log_n
        ctx = g.HContext(log_n)
        ad, bd, cd = _inputs(workload, log_n)
        want_m, want_s = ctx.h_compute(ad, bd, cd)
        hm, hs = g.empty_fr(n), g.empty_fr(n)
        hm.fill_(-1)
        hs.fill_(-1)
        ctx.h_compute_noalloc(ad, bd, cd, hm, hs)
        _same(hm, want_m, "h_mont 2^%d" % log_n)
        _same(hs, want_s, "h_std 2^%d" % log_n)
        ctx.release()


def test_noalloc_refuses_domains_above_its_limit():
    import torch
    g.load()
    log_n = 23
    say("limit: 2^%d refused" % log_n)
    ctx = g.HContext(log_n)
    n = 1 << log_n
    x = torch.zeros((n, 8), dtype=torch.int32, device="cuda")
    h1, h2 = g.empty_fr(n), g.empty_fr(n)
    with pytest.raises(g.G16Error) as e:
        ctx.h_compute_noalloc(x, x, x, h1, h2)
    assert e.value.code == g.G16_ENOSPACE
    # argument errors as g16_h_compute
    with pytest.raises(g.G16Error) as e:
        ctx.h_compute_noalloc(x, x, x, x, h2)
    assert e.value.code == g.G16_EALIAS
    ctx.release()
