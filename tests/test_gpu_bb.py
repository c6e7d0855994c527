"""The BabyBear Reed-Solomon encoding transform of the HIP library (through the C ABI)
against the BabyBear oracle, word for word.

Inputs come from the seeded generator in standard form; the GPU converts them with its
own kernel (g16_bb_to_mont) and the oracle with its own arithmetic, and both
conversions are compared.  Shapes cover every code path: the one-kernel small domains
(2^1..2^4), one batch (2^5..2^8), two and three batches, one to 32+ columns (the first
batch's staged load takes its row blocks and columns in different proportions),
several matrices, every extension rate used by the WHIR grids (0..3), and the
benchmark's shapes at full size."""
import sys

import numpy as np
import pytest

from groth16_polynomial_amd import binding as g
from groth16_polynomial_amd import synth
from oracle import bb

pytestmark = pytest.mark.gpu

P = synth.BB_MODULUS


def say(*a):
    print("[gpu-bb]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "the GPU tests need a HIP device"
    g.load()
    yield torch
    torch.cuda.synchronize()


def host(t):
    import torch
    torch.cuda.synchronize()
    return g.bb_to_host(t)


def same(got, want, what):
    got, want = np.asarray(got, np.uint32).reshape(-1), np.asarray(want, np.uint32).reshape(-1)
    assert got.shape == want.shape, what
    bad = np.flatnonzero(got != want)
    assert len(bad) == 0, "%s: %d of %d words differ, first at %s" % (what, len(bad), len(got),
                                                                      bad[:8].tolist())


def _case(log_n, log_w=0, count=1, rate=0, workload=30, values=None):
    log_in = log_n - rate
    say("bb lde log_n=%d log_w=%d count=%d rate=%d" % (log_n, log_w, count, rate))
    x = synth.bb_lde_input(workload, log_in, log_w, count) if values is None else values
    xd = g.bb_to_mont(g.bb_to_device(x))
    xm = bb.to_mont(x)
    same(host(xd), xm, "to Montgomery")
    ctx = g.BbContext(log_n)
    y = ctx.lde(xd, log_in=log_in, log_w=log_w, count=count)
    same(host(y), bb.ntt_mont(xm, log_n, log_w=log_w, count=count, log_in=log_in),
         "lde 2^%d x 2^%d x %d rate %d" % (log_n, log_w, count, rate))
    same(host(g.bb_from_mont(y)), bb.from_mont(host(y)), "from Montgomery")
    ctx.release()
    return y


@pytest.mark.parametrize("log_n", list(range(1, 19)))
def test_bb_single_vector(log_n):
    _case(log_n)


@pytest.mark.parametrize("log_n,log_w,count,rate", [
    (3, 2, 3, 1), (4, 6, 1, 0), (5, 1, 2, 0), (7, 3, 1, 2), (9, 2, 2, 1), (9, 5, 1, 0),
    (10, 7, 1, 3), (12, 3, 4, 1), (13, 4, 1, 2), (16, 1, 3, 1), (17, 3, 1, 1), (18, 6, 1, 2),
    (20, 0, 2, 1), (21, 2, 1, 3)])
def test_bb_matrices_and_rates(log_n, log_w, count, rate):
    _case(log_n, log_w, count, rate, workload=31 + log_n)


def test_bb_extreme_values():
    """Inputs at the edges of [0, p): the additions and Shoup products at their bounds."""
    log_n = 12
    vals = np.array([P - 1, 0, 1, P - 2, (1 << 31) - (1 << 27), 1 << 30] * (1 << 12),
                    np.uint32)[: 1 << log_n]
    _case(log_n, values=vals)


@pytest.mark.parametrize("log_n,log_w,rate", [(24, 0, 1), (22, 3, 1), (24, 1, 1)])
def test_bb_benchmark_shapes(log_n, log_w, rate):
    """The benchmark's encodings at full size: one polynomial of 2^23 coefficients at rate
    1/2, and 2^24 coefficients folded into 2^3 and 2^1 columns at rate 1/2 (the WHIR
    grid's n = 24 cells with fold 3 and fold 1)."""
    _case(log_n, log_w, 1, rate, workload=40)


def test_bb_edges_and_errors():
    import torch
    ctx = g.BbContext(10)
    x = g.bb_to_mont(g.bb_to_device(synth.uniform_bb(5, 1024)))
    # an empty batch enqueues nothing
    lib = g.load()
    assert lib.g16_bb_lde(ctx.handle, 10, 0, 0, x.data_ptr(), x.data_ptr(), None) == g.G16_OK
    # log_in above the domain, in place (overlap), a short output, a host pointer
    y = torch.empty(1024, dtype=torch.int32, device="cuda")
    assert lib.g16_bb_lde(ctx.handle, 11, 0, 1, x.data_ptr(), y.data_ptr(), None) == g.G16_EINVAL
    assert lib.g16_bb_lde(ctx.handle, 10, 0, 1, x.data_ptr(), x.data_ptr(), None) == g.G16_EALIAS
    host_buf = np.zeros(1024, np.uint32)
    assert lib.g16_bb_lde(ctx.handle, 10, 0, 1, x.data_ptr(), host_buf.ctypes.data,
                          None) == g.G16_EINVAL
    assert lib.g16_bb_lde(ctx.handle, 10, 11, 1, x.data_ptr(), y.data_ptr(), None) == g.G16_EINVAL
    torch.cuda.synchronize()
    ctx.release()
    assert lib.g16_bb_release(ctypes_void(0x1000)) == g.G16_ESTATE


def ctypes_void(v):
    import ctypes
    return ctypes.c_void_p(v)
