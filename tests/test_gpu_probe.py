"""The instruction-rate probe runs the chains it claims: every lane's result equals the
host's computation of the same chains, for each instruction."""
import sys

import pytest

from groth16_polynomial_amd import probe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("op", [0, 1, 2, 3, 4, 5])
def test_probe_chains_match_host(op):
    import torch
    assert torch.cuda.is_available()
    print("[gpu-probe] op %s" % probe.OPS[op], flush=True)
    sys.stdout.flush()
    r = probe.run(op, blocks=64, iters=300, seed=777, reps=1)
    assert r["results_match"], r
    assert r["lane_ops_per_s_t"] > 0
