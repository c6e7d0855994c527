"""The seeded input generator: stream definition, rejection sampling, workload shapes."""
import os

import numpy as np
import pytest

from groth16_polynomial_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gather_row_stats.txt")


def splitmix64_sequential(seed, count):
    """SplitMix64 written as the stateful generator (Steele, Lea, Flood 2014)."""
    m = (1 << 64) - 1
    state = seed
    out = []
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & m
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & m
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & m
        out.append(z ^ (z >> 31))
    return out


def test_splitmix_counter_form_matches_stateful_form():
    for seed in (0, 1, 1234567, synth.seed_for(3, 1)):
        want = splitmix64_sequential(seed, 50)
        got = [int(v) for v in synth.splitmix64(seed, 50)]
        assert got == want
        # any window of the stream can be drawn on its own
        assert [int(v) for v in synth.splitmix64(seed, 10, 40)] == want[40:]


def test_uniform_fr_canonical_and_deterministic():
    a = synth.uniform_fr(7, 5000)
    assert a.shape == (5000, 8) and a.dtype == np.uint32
    vals = synth.fr_to_ints(a)
    assert all(0 <= v < synth.R_MODULUS for v in vals)
    assert (synth.uniform_fr(7, 5000) == a).all()
    # a shorter draw is a prefix of a longer one
    assert (synth.uniform_fr(7, 1234) == a[:1234]).all()
    # the candidates follow the stated rule: four outputs per candidate, top limb masked
    raw = synth.splitmix64(7, 4 * 40).reshape(40, 4)
    cands = [int(l0) | int(l1) << 64 | int(l2) << 128 | (int(l3) & ((1 << 62) - 1)) << 192
             for l0, l1, l2, l3 in raw]
    kept = [c for c in cands if c < synth.R_MODULUS]
    assert vals[:len(kept)] == kept
    # top bits are spread: about 3/4 of candidates kept, values fill [0, r)
    assert max(vals) > synth.R_MODULUS * 0.99 and min(vals) < synth.R_MODULUS * 0.01


def test_int_layout_round_trip():
    vals = [0, 1, synth.R_MODULUS - 1, 2**255 + 12345, 2**32 - 1]
    assert synth.fr_to_ints(synth.ints_to_fr(vals)) == vals


def _golden_rows():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                p = line.split()
                rows[p[0]] = dict(log_n=int(p[1]), a=(float(p[2]), int(p[3]), int(p[4])),
                                  b=(float(p[5]), int(p[6]), int(p[7])))
    return rows


def _stats(m):
    lens = np.diff(m.row_ptr.astype(np.int64))
    nz = lens[lens > 0]
    return float(nz.mean()), int((lens == 0).sum()), int(lens.max())


def test_gather_shape_matches_page_measurements():
    g = _golden_rows()["js_16x16_d32"]
    assert g["log_n"] == 18
    a, b, w = synth.gather_inputs(4)
    assert a.row_ptr.shape == ((1 << 18) + 1,)
    for m, (mean, empty, longest) in ((a, g["a"]), (b, g["b"])):
        got_mean, got_empty, got_long = _stats(m)
        assert got_empty == empty
        # geometric lengths: the sample mean is within 1% of the target mean
        target = synth.GATHER_2_18["a_mean"] if m is a else synth.GATHER_2_18["b_mean"]
        assert abs(got_mean - target) < 0.01 * target
        assert abs(target - mean) <= 0.011          # 1.69 printed vs 1.70 generated for B
        assert got_long <= synth.GATHER_2_18["cap"] and got_long <= 95
        assert m.signal.max() < synth.GATHER_2_18["n_witness"]
        assert len(m.signal) == m.nnz and m.value.shape == (m.nnz, 8)
    vals = synth.fr_to_ints(w)
    small = sum(1 for v in vals if v in (0, 1))
    assert abs(small / len(vals) - 0.9) < 0.005
    ones = sum(1 for v in vals if v == 1)
    assert abs(ones / small - 0.5) < 0.01


@pytest.mark.parametrize("rows", [64, 1000, 4096])
def test_gather_small_shapes(rows):
    a, b, w = synth.gather_inputs(4, rows=rows, n_witness=777)
    assert a.row_ptr.shape == (rows + 1,) and b.row_ptr.shape == (rows + 1,)
    assert a.row_ptr[0] == 0 and (np.diff(a.row_ptr.astype(np.int64)) >= 0).all()
    assert a.signal.max(initial=0) < 777 and w.shape == (777, 8)
