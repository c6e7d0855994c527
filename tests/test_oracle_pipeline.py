"""Pins of the oracle's H pipeline.

H_i = a(s w^i) b(s w^i) - c(s w^i), where a, b, c interpolate A, B, C on the n-th
roots of unity and s is the coset shift (the NTT_CU page, "THE ALGORITHM IS THE CPU
BACKEND'S, EXACTLY"; the POINTWISE_CU page, "NO DIVISION BY Z(coset)").  The pins:
  * closed form for small n: the polynomial P = a b - c in Python integers, its exact
    division by x^n - 1 (zero remainder when C = A o B), and H_i = P(s w^i) =
    -2 Q(s w^i) because (s w^i)^n = s^n = -1;
  * Lagrange / barycentric evaluation in Python at sampled indices for larger n;
  * the oracle's own barycentric route (oracle_h_at) against its DIT route;
  * the invariant that Q has degree <= n - 2, seen as a zero top coefficient of the
    inverse transform of H;
  * the two encodings agree: h_mont = h_std * 2^256 mod r.
"""
import numpy as np
import pytest

import oracle
from groth16_polynomial_amd import synth
from tests import intref

R = synth.R_MODULUS
ints = synth.fr_to_ints
fr = synth.ints_to_fr


def _inputs(log_n, workload=1, c_is_product=True):
    a, b = synth.h_inputs(workload, log_n)
    am, bm = oracle.to_mont(a), oracle.to_mont(b)
    if c_is_product:
        cm = oracle.pointwise_mul_mont(am, bm)
    else:
        cm = oracle.to_mont(synth.random_c(workload, log_n))
    return am, bm, cm


def test_pointwise_product_against_python():
    am, bm, cm = _inputs(8)
    A, B, C = (ints(oracle.from_mont(v)) for v in (am, bm, cm))
    assert C == [x * y % R for x, y in zip(A, B)]


@pytest.mark.parametrize("log_n", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("c_is_product", [True, False])
def test_closed_form_small(log_n, c_is_product):
    n = 1 << log_n
    am, bm, cm = _inputs(log_n, workload=log_n, c_is_product=c_is_product)
    A, B, C = (ints(oracle.from_mont(v)) for v in (am, bm, cm))
    omega, shift, _ = oracle.domain_roots(log_n)
    a, b, c = (intref.idft(v, omega) for v in (A, B, C))
    P = intref.poly_sub(intref.poly_mul(a, b), c)
    Q, rem = intref.divmod_xn_minus_1(P, n)
    if c_is_product:
        assert rem == [0] * n            # A*B - C vanishes on the domain
        assert len(Q) <= n - 1           # deg Q <= n - 2
    h_mont, h_std = oracle.h_pipeline(log_n, am, bm, cm)
    xs = [shift * pow(omega, i, R) % R for i in range(n)]
    want = [intref.horner(P, x) for x in xs]
    assert ints(h_std) == want
    if c_is_product:
        assert want == [(-2 * intref.horner(Q, x)) % R for x in xs]
    assert ints(h_mont) == [h * (1 << 256) % R for h in want]


def test_lagrange_sampled_2_12():
    log_n = 12
    n = 1 << log_n
    am, bm, cm = _inputs(log_n, workload=1)
    A, B, C = (ints(oracle.from_mont(v)) for v in (am, bm, cm))
    omega, shift, _ = oracle.domain_roots(log_n)
    h_mont, h_std = oracle.h_pipeline(log_n, am, bm, cm)
    hs = ints(h_std)
    rng = np.random.default_rng(12)
    for i in [0, 1, n - 1] + [int(v) for v in rng.integers(0, n, 5)]:
        x = shift * pow(omega, i, R) % R
        va, vb, vc = (intref.barycentric_eval(v, omega, x) for v in (A, B, C))
        assert hs[i] == (va * vb - vc) % R
    # the O(n) barycentric form itself agrees with Lagrange written out, at n = 64
    small = A[:64]
    w64, s64, _ = oracle.domain_roots(6)
    assert intref.barycentric_eval(small, w64, s64) == intref.lagrange_eval(small, w64, s64)


@pytest.mark.parametrize("log_n", [9, 16])
def test_oracle_barycentric_route_matches_dit_route(log_n):
    n = 1 << log_n
    am, bm, cm = _inputs(log_n, workload=3)
    h_mont, h_std = oracle.h_pipeline(log_n, am, bm, cm)
    idx = np.array([0, 1, 2, n // 2, n - 1, 12345 % n], np.uint32)
    hm, hs = oracle.h_at(log_n, am, bm, cm, idx)
    assert (hm == h_mont[idx]).all() and (hs == h_std[idx]).all()


@pytest.mark.parametrize("log_n", [4, 10, 14])
def test_quotient_degree_invariant(log_n):
    """With C = A o B, iNTT(H) over the coset has a zero top coefficient, and
    q_j = -1/2 s^-j iNTT(H)_j are the coefficients of Q = (AB - C)/(x^n - 1)."""
    n = 1 << log_n
    am, bm, cm = _inputs(log_n, workload=5)
    _, h_std = oracle.h_pipeline(log_n, am, bm, cm)
    coeffs = ints(oracle.ntt(h_std, log_n, inverse=True))
    assert coeffs[n - 1] == 0
    if log_n <= 4:
        A, B, C = (ints(oracle.from_mont(v)) for v in (am, bm, cm))
        omega, shift, _ = oracle.domain_roots(log_n)
        a, b, c = (intref.idft(v, omega) for v in (A, B, C))
        Q, _ = intref.divmod_xn_minus_1(intref.poly_sub(intref.poly_mul(a, b), c), n)
        Q = Q + [0] * (n - len(Q))
        half = pow(2, -1, R)
        sinv = pow(shift, -1, R)
        assert Q == [(-half) * pow(sinv, j, R) * coeffs[j] % R for j in range(n)]


def test_invariant_detects_c_not_product():
    log_n = 10
    am, bm, cm = _inputs(log_n, workload=5, c_is_product=False)
    _, h_std = oracle.h_pipeline(log_n, am, bm, cm)
    assert ints(oracle.ntt(h_std, log_n, inverse=True))[-1] != 0


def test_dual_encoding_large():
    log_n = 13
    am, bm, cm = _inputs(log_n, workload=2)
    h_mont, h_std = oracle.h_pipeline(log_n, am, bm, cm)
    assert (oracle.to_mont(h_std) == h_mont).all()
    assert all(v < R for v in ints(h_std)) and all(v < R for v in ints(h_mont))


def test_zero_and_degenerate_inputs():
    log_n = 5
    n = 1 << log_n
    z = fr([0] * n)
    hm, hs = oracle.h_pipeline(log_n, z, z, z)
    assert ints(hs) == [0] * n and ints(hm) == [0] * n
    # constant A = 1, B = 1, C = 1: a = b = c = 1 as polynomials, H = 1*1 - 1 = 0
    one = oracle.to_mont(fr([1] * n))
    hm, hs = oracle.h_pipeline(log_n, one, one, one)
    assert ints(hs) == [0] * n
    # A = 1, B = 1, C = 0: H = 1 everywhere on the coset
    hm, hs = oracle.h_pipeline(log_n, one, one, z)
    assert ints(hs) == [1] * n


@pytest.mark.parametrize("log_n", [3, 11])
def test_coset_eval_is_the_pipeline_first_half(log_n):
    """Coset evaluations of one vector: Horner of its interpolant at s w^i, and the
    pipeline's H equals the pointwise combination of three such vectors."""
    n = 1 << log_n
    am, bm, cm = _inputs(log_n, workload=6, c_is_product=False)
    ca, cb, cc = (oracle.coset_eval(log_n, v) for v in (am, bm, cm))
    omega, shift, _ = oracle.domain_roots(log_n)
    coeffs = ints(oracle.ntt(oracle.from_mont(am), log_n, inverse=True))
    got = ints(oracle.from_mont(ca))
    for i in (0, 1, n // 2, n - 1):
        assert got[i] == intref.horner(coeffs, shift * pow(omega, i, R) % R)
    H = oracle.field_op("sub", oracle.field_op("mul", oracle.from_mont(ca), oracle.from_mont(cb)),
                        oracle.from_mont(cc))
    _, h_std = oracle.h_pipeline(log_n, am, bm, cm)
    assert (H == h_std).all()


def test_thread_count_does_not_change_results():
    """The oracle splits independent loops over threads; the same inputs give the same
    words on one thread and on several (H pipeline, both encodings, and the sampled
    barycentric route)."""
    log_n = 13
    a, b = synth.h_inputs(17, log_n)
    am, bm = oracle.to_mont(a), oracle.to_mont(b)
    cm = oracle.pointwise_mul_mont(am, bm)
    idx = np.array([0, 1, 4095, (1 << log_n) - 1], np.uint32)
    prev = oracle.set_threads(1)
    try:
        one = oracle.h_pipeline(log_n, am, bm, cm)
        one_at = oracle.h_at(log_n, am, bm, cm, idx)
        oracle.set_threads(8)
        many = oracle.h_pipeline(log_n, am, bm, cm)
        many_at = oracle.h_at(log_n, am, bm, cm, idx)
    finally:
        oracle.set_threads(prev)
    for x, y in zip(one + one_at, many + many_at):
        assert np.array_equal(x, y)
    assert np.array_equal(one[0][idx], one_at[0])
