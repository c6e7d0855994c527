"""Pins of the MSM oracle (oracle/msm_oracle.c) against what the mathematics fixes:
the BN254 moduli from the curve family's closed form, the field operations against
Python integers, the group order (r G is the point at infinity), the textbook affine
group law against the Jacobian formulas, linearity of scalar multiplication, and the
MSM against its definition on tiny cases and against one scalar multiple on random
ones."""
import numpy as np
import pytest

from groth16_polynomial_amd import synth
from oracle import msm

R = synth.R_MODULUS
# BN curves (Barreto and Naehrig, "Pairing-friendly elliptic curves of prime order",
# SAC 2005): p = 36u^4 + 36u^3 + 24u^2 + 6u + 1 and r = 36u^4 + 36u^3 + 18u^2 + 6u + 1;
# BN254 takes u = 4965661367192848881.
U = 4965661367192848881
P = 36 * U**4 + 36 * U**3 + 24 * U**2 + 6 * U + 1
G = (1, 2)


def rand_ints(seed, n, mod):
    """n integers below mod from the seeded generator (four 64-bit draws each)."""
    raw = synth.splitmix64(seed, 4 * n).reshape(n, 4)
    return [sum(int(x) << (64 * j) for j, x in enumerate(row.tolist())) % mod for row in raw]


def pt(words):
    return msm.words_to_points(words)


def test_moduli_closed_form():
    assert msm.modulus() == P
    assert R == 36 * U**4 + 36 * U**3 + 18 * U**2 + 6 * U + 1


def test_field_ops_against_python():
    xs = [0, 1, 2, P - 1, P - 2, (1 << 256) % P, P // 2] + rand_ints(1, 300, P)
    ys = list(reversed(xs))
    a, b = msm.to_words(xs), msm.to_words(ys)
    assert msm.from_words(msm.fp_op("add", a, b)) == [(x + y) % P for x, y in zip(xs, ys)]
    assert msm.from_words(msm.fp_op("sub", a, b)) == [(x - y) % P for x, y in zip(xs, ys)]
    assert msm.from_words(msm.fp_op("mul", a, b)) == [x * y % P for x, y in zip(xs, ys)]
    inv = msm.from_words(msm.fp_op("inv", a))
    assert inv == [pow(x, -1, P) if x else 0 for x in xs]
    assert msm.from_words(msm.to_mont(a)) == [x * (1 << 256) % P for x in xs]
    assert msm.from_words(msm.from_mont(msm.to_mont(a))) == xs
    # a large batch: Barrett's quotient estimate is short only rarely
    big = rand_ints(2, 20000, P)
    big2 = rand_ints(3, 20000, P)
    got = msm.from_words(msm.fp_op("mul", msm.to_words(big), msm.to_words(big2)))
    assert got == [x * y % P for x, y in zip(big, big2)]


def test_non_canonical_input_is_refused():
    with pytest.raises(ValueError):
        msm.fp_op("add", msm.to_words([P]), msm.to_words([1]))


def test_generator_and_group_order():
    assert msm.on_curve(msm.points_to_words([G]))
    ks = [1, 2, 3, R - 1, R, R + 5, 5, 0, (1 << 256) - 1]
    out = pt(msm.scalar_mul(msm.to_words(ks)))
    assert out[0] == G
    assert out[3] == (1, P - 2)            # (r - 1) G = -G
    assert out[4] is None                  # r G = infinity: the group order is r
    assert out[5] == out[6]                # (r + 5) G = 5 G
    assert out[7] is None
    assert out[8] == pt(msm.scalar_mul(msm.to_words([((1 << 256) - 1) % R])))[0]
    assert msm.on_curve(msm.points_to_words([q for q in out if q is not None]))


def test_affine_law_against_jacobian():
    a = rand_ints(4, 40, R)
    b = rand_ints(5, 40, R)
    pa, pb = msm.scalar_mul(msm.to_words(a)), msm.scalar_mul(msm.to_words(b))
    assert msm.on_curve(pa) and msm.on_curve(pb)
    assert np.array_equal(msm.affine_op("add", pa, pb), msm.jacobian_op("add", pa, pb))
    assert np.array_equal(msm.affine_op("double", pa), msm.jacobian_op("double", pa))
    # special cases: P + P, P + (-P), P + infinity, infinity + infinity
    neg = msm.affine_op("neg", pa)
    inf = np.zeros_like(pa)
    assert np.array_equal(msm.affine_op("add", pa, pa), msm.affine_op("double", pa))
    assert np.array_equal(msm.jacobian_op("add", pa, pa), msm.affine_op("double", pa))
    assert not msm.affine_op("add", pa, neg).any()
    assert not msm.jacobian_op("add", pa, neg).any()
    assert np.array_equal(msm.affine_op("add", pa, inf), pa)
    assert np.array_equal(msm.jacobian_op("add", inf, pa), pa)
    assert not msm.jacobian_op("double", inf).any()


def test_linearity_of_scalar_multiplication():
    a = rand_ints(6, 30, R)
    b = rand_ints(7, 30, R)
    pa, pb = msm.scalar_mul(msm.to_words(a)), msm.scalar_mul(msm.to_words(b))
    s = msm.scalar_mul(msm.to_words([(x + y) % R for x, y in zip(a, b)]))
    assert np.array_equal(msm.affine_op("add", pa, pb), s)
    # a (b G) = (a b) G
    for i in range(5):
        lhs = msm.scalar_mul(msm.to_words([a[i]]), pt(pb[i:i + 1])[0])
        rhs = msm.scalar_mul(msm.to_words([a[i] * b[i] % R]))
        assert np.array_equal(lhs, rhs)


def test_msm_tiny_cases_by_definition():
    bases = msm.scalar_mul(msm.to_words(rand_ints(8, 4, R)))
    # all-one scalars: the plain sum
    ones = msm.to_words([1, 1, 1, 1])
    s = bases[0:1]
    for i in range(1, 4):
        s = msm.affine_op("add", s, bases[i:i + 1])
    assert np.array_equal(msm.msm(ones, bases), s[0])
    # zeros: infinity; a single term: one scalar multiple
    assert not msm.msm(msm.to_words([0, 0, 0, 0]), bases).any()
    k = rand_ints(9, 1, R)
    assert np.array_equal(msm.msm(msm.to_words(k), bases[:1]),
                          msm.scalar_mul(msm.to_words(k), pt(bases[:1])[0])[0])
    # k P + (-k) P = infinity; repeated bases add up
    two = msm.to_words([k[0], R - k[0]])
    assert not msm.msm(two, np.concatenate([bases[:1], bases[:1]])).any()
    assert np.array_equal(msm.msm(msm.to_words([3, 4]), np.concatenate([bases[:1], bases[:1]])),
                          msm.scalar_mul(msm.to_words([7]), pt(bases[:1])[0])[0])
    # an empty MSM is infinity
    assert not msm.msm(np.zeros((0, 8), np.uint32), np.zeros((0, 16), np.uint32)).any()


@pytest.mark.parametrize("n", [17, 200])
def test_msm_against_one_scalar_multiple(n):
    """With bases s_i G, sum_i k_i (s_i G) = (sum_i k_i s_i mod r) G."""
    s = rand_ints(10 + n, n, R)
    k = rand_ints(20 + n, n, 1 << 256)      # full 256-bit scalars, not reduced
    bases = msm.scalar_mul(msm.to_words(s))
    want = msm.scalar_mul(msm.to_words([sum(x * y for x, y in zip(k, s)) % R]))[0]
    assert np.array_equal(msm.msm(msm.to_words(k), bases), want)
