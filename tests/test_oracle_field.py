"""Pins of the oracle's field layer against Python's own big-integer arithmetic and
against closed-form facts about the BN254 scalar field."""
import random

import numpy as np
import pytest

import oracle
from groth16_polynomial_amd import synth
from tests import intref

R = synth.R_MODULUS
EDGE = [0, 1, 2, R - 1, R - 2, (R - 1) // 2, (R + 1) // 2, pow(2, 256, R), 2**253, 2**128,
        2**64 - 1, 2**64, 2**192 + 5]


def _values(n, seed):
    rng = random.Random(seed)
    return EDGE + [rng.randrange(R) for _ in range(n)]


def test_modulus_is_the_bn254_scalar_prime():
    assert oracle.modulus() == R
    assert R.bit_length() == 254
    assert intref.is_probable_prime(R)
    # r - 1 = 2^28 * odd: the largest power-of-two domain is 2^28, so a primitive
    # 2n-th root exists for n up to 2^27
    t, s = R - 1, 0
    while t % 2 == 0:
        t //= 2
        s += 1
    assert s == 28


def test_start_up_constants():
    c = oracle.constants()
    assert c["barrett_mu"] == (1 << 512) // R
    assert c["r_mod_r"] == (1 << 256) % R
    g = c["root_2_28"]
    assert pow(g, 1 << 28, R) == 1 and pow(g, 1 << 27, R) == R - 1   # primitive 2^28-th root
    # 5 is a quadratic non-residue (Euler's criterion), so 5^((r-1)/2^28) has order 2^28
    assert pow(5, (R - 1) // 2, R) == R - 1


@pytest.mark.parametrize("op", ["add", "sub", "mul"])
def test_field_ops_against_python_ints(op):
    xs = _values(3000, 1)
    ys = list(reversed(_values(3000, 2)))
    got = synth.fr_to_ints(oracle.field_op(op, synth.ints_to_fr(xs), synth.ints_to_fr(ys)))
    f = {"add": lambda a, b: (a + b) % R, "sub": lambda a, b: (a - b) % R,
         "mul": lambda a, b: a * b % R}[op]
    assert got == [f(a, b) for a, b in zip(xs, ys)]


def test_mul_large_random_batch():
    """Barrett's quotient estimate falls one short about once in 3000 products; a
    large batch exercises the final correction many times."""
    x = synth.uniform_fr(21, 200000)
    y = synth.uniform_fr(22, 200000)
    got = synth.fr_to_ints(oracle.field_op("mul", x, y))
    assert got == [a * b % R for a, b in zip(synth.fr_to_ints(x), synth.fr_to_ints(y))]


def test_mul_exhaustive_edge_pairs():
    xs = [a for a in EDGE for _ in EDGE]
    ys = [b for _ in EDGE for b in EDGE]
    got = synth.fr_to_ints(oracle.field_op("mul", synth.ints_to_fr(xs), synth.ints_to_fr(ys)))
    assert got == [a * b % R for a, b in zip(xs, ys)]


def test_montgomery_conversion():
    xs = _values(2000, 3)
    m = oracle.to_mont(synth.ints_to_fr(xs))
    assert synth.fr_to_ints(m) == [x * (1 << 256) % R for x in xs]
    assert synth.fr_to_ints(oracle.from_mont(m)) == xs


def test_pow_and_inverse():
    rng = random.Random(4)
    for _ in range(20):
        a, e = rng.randrange(1, R), rng.randrange(1 << 256)
        assert oracle.pow_int(a, e) == pow(a, e, R)
        assert oracle.inv_int(a) == pow(a, -1, R)
    assert oracle.inv_int(1) == 1 and oracle.inv_int(R - 1) == R - 1
    with pytest.raises(ValueError):
        oracle.inv_int(0)


@pytest.mark.parametrize("log_n", list(range(1, 28)))
def test_domain_roots_closed_form(log_n):
    n = 1 << log_n
    omega, shift, size_inv = oracle.domain_roots(log_n)
    # shift: a primitive 2n-th root (shift^n = -1), and the domain root is its square
    assert pow(shift, 2 * n, R) == 1 and pow(shift, n, R) == R - 1
    assert omega == shift * shift % R
    assert pow(omega, n, R) == 1 and pow(omega, n // 2, R) == R - 1
    assert size_inv * n % R == 1
    # the coset does not meet the domain: shift^n = -1 != 1
    # and the convention of the design notes (reading c1): shift = (5^((r-1)/2^28))^(2^(27-L))
    assert shift == pow(pow(5, (R - 1) >> 28, R), 1 << (27 - log_n), R)


def test_domain_roots_reject_bad_sizes():
    for bad in (0, 28, 40):
        with pytest.raises(ValueError):
            oracle.domain_roots(bad)
