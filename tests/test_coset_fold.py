"""The schedule the kernels use for the coset shift and 1/n, checked in Python integers
(no GPU): between the inverse and the forward transform each element at position p of
the bit-reversed coefficient vector is multiplied by kappa[p mod 4] = n^-1 s^(2^(L-1) p_0 +
2^(L-2) p_1), and the forward pass on each bit b >= 2 multiplies its twiddles by
sigma_b = s^(2^(L-1-b)).  The forward transform over that vector must give the coset
evaluations n^-1 sum_j c_j (s w^k)^j (the coset step of the H pipeline: multiply c_j by
s^j, scale by 1/n, evaluate on the subgroup), for every size and for a few vectors,
including the unit vectors that single out each factor."""
import random

import pytest

from groth16_polynomial_amd import synth

R = synth.R_MODULUS


def bitrev(x, bits):
    return int(format(x, "0%db" % bits)[::-1], 2) if bits else 0


def roots(log_n):
    # a primitive 2n-th root s (5 generates the multiplicative group of Fr) and w = s^2
    s = pow(5, (R - 1) >> (log_n + 1), R)
    return s, s * s % R


def folded_schedule(coeffs, log_n):
    n = 1 << log_n
    s, w = roots(log_n)
    n_inv = pow(n, R - 2, R)
    x = [coeffs[bitrev(p, log_n)] for p in range(n)]
    for p in range(n):
        e = (p & 1) << (log_n - 1)
        if log_n >= 2:
            e += ((p >> 1) & 1) << (log_n - 2)
        x[p] = x[p] * n_inv % R * pow(s, e, R) % R
    for b in range(log_n):  # forward order, bit-reversed in, natural out
        half = 1 << b
        sigma = pow(s, 1 << (log_n - 1 - b), R) if b >= 2 else 1
        for i in range(n):
            if i & half:
                continue
            tw = pow(w, (i % half) * (n >> (b + 1)), R) * sigma % R
            u, v = x[i], x[i + half] * tw % R
            x[i], x[i + half] = (u + v) % R, (u - v) % R
    return x


def coset_direct(coeffs, log_n):
    n = 1 << log_n
    s, w = roots(log_n)
    n_inv = pow(n, R - 2, R)
    out = []
    for k in range(n):
        z = s * pow(w, k, R) % R
        acc, zj = 0, 1
        for c in coeffs:
            acc = (acc + c * zj) % R
            zj = zj * z % R
        out.append(acc * n_inv % R)
    return out


@pytest.mark.parametrize("log_n", range(1, 8))
def test_folded_coset_shift_matches_definition(log_n):
    n = 1 << log_n
    rng = random.Random(9000 + log_n)
    vecs = [[rng.randrange(R) for _ in range(n)]]
    vecs += [[1 if j == t else 0 for j in range(n)] for t in range(n)]  # c = unit vectors
    for c in vecs:
        assert folded_schedule(c, log_n) == coset_direct(c, log_n)


def test_dropping_a_fold_is_caught():
    """A schedule without sigma on one bit (or with kappa's bit 1 dropped) is wrong, so the
    check above pins every factor."""
    log_n, n = 5, 32
    c = [random.Random(1).randrange(R) for _ in range(n)]
    want = coset_direct(c, log_n)
    s, w = roots(log_n)
    n_inv = pow(n, R - 2, R)
    for missing in ("kappa_bit1", "sigma_3"):
        x = [c[bitrev(p, log_n)] for p in range(n)]
        for p in range(n):
            e = (p & 1) << (log_n - 1)
            if missing != "kappa_bit1":
                e += ((p >> 1) & 1) << (log_n - 2)
            x[p] = x[p] * n_inv % R * pow(s, e, R) % R
        for b in range(log_n):
            half = 1 << b
            sigma = pow(s, 1 << (log_n - 1 - b), R) if b >= 2 and not (
                missing == "sigma_3" and b == 3) else 1
            for i in range(n):
                if i & half:
                    continue
                tw = pow(w, (i % half) * (n >> (b + 1)), R) * sigma % R
                u, v = x[i], x[i + half] * tw % R
                x[i], x[i + half] = (u + v) % R, (u - v) % R
        assert x != want, missing
