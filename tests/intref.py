"""Definitions written with Python's arbitrary-precision integers, used to pin the
oracle.  None of this shares code with the oracle (C, Barrett reduction) or with the
HIP library (Montgomery limbs): the arithmetic here is Python's own `*`, `%` and
`pow`, and each function is the textbook definition, not an algorithm of the pages.
"""
from __future__ import annotations

from groth16_polynomial_amd.synth import R_MODULUS as R


def inv(a: int) -> int:
    return pow(a, -1, R)


def dft(xs, w: int):
    """y_i = sum_j x_j w^(i j) (the definition of the transform at root w)."""
    n = len(xs)
    out = []
    for i in range(n):
        wi = pow(w, i, R)
        acc, p = 0, 1
        for x in xs:
            acc += x * p
            p = p * wi % R
        out.append(acc % R)
    return out


def idft(ys, w: int):
    n = len(ys)
    ninv = inv(n)
    return [v * ninv % R for v in dft(ys, inv(w))]


def horner(coeffs, x: int) -> int:
    acc = 0
    for c in reversed(coeffs):
        acc = (acc * x + c) % R
    return acc


def poly_mul(a, b):
    out = [0] * (len(a) + len(b) - 1)
    for i, x in enumerate(a):
        if x:
            for j, y in enumerate(b):
                out[i + j] += x * y
    return [v % R for v in out]


def poly_sub(a, b):
    m = max(len(a), len(b))
    a = list(a) + [0] * (m - len(a))
    b = list(b) + [0] * (m - len(b))
    return [(x - y) % R for x, y in zip(a, b)]


def divmod_xn_minus_1(p, n: int):
    """Quotient and remainder of p(x) by x^n - 1 (schoolbook long division)."""
    p = list(p)
    if len(p) <= n:
        return [0], p
    q = [0] * (len(p) - n)
    for k in range(len(p) - 1, n - 1, -1):
        c = p[k] % R
        if c:
            q[k - n] = c
            p[k] = 0
            p[k - n] = (p[k - n] + c) % R     # subtract c * x^(k-n) * (x^n - 1)
    return q, [v % R for v in p[:n]]


def lagrange_eval(values, omega: int, x: int) -> int:
    """Value at x of the polynomial of degree < n through (omega^j, values[j]), by
    Lagrange interpolation written out term by term (O(n^2), small n only)."""
    n = len(values)
    pts = [pow(omega, j, R) for j in range(n)]
    total = 0
    for j, yj in enumerate(values):
        num, den = 1, 1
        for m, xm in enumerate(pts):
            if m != j:
                num = num * (x - xm) % R
                den = den * (pts[j] - xm) % R
        total += yj * num * inv(den)
    return total % R


def barycentric_eval(values, omega: int, x: int) -> int:
    """Same value as lagrange_eval in O(n) Python operations, using
    L_j(x) = omega^j (x^n - 1) / (n (x - omega^j)) on the n-th roots of unity."""
    n = len(values)
    acc, wj = 0, 1
    for yj in values:
        acc += yj * wj * inv((x - wj) % R)
        wj = wj * omega % R
    return acc * (pow(x, n, R) - 1) * inv(n) % R


def is_probable_prime(m: int) -> bool:
    """Deterministic Miller-Rabin over the first 20 prime bases."""
    if m < 2:
        return False
    small = [2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41, 43, 47, 53, 59, 61, 67, 71]
    for p in small:
        if m % p == 0:
            return m == p
    d, s = m - 1, 0
    while d % 2 == 0:
        d //= 2
        s += 1
    for a in small:
        x = pow(a, d, m)
        if x in (1, m - 1):
            continue
        for _ in range(s - 1):
            x = x * x % m
            if x == m - 1:
                break
        else:
            return False
    return True
