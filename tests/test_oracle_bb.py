"""Pins of the BabyBear NTT oracle (oracle/bb_oracle.c) against what the mathematics
fixes, independently of the oracle's own code: Python integers for the field and the
Montgomery conversion, the transform's definition (an O(n^2) sum) for small sizes, the
closed forms of the roots, special vectors, the round trip, the low-degree extension's
restriction to the smaller domain, Horner evaluation at scattered points, and the matrix
layout column by column.  Planted mistakes in a copy of the C source must each make a
pin fail."""
import multiprocessing as mp
import random

import numpy as np
import pytest

from oracle import bb

P = (1 << 31) - (1 << 27) + 1
R32 = (1 << 32) % P


def mont(xs):
    return [x * R32 % P for x in xs]


def unmont(ys):
    inv = pow(R32, P - 2, P)
    return [y * inv % P for y in ys]


def py_dft(xs, w):
    n = len(xs)
    return [sum(x * pow(w, i * j, P) for j, x in enumerate(xs)) % P for i in range(n)]


def rand_elems(seed, n):
    rng = random.Random(seed)
    return [rng.randrange(P) for _ in range(n)]


def test_modulus_and_generator():
    assert bb.modulus() == P
    # p is prime (deterministic Miller-Rabin bases for n < 3.4e14), p - 1 = 2^27 * 15
    d, s = P - 1, 0
    while d % 2 == 0:
        d //= 2
        s += 1
    assert (s, d) == (27, 15)
    for a in (2, 3, 5, 7, 11, 13, 17):
        x = pow(a, d, P)
        assert x in (1, P - 1) or any(pow(x, 1 << r, P) == P - 1 for r in range(1, s))
    g = bb.generator()
    assert g == 31
    for q in (2, 3, 5):
        assert pow(g, (P - 1) // q, P) != 1
    # and no smaller element generates the group
    for h in range(2, 31):
        assert any(pow(h, (P - 1) // q, P) == 1 for q in (2, 3, 5))


@pytest.mark.parametrize("L", list(range(0, 28)))
def test_roots_closed_form(L):
    w, size_inv = bb.roots(L)
    assert pow(w, 1 << L, P) == 1
    if L:
        assert pow(w, 1 << (L - 1), P) == P - 1
    assert (1 << L) * size_inv % P == 1
    assert w == pow(pow(31, (P - 1) >> 27, P), 1 << (27 - L), P)


def test_field_ops_and_conversions():
    xs = [0, 1, 2, P - 1, P - 2, (1 << 31) % P, (1 << 30)] + rand_elems(1, 3000)
    ys = list(reversed(xs))
    a, b = np.array(xs, np.uint32), np.array(ys, np.uint32)
    assert bb.field_op("add", a, b).tolist() == [(x + y) % P for x, y in zip(xs, ys)]
    assert bb.field_op("sub", a, b).tolist() == [(x - y) % P for x, y in zip(xs, ys)]
    assert bb.field_op("mul", a, b).tolist() == [x * y % P for x, y in zip(xs, ys)]
    assert bb.to_mont(a).tolist() == mont(xs)
    assert bb.from_mont(bb.to_mont(a)).tolist() == xs
    with pytest.raises(ValueError):
        bb.field_op("add", np.array([P], np.uint32), np.array([0], np.uint32))


@pytest.mark.parametrize("L", [0, 1, 2, 3, 5, 6])
def test_dft_naive_is_the_definition(L):
    xs = rand_elems(10 + L, 1 << L)
    w, _ = bb.roots(L)
    assert bb.dft_naive(np.array(xs, np.uint32), L).tolist() == py_dft(xs, w)
    inv = [v * pow(1 << L, P - 2, P) % P for v in py_dft(xs, pow(w, P - 2, P))]
    assert bb.dft_naive(np.array(xs, np.uint32), L, inverse=True).tolist() == inv


@pytest.mark.parametrize("L", [1, 2, 4, 7])
def test_ntt_against_definition(L):
    xs = rand_elems(20 + L, 1 << L)
    w, _ = bb.roots(L)
    got = unmont(bb.ntt_mont(np.array(mont(xs), np.uint32), L).tolist())
    assert got == py_dft(xs, w)


def test_brute_force_two_points():
    x0, x1 = 123456789, P - 5
    got = unmont(bb.ntt_mont(np.array(mont([x0, x1]), np.uint32), 1).tolist())
    assert got == [(x0 + x1) % P, (x0 - x1) % P]


def test_special_vectors():
    L, n = 9, 1 << 9
    w, _ = bb.roots(L)
    e0 = [1] + [0] * (n - 1)
    assert unmont(bb.ntt_mont(np.array(mont(e0), np.uint32), L).tolist()) == [1] * n
    ones = [1] * n
    assert unmont(bb.ntt_mont(np.array(mont(ones), np.uint32), L).tolist()) == [n] + [0] * (n - 1)
    e1 = [0, 1] + [0] * (n - 2)
    assert unmont(bb.ntt_mont(np.array(mont(e1), np.uint32), L).tolist()) == \
        [pow(w, i, P) for i in range(n)]
    assert not bb.ntt_mont(np.zeros(n, np.uint32), L).any()


def test_linearity_and_round_trip():
    for L in (3, 10, 16):
        n = 1 << L
        x, y = rand_elems(30 + L, n), rand_elems(40 + L, n)
        alpha = 987654321
        fx = unmont(bb.ntt_mont(np.array(mont(x), np.uint32), L).tolist())
        fy = unmont(bb.ntt_mont(np.array(mont(y), np.uint32), L).tolist())
        comb = [(a + alpha * b) % P for a, b in zip(x, y)]
        fc = unmont(bb.ntt_mont(np.array(mont(comb), np.uint32), L).tolist())
        assert fc == [(a + alpha * b) % P for a, b in zip(fx, fy)]
        back = bb.ntt_mont(bb.ntt_mont(np.array(mont(x), np.uint32), L), L, inverse=True)
        assert unmont(back.tolist()) == x


def test_horner_at_scattered_points():
    """Evaluations of a 2^14 transform at scattered indices are the polynomial's values at
    the powers of the root (Horner's rule in Python)."""
    L = 14
    xs = rand_elems(50, 1 << L)
    w, _ = bb.roots(L)
    got = unmont(bb.ntt_mont(np.array(mont(xs), np.uint32), L).tolist())
    for i in (0, 1, 2, 777, 8191, 8192, (1 << L) - 1):
        pt, acc = pow(w, i, P), 0
        for c in reversed(xs):
            acc = (acc * pt + c) % P
        assert got[i] == acc, i


@pytest.mark.parametrize("L,rate", [(6, 1), (10, 2), (12, 3), (9, 0)])
def test_low_degree_extension(L, rate):
    """The zero-padded transform on 2^L points restricted to the subgroup of 2^(L-rate)
    points (every 2^rate-th output) is the transform of the unpadded coefficients, and at
    small sizes every output is the definition's value."""
    k = L - rate
    xs = rand_elems(60 + L, 1 << k)
    big = bb.ntt_mont(np.array(mont(xs), np.uint32), L, log_in=k)
    small = bb.ntt_mont(np.array(mont(xs), np.uint32), k)
    assert big[:: 1 << rate].tolist() == small.tolist()
    if L <= 10:
        w, _ = bb.roots(L)
        assert unmont(big.tolist()) == py_dft(xs + [0] * ((1 << L) - len(xs)), w)


def test_matrix_columns_and_batches():
    """Row-major matrices of 2^lw columns: column c of the output is the transform of
    column c alone; several matrices one after another are independent."""
    L, lw, count, log_in = 8, 3, 2, 7
    w = 1 << lw
    m = np.array(mont(rand_elems(70, count * w << log_in)), np.uint32)
    out = bb.ntt_mont(m, L, log_w=lw, count=count, log_in=log_in).reshape(count, 1 << L, w)
    src = m.reshape(count, 1 << log_in, w)
    for v in range(count):
        for c in range(w):
            one = bb.ntt_mont(np.ascontiguousarray(src[v, :, c]), L, log_in=log_in)
            assert out[v, :, c].tolist() == one.tolist()


# ------------------------------------------------------------------ sharpness

MUTATIONS = [
    ("butterfly outputs swapped",
     "x[start + j] = add_p(u, v);\n                x[start + j + half] = sub_p(u, v);",
     "x[start + j] = sub_p(u, v);\n                x[start + j + half] = add_p(u, v);"),
    ("twiddle index without stride", "tw[j * step]", "tw[j]"),
    ("bit reversal dropped", "if (j > i) { u64 t = x[i]; x[i] = x[j]; x[j] = t; }", ""),
    ("another generator", "const u64 q[3] = {2, 3, 5};", "const u64 q[3] = {2, 3, 3};"),
    ("padding rows read", "if (i < h_in) {", "if (1) {"),
    ("column-major read", "u32 y = src[i * w + c];", "u32 y = src[c * h_in + i];"),
    ("no Montgomery on output", "dst[i * w + c] = (u32)to_mont(mul_p(col[i], scale));",
     "dst[i * w + c] = (u32)mul_p(col[i], scale);"),
    ("subtraction without wrap", "static u64 sub_p(u64 a, u64 b) { return (a + P - b) % P; }",
     "static u64 sub_p(u64 a, u64 b) { return (a - b) % P; }"),
]


def _pins_pass() -> bool:
    try:
        if bb.generator() != 31:
            return False
        for L in (1, 4, 7):
            xs = rand_elems(80 + L, 1 << L)
            w, _ = bb.roots(L)
            if pow(w, 1 << (L - 1), P) != P - 1:
                return False
            if unmont(bb.ntt_mont(np.array(mont(xs), np.uint32), L).tolist()) != py_dft(xs, w):
                return False
        xs = rand_elems(90, 32)
        big = bb.ntt_mont(np.array(mont(xs), np.uint32), 6, log_in=5)
        w6, _ = bb.roots(6)
        if unmont(big.tolist()) != py_dft(xs + [0] * 32, w6):
            return False
        m = np.array(mont(rand_elems(91, 64)), np.uint32)
        out = bb.ntt_mont(m, 4, log_w=2).reshape(16, 4)
        for c in range(4):
            col = unmont(m.reshape(16, 4)[:, c].tolist())
            if unmont(out[:, c].tolist()) != py_dft(col, bb.roots(4)[0]):
                return False
    except ValueError:
        return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


def _child(path, q):
    with bb.use_library(bb.open_library(path)):
        q.put(_pins_pass())


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = bb.source_text()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %s" % name
    path = bb.compile_source(src.replace(old, new), str(tmp_path / "libbb_mut.so"))
    ctx = mp.get_context("fork")
    q = ctx.Queue()
    p = ctx.Process(target=_child, args=(path, q))
    p.start()
    p.join(30)
    if p.is_alive():
        p.kill()
        p.join()
        return
    assert p.exitcode == 0 or p.exitcode < 0, "mutated oracle child failed: %s" % name
    if p.exitcode == 0:
        assert q.get(timeout=5) is False, "pins did not catch: %s" % name
