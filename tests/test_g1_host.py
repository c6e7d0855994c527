"""The library's base field, G1 formulas and MSM digit recoding (fp.hpp, g1.hpp,
msm_digit.hpp) compiled for the host and checked against Python integers and the MSM
oracle; and the host-side window combination of libg16.so (g16_msm_g1_finish) against
the oracle's MSM by definition.  The same sources are compiled for gfx950; the GPU tests
check the device build."""
import ctypes
import os
import random
import subprocess

import numpy as np
import pytest

from groth16_polynomial_amd import binding, synth
from oracle import msm

R = synth.R_MODULUS
P = msm.modulus()
RR = 1 << 256
RINV = pow(RR, -1, P)
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("g1host") / "g1_host_driver")
    cmd = ["/opt/rocm/bin/hipcc", "--offload-host-only", "-O2", "-std=c++17",
           "-I", os.path.join(ROOT, "groth16_polynomial_amd", "csrc"),
           "-o", exe, os.path.join(HERE, "g1_host_driver.cpp")]
    subprocess.check_call(cmd, stderr=subprocess.DEVNULL)
    return exe


def run(exe, lines):
    inp = "".join(" ".join([op] + ["%x" % v for v in args]) + "\n" for op, *args in lines)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return out.splitlines()


def ints_of(line):
    return [int(v, 16) for v in line.split()]


def rand_below(rng, m, n):
    return [rng.randrange(m) for _ in range(n)]


EDGE = [0, 1, 2, P - 1, P - 2, RR % P, (P - 1) // 2, 2**253, 2**64 - 1]


def test_field(driver):
    rng = random.Random(11)
    xs = EDGE + rand_below(rng, P, 2000)
    ys = list(reversed(EDGE)) + rand_below(rng, P, 2000)
    lines = [(op, x, y) for x, y in zip(xs, ys) for op in ("fpmul", "fpadd", "fpsub")]
    got = [ints_of(l)[0] for l in run(driver, lines)]
    want = []
    for x, y in zip(xs, ys):
        want += [x * y * RINV % P, (x + y) % P, (x - y) % P]
    assert got == want
    one = [("fpinv", x) for x in xs[:300]] + [("tomont", x) for x in xs[:300]] + \
          [("frommont", x) for x in xs[:300]] + [("fpneg", x) for x in xs[:300]]
    got = [ints_of(l)[0] for l in run(driver, one)]
    inv = [pow(x * RINV, -1, P) * RR % P if x else 0 for x in xs[:300]]   # Montgomery domain
    assert got == inv + [x * RR % P for x in xs[:300]] + [x * RINV % P for x in xs[:300]] + \
        [(-x) % P for x in xs[:300]]


def test_field_digits(driver):
    """The 29-bit digit form: products, sums, differences and a lazy chain, all through
    the conversions in and out of the canonical 2^256 form."""
    rng = random.Random(12)
    xs = EDGE + rand_below(rng, P, 2000)
    ys = list(reversed(EDGE)) + rand_below(rng, P, 2000)
    lines = [(op, x, y) for x, y in zip(xs, ys)
             for op in ("f29mul", "f29add", "f29sub", "f29canon", "f29lazy")]
    got = [ints_of(l)[0] for l in run(driver, lines)]
    want = []
    for x, y in zip(xs, ys):
        d = (x - 7 * y) % P
        want += [x * y * RINV % P, (x + y) % P, (x - y) % P, x,
                 (d * d * RINV - 5 * x * y * RINV) % P]
    assert got == want
    zs = rand_below(rng, P, 2000)
    ws = list(reversed(zs))
    lines = [("f29sqr", x) for x in xs] + \
        [("f29mulsub", x, y, z, w) for x, y, z, w in zip(xs, ys, zs + EDGE, ws + EDGE)]
    got = [ints_of(l)[0] for l in run(driver, lines)]
    want = [x * x * RINV % P for x in xs] + \
        [(x * y - z * w) * RINV % P for x, y, z, w in zip(xs, ys, zs + EDGE, ws + EDGE)]
    assert got == want


def test_digit_zero_test(driver):
    """The exact zero test of the digit form on lazy values: 32 (a + b) is a multiple of p
    (nonzero digits) when a + b = p, and 32 (a - b) when a = b; one off is not zero."""
    rng = random.Random(13)
    cases = []
    for _ in range(300):
        a = rng.randrange(1, P)
        cases += [(a, P - a), (a, a), (a, (P - a + 1) % P), (a, (a + 1) % P), (a, rng.randrange(P))]
    cases += [(0, 0), (1, P - 1), (P - 1, 1), (P - 1, P - 1)]
    got = run(driver, [("f29zero", a, b) for a, b in cases])
    for (a, b), line in zip(cases, got):
        s, d = (int(v) for v in line.split())
        assert s == int((a + b) % P == 0), (a, b)
        assert d == int((a - b) % P == 0), (a, b)


def _points(seed, n):
    ks = [random.Random(seed + i).randrange(1, R) for i in range(n)]
    return msm.words_to_points(msm.scalar_mul(msm.to_words(ks)))


def _oracle_add(ps, qs):
    return msm.words_to_points(msm.affine_op("add", msm.points_to_words(ps),
                                             msm.points_to_words(qs)))


def _oracle_dbl(ps):
    return msm.words_to_points(msm.affine_op("double", msm.points_to_words(ps)))


def _flat(p):
    return (0, 0) if p is None else p


def _out(lines):
    res = []
    for l in lines:
        x, y = ints_of(l)
        res.append(None if x == 0 and y == 0 else (x, y))
    return res


def test_point_formulas_against_oracle(driver):
    ps, qs = _points(100, 60), _points(200, 60)
    neg = msm.words_to_points(msm.affine_op("neg", msm.points_to_words(ps)))
    p2 = _oracle_dbl(ps)
    q2 = _oracle_dbl(qs)
    lines = []
    for p, q in zip(ps, qs):
        lines += [("madd", *_flat(p), *_flat(q)), ("madd1", *_flat(p), *_flat(q)),
                  ("add", *_flat(p), *_flat(q)), ("add1", *_flat(p), *_flat(q)),
                  ("dbl", *_flat(p)), ("dblaff", *_flat(p))]
    got = _out(run(driver, lines))
    want = []
    s1 = _oracle_add(p2, qs)
    s2 = _oracle_add(ps, qs)
    s3 = _oracle_add(p2, q2)
    d4 = _oracle_dbl(p2)
    for i in range(len(ps)):
        want += [s1[i], s2[i], s3[i], s2[i], d4[i], p2[i]]
    assert got == want


def test_point_formulas_in_digits(driver):
    """The same formulas instantiated on the 29-bit digit form (what the device runs)."""
    ps, qs = _points(110, 60), _points(210, 60)
    p2 = _oracle_dbl(ps)
    q2 = _oracle_dbl(qs)
    lines = []
    for p, q in zip(ps, qs):
        lines += [("madd29", *p, *q), ("madd129", *p, *q), ("add29", *p, *q), ("add129", *p, *q)]
    got = _out(run(driver, lines))
    s1, s2, s3 = _oracle_add(p2, qs), _oracle_add(ps, qs), _oracle_add(p2, q2)
    want = []
    for i in range(len(ps)):
        want += [s1[i], s2[i], s3[i], s2[i]]
    assert got == want
    neg = msm.words_to_points(msm.affine_op("neg", msm.points_to_words(ps)))
    inf = (0, 0)
    lines = []
    for p, m in zip(ps[:10], neg[:10]):
        lines += [("madd129", *p, *p), ("madd129", *p, *m), ("add129", *p, *p),
                  ("add129", *p, *m), ("madd129", *inf, *p), ("madd129", *p, *inf),
                  ("add129", *inf, *inf)]
    got = _out(run(driver, lines))
    want = []
    for p, d in zip(ps[:10], p2[:10]):
        want += [d, None, d, None, p, p, None]
    assert got == want
    ks = [0, 1, 2, 3, 255, 32767, 65535, 123456789]
    got = _out(run(driver, [("mulsmall29", k, *p) for p in ps[:4] for k in ks]))
    want = []
    for p in ps[:4]:
        want += msm.words_to_points(msm.scalar_mul(msm.to_words(ks), p))
    assert got == want


def test_point_special_cases(driver):
    ps = _points(300, 12)
    neg = msm.words_to_points(msm.affine_op("neg", msm.points_to_words(ps)))
    p2 = _oracle_dbl(ps)
    inf = (0, 0)
    lines = []
    for p, m in zip(ps, neg):
        lines += [("madd1", *p, *p),          # P + P: doubling
                  ("madd1", *p, *m),          # P + (-P): infinity
                  ("add1", *p, *p), ("add1", *p, *m),
                  ("madd1", *inf, *p),        # infinity + P
                  ("madd1", *p, *inf),        # P + infinity
                  ("add1", *inf, *p), ("add1", *p, *inf), ("add1", *inf, *inf),
                  ("dbl", *inf)]
    got = _out(run(driver, lines))
    want = []
    for p, d in zip(ps, p2):
        want += [d, None, d, None, p, p, p, p, None, None]
    assert got == want


def test_mul_small(driver):
    ps = _points(400, 8)
    ks = [0, 1, 2, 3, 7, 8, 255, 4096, 32767, 65535, 1 << 20, 123456789]
    lines = [("mulsmall", k, *p) for p in ps for k in ks]
    got = _out(run(driver, lines))
    want = []
    for p in ps:
        want += msm.words_to_points(msm.scalar_mul(msm.to_words(ks), p))
    assert got == want


@pytest.mark.parametrize("c", [1, 2, 3, 4, 5, 7, 8, 9, 11, 12, 13, 15, 16, 17, 20, 23, 24])
def test_signed_digits_recompose(driver, c):
    rng = random.Random(c)
    ks = [0, 1, 2, R - 1, R - 2, 2**253, 2**254 - 1, (1 << (c - 1)), (1 << c) - 1] + \
        rand_below(rng, R, 200)
    got = run(driver, [("digits", c, k) for k in ks])
    windows = -(-255 // c)
    for k, line in zip(ks, got):
        ds = [int(v) for v in line.split()]
        assert len(ds) == windows
        assert all(1 - (1 << (c - 1)) <= d <= 1 << (c - 1) for d in ds), (c, k)
        assert sum(d << (c * w) for w, d in enumerate(ds)) == k, (c, k)


@pytest.mark.parametrize("c", [1, 2, 3, 9, 15, 16])
def test_digit_codes(driver, c):
    """The 16-bit digit codes: every digit of [1 - 2^(c-1), 2^(c-1)] gets a distinct code
    below 2^c; decoding gives the bucket row |d| - 1 and the sign, and only the zero digit
    decodes as empty."""
    half = 1 << (c - 1)
    ds = list(range(1 - half, half + 1)) if c <= 9 else \
        [1 - half, 2 - half, -2, -1, 0, 1, 2, 12345, half - 1, half]
    got = run(driver, [("code", c, d & 0xffffffff) for d in ds])
    codes = set()
    for d, line in zip(ds, got):
        code, nz, row, neg = (int(v) for v in line.split())
        assert 0 <= code < 1 << c
        codes.add(code)
        assert nz == int(d != 0)
        if d:
            assert (row, neg) == (abs(d) - 1, int(d < 0)), d
    assert len(codes) == len(ds)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from groth16_polynomial_amd import build
        build.build()
    return binding.load()


def _xyzz_words(points, rng):
    """Affine points -> XYZZ Montgomery words with a random Z (Z^2, Z^3 scaling)."""
    out = np.zeros((len(points), 32), np.uint32)
    for i, pt in enumerate(points):
        if pt is None:
            continue
        z = rng.randrange(1, P)
        zz, zzz = z * z % P, z * z * z % P
        vals = [pt[0] * zz % P, pt[1] * zzz % P, zz, zzz]
        out[i] = msm.to_words([v * RR % P for v in vals]).reshape(-1)
    return out


@pytest.mark.parametrize("c", [1, 4, 13, 16])
def test_host_window_combination(lib, c):
    """g16_msm_g1_finish (host code of libg16.so) = sum_w 2^(cw) W_w by the oracle."""
    rng = random.Random(50 + c)
    windows = binding.load().g16_msm_g1_window_count(c)
    assert windows == -(-255 // c)
    pts = _points(500 + c, windows)
    pts[windows // 2] = None                        # an infinite window sum too
    sums = _xyzz_words(pts, rng)
    out = np.zeros(16, np.uint32)
    rc = lib.g16_msm_g1_finish(c, sums.ctypes.data, out.ctypes.data)
    assert rc == 0
    scal = [1 << (c * w) for w in range(windows)]
    want = msm.msm(msm.to_words([s % R for s in scal]), msm.points_to_words(pts))
    assert np.array_equal(out, want)
    assert lib.g16_msm_g1_finish(0, sums.ctypes.data, out.ctypes.data) == binding.G16_EINVAL
    assert lib.g16_msm_g1_finish(17, sums.ctypes.data, out.ctypes.data) == binding.G16_EINVAL


def test_generated_columns_up_to_date():
    """fp29_cols.hpp is what fp29_cols_gen.py writes (the device's column chains)."""
    gen = os.path.join(ROOT, "groth16_polynomial_amd", "csrc", "fp29_cols_gen.py")
    assert subprocess.run(["python3", gen, "--check"]).returncode == 0
