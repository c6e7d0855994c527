"""The library's Fr layer (fr.hpp) compiled for the host and checked against Python
integers: Montgomery product, add, sub, conversions, powers and inverse.  The same
source is compiled for gfx950; the GPU tests check the device build."""
import os
import random
import subprocess

import pytest

from groth16_polynomial_amd import synth

R = synth.R_MODULUS
RR = 1 << 256
RINV = pow(RR, -1, R)
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("frhost") / "fr_host_driver")
    cmd = ["/opt/rocm/bin/hipcc", "--offload-host-only", "-O2", "-std=c++17",
           "-I", os.path.join(ROOT, "groth16_polynomial_amd", "csrc"),
           "-o", exe, os.path.join(HERE, "fr_host_driver.cpp")]
    subprocess.check_call(cmd, stderr=subprocess.DEVNULL)
    return exe


def run(exe, lines):
    inp = "".join("%s %x %x\n" % (op, a, b) for op, a, b in lines)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return [int(v, 16) for v in out.split()]


EDGE = [0, 1, 2, R - 1, R - 2, RR % R, (R - 1) // 2, 2**253, 2**64 - 1, 2**128 + 3]


def test_mont_mul_add_sub(driver):
    rng = random.Random(7)
    xs = EDGE + [rng.randrange(R) for _ in range(3000)]
    ys = list(reversed(EDGE)) + [rng.randrange(R) for _ in range(3000)]
    lines = [(op, x, y) for x, y in zip(xs, ys) for op in ("mul", "add", "sub")]
    got = run(driver, lines)
    want = []
    for x, y in zip(xs, ys):
        want += [x * y * RINV % R, (x + y) % R, (x - y) % R]
    assert got == want


def test_mul_edge_pairs(driver):
    lines = [("mul", x, y) for x in EDGE for y in EDGE]
    assert run(driver, lines) == [x * y * RINV % R for _, x, y in lines]


def test_conversions_pow_inv(driver):
    rng = random.Random(8)
    xs = EDGE + [rng.randrange(R) for _ in range(500)]
    got = run(driver, [("tomont", x, 0) for x in xs] + [("frommont", x, 0) for x in xs])
    assert got == [x * RR % R for x in xs] + [x * RINV % R for x in xs]
    # powers and inverses act on Montgomery representatives
    cases = [(rng.randrange(1, R), rng.randrange(1 << 64)) for _ in range(20)]
    got = run(driver, [("pow", x * RR % R, e) for x, e in cases])
    assert got == [pow(x, e, R) * RR % R for x, e in cases]
    got = run(driver, [("inv", x * RR % R, 0) for x, _ in cases])
    assert got == [pow(x, -1, R) * RR % R for x, _ in cases]


def test_table_product_radix_2_261(driver):
    """fr_mul_tab: the nine-limb product with Montgomery radix 2^261, x * w * 2^-261."""
    rng = random.Random(9)
    xs = EDGE + [rng.randrange(R) for _ in range(3000)]
    ws = list(reversed(EDGE)) + [rng.randrange(R) for _ in range(3000)]
    inv261 = pow(1 << 261, -1, R)
    got = run(driver, [("mul29", x, w) for x, w in zip(xs, ws)])
    assert got == [x * w * inv261 % R for x, w in zip(xs, ws)]
    # the 2^261-form table entry w * 2^261 turns it into the ordinary product form
    got = run(driver, [("mul29", x, w * (1 << 261) % R) for x, w in zip(xs, ws)])
    assert got == [x * w % R for x, w in zip(xs, ws)]
    # limb repacking is the identity on 256-bit values
    vals = [rng.randrange(1 << 256) for _ in range(200)] + [0, (1 << 256) - 1]
    assert run(driver, [("unpack29", v, 0) for v in vals]) == vals


def test_lazy_range_helpers(driver):
    """The in-kernel lazy forms: [0, 4r) -> [0, 2r) and -> canonical, a + b and a + 2r - b
    without reduction, and the unreduced 2^261 product (below 2r for any 256-bit x)."""
    rng = random.Random(10)
    x4 = [0, 1, R - 1, R, 2 * R - 1, 2 * R, 3 * R + 5, 4 * R - 1] + \
        [rng.randrange(4 * R) for _ in range(2000)]
    got = run(driver, [("red2r", x, 0) for x in x4] + [("canon4r", x, 0) for x in x4])
    n = len(x4)
    assert got[:n] == [x - 2 * R if x >= 2 * R else x for x in x4]
    assert got[n:] == [x % R for x in x4]
    a2 = [rng.randrange(2 * R) for _ in range(2000)] + [0, 2 * R - 1]
    b2 = [rng.randrange(2 * R + 1) for _ in range(2000)] + [2 * R, 0]
    got = run(driver, [("addlazy", a, b) for a, b in zip(a2, b2)] +
              [("sublazy", a, b) for a, b in zip(a2, b2)])
    m = len(a2)
    assert got[:m] == [a + b for a, b in zip(a2, b2)]
    assert got[m:] == [a + 2 * R - b for a, b in zip(a2, b2)]
    assert all(0 <= v < 4 * R for v in got[m:])
    xs = [rng.randrange(1 << 256) for _ in range(2000)] + [(1 << 256) - 1]
    ws = [rng.randrange(R) for _ in range(len(xs) - 1)] + [R - 1]
    inv261 = pow(1 << 261, -1, R)
    got = run(driver, [("mul29lazy", x, w) for x, w in zip(xs, ws)])
    assert [v % R for v in got] == [x * w * inv261 % R for x, w in zip(xs, ws)]
    assert all(v < 2 * R for v in got)
