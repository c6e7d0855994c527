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


def test_constant_2_261(driver):
    """2^261 mod r, the constant the table builder multiplies by."""
    assert run(driver, [("c261", 0, 0)]) == [(1 << 261) % R]
