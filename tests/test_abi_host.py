"""The C ABI on the CPU: the library loads, exports every symbol include/g16.h
declares, and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

from groth16_polynomial_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "g16.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "batch_split.txt")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from groth16_polynomial_amd import build
        build.build()
    return binding.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(g16_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
    # and the binding wraps exactly the declared set
    assert sorted(binding.SIGNATURES) == names


def test_version_and_strerror(lib):
    assert binding.abi_version() == 1
    for code in range(-6, 1):
        assert binding.strerror(code)
    assert binding.strerror(-99) == "unknown status"


def test_workspace_bytes(lib):
    assert binding.workspace_bytes(0) == 0
    assert binding.workspace_bytes(28) == 0
    for L in (1, 2, 12, 20, 27):
        n = 1 << L
        rnd = lambda x: -(-x // 256) * 256
        assert binding.workspace_bytes(L) == 3 * rnd(n * 80) + 3 * rnd(n * 32) + rnd(4 * 80)


def test_bb_workspace_bytes(lib):
    f = lib.g16_bb_workspace_bytes
    assert f(0) == 0 and f(28) == 0
    rnd = lambda x: -(-x // 256) * 256
    for L in (1, 2, 12, 20, 27):
        e = (1 << L) - 1
        assert f(L) == rnd(8 * e) + rnd(4 * e)   # Shoup pairs, then the 4-byte form


def test_batch_scratch_bytes(lib):
    f = lib.g16_h_batch_scratch_bytes
    assert f(0, 1) == 0 and f(28, 1) == 0            # log_n out of range
    assert f(12, 0) == 0                             # an empty batch needs nothing
    assert f(12, 5) == 5 * 4096 * 32
    assert f(20, 16) == 16 * (1 << 20) * 32
    assert f(1, 16384) == 16384 * 2 * 32             # the proof-count limit itself
    assert f(1, 16385) == 0                          # beyond it
    assert f(27, 16) == 16 * (1 << 27) * 32          # 2^31 elements: the element limit
    assert f(27, 17) == 0


def test_msm_sizes(lib):
    """Window counts, default widths and workspace limits of the G1 MSM (host only)."""
    assert lib.g16_msm_g1_window_count(0) == 0 and lib.g16_msm_g1_window_count(17) == 0
    for c in range(1, 17):
        assert lib.g16_msm_g1_window_count(c) == -(-255 // c)
    for log_n in range(0, 27):
        c = lib.g16_msm_g1_window_bits(1 << log_n)
        assert 1 <= c <= 16
        assert lib.g16_msm_g1_workspace_bytes(1 << log_n, 0) > 0
    assert lib.g16_msm_g1_window_bits(1 << 20) == 16
    assert lib.g16_msm_g1_workspace_bytes(0, 16) == 0            # empty: nothing needed
    assert lib.g16_msm_g1_workspace_bytes(1 << 20, 17) == 0      # c beyond the LDS counters
    assert lib.g16_msm_g1_workspace_bytes(1 << 28, 16) == 0      # windows * n reaches 2^32
    assert lib.g16_msm_g1_workspace_bytes((1 << 28) - 1, 16) > 0
    fake = ctypes.c_void_p(0x100000)
    assert lib.g16_msm_g1(16, fake, fake, 17, fake, 1 << 20, None, None) == binding.G16_EINVAL
    assert lib.g16_g1_generator_mul(0, fake, fake, None) == binding.G16_EINVAL
    assert lib.g16_msm_g1_finish(16, None, None) == binding.G16_EINVAL


def test_batch_plan_matches_page(lib):
    with open(GOLDEN) as f:
        rows = [list(map(int, l.split())) for l in f if l.strip() and not l.startswith("#")]
    for row in rows:
        L, kmax, want = row[0], row[1], row[2:]
        assert sorted(binding.batch_plan(L, kmax)) == sorted(want)


@pytest.mark.parametrize("kmax", list(range(1, 13)))
def test_batch_plan_rule(lib, kmax):
    for L in range(1, 28):
        ks = binding.batch_plan(L, kmax)
        assert sum(ks) == L
        assert len(ks) == -(-L // kmax)                 # ceil(log n / kmax) batches
        assert max(ks) <= kmax and max(ks) - min(ks) <= 1   # near-equal, no tiny tail
        assert ks == sorted(ks, reverse=True)


def test_default_batch_plan(lib, monkeypatch):
    """kmax = 0 without G16_MAX_K: the near-equal split under a cap of 10, except the
    measured plans at 2^21, 2^22, 2^23, 2^25 and 2^26; from 2^12 up every batch keeps 6..10
    passes (no tiny tail)."""
    monkeypatch.delenv("G16_MAX_K", raising=False)
    measured = {21: [6, 7, 8], 22: [8, 6, 8], 23: [8, 7, 8], 25: [10, 8, 7], 26: [10, 8, 8]}
    for L in range(1, 28):
        ks = binding.batch_plan(L, 0)
        assert ks == measured.get(L, binding.batch_plan(L, 10)), L
        assert sum(ks) == L and len(ks) == -(-L // 10)
        if L >= 12:
            assert 6 <= min(ks) and max(ks) <= 10
    monkeypatch.setenv("G16_MAX_K", "10")
    assert binding.batch_plan(22, 0) == [8, 7, 7]


def test_batch_plan_errors(lib):
    for bad_L in (0, 28):
        with pytest.raises(binding.G16Error):
            binding.batch_plan(bad_L, 10)
    with pytest.raises(binding.G16Error):
        binding.batch_plan(10, 13)


def test_host_side_argument_errors(lib):
    """Paths that return before any HIP call."""
    P = ctypes.c_void_p
    ctx = ctypes.c_void_p()
    fake = P(0x100000)  # never dereferenced: every case below fails its host checks first
    assert lib.g16_h_prepare(20, fake, 1 << 30, None, None) == binding.G16_EINVAL
    assert lib.g16_h_prepare(20, None, 1 << 30, None, ctypes.byref(ctx)) == binding.G16_EINVAL
    assert lib.g16_h_prepare(0, fake, 1 << 30, None, ctypes.byref(ctx)) == binding.G16_ERANGE
    assert lib.g16_h_prepare(28, fake, 1 << 30, None, ctypes.byref(ctx)) == binding.G16_ERANGE
    assert lib.g16_h_prepare(20, fake, 1000, None, ctypes.byref(ctx)) == binding.G16_ENOSPACE
    assert lib.g16_h_prepare(12, P(0x100010), 1 << 30, None, ctypes.byref(ctx)) == \
        binding.G16_EINVAL  # misaligned
    assert lib.g16_release(None) == binding.G16_EINVAL
    assert lib.g16_ctx_log_n(None) == 0
    assert lib.g16_domain_roots(None, None, None, None) == binding.G16_EINVAL
    for f in ("g16_ntt_forward", "g16_ntt_inverse", "g16_coset_eval"):
        assert getattr(lib, f)(None, fake, fake, None) == binding.G16_EINVAL
    assert lib.g16_h_compute(None, fake, fake, fake, fake, fake, None) == binding.G16_EINVAL
    assert lib.g16_h_compute_batch(None, 2, fake, fake, fake, fake, fake, fake, 1 << 20,
                                   None) == binding.G16_EINVAL
    # h_join: zero length, NULLs, outputs overlapping each other or an input
    assert lib.g16_h_join(0, fake, fake, fake, P(0x200000), P(0x300000), None) == \
        binding.G16_EINVAL
    assert lib.g16_h_join(16, None, fake, fake, P(0x200000), P(0x300000), None) == \
        binding.G16_EINVAL
    assert lib.g16_h_join(16, fake, fake, fake, P(0x200000), P(0x200100), None) == \
        binding.G16_EALIAS
    assert lib.g16_h_join(16, fake, fake, fake, P(0x100100), P(0x300000), None) == \
        binding.G16_EALIAS
    # element-wise: partial overlap of in and out
    assert lib.g16_fr_mul(16, fake, fake, P(0x100020), None) == binding.G16_EALIAS
    assert lib.g16_to_mont(0, fake, fake, None) == binding.G16_EINVAL
    # gather: zero rows, null witness, outputs overlapping
    z = P(0x400000)
    assert lib.g16_gather_abc(0, z, z, z, 1, z, z, z, 1, z, 1, P(1 << 24), P(2 << 24),
                              P(3 << 24), None) == binding.G16_EINVAL
    assert lib.g16_gather_abc(8, z, z, z, 1, z, z, z, 1, None, 1, P(1 << 24), P(2 << 24),
                              P(3 << 24), None) == binding.G16_EINVAL
    assert lib.g16_gather_abc(8, z, z, z, 1, z, z, z, 1, z, 1, P(1 << 24), P(1 << 24),
                              P(3 << 24), None) == binding.G16_EALIAS


def test_probe_library_exports_its_header():
    """libg16_probe.so loads and exports what include/g16_probe.h declares."""
    from groth16_polynomial_amd import probe
    if not os.path.exists(probe.PROBE_PATH):
        from groth16_polynomial_amd import build
        build.build()
    text = open(os.path.join(ROOT, "include", "g16_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(g16_\w+)\s*\(", text)))
    assert names == ["g16_probe_rate"]
    lib = probe.load()
    for name in names:
        assert hasattr(lib, name), name
    # host-side argument checks (nothing is launched)
    assert lib.g16_probe_rate(9, 1, 1, 0, None, None, None) == -1


def test_probe_host_reference_small():
    """The probe's host reference of its chains, against plain Python integers."""
    from groth16_polynomial_amd import probe
    blocks, iters, seed = 1, 5, 99
    got = probe.expected(0, blocks, iters, seed)
    m = (1 << 64) - 1
    for gid in (0, 1, 200):
        x = ((gid * 2654435761) & 0xffffffff) ^ seed
        want = 0
        for k in range(8):
            a = ((gid + k) * 0x9E3779B97F4A7C15) & m
            for _ in range(iters):
                a = (a + x * (seed | 1)) & m
            want ^= a
        assert int(got[gid]) == want
    got3 = probe.expected(3, blocks, iters, seed)
    for gid in (0, 7):
        x = ((gid * 2654435761) & 0xffffffff) ^ seed
        want = 0
        for k in range(8):
            a = (((gid + k) * 0x9E3779B9) | 1) & 0xffffffff
            for _ in range(iters):
                a = (a * x) & 0xffffffff
            want ^= a
        assert int(got3[gid]) == want


def test_release_of_unknown_context_is_refused(lib):
    """g16_release and the context calls refuse a pointer that is not a live context
    (never handed out, or released before) without reading through it."""
    bogus = ctypes.c_void_p(0x1000)
    assert lib.g16_release(bogus) == binding.G16_ESTATE
    assert lib.g16_ctx_log_n(bogus) == 0
    assert lib.g16_h_stage_count(bogus) == binding.G16_ESTATE
    assert lib.g16_release(None) == binding.G16_EINVAL
