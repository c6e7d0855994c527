"""ctypes wrapper of the C oracle (oracle.c).  TEST INFRASTRUCTURE ONLY.

Arrays cross as numpy uint32 arrays of shape (n, 8): little-endian 32-bit words of
each 256-bit element, i.e. the same bytes as four little-endian 64-bit limbs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-pthread", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_SIGNATURES = {
    "oracle_modulus": "P",
    "oracle_set_threads": "I",
    "oracle_constants": "PPP",
    "oracle_field_op": "IZPPP",
    "oracle_pow": "PPP",
    "oracle_inv": "PP",
    "oracle_convert": "IZPP",
    "oracle_domain_roots": "UPPP",
    "oracle_ntt": "UIP",
    "oracle_dft_naive": "UIPP",
    "oracle_h_pipeline": "UPPPPP",
    "oracle_coset_eval": "UPP",
    "oracle_h_at": "UPPPZPPP",
    "oracle_pointwise_mul_mont": "ZPPP",
    "oracle_gather": "ZPPPPPPPZPPP",
}
_CT = {"P": ctypes.c_void_p, "U": ctypes.c_uint, "Z": ctypes.c_size_t, "I": ctypes.c_int}


def open_library(path: str):
    """Load an oracle shared library (the default one, or a test's mutated copy)."""
    lib = ctypes.CDLL(path)
    for name, codes in _SIGNATURES.items():
        f = getattr(lib, name)
        f.argtypes = [_CT[c] for c in codes]
        f.restype = ctypes.c_int
    return lib


def compile_source(source: str, out_path: str) -> str:
    """Compile oracle C source text to a shared library at out_path."""
    src_path = out_path + ".c"
    with open(src_path, "w") as f:
        f.write(source)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", "-o",
                           out_path, src_path])
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


_override = None


class use_library:
    """Context manager: route the module functions to another oracle library."""

    def __init__(self, lib):
        self.lib = lib

    def __enter__(self):
        global _override
        self.prev = _override
        _override = self.lib
        return self.lib

    def __exit__(self, *exc):
        global _override
        _override = self.prev
        return False


def default_threads() -> int:
    """Threads the oracle uses unless told otherwise: G16_ORACLE_THREADS, else the
    host's cores, at most 16."""
    env = os.environ.get("G16_ORACLE_THREADS")
    if env:
        return max(1, min(256, int(env)))
    return max(1, min(16, os.cpu_count() or 1))


def _load():
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = open_library(_LIB)
        _lib.oracle_set_threads(default_threads())
    return _lib


def set_threads(threads: int) -> int:
    """Threads for the transforms, element-wise loops and barycentric sums; returns the
    previous setting.  Results do not depend on it."""
    return _load().oracle_set_threads(int(threads))


def _arr(x, rows=None) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.uint32)
    a = a.reshape(-1, 8)
    if rows is not None and a.shape[0] != rows:
        raise ValueError("expected %d elements, got %d" % (rows, a.shape[0]))
    return a


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s failed (%d)" % (what, rc))


def _one(v: int) -> np.ndarray:
    m = (1 << 32) - 1
    return np.array([(v >> (32 * i)) & m for i in range(8)], dtype=np.uint32)


def _int(w: np.ndarray) -> int:
    w = np.asarray(w, dtype=np.uint32).reshape(8)
    return sum(int(x) << (32 * i) for i, x in enumerate(w.tolist()))


# ------------------------------------------------------------------ scalar helpers (ints)

def modulus() -> int:
    out = np.zeros(8, np.uint32)
    _check(_load().oracle_modulus(_ptr(out)), "modulus")
    return _int(out)


def constants() -> dict:
    mu = np.zeros(10, np.uint32)
    rr = np.zeros(8, np.uint32)
    root = np.zeros(8, np.uint32)
    _check(_load().oracle_constants(_ptr(mu), _ptr(rr), _ptr(root)), "constants")
    mu_int = sum(int(x) << (32 * i) for i, x in enumerate(mu.tolist()))
    return {"barrett_mu": mu_int, "r_mod_r": _int(rr), "root_2_28": _int(root)}


def pow_int(a: int, e: int) -> int:
    out = np.zeros(8, np.uint32)
    ea, ee = _one(a), _one(e)
    _check(_load().oracle_pow(_ptr(ea), _ptr(ee), _ptr(out)), "pow")
    return _int(out)


def inv_int(a: int) -> int:
    out = np.zeros(8, np.uint32)
    ea = _one(a)
    _check(_load().oracle_inv(_ptr(ea), _ptr(out)), "inv")
    return _int(out)


def domain_roots(log_n: int):
    """(omega, shift, size_inv) of the 2^log_n domain, standard-form ints."""
    w, s, si = (np.zeros(8, np.uint32) for _ in range(3))
    _check(_load().oracle_domain_roots(log_n, _ptr(w), _ptr(s), _ptr(si)), "domain_roots")
    return _int(w), _int(s), _int(si)


# ------------------------------------------------------------------ array functions

def field_op(op: str, a, b) -> np.ndarray:
    code = {"add": 0, "sub": 1, "mul": 2}[op]
    a = _arr(a)
    b = _arr(b, a.shape[0])
    out = np.empty_like(a)
    _check(_load().oracle_field_op(code, a.shape[0], _ptr(a), _ptr(b), _ptr(out)), op)
    return out


def to_mont(x) -> np.ndarray:
    x = _arr(x)
    out = np.empty_like(x)
    _check(_load().oracle_convert(0, x.shape[0], _ptr(x), _ptr(out)), "to_mont")
    return out


def from_mont(x) -> np.ndarray:
    x = _arr(x)
    out = np.empty_like(x)
    _check(_load().oracle_convert(1, x.shape[0], _ptr(x), _ptr(out)), "from_mont")
    return out


def ntt(x, log_n: int, inverse: bool = False) -> np.ndarray:
    """Standard-form transform (natural order in and out)."""
    out = _arr(x, 1 << log_n).copy()
    _check(_load().oracle_ntt(log_n, int(inverse), _ptr(out)), "ntt")
    return out


def ntt_mont(x_mont, log_n: int, inverse: bool = False) -> np.ndarray:
    """The same transform on Montgomery-form input and output."""
    return to_mont(ntt(from_mont(x_mont), log_n, inverse))


def dft_naive(x, log_n: int, inverse: bool = False) -> np.ndarray:
    x = _arr(x, 1 << log_n)
    out = np.empty_like(x)
    _check(_load().oracle_dft_naive(log_n, int(inverse), _ptr(x), _ptr(out)), "dft_naive")
    return out


def coset_eval(log_n: int, x_mont) -> np.ndarray:
    """One vector's coset evaluations x(s w^i), Montgomery in and out."""
    x = _arr(x_mont, 1 << log_n)
    out = np.empty_like(x)
    _check(_load().oracle_coset_eval(log_n, _ptr(x), _ptr(out)), "coset_eval")
    return out


def h_pipeline(log_n: int, a_mont, b_mont, c_mont):
    """(h_mont, h_std) of the full pipeline on Montgomery inputs."""
    n = 1 << log_n
    a, b, c = _arr(a_mont, n), _arr(b_mont, n), _arr(c_mont, n)
    hm = np.empty_like(a)
    hs = np.empty_like(a)
    _check(_load().oracle_h_pipeline(log_n, _ptr(a), _ptr(b), _ptr(c), _ptr(hm), _ptr(hs)),
           "h_pipeline")
    return hm, hs


def h_at(log_n: int, a_mont, b_mont, c_mont, indices):
    """(h_mont, h_std) at the given indices only, by barycentric evaluation."""
    n = 1 << log_n
    a, b, c = _arr(a_mont, n), _arr(b_mont, n), _arr(c_mont, n)
    idx = np.ascontiguousarray(indices, dtype=np.uint32)
    hm = np.empty((len(idx), 8), np.uint32)
    hs = np.empty((len(idx), 8), np.uint32)
    _check(_load().oracle_h_at(log_n, _ptr(a), _ptr(b), _ptr(c), len(idx), _ptr(idx),
                               _ptr(hm), _ptr(hs)), "h_at")
    return hm, hs


def pointwise_mul_mont(a_mont, b_mont) -> np.ndarray:
    a = _arr(a_mont)
    b = _arr(b_mont, a.shape[0])
    out = np.empty_like(a)
    _check(_load().oracle_pointwise_mul_mont(a.shape[0], _ptr(a), _ptr(b), _ptr(out)),
           "pointwise_mul")
    return out


def gather(row_ptr_a, signal_a, value_a_mont, row_ptr_b, signal_b, value_b_mont,
           witness_mont):
    """(out_a, out_b, out_c) Montgomery, one element per CSR row."""
    rpa = np.ascontiguousarray(row_ptr_a, dtype=np.uint32)
    rpb = np.ascontiguousarray(row_ptr_b, dtype=np.uint32)
    if rpa.shape != rpb.shape:
        raise ValueError("A and B must have the same number of rows")
    rows = rpa.shape[0] - 1
    sa = np.ascontiguousarray(signal_a, dtype=np.uint32)
    sb = np.ascontiguousarray(signal_b, dtype=np.uint32)
    va = _arr(value_a_mont, int(rpa[-1]))
    vb = _arr(value_b_mont, int(rpb[-1]))
    w = _arr(witness_mont)
    oa, ob, oc = (np.empty((rows, 8), np.uint32) for _ in range(3))
    _check(_load().oracle_gather(rows, _ptr(rpa), _ptr(sa), _ptr(va), _ptr(rpb), _ptr(sb),
                                 _ptr(vb), _ptr(w), w.shape[0], _ptr(oa), _ptr(ob), _ptr(oc)),
           "gather")
    return oa, ob, oc
