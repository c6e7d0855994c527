"""ctypes wrapper of the BabyBear NTT oracle (bb_oracle.c).  TEST INFRASTRUCTURE ONLY.

Arrays cross as numpy uint32 arrays (one word per element, values < p)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bb_oracle.c")
_LIB = os.path.join(_HERE, "libbb_oracle.so")
_lib = None

P = 2013265921

_SIGNATURES = {
    "bb_oracle_modulus": "P",
    "bb_oracle_generator": "P",
    "bb_oracle_roots": "UPP",
    "bb_oracle_field_op": "IZPPP",
    "bb_oracle_convert": "IZPP",
    "bb_oracle_dft_naive": "UIPP",
    "bb_oracle_ntt": "UUZUIPP",
}
_CT = {"P": ctypes.c_void_p, "U": ctypes.c_uint, "Z": ctypes.c_size_t, "I": ctypes.c_int}


def build(force: bool = True) -> str:
    """Compile bb_oracle.c with gcc into oracle/libbb_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def open_library(path: str):
    lib = ctypes.CDLL(path)
    for name, codes in _SIGNATURES.items():
        f = getattr(lib, name)
        f.argtypes = [_CT[c] for c in codes]
        f.restype = ctypes.c_int
    return lib


def compile_source(source: str, out_path: str) -> str:
    """Compile oracle C source text (a test's mutated copy) to a shared library."""
    src_path = out_path + ".c"
    with open(src_path, "w") as f:
        f.write(source)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", out_path,
                           src_path])
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


def _load():
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = open_library(_LIB)
    return _lib


def _arr(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.uint32).reshape(-1)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("BabyBear oracle %s failed (%d)" % (what, rc))


def modulus() -> int:
    v = ctypes.c_uint32()
    _check(_load().bb_oracle_modulus(ctypes.byref(v)), "modulus")
    return v.value


def generator() -> int:
    v = ctypes.c_uint32()
    _check(_load().bb_oracle_generator(ctypes.byref(v)), "generator")
    return v.value


def roots(log_n: int):
    """(omega, n^-1) of the 2^log_n domain, standard form."""
    w, s = ctypes.c_uint32(), ctypes.c_uint32()
    _check(_load().bb_oracle_roots(log_n, ctypes.byref(w), ctypes.byref(s)), "roots")
    return w.value, s.value


def field_op(op: str, a, b) -> np.ndarray:
    a, b = _arr(a), _arr(b)
    out = np.empty_like(a)
    _check(_load().bb_oracle_field_op({"add": 0, "sub": 1, "mul": 2}[op], a.size, _ptr(a),
                                      _ptr(b), _ptr(out)), op)
    return out


def to_mont(x) -> np.ndarray:
    x = _arr(x)
    out = np.empty_like(x)
    _check(_load().bb_oracle_convert(0, x.size, _ptr(x), _ptr(out)), "to_mont")
    return out


def from_mont(x) -> np.ndarray:
    x = _arr(x)
    out = np.empty_like(x)
    _check(_load().bb_oracle_convert(1, x.size, _ptr(x), _ptr(out)), "from_mont")
    return out


def dft_naive(x, log_n: int, inverse: bool = False) -> np.ndarray:
    x = _arr(x)
    out = np.empty_like(x)
    _check(_load().bb_oracle_dft_naive(log_n, int(inverse), _ptr(x), _ptr(out)), "dft_naive")
    return out


def ntt_mont(x_mont, log_n: int, log_w: int = 0, count: int = 1, log_in: int | None = None,
             inverse: bool = False) -> np.ndarray:
    """`count` row-major matrices of 2^log_in rows and 2^log_w columns (Montgomery) ->
    the same number of 2^log_n-row matrices: each column zero-padded and transformed."""
    log_in = log_n if log_in is None else log_in
    x = _arr(x_mont)
    if x.size != count << (log_in + log_w):
        raise ValueError("expected %d elements, got %d" % (count << (log_in + log_w), x.size))
    out = np.empty(count << (log_n + log_w), np.uint32)
    _check(_load().bb_oracle_ntt(log_n, log_w, count, log_in, int(inverse), _ptr(x), _ptr(out)),
           "ntt")
    return out
