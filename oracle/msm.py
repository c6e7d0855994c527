"""ctypes wrapper of the MSM oracle (msm_oracle.c).  TEST INFRASTRUCTURE ONLY.

Points cross as numpy uint32 arrays of shape (n, 16): x then y, each eight
little-endian 32-bit words in standard form; the point at infinity is (0, 0).
Scalars and field elements are (n, 8) arrays of the same word layout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msm_oracle.c")
_LIB = os.path.join(_HERE, "libmsm_oracle.so")
_lib = None
_override = None

GENERATOR = (1, 2)

_SIGNATURES = {
    "msm_oracle_modulus": "P",
    "msm_oracle_fp_op": "IZPPP",
    "msm_oracle_on_curve": "ZPP",
    "msm_oracle_affine_op": "IZPPP",
    "msm_oracle_jacobian_op": "IZPPP",
    "msm_oracle_scalar_mul": "ZPPP",
    "msm_oracle_msm": "ZPPP",
}
_CT = {"P": ctypes.c_void_p, "Z": ctypes.c_size_t, "I": ctypes.c_int}


def build(force: bool = True) -> str:
    """Compile msm_oracle.c with gcc into oracle/libmsm_oracle.so."""
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
    src_path = out_path + ".c"
    with open(src_path, "w") as f:
        f.write(source)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", out_path,
                           src_path])
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


class use_library:
    """Context manager: route the module functions to another MSM oracle library."""

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


def _words(x, width: int) -> np.ndarray:
    a = np.ascontiguousarray(x, dtype=np.uint32)
    return a.reshape(-1, width)


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("msm oracle %s failed (%d)" % (what, rc))


# ------------------------------------------------------------------ int helpers

def to_words(values, width: int = 8) -> np.ndarray:
    """Python ints -> (n, width) uint32 words, little-endian."""
    m = (1 << 32) - 1
    vals = list(values)
    out = np.zeros((len(vals), width), np.uint32)
    for i, v in enumerate(vals):
        for j in range(width):
            out[i, j] = (v >> (32 * j)) & m
    return out


def from_words(a) -> list:
    a = np.asarray(a, dtype=np.uint32)
    a = a.reshape(-1, a.shape[-1])
    return [sum(int(x) << (32 * j) for j, x in enumerate(row.tolist())) for row in a]


def points_to_words(points) -> np.ndarray:
    """[(x, y) or None] -> (n, 16) words; None is the point at infinity."""
    flat = []
    for pt in points:
        x, y = (0, 0) if pt is None else pt
        flat.append(x | (y << 256))
    return to_words(flat, 16)


def words_to_points(a) -> list:
    out = []
    for v in from_words(np.asarray(a, dtype=np.uint32).reshape(-1, 16)):
        x, y = v & ((1 << 256) - 1), v >> 256
        out.append(None if x == 0 and y == 0 else (x, y))
    return out


# ------------------------------------------------------------------ field

def modulus() -> int:
    out = np.zeros(8, np.uint32)
    _check(_load().msm_oracle_modulus(_p(out)), "modulus")
    return from_words(out)[0]


def fp_op(op: str, a, b=None) -> np.ndarray:
    code = {"add": 0, "sub": 1, "mul": 2, "inv": 3, "to_mont": 4, "from_mont": 5}[op]
    a = _words(a, 8)
    bb = _words(b, 8) if b is not None else None
    if bb is not None and bb.shape != a.shape:
        raise ValueError("operand shapes differ")
    out = np.empty_like(a)
    _check(_load().msm_oracle_fp_op(code, a.shape[0], _p(a), _p(bb) if bb is not None else None,
                                    _p(out)), op)
    return out


def to_mont(a) -> np.ndarray:
    return fp_op("to_mont", a)


def from_mont(a) -> np.ndarray:
    return fp_op("from_mont", a)


def points_to_mont(pts) -> np.ndarray:
    """(n, 16) standard-form points -> Montgomery coordinates (infinity stays (0, 0))."""
    p = _words(pts, 16)
    out = np.empty_like(p)
    out[:, :8] = to_mont(p[:, :8])
    out[:, 8:] = to_mont(p[:, 8:])
    return out


def points_from_mont(pts) -> np.ndarray:
    p = _words(pts, 16)
    out = np.empty_like(p)
    out[:, :8] = from_mont(p[:, :8])
    out[:, 8:] = from_mont(p[:, 8:])
    return out


# ------------------------------------------------------------------ curve

def on_curve(pts) -> bool:
    p = _words(pts, 16)
    ok = ctypes.c_int(0)
    _check(_load().msm_oracle_on_curve(p.shape[0], _p(p), ctypes.byref(ok)), "on_curve")
    return bool(ok.value)


def affine_op(op: str, a, b=None) -> np.ndarray:
    code = {"add": 0, "double": 1, "neg": 2}[op]
    a = _words(a, 16)
    bb = _words(b, 16) if b is not None else a
    out = np.empty_like(a)
    _check(_load().msm_oracle_affine_op(code, a.shape[0], _p(a), _p(bb), _p(out)), op)
    return out


def jacobian_op(op: str, a, b=None) -> np.ndarray:
    code = {"add": 0, "double": 1}[op]
    a = _words(a, 16)
    bb = _words(b, 16) if b is not None else a
    out = np.empty_like(a)
    _check(_load().msm_oracle_jacobian_op(code, a.shape[0], _p(a), _p(bb), _p(out)), op)
    return out


def scalar_mul(scalars, point=GENERATOR) -> np.ndarray:
    """k_i P for each scalar (P the generator by default): (n, 16) standard form."""
    k = _words(scalars, 8)
    pt = points_to_words([point])
    out = np.empty((k.shape[0], 16), np.uint32)
    _check(_load().msm_oracle_scalar_mul(k.shape[0], _p(k), _p(pt), _p(out)), "scalar_mul")
    return out


def msm(scalars, bases) -> np.ndarray:
    """sum_i k_i P_i, (16,) words standard form."""
    k = _words(scalars, 8)
    b = _words(bases, 16)
    if b.shape[0] != k.shape[0]:
        raise ValueError("%d scalars, %d bases" % (k.shape[0], b.shape[0]))
    out = np.empty(16, np.uint32)
    _check(_load().msm_oracle_msm(k.shape[0], _p(k), _p(b), _p(out)), "msm")
    return out
