"""ctypes binding of libg16.so (include/g16.h).

Argument marshalling only: every step of the pipeline runs in the HIP library.  Field
vectors are torch tensors on the current HIP device holding n elements of 32 bytes
(shape (n, 8) int32 is the usual carrier; any contiguous dtype with 32 bytes per
element works).  Calls enqueue on torch's current stream and do not synchronise.
There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libg16.so")

G16_OK = 0
G16_EINVAL = -1
G16_ERANGE = -2
G16_ENOSPACE = -3
G16_EALIAS = -4
G16_EHIP = -5
G16_ESTATE = -6

# Every symbol the header declares, with its ctypes signature.
_P, _U32, _U64, _SZ, _I = (ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64,
                           ctypes.c_size_t, ctypes.c_int)
SIGNATURES = {
    "g16_abi_version": (ctypes.c_uint32, []),
    "g16_strerror": (ctypes.c_char_p, [_I]),
    "g16_h_workspace_bytes": (_SZ, [_U32]),
    "g16_batch_plan": (_I, [_U32, _U32, _P, _U32]),
    "g16_h_prepare": (_I, [_U32, _P, _SZ, _P, ctypes.POINTER(_P)]),
    "g16_release": (_I, [_P]),
    "g16_ctx_log_n": (_U32, [_P]),
    "g16_domain_roots": (_I, [_P, _P, _P, _P]),
    "g16_ntt_forward": (_I, [_P, _P, _P, _P]),
    "g16_ntt_inverse": (_I, [_P, _P, _P, _P]),
    "g16_coset_eval": (_I, [_P, _P, _P, _P]),
    "g16_h_compute": (_I, [_P, _P, _P, _P, _P, _P, _P]),
    "g16_h_compute_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P]),
    "g16_h_batch_scratch_bytes": (_SZ, [_U32, _U64]),
    "g16_h_compute_batch": (_I, [_P, _U64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "g16_h_stage_count": (_I, [_P]),
    "g16_h_stage": (_I, [_P, _U32, _P, _P, _P, _P, _P, _P]),
    "g16_h_join": (_I, [_U64, _P, _P, _P, _P, _P, _P]),
    "g16_gather_abc": (_I, [_U64, _P, _P, _P, _U64, _P, _P, _P, _U64, _P, _U64, _P, _P, _P,
                            _P]),
    "g16_to_mont": (_I, [_U64, _P, _P, _P]),
    "g16_from_mont": (_I, [_U64, _P, _P, _P]),
    "g16_fr_mul": (_I, [_U64, _P, _P, _P, _P]),
    "g16_msm_g1_window_bits": (_U32, [_U64]),
    "g16_msm_g1_window_count": (_U32, [_U32]),
    "g16_msm_g1_workspace_bytes": (_SZ, [_U64, _U32]),
    "g16_msm_g1": (_I, [_U64, _P, _P, _U32, _P, _SZ, _P, _P]),
    "g16_msm_g1_finish": (_I, [_U32, _P, _P]),
    "g16_g1_generator_mul": (_I, [_U64, _P, _P, _P]),
    "g16_bb_workspace_bytes": (_SZ, [_U32]),
    "g16_bb_batch_plan": (_I, [_U32, _P, _U32]),
    "g16_bb_prepare": (_I, [_U32, _P, _SZ, _P, ctypes.POINTER(_P)]),
    "g16_bb_release": (_I, [_P]),
    "g16_bb_lde": (_I, [_P, _U32, _U32, _U64, _P, _P, _P]),
    "g16_bb_to_mont": (_I, [_U64, _P, _P, _P]),
    "g16_bb_from_mont": (_I, [_U64, _P, _P, _P]),
}

_lib = None


class G16Error(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (what, strerror(code), code))


def load(path: str = LIB_PATH):
    """Load libg16.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError("libg16.so is not built (%s); run __graft_entry__.build() or "
                               "python -m groth16_polynomial_amd.build" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load().g16_strerror(code).decode()


def _check(rc: int, what: str):
    if rc != G16_OK:
        raise G16Error(rc, what)


def abi_version() -> int:
    return load().g16_abi_version()


def workspace_bytes(log_n: int) -> int:
    return load().g16_h_workspace_bytes(log_n)


def batch_plan(log_n: int, kmax: int = 0) -> list:
    """Pass batches (lowest bits first) of a 2^log_n transform."""
    ks = (ctypes.c_uint32 * 32)()
    rc = load().g16_batch_plan(log_n, kmax, ks, 32)
    if rc < 0:
        raise G16Error(rc, "g16_batch_plan")
    return list(ks[:rc])


# ------------------------------------------------------------------ tensor helpers

def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t, n: int | None = None, what: str = "tensor") -> int:
    """Device pointer of a contiguous GPU tensor holding n 32-byte elements."""
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    nbytes = t.numel() * t.element_size()
    if n is not None and nbytes != 32 * n:
        raise ValueError("%s holds %d bytes, expected %d elements of 32 bytes"
                         % (what, nbytes, n))
    return t.data_ptr()


def n_elements(t) -> int:
    nbytes = t.numel() * t.element_size()
    if nbytes % 32:
        raise ValueError("tensor size is not a whole number of 32-byte elements")
    return nbytes // 32


def empty_fr(n: int, device=None):
    """An uninitialised (n, 8) int32 tensor on the GPU."""
    torch = _torch()
    return torch.empty((n, 8), dtype=torch.int32, device=device or "cuda")


def to_device(words: np.ndarray, device=None):
    """(n, 8) uint32 numpy array -> (n, 8) int32 GPU tensor with the same bytes."""
    torch = _torch()
    a = np.ascontiguousarray(words, dtype=np.uint32).reshape(-1, 8)
    return torch.from_numpy(a.view(np.int32).copy()).to(device or "cuda")


def to_host(t) -> np.ndarray:
    """GPU tensor of 32-byte elements -> (n, 8) uint32 numpy array."""
    torch = _torch()
    b = t.detach().contiguous().view(torch.int32).reshape(-1, 8).cpu().numpy()
    return b.view(np.uint32)


# ------------------------------------------------------------------ context

class HContext:
    """A prepared 2^log_n domain: resident tables and scratch in a torch-owned workspace."""

    def __init__(self, log_n: int, device=None, stream=None):
        torch = _torch()
        self.log_n = log_n
        self.n = 1 << log_n
        nbytes = workspace_bytes(log_n)
        if nbytes == 0:
            _check(G16_ERANGE, "g16_h_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
        ctx = ctypes.c_void_p()
        _check(load().g16_h_prepare(log_n, self.workspace.data_ptr(), nbytes,
                                    _stream(stream), ctypes.byref(ctx)), "g16_h_prepare")
        self._ctx = ctx

    @property
    def handle(self) -> int:
        if self._ctx is None or not self._ctx.value:
            raise RuntimeError("context released")
        return self._ctx.value

    def release(self):
        if self._ctx is not None and self._ctx.value:
            _check(load().g16_release(self._ctx), "g16_release")
        self._ctx = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass

    def domain_roots(self):
        """(omega, shift, size_inv) as Python ints, Montgomery form."""
        bufs = [ctypes.create_string_buffer(32) for _ in range(3)]
        _check(load().g16_domain_roots(self.handle, *[ctypes.addressof(b) for b in bufs]),
               "g16_domain_roots")
        return tuple(int.from_bytes(b.raw, "little") for b in bufs)

    def _unary(self, fname, x, out, stream):
        out = empty_fr(self.n, x.device) if out is None else out
        _check(getattr(load(), fname)(self.handle, _ptr(x, self.n, "in"),
                                      _ptr(out, self.n, "out"), _stream(stream)), fname)
        return out

    def ntt_forward(self, x, out=None, stream=None):
        return self._unary("g16_ntt_forward", x, out, stream)

    def ntt_inverse(self, x, out=None, stream=None):
        return self._unary("g16_ntt_inverse", x, out, stream)

    def coset_eval(self, x, out=None, stream=None):
        return self._unary("g16_coset_eval", x, out, stream)

    def h_compute(self, a, b, c, h_mont=None, h_std=None, stream=None):
        h_mont = empty_fr(self.n, a.device) if h_mont is None else h_mont
        h_std = empty_fr(self.n, a.device) if h_std is None else h_std
        _check(load().g16_h_compute(self.handle, _ptr(a, self.n, "a"), _ptr(b, self.n, "b"),
                                    _ptr(c, self.n, "c"), _ptr(h_mont, self.n, "h_mont"),
                                    _ptr(h_std, self.n, "h_std"), _stream(stream)),
               "g16_h_compute")
        return h_mont, h_std

    def h_compute_noalloc(self, a, b, c, h_mont, h_std, stream=None):
        """g16_h_compute_noalloc: h_compute with the library's own device scratch
        (outputs must be given: the call allocates nothing)."""
        _check(load().g16_h_compute_noalloc(
            self.handle, _ptr(a, self.n, "a"), _ptr(b, self.n, "b"), _ptr(c, self.n, "c"),
            _ptr(h_mont, self.n, "h_mont"), _ptr(h_std, self.n, "h_std"), _stream(stream)),
            "g16_h_compute_noalloc")
        return h_mont, h_std

    def h_compute_batch(self, a, b, c, h_mont=None, h_std=None, scratch=None, stream=None):
        """H of P proofs at once: a, b, c hold P vectors of n elements back to back (for
        instance (P, n, 8) int32); returns (h_mont, h_std) of the same shape as a."""
        total = n_elements(a)
        if total % self.n:
            raise ValueError("a holds %d elements, not a whole number of %d-element vectors"
                             % (total, self.n))
        proofs = total // self.n
        h_mont = _torch().empty_like(a) if h_mont is None else h_mont
        h_std = _torch().empty_like(a) if h_std is None else h_std
        need = load().g16_h_batch_scratch_bytes(self.log_n, proofs)
        if scratch is None:
            scratch = empty_fr(max(need // 32, 1), a.device)
        sbytes = scratch.numel() * scratch.element_size()
        _check(load().g16_h_compute_batch(
            self.handle, proofs, _ptr(a, total, "a"), _ptr(b, total, "b"),
            _ptr(c, total, "c"), _ptr(h_mont, total, "h_mont"), _ptr(h_std, total, "h_std"),
            _ptr(scratch, None, "scratch"), sbytes, _stream(stream)), "g16_h_compute_batch")
        return h_mont, h_std

    def stage_count(self) -> int:
        rc = load().g16_h_stage_count(self.handle)
        if rc < 0:
            raise G16Error(rc, "g16_h_stage_count")
        return rc

    def h_stage(self, stage, a, b, c, h_mont, h_std, stream=None):
        """Enqueue one stage (kernel launch) of h_compute."""
        _check(load().g16_h_stage(self.handle, stage, _ptr(a, self.n, "a"),
                                  _ptr(b, self.n, "b"), _ptr(c, self.n, "c"),
                                  _ptr(h_mont, self.n, "h_mont"), _ptr(h_std, self.n, "h_std"),
                                  _stream(stream)), "g16_h_stage")


# ------------------------------------------------------------------ free functions

def h_join(a, b, c, h_mont=None, h_std=None, stream=None):
    n = n_elements(a)
    h_mont = empty_fr(n, a.device) if h_mont is None else h_mont
    h_std = empty_fr(n, a.device) if h_std is None else h_std
    _check(load().g16_h_join(n, _ptr(a, n, "a"), _ptr(b, n, "b"), _ptr(c, n, "c"),
                             _ptr(h_mont, n, "h_mont"), _ptr(h_std, n, "h_std"),
                             _stream(stream)), "g16_h_join")
    return h_mont, h_std


def gather_abc(row_ptr_a, signal_a, value_a, row_ptr_b, signal_b, value_b, witness,
               out_a=None, out_b=None, out_c=None, stream=None):
    """CSR gather.  row_ptr_* / signal_* are int32 GPU tensors (bit patterns of u32)."""
    n_rows = row_ptr_a.numel() - 1
    if row_ptr_b.numel() - 1 != n_rows:
        raise ValueError("A and B must have the same number of rows")
    nnz_a, nnz_b = signal_a.numel(), signal_b.numel()
    n_w = n_elements(witness)
    dev = witness.device
    outs = [empty_fr(n_rows, dev) if o is None else o for o in (out_a, out_b, out_c)]

    def raw(t):
        if t.numel() == 0:
            return None
        if not t.is_cuda or not t.is_contiguous() or t.element_size() != 4:
            raise ValueError("index arrays must be contiguous 32-bit GPU tensors")
        return t.data_ptr()

    _check(load().g16_gather_abc(n_rows, raw(row_ptr_a), raw(signal_a),
                                 _ptr(value_a, nnz_a, "value_a") if nnz_a else None, nnz_a,
                                 raw(row_ptr_b), raw(signal_b),
                                 _ptr(value_b, nnz_b, "value_b") if nnz_b else None, nnz_b,
                                 _ptr(witness, n_w, "witness"), n_w,
                                 _ptr(outs[0], n_rows), _ptr(outs[1], n_rows),
                                 _ptr(outs[2], n_rows), _stream(stream)), "g16_gather_abc")
    return tuple(outs)


def _elementwise(fname, x, out, stream, y=None):
    n = n_elements(x)
    out = empty_fr(n, x.device) if out is None else out
    args = [n, _ptr(x, n, "in")]
    if y is not None:
        args.append(_ptr(y, n, "b"))
    args += [_ptr(out, n, "out"), _stream(stream)]
    _check(getattr(load(), fname)(*args), fname)
    return out


def to_mont(x, out=None, stream=None):
    return _elementwise("g16_to_mont", x, out, stream)


def from_mont(x, out=None, stream=None):
    return _elementwise("g16_from_mont", x, out, stream)


def fr_mul(a, b, out=None, stream=None):
    return _elementwise("g16_fr_mul", a, out, stream, y=b)


# ------------------------------------------------------------------ G1 MSM

G1_AFF_BYTES = 64
G1_XYZZ_BYTES = 128


def msm_window_bits(n: int) -> int:
    return load().g16_msm_g1_window_bits(n)


def msm_window_count(c: int) -> int:
    return load().g16_msm_g1_window_count(c)


def msm_workspace_bytes(n: int, c: int = 0) -> int:
    return load().g16_msm_g1_workspace_bytes(n, c)


def g1_generator_mul(scalars, out=None, stream=None):
    """k_i G for 32-byte scalars on the GPU: affine bases, (n, 16) int32, Montgomery form."""
    n = n_elements(scalars)
    torch = _torch()
    out = torch.empty((n, 16), dtype=torch.int32, device=scalars.device) if out is None else out
    if out.numel() * out.element_size() != n * G1_AFF_BYTES:
        raise ValueError("out must hold %d affine points" % n)
    _check(load().g16_g1_generator_mul(n, _ptr(scalars, n, "scalars"), out.data_ptr(),
                                       _stream(stream)), "g16_g1_generator_mul")
    return out


class MsmG1:
    """Workspace for G1 MSMs of up to n terms with window width c (0: the default)."""

    def __init__(self, n: int, c: int = 0, device=None):
        torch = _torch()
        self.n = n
        self.c = c or msm_window_bits(n)
        self.windows = msm_window_count(self.c)
        nbytes = msm_workspace_bytes(n, self.c) if n else 0
        if n and nbytes == 0:
            raise G16Error(G16_EINVAL, "g16_msm_g1_workspace_bytes")
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8,
                                     device=device or "cuda")
        self.sums = torch.empty((self.windows, 32), dtype=torch.int32, device=device or "cuda")

    def window_sums(self, scalars, bases, stream=None):
        """Enqueue the MSM; returns the (windows, 32) int32 XYZZ window sums on the GPU."""
        n = n_elements(scalars)
        if n > self.n:
            raise ValueError("%d terms, workspace for %d" % (n, self.n))
        if bases.numel() * bases.element_size() != n * G1_AFF_BYTES:
            raise ValueError("bases must hold %d affine points" % n)
        ws = self.workspace
        _check(load().g16_msm_g1(n, scalars.data_ptr() if n else None,
                                 bases.data_ptr() if n else None, self.c,
                                 ws.data_ptr(), ws.numel(), self.sums.data_ptr(),
                                 _stream(stream)), "g16_msm_g1")
        return self.sums

    def finish(self, sums_host: np.ndarray) -> np.ndarray:
        """Host combination of the window sums: (16,) uint32 affine result, standard form."""
        s = np.ascontiguousarray(sums_host, dtype=np.uint32).reshape(self.windows, 32)
        out = np.zeros(16, np.uint32)
        _check(load().g16_msm_g1_finish(self.c, s.ctypes.data, out.ctypes.data),
               "g16_msm_g1_finish")
        return out

    def __call__(self, scalars, bases, stream=None) -> np.ndarray:
        """The whole MSM (synchronises the stream to read the window sums back)."""
        sums = self.window_sums(scalars, bases, stream)
        return self.finish(to_host(sums).reshape(self.windows, 32))


# ------------------------------------------------------------------ BabyBear transform

def bb_batch_plan(log_n: int) -> list:
    ks = (ctypes.c_uint32 * 8)()
    rc = load().g16_bb_batch_plan(log_n, ks, 8)
    if rc < 0:
        raise G16Error(rc, "g16_bb_batch_plan")
    return list(ks[:rc])


def bb_to_device(words: np.ndarray, device=None):
    """uint32 numpy array -> int32 GPU tensor with the same bytes."""
    torch = _torch()
    a = np.ascontiguousarray(words, dtype=np.uint32).reshape(-1)
    return torch.from_numpy(a.view(np.int32).copy()).to(device or "cuda")


def bb_to_host(t) -> np.ndarray:
    return t.detach().contiguous().view(_torch().int32).reshape(-1).cpu().numpy().view(np.uint32)


def _bb_words(t, what):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous GPU tensor" % what)
    nbytes = t.numel() * t.element_size()
    if nbytes % 4:
        raise ValueError("%s is not a whole number of 32-bit words" % what)
    return nbytes // 4


def bb_to_mont(x, out=None, stream=None):
    n = _bb_words(x, "x")
    out = _torch().empty_like(x) if out is None else out
    _check(load().g16_bb_to_mont(n, x.data_ptr(), out.data_ptr(), _stream(stream)),
           "g16_bb_to_mont")
    return out


def bb_from_mont(x, out=None, stream=None):
    n = _bb_words(x, "x")
    out = _torch().empty_like(x) if out is None else out
    _check(load().g16_bb_from_mont(n, x.data_ptr(), out.data_ptr(), _stream(stream)),
           "g16_bb_from_mont")
    return out


class BbContext:
    """A prepared 2^log_n BabyBear domain: the twiddle levels in a torch-owned workspace."""

    def __init__(self, log_n: int, device=None, stream=None):
        torch = _torch()
        self.log_n = log_n
        nbytes = load().g16_bb_workspace_bytes(log_n)
        if nbytes == 0:
            _check(G16_ERANGE, "g16_bb_workspace_bytes")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
        ctx = ctypes.c_void_p()
        _check(load().g16_bb_prepare(log_n, self.workspace.data_ptr(), nbytes, _stream(stream),
                                     ctypes.byref(ctx)), "g16_bb_prepare")
        self._ctx = ctx

    @property
    def handle(self) -> int:
        if self._ctx is None or not self._ctx.value:
            raise RuntimeError("context released")
        return self._ctx.value

    def release(self):
        if self._ctx is not None and self._ctx.value:
            _check(load().g16_bb_release(self._ctx), "g16_bb_release")
        self._ctx = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass

    def lde(self, x, log_in: int | None = None, log_w: int = 0, count: int = 1, out=None,
            stream=None):
        """`count` row-major matrices of 2^log_in rows and 2^log_w columns (Montgomery, a
        GPU tensor of 32-bit words) -> their columns' values on the 2^log_n-th roots of
        unity (2^log_n rows each)."""
        torch = _torch()
        log_in = self.log_n if log_in is None else log_in
        n_in = count << (log_in + log_w)
        if _bb_words(x, "x") != n_in:
            raise ValueError("x holds %d words, expected %d" % (_bb_words(x, "x"), n_in))
        n_out = count << (self.log_n + log_w)
        out = torch.empty(n_out, dtype=torch.int32, device=x.device) if out is None else out
        if _bb_words(out, "out") != n_out:
            raise ValueError("out holds the wrong number of words")
        _check(load().g16_bb_lde(self.handle, log_in, log_w, count, x.data_ptr(),
                                 out.data_ptr(), _stream(stream)), "g16_bb_lde")
        return out
