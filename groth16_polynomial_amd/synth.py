"""Seeded synthetic inputs for the H-polynomial pipeline.

This module is the only code shared by the GPU path's tests/bench and the CPU
oracle.  It holds no field arithmetic of the method: it draws integers, compares
them against the BN254 scalar modulus r (rejection sampling) and lays them out as
little-endian 8 x u32 words.  Every value it returns is a canonical integer in
[0, r) in STANDARD form (not Montgomery); each consumer converts to Montgomery
form with its own arithmetic.

Random stream: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014).  Output i (0-based) of the stream with seed S
is mix(S + (i + 1) * 0x9E3779B97F4A7C15), so any block of it can be drawn
without running the ones before it.

Workload shapes follow the pages:
* uniform Fr vectors for the H pipeline and the standalone transform (the
  NTT_CU page, "BATCHING" section, domain sizes 2^12 .. 2^22 of the prover);
* the sparse R1CS rows of the gather front end follow the row statistics the
  GATHER_CU page measures in its "WHY ONE THREAD PER ROW" section (mean
  row length of non-empty rows, count of empty rows, longest row).
"""
from __future__ import annotations

import numpy as np

# BN254 scalar field modulus r (254 bits).
R_MODULUS = 21888242871839275222246405745257275088548364400416034343698204186575808495617
_R_LIMBS64 = tuple((R_MODULUS >> (64 * i)) & 0xFFFFFFFFFFFFFFFF for i in range(4))

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

SEED_BASE = 0x6731360000000000

# Stream numbers inside one workload's seed space.
STREAM_A = 1
STREAM_B = 2
STREAM_WITNESS_SELECT = 3
STREAM_CSR_LENGTHS = 4
STREAM_CSR_COLUMNS = 5
STREAM_CSR_VALUES = 6
STREAM_VECTOR = 7
STREAM_C = 8
STREAM_WITNESS_VALUES = 9


def seed_for(workload: int, stream: int) -> int:
    """Seed of `stream` inside workload number `workload` (1-based)."""
    return (SEED_BASE + 16 * workload + stream) & 0xFFFFFFFFFFFFFFFF


def splitmix64(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream seeded with `seed`."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def _below_r(l0, l1, l2, l3) -> np.ndarray:
    """Lexicographic (l3, l2, l1, l0) < r, limb-wise on uint64 arrays."""
    r0, r1, r2, r3 = (np.uint64(v) for v in _R_LIMBS64)
    lt = l3 < r3
    eq = l3 == r3
    lt |= eq & (l2 < r2)
    eq &= l2 == r2
    lt |= eq & (l1 < r1)
    eq &= l1 == r1
    lt |= eq & (l0 < r0)
    return lt


def uniform_fr(seed: int, n: int) -> np.ndarray:
    """n uniform elements of [0, r), standard form, shape (n, 8) uint32 LE limbs.

    Candidate j takes stream outputs 4j .. 4j+3 as 64-bit limbs, least significant
    first, masks the top limb to 62 bits (so the candidate is < 2^254) and is kept
    iff it is < r.  About 3 in 4 candidates are kept.
    """
    out = np.empty((n, 4), dtype=np.uint64)
    got = 0
    cand = 0
    mask = np.uint64((1 << 62) - 1)
    while got < n:
        want = max(1024, int((n - got) * 1.34) + 64)
        w = splitmix64(seed, 4 * want, 4 * cand).reshape(want, 4)
        w[:, 3] &= mask
        keep = w[_below_r(w[:, 0], w[:, 1], w[:, 2], w[:, 3])]
        take = min(len(keep), n - got)
        out[got:got + take] = keep[:take]
        got += take
        cand += want
    return out.view(np.uint32).reshape(n, 8).copy()


# BabyBear modulus (the WHIR forum post's field), for the Reed-Solomon encoding workload.
BB_MODULUS = (1 << 31) - (1 << 27) + 1


def uniform_bb(seed: int, n: int) -> np.ndarray:
    """n uniform elements of [0, p) for BabyBear p, standard form, uint32.  Candidate j is
    the low 31 bits of stream output j, kept iff it is < p (15 in 16 are kept)."""
    out = np.empty(n, dtype=np.uint32)
    got = 0
    cand = 0
    while got < n:
        want = max(1024, int((n - got) * 1.08) + 64)
        z = (splitmix64(seed, want, cand) & np.uint64(0x7FFFFFFF)).astype(np.uint32)
        keep = z[z < np.uint32(BB_MODULUS)]
        take = min(len(keep), n - got)
        out[got:got + take] = keep[:take]
        got += take
        cand += want
    return out


def bb_lde_input(workload: int, log_in: int, log_w: int, count: int = 1) -> np.ndarray:
    """The coefficients of a Reed-Solomon encoding workload: `count` row-major matrices of
    2^log_in rows and 2^log_w columns of uniform BabyBear elements (standard form), as a
    flat uint32 array."""
    return uniform_bb(seed_for(workload, STREAM_VECTOR), count << (log_in + log_w))


def unit_floats(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Uniform doubles in [0, 1) from the top 53 bits of each stream output."""
    z = splitmix64(seed, count, start)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def fr_to_ints(words: np.ndarray) -> list:
    """(n, 8) uint32 LE limbs -> list of Python ints (test helper; no arithmetic mod r)."""
    w = np.ascontiguousarray(words, dtype=np.uint32).reshape(-1, 8)
    q = w.view(np.uint64).reshape(-1, 4)
    return [int(a) | (int(b) << 64) | (int(c) << 128) | (int(d) << 192)
            for a, b, c, d in q.tolist()]


def ints_to_fr(values) -> np.ndarray:
    """List of ints in [0, 2^256) -> (n, 8) uint32 LE limbs."""
    vals = list(values)
    q = np.empty((len(vals), 4), dtype=np.uint64)
    m = (1 << 64) - 1
    for i, v in enumerate(vals):
        q[i] = [v & m, (v >> 64) & m, (v >> 128) & m, (v >> 192) & m]
    return q.view(np.uint32).reshape(len(vals), 8).copy()


# --------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------

def h_inputs(workload: int, log_n: int):
    """A and B of an H-pipeline workload: two uniform Fr vectors (standard form).

    C is not drawn: the workloads use C = A o B (pointwise), which each side forms
    with its own field multiply.
    """
    n = 1 << log_n
    return (uniform_fr(seed_for(workload, STREAM_A), n),
            uniform_fr(seed_for(workload, STREAM_B), n))


def random_c(workload: int, log_n: int) -> np.ndarray:
    """An independent uniform C, for cases where C is not A o B."""
    return uniform_fr(seed_for(workload, STREAM_C), 1 << log_n)


def ntt_input(workload: int, log_n: int) -> np.ndarray:
    """One uniform Fr vector for the standalone transform workload."""
    return uniform_fr(seed_for(workload, STREAM_VECTOR), 1 << log_n)


class CsrMatrix:
    """A CSR matrix of Fr coefficients: row_ptr u32[n+1], signal u32[nnz], value (nnz, 8)."""

    def __init__(self, row_ptr: np.ndarray, signal: np.ndarray, value: np.ndarray):
        self.row_ptr = row_ptr
        self.signal = signal
        self.value = value

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])


def _row_lengths(seed: int, rows: int, nonempty: int, mean: float, cap: int) -> np.ndarray:
    """Geometric lengths on {1, 2, ...} with the given mean, capped, for the first
    `nonempty` rows; the trailing rows are empty padding of the domain."""
    lengths = np.zeros(rows, dtype=np.int64)
    if nonempty:
        p = 1.0 / mean
        u = 1.0 - unit_floats(seed, nonempty)            # (0, 1]
        k = 1 + np.floor(np.log(u) / np.log1p(-p)).astype(np.int64)
        lengths[:nonempty] = np.minimum(k, cap)
    return lengths


def csr_matrix(workload: int, which: int, rows: int, nonempty: int, mean: float,
               cap: int, n_witness: int) -> CsrMatrix:
    """One synthetic constraint matrix (which = 0 for A, 1 for B)."""
    sub = which << 48  # flips a high seed bit for B, so A and B draw unrelated streams
    lengths = _row_lengths(seed_for(workload, STREAM_CSR_LENGTHS) ^ sub, rows, nonempty,
                           mean, cap)
    row_ptr = np.zeros(rows + 1, dtype=np.uint32)
    row_ptr[1:] = np.cumsum(lengths)
    nnz = int(row_ptr[-1])
    cols = splitmix64(seed_for(workload, STREAM_CSR_COLUMNS) ^ sub, nnz) % np.uint64(n_witness)
    vals = uniform_fr(seed_for(workload, STREAM_CSR_VALUES) ^ sub, nnz)
    return CsrMatrix(row_ptr, cols.astype(np.uint32), vals)


def witness(workload: int, n_witness: int, p_small: float = 0.9) -> np.ndarray:
    """Witness vector: each slot is 0 or 1 (equally likely) with probability p_small,
    otherwise a uniform Fr element.  Standard form, (n_witness, 8) uint32."""
    sel = splitmix64(seed_for(workload, STREAM_WITNESS_SELECT), n_witness)
    u = (sel >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
    small = u < p_small
    out = np.zeros((n_witness, 8), dtype=np.uint32)
    out[small, 0] = (sel[small] & np.uint64(1)).astype(np.uint32)
    big = np.flatnonzero(~small)
    if len(big):
        out[big] = uniform_fr(seed_for(workload, STREAM_WITNESS_VALUES), len(big))
    return out


# Row statistics of the largest proving key the gather page measures (domain 2^18):
# empty rows per matrix and the longest row; the non-empty mean lengths are
# 1.13 (A) and 1.70 (B).
GATHER_2_18 = dict(rows=1 << 18, n_witness=500_000,
                   a_nonempty=(1 << 18) - 121_848, a_mean=1.13,
                   b_nonempty=(1 << 18) - 121_883, b_mean=1.70, cap=95)


def gather_inputs(workload: int, rows: int = GATHER_2_18["rows"],
                  n_witness: int = GATHER_2_18["n_witness"],
                  a_nonempty: int | None = None, b_nonempty: int | None = None,
                  a_mean: float = GATHER_2_18["a_mean"], b_mean: float = GATHER_2_18["b_mean"],
                  cap: int = GATHER_2_18["cap"]):
    """CSR A, CSR B and the witness for the gather front end.

    Defaults reproduce the 2^18 shape; smaller `rows` keep the same empty-row
    fraction (about 46%) unless a_nonempty / b_nonempty are given.
    """
    full = GATHER_2_18["rows"]
    if a_nonempty is None:
        a_nonempty = (rows * GATHER_2_18["a_nonempty"]) // full
    if b_nonempty is None:
        b_nonempty = (rows * GATHER_2_18["b_nonempty"]) // full
    a = csr_matrix(workload, 0, rows, a_nonempty, a_mean, cap, n_witness)
    b = csr_matrix(workload, 1, rows, b_nonempty, b_mean, cap, n_witness)
    w = witness(workload, n_witness)
    return a, b, w
