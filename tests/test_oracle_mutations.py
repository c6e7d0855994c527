"""The pins must be sharp: each plausible mistake planted in a copy of the oracle's C
source (a dropped term, a wrong sign or index, a transposed operand) makes at least one
pin fail.  The mutated copies are compiled with gcc into a temporary directory and run
on the CPU only."""
import multiprocessing as mp

import numpy as np
import pytest

import oracle
from groth16_polynomial_amd import synth
from tests import intref

R = synth.R_MODULUS
ints = synth.fr_to_ints
fr = synth.ints_to_fr

# (name, original text, planted text)
MUTATIONS = [
    ("coset shift by the domain root", "shift_job job = {x, shift};", "shift_job job = {x, omega};"),
    ("shift applied one index late", "x[j] = fe_mul(x[j], sj);\n        sj = fe_mul(sj, shift);",
     "sj = fe_mul(sj, shift);\n        x[j] = fe_mul(x[j], sj);"),
    ("size_inv dropped", "for (size_t i = lo; i < hi; ++i) x[i] = fe_mul(x[i], size_inv);", ""),
    ("twiddle index without stride", "tw[j * step]", "tw[j]"),
    ("butterfly outputs swapped", "x[start + j] = fe_add(u, v);\n        x[start + j + half] = fe_sub(u, v);",
     "x[start + j] = fe_sub(u, v);\n        x[start + j + half] = fe_add(u, v);"),
    ("bit reversal dropped", "if (j > i) { fe t = x[i]; x[i] = x[j]; x[j] = t; }", ""),
    ("H operands transposed", "fe h = fe_sub(fe_mul(v[0][i], v[1][i]), v[2][i]);",
     "fe h = fe_sub(v[2][i], fe_mul(v[0][i], v[1][i]));"),
    ("h_std and h_mont swapped", "memcpy(h_std + 4 * i, h.v, 32);\n        fe hm = to_mont(h);\n        memcpy(h_mont + 4 * i, hm.v, 32);",
     "memcpy(h_mont + 4 * i, h.v, 32);\n        fe hm = to_mont(h);\n        memcpy(h_std + 4 * i, hm.v, 32);"),
    ("subtraction without wrap", "if (sub_n(d.v, a.v, b.v, 4)) add_n(d.v, d.v, MOD.v, 4);",
     "sub_n(d.v, a.v, b.v, 4);"),
    ("Barrett final correction dropped", "while (geq_n(rr, m5, 5)) sub_n(rr, rr, m5, 5);", ""),
    ("Barrett quotient from the wrong limbs", "memcpy(q3, q2 + 5, sizeof q3);",
     "memcpy(q3, q2 + 4, sizeof q3);"),
    ("inverse uses the forward root", "dit_in_place(x, L, fe_inv(omega));", "dit_in_place(x, L, omega);"),
    ("wrong non-residue", "ROOT_2_28 = fe_pow(fe_small(5), e);", "ROOT_2_28 = fe_pow(fe_small(7), e);"),
    ("gather ignores the coefficient", "acc[m] = fe_add(acc[m], fe_mul(from_mont(v), from_mont(w)));",
     "acc[m] = fe_add(acc[m], from_mont(w));"),
    ("gather C from A twice", "fe c = to_mont(fe_mul(acc[0], acc[1]));", "fe c = to_mont(fe_mul(acc[0], acc[0]));"),
    ("barycentric scale dropped", "fe va = fe_mul(sum[0], scale), vb = fe_mul(sum[1], scale), vc = fe_mul(sum[2], scale);",
     "fe va = sum[0], vb = sum[1], vc = sum[2];"),
]


def _pins_pass() -> bool:
    """A quick subset of the pins, run against whatever library is installed."""
    try:
        # field layer against Python integers (includes values near r)
        xs = [0, 1, R - 1, R - 2, pow(2, 256, R)] + [int(v) for v in ints(synth.uniform_fr(9, 400))]
        ys = list(reversed(xs))
        if ints(oracle.field_op("mul", fr(xs), fr(ys))) != [a * b % R for a, b in zip(xs, ys)]:
            return False
        if ints(oracle.field_op("sub", fr(xs), fr(ys))) != [(a - b) % R for a, b in zip(xs, ys)]:
            return False
        # a large random batch: Barrett's quotient estimate is one short only about
        # once in 3000 products, so a few hundred products would miss a lost correction
        big_x = synth.uniform_fr(11, 100000)
        big_y = synth.uniform_fr(12, 100000)
        got = ints(oracle.field_op("mul", big_x, big_y))
        if got != [a * b % R for a, b in zip(ints(big_x), ints(big_y))]:
            return False
        # roots: closed form
        omega, shift, size_inv = oracle.domain_roots(5)
        if pow(shift, 32, R) != R - 1 or omega != shift * shift % R:
            return False
        # the root convention (generator 5) that both sides follow
        if shift != pow(pow(5, (R - 1) >> 28, R), 1 << 22, R):
            return False
        # transform against the definition
        x = synth.uniform_fr(10, 16)
        if ints(oracle.ntt(x, 4)) != intref.dft(ints(x), oracle.domain_roots(4)[0]):
            return False
        w4 = oracle.domain_roots(4)[0]
        if ints(oracle.ntt(x, 4, inverse=True)) != intref.idft(ints(x), w4):
            return False
        # pipeline closed form, n = 16
        n = 16
        a, b = synth.h_inputs(7, 4)
        am, bm = oracle.to_mont(a), oracle.to_mont(b)
        cm = oracle.to_mont(synth.random_c(7, 4))
        A, B, C = ints(a), ints(b), ints(oracle.from_mont(cm))
        w, s, _ = oracle.domain_roots(4)
        pa, pb, pc = (intref.idft(v, w) for v in (A, B, C))
        P = intref.poly_sub(intref.poly_mul(pa, pb), pc)
        want = [intref.horner(P, s * pow(w, i, R) % R) for i in range(n)]
        hm, hs = oracle.h_pipeline(4, am, bm, cm)
        if ints(hs) != want or ints(hm) != [v * (1 << 256) % R for v in want]:
            return False
        hm2, hs2 = oracle.h_at(4, am, bm, cm, np.arange(n, dtype=np.uint32))
        if ints(hs2) != want:
            return False
        # gather against a Python sparse dot product
        ma, mb, wt = synth.gather_inputs(4, rows=64, n_witness=50)
        oa, ob, oc = oracle.gather(ma.row_ptr, ma.signal, oracle.to_mont(ma.value), mb.row_ptr,
                                   mb.signal, oracle.to_mont(mb.value), oracle.to_mont(wt))
        wi, va, vb = ints(wt), ints(ma.value), ints(mb.value)
        ra = [sum(va[k] * wi[ma.signal[k]] for k in range(ma.row_ptr[i], ma.row_ptr[i + 1])) % R
              for i in range(64)]
        rb = [sum(vb[k] * wi[mb.signal[k]] for k in range(mb.row_ptr[i], mb.row_ptr[i + 1])) % R
              for i in range(64)]
        if ints(oracle.from_mont(oa)) != ra or ints(oracle.from_mont(oc)) != \
                [p * q % R for p, q in zip(ra, rb)]:
            return False
    except ValueError:
        return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


def _child(path, q):
    with oracle.use_library(oracle.open_library(path)):
        q.put(_pins_pass())


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %s" % name
    path = oracle.compile_source(src.replace(old, new), str(tmp_path / "liboracle_mut.so"))
    # Some mistakes (a broken reduction) make the oracle loop for ever; a pin run that
    # does not finish within the limit counts as caught.
    ctx = mp.get_context("fork")
    q = ctx.Queue()
    p = ctx.Process(target=_child, args=(path, q))
    p.start()
    p.join(20)
    if p.is_alive():
        p.kill()
        p.join()
        return
    assert p.exitcode == 0 or p.exitcode < 0, "mutated oracle child failed: %s" % name
    if p.exitcode == 0:
        assert q.get(timeout=5) is False, "pins did not catch: %s" % name
