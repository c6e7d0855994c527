"""The device product (fr29.hpp) spells each column of its digit products out as an
asm block of multiply-adds.  These tests read the header and check every block against
the column it stands for, so that a dropped, doubled or misindexed multiply-add fails
on the CPU:

* quotient columns C = 8..16 of x w': one x_i w'_(C-i) for every i with both indices in
  0..8;
* low columns C = 0..8 of x w + q (-r): one x_i w_(C-i) and one q_i (-r)_(C-i) for every
  i in 0..C;
* the first multiply-add of columns 8 (quotient) and 0 (low) starts from zero and its
  accumulator is a write-only, early-clobber operand; every other block reads the
  carry of the column below through a read-write operand;
* the table digits b come in VGPRs or SGPRs (one constraint set each), and both column
  functions instantiate the blocks with each set.
"""
import os
import re

import pytest

HDR = os.path.join(os.path.dirname(__file__), "..", "groth16_polynomial_amd", "csrc", "fr29.hpp")


def _blocks(fn):
    src = open(HDR).read()
    macro = {"col_q": "G16_COL_Q", "col_y": "G16_COL_Y"}[fn]
    start = src.index(f"#define {macro}(BOPS)")
    end = src.index("\n\n", start)
    body = src[start:end]
    out = {}
    for m in re.finditer(r"constexpr \(C == (\d+)\) \{(.*?)\"vcc\"\);", body, re.S):
        c = int(m.group(1))
        text = m.group(2)
        ops = [(k, int(i), int(j)) for k, i, j in re.findall(r"G16_(X0|X|Q)\((\d+), (\d+)\)", text)]
        assert "BOPS(b)" in text, c
        acc = re.search(r"\[acc\] \"([=&+v]+)\"", text).group(1)
        out[c] = (ops, acc)
    return out


def test_macros_are_the_multiply_adds():
    src = open(HDR).read()
    assert '#define G16_X(i, j) "v_mad_i64_i32 %[acc], vcc, %[x" #i "], %[b" #j "], %[acc]' in src
    assert '#define G16_X0(i, j) "v_mad_i64_i32 %[acc], vcc, %[x" #i "], %[b" #j "], 0' in src
    assert '#define G16_Q(i, j) "v_mad_i64_i32 %[acc], vcc, %[q" #i "], %[m" #j "], %[acc]' in src
    for tag, con, expr in (("x", "v", "v[{k}]"), ("b", "v", "v[{k}]"), ("b", "s", "v[{k}]"),
                           ("q", "v", "v[{k}]"), ("m", "s", "mr29_digit({k})")):
        for k in range(9):
            assert f'[{tag}{k}] "{con}"({expr.format(k=k)})' in src, (tag, k)


def test_quotient_columns():
    blocks = _blocks("col_q")
    assert sorted(blocks) == list(range(8, 17))
    for c, (ops, acc) in blocks.items():
        want = {(i, c - i) for i in range(9) if 0 <= c - i <= 8}
        got = [(i, j) for _, i, j in ops]
        assert len(got) == len(set(got)) and set(got) == want, c
        assert all(k in ("X", "X0") for k, _, _ in ops)
        kinds = [k for k, _, _ in ops]
        if c == 8:
            assert kinds[0] == "X0" and kinds.count("X0") == 1 and acc == "=&v"
        else:
            assert "X0" not in kinds and acc == "+v"


def test_low_columns():
    blocks = _blocks("col_y")
    assert sorted(blocks) == list(range(0, 9))
    for c, (ops, acc) in blocks.items():
        want = {(i, c - i) for i in range(c + 1)}
        xs = [(i, j) for k, i, j in ops if k in ("X", "X0")]
        qs = [(i, j) for k, i, j in ops if k == "Q"]
        assert len(xs) == len(set(xs)) and set(xs) == want, c
        assert len(qs) == len(set(qs)) and set(qs) == want, c
        kinds = [k for k, _, _ in ops]
        if c == 0:
            assert kinds[0] == "X0" and kinds.count("X0") == 1 and acc == "=&v"
        else:
            assert "X0" not in kinds and acc == "+v"


@pytest.mark.parametrize("total", [135])
def test_product_count(total):
    n = sum(len(ops) for ops, _ in _blocks("col_q").values())
    n += sum(len(ops) for ops, _ in _blocks("col_y").values())
    assert n == total


def test_both_operand_sets_instantiated():
    src = open(HDR).read()
    for fn, macro in (("col_q", "G16_COL_Q"), ("col_y", "G16_COL_Y")):
        start = src.index(f"__device__ __forceinline__ void {fn}(")
        body = src[start:src.index("\n}\n", start)]
        assert f"{macro}(G16_BOPS_S)" in body and f"{macro}(G16_BOPS)" in body
