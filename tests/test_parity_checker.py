"""Pins of the parity checker (CPU): it must reject wrong long-context outputs.

At long context every output value is an average over thousands of
unit-variance values, so its magnitude is ~1e-2 and the elementwise bound of
test_verify_splitkv.py (atol 2e-2) cannot tell a correct output from zero.
These cases show that the checker's relative-L2 bound does: the oracle's own
output rounded to bf16 (what a correct kernel stores) passes; an all-zero
output, a halved output and the output of the same batch with the first
eighth of one sequence's prefix dropped (a lost range) fail, although the
first two pass the elementwise bound alone.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import BF16_TOL, compare
from speculative_decoding_attention_amd import workloads as W


@pytest.fixture(scope="module")
def long_case():
    # headline geometry at two sequences of 8k: 16/2 heads, D=256, scattered pool
    p = W.make_problem([8192, 8192], 4, 16, 2, 256, k_scale=0.5, v_scale=0.25, pool_factor=2,
                       permute=True, seed=3, name="checker")
    args = lambda idx, indptr: (p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, indptr, idx,
                                p.sm_scale, p.k_scale, p.v_scale)
    ref = oracle.verify_attn(*args(p.kv_indices, p.kv_indptr))
    # sequence 0 without its first 1024 prefix tokens
    idx = torch.cat([p.kv_indices[1024:8192], p.kv_indices[8192:]])
    indptr = torch.tensor([0, 7168, 7168 + 8192], dtype=torch.int32)
    dropped = oracle.verify_attn(*args(idx, indptr))
    return ref, dropped


def test_outputs_are_small_at_long_context(long_case):
    ref, _ = long_case
    assert float(np.abs(ref).max()) < BF16_TOL["atol"]


def test_correct_bf16_output_passes(long_case):
    ref, _ = long_case
    stored = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    elem_ok, l2_ok, _, rel = compare(stored, ref, BF16_TOL)
    assert elem_ok and l2_ok and rel < 3e-3


@pytest.mark.parametrize("wrong", ["zero", "half", "dropped range"])
def test_wrong_outputs_fail(long_case, wrong):
    ref, dropped = long_case
    got = {"zero": np.zeros_like(ref), "half": 0.5 * ref, "dropped range": dropped}[wrong]
    elem_ok, l2_ok, _, rel = compare(got, ref, BF16_TOL)
    assert not l2_ok, "relative L2 %.3e" % rel
    if wrong != "dropped range":
        assert elem_ok  # the elementwise bound alone would have accepted it
