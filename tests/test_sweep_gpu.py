"""Seeded sweep of random verify shapes: HIP path (C ABI) against the fp64 oracle.

Each case draws, from its own seed, a batch size (up to 80, so index-pointer
walks cross the first 64 sequences), prefix lengths (ragged with empty
sequences, or uniform multiples of 64, the shape whose ranges start where the
prefix pass copies its first indices before reading kv_indptr), l_ext, the GQA
ratio, the head dim, the pool dtype, a contiguous or scattered pool and the
split mode.  A second sweep adds value head dims apart from D, batches of up
to 600 sequences (past the resident prefix workgroups) and kv_indices buffers
of up to 4x the batch's tokens whose unused tail holds other valid pool rows.
Sizes stay small enough for the oracle to finish in about a second per case.
Tolerances (elementwise and relative L2) from tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import BF16_TOL, FP8_TOL, assert_close
from speculative_decoding_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def va():
    from speculative_decoding_attention_amd import verify_attn
    return verify_attn


def draw_case(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 256]))
    fp8 = bool(rng.random() < 0.4)
    h_kv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    l_ext = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    while group * l_ext > 128:
        l_ext = max(1, l_ext // 2)
    bs = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 70, 80]))
    # keep the oracle's work (tokens x query heads x draft rows) near 4M
    budget = max(64, int(4e6 / (h_kv * group * l_ext * bs)))
    if rng.random() < 0.3:
        lens = [64 * int(rng.integers(1, max(2, min(budget, 8192) // 64 + 1)))] * bs
    else:
        lens = rng.integers(0, max(2, min(budget, 6000)), bs).tolist()
        lens = [0 if rng.random() < 0.1 else int(n) for n in lens]
    split = {}
    r = rng.random()
    if r < 0.2:
        split = dict(split_tokens=int(rng.choice([64, 128, 320])))
    elif r < 0.35:
        split = dict(n_splits=int(rng.choice([1, 3, 8])))
    permute = bool(rng.random() < 0.6)
    return dict(lens=lens, l_ext=l_ext, h_q=h_kv * group, h_kv=h_kv, d=d, fp8=fp8, split=split,
                permute=permute)


@pytest.mark.parametrize("seed", range(40))
def test_random_shape(va, seed):
    c = draw_case(1000 + seed)
    p = W.make_problem(c["lens"], c["l_ext"], c["h_q"], c["h_kv"], c["d"],
                       kv_dtype=torch.float8_e4m3fn if c["fp8"] else torch.bfloat16,
                       k_scale=0.5, v_scale=0.75, pool_factor=2 if c["permute"] else None,
                       permute=c["permute"], seed=2000 + seed, name="sweep %d" % seed)
    print("case %d: bs %d, lens %s..., l_ext %d, heads %d/%d, d %d, %s, %s, %s" % (
        seed, p.bs, c["lens"][:4], c["l_ext"], c["h_q"], c["h_kv"], c["d"], "fp8" if c["fp8"] else "bf16",
        "scattered" if c["permute"] else "contiguous", c["split"] or "auto"), flush=True)
    pg = p.to(torch.device("cuda", 0))
    out = va.verify_attn_run(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr,
                             pg.kv_indices, pg.l_ext, pg.sm_scale, pg.k_scale, pg.v_scale, **c["split"])
    torch.cuda.synchronize()
    ref = oracle.verify_attn(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr,
                             p.kv_indices, p.sm_scale, p.k_scale, p.v_scale)
    assert_close(out, ref, FP8_TOL if c["fp8"] else BF16_TOL, p.name)


def draw_wide_case(seed):
    """A second sweep: value head dims apart from D, batches past the
    resident prefix workgroups (up to 600 sequences, plan mode 3) and
    kv_indices buffers of 1-4x the batch's tokens."""
    rng = np.random.default_rng(seed)
    d, dv = [(64, 64), (128, 128), (256, 256), (64, 128), (128, 64), (128, 256), (256, 128)][int(rng.integers(7))]
    fp8 = bool(rng.random() < 0.4)
    h_kv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 4, 8]))
    l_ext = int(rng.choice([1, 2, 4]))
    bs = int(rng.choice([1, 7, 64, 65, 300, 600]))
    budget = max(64, int(3e6 / (h_kv * group * l_ext * bs)))
    lens = rng.integers(0, max(2, min(budget, 6000)), bs).tolist()
    lens = [0 if rng.random() < 0.05 else int(n) for n in lens]
    capacity = int(rng.choice([1, 2, 4]))
    split = dict(split_tokens=int(rng.choice([64, 256]))) if rng.random() < 0.15 else {}
    return dict(lens=lens, l_ext=l_ext, h_q=h_kv * group, h_kv=h_kv, d=d, dv=dv, fp8=fp8, capacity=capacity,
                split=split)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_wide(va, seed):
    c = draw_wide_case(5000 + seed)
    p = W.make_problem(c["lens"], c["l_ext"], c["h_q"], c["h_kv"], c["d"], c["dv"],
                       kv_dtype=torch.float8_e4m3fn if c["fp8"] else torch.bfloat16,
                       k_scale=0.5, v_scale=0.75, pool_factor=2, permute=True, seed=6000 + seed,
                       name="wide sweep %d" % seed)
    print("case %d: bs %d, T %d, l_ext %d, heads %d/%d, d %d/%d, %s, kv_indices x%d, %s" % (
        seed, p.bs, p.total_prefix, c["l_ext"], c["h_q"], c["h_kv"], c["d"], c["dv"],
        "fp8" if c["fp8"] else "bf16", c["capacity"], c["split"] or "auto"), flush=True)
    dev = torch.device("cuda", 0)
    pg = p.to(dev)
    # the unused tail of the buffer holds other valid pool rows: read as
    # indices they would change the output, but never leave the pool
    g = torch.Generator().manual_seed(7000 + seed)
    rows = p.k_buf.shape[0]
    idx = torch.randint(0, rows, (c["capacity"] * max(1, p.total_prefix),), generator=g).to(torch.int64)
    idx[:p.total_prefix] = p.kv_indices
    idx = idx.to(dev)
    out = va.verify_attn_run(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr, idx,
                             pg.l_ext, pg.sm_scale, pg.k_scale, pg.v_scale, **c["split"])
    torch.cuda.synchronize()
    ref = oracle.verify_attn(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr,
                             p.kv_indices, p.sm_scale, p.k_scale, p.v_scale)
    assert_close(out, ref, FP8_TOL if c["fp8"] else BF16_TOL, p.name)
