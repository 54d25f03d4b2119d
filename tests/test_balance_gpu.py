"""Run-time balancing of long prefix ranges (the plan's balance = 1) on the GPU.

With the automatic split, long ranges are shared at run time: workgroups that
run out of work take the back part of another range (one compare-and-swap on
that range's control word) and the combine pass merges the taken part like a
range of its own.  These tests run shapes whose plan turns balancing on and
check, against the fp64 oracle at the tolerance of the parity tests:

* the output on every value, for ragged prefixes whose short last ranges make
  workgroups finish early (so parts are taken for certain), and the control
  words left in the workspace: every range fully covered, taken parts inside
  the range;
* repeated runs (the schedule depends on timing, the result may not);
* the same ranges under a static schedule (explicit split_tokens);
* HIP-graph replays with the inputs refilled between replays (the control
  words are reset by a kernel inside the captured call).
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

BF16_TOL = dict(atol=2e-2, rtol=1e-2)
STEAL_CHUNK = 4                 # tiles per owner claim (two chunks are held from the start)
NONE = 0xFFFFFFFF               # owner end not set


@pytest.fixture(scope="module")
def va():
    from speculative_decoding_attention_amd import verify_attn
    return verify_attn


def dev():
    return torch.device("cuda", 0)


def assert_close(gpu, ref, what):
    g = gpu.float().cpu().double().numpy()
    assert np.isfinite(g).all(), what + ": non-finite GPU output"
    err = np.abs(g - ref)
    bad = err > BF16_TOL["atol"] + BF16_TOL["rtol"] * np.abs(ref)
    print("%s: max abs err %.3e over %d values" % (what, float(err.max()), err.size), flush=True)
    assert not bad.any(), "%s: %d/%d values out of tolerance" % (what, int(bad.sum()), bad.size)


def long_problem(seed=11):
    # 65536 prefix tokens over two sequences, 8 KV heads, D = 256: 1024-token
    # ranges (32 tiles of 32 tokens) on 256 CUs; each sequence's last range
    # is short, so its workgroups finish early and take work from the others
    return W.make_problem([40000, 25536], 4, 16, 8, 256, k_scale=0.5, v_scale=0.25,
                          pool_factor=2, permute=True, seed=seed, device=dev(), name="balanced")


def oracle_of(pg):
    return oracle.verify_attn(pg.q.cpu(), pg.k_ext.cpu(), pg.v_ext.cpu(), pg.k_buf.cpu(),
                              pg.v_buf.cpu(), pg.qo_indptr.cpu(), pg.kv_indptr.cpu(),
                              pg.kv_indices.cpu(), pg.sm_scale, pg.k_scale, pg.v_scale)


def desc_plan(va, pg, **kw):
    out = torch.empty(pg.q.shape[0], pg.h_q, pg.v_head_dim, dtype=torch.bfloat16, device=dev())
    desc = va.make_desc(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.kv_indices, out, pg.bs, **kw)
    return out, desc, va.verify_attn_plan(desc, pg.l_ext, 0)


def run(va, pg, ws=None, **kw):
    out = va.verify_attn_run(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr,
                             pg.kv_indices, pg.l_ext, pg.sm_scale, pg.k_scale, pg.v_scale,
                             workspace=ws, **kw)
    torch.cuda.synchronize()
    return out


def range_tiles(pg, plan):
    """Exact tile count of every work item (range-major, then KV head)."""
    c, tn = plan.split_tokens, plan.tile_tokens
    caps = []
    for n in pg.prefix_lens:
        for s in range(-(-n // c)):
            caps.append(-(-(min(n, (s + 1) * c) - s * c) // tn))
    caps += [0] * (plan.range_slots - len(caps))
    return np.repeat(np.asarray(caps, np.int64), pg.h_kv * plan.row_chunks)


def test_balanced_full_parity_and_control_words(va):
    pg = long_problem()
    _, desc, plan = desc_plan(va, pg)
    assert plan.balance == 1, "this shape must plan balancing (256 CUs)"
    ws = va.alloc_workspace(desc, pg.l_ext, dev())
    out = run(va, pg, ws=ws)
    assert_close(out, oracle_of(pg), "balanced full")

    n_items = plan.range_slots * pg.h_kv * plan.row_chunks
    words = ws[plan.ctrl_offset:plan.ctrl_offset + 8 * n_items].view(torch.int64).cpu().numpy()
    low = (words & 0xFFFFFFFF).astype(np.int64)
    tail = ((words >> 32) & 0xFFFFFFFF).astype(np.int64)
    cap = range_tiles(pg, plan)
    taken = tail != NONE
    print("balanced: %d of %d ranges had their back part taken" % (int(taken.sum()), n_items), flush=True)
    assert taken.any(), "no part was taken although short ranges finish early"
    # a taken part starts past the owner's first two chunks and leaves a
    # non-empty back part; a range never taken was claimed to its end by its
    # owner (or marked as having nothing to take)
    assert (tail[taken] >= 2 * STEAL_CHUNK).all() and (tail[taken] < cap[taken]).all()
    assert (low >= 2 * STEAL_CHUNK).all()
    assert (low[~taken] >= cap[~taken]).all()


def test_balanced_repeats_stay_within_tolerance(va):
    pg = long_problem(seed=12)
    ref = oracle_of(pg)
    first = run(va, pg)
    for rep in range(3):
        out = run(va, pg)
        assert_close(out, ref, "balanced repeat %d" % rep)
        # runs differ only by the order partial results are summed in
        assert float((out.float() - first.float()).abs().max()) <= 1e-2


def test_balanced_matches_static_schedule(va):
    pg = long_problem(seed=13)
    _, _, plan = desc_plan(va, pg)
    assert plan.balance == 1
    dyn = run(va, pg)
    _, _, splan = desc_plan(va, pg, split_tokens=plan.split_tokens)
    assert splan.balance == 0
    static = run(va, pg, split_tokens=plan.split_tokens)
    assert float((dyn.float() - static.float()).abs().max()) <= 1e-2
    assert_close(static, oracle_of(pg), "static schedule")


def test_balanced_graph_replays(va):
    p = long_problem(seed=14)
    runner = va.VerifyAttn(p.h_q, p.h_kv, p.head_dim, p.l_ext, p.k_buf.dtype, max_bs=p.bs,
                           max_kv_indices=p.kv_indices.numel(), device=dev())
    out = torch.empty(p.q.shape[0], p.h_q, p.v_head_dim, dtype=torch.bfloat16, device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        runner(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr, p.kv_indices,
               p.sm_scale, out=out, k_scale=p.k_scale, v_scale=p.v_scale)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        runner(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr, p.kv_indices,
               p.sm_scale, out=out, k_scale=p.k_scale, v_scale=p.v_scale)
    for rep in range(2):
        fresh = long_problem(seed=200 + rep)
        for name in ("q", "k_ext", "v_ext", "k_buf", "v_buf", "kv_indices"):
            getattr(p, name).copy_(getattr(fresh, name))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_close(out, oracle_of(p), "balanced graph replay %d" % rep)


def test_static_sized_workspace_runs_the_static_schedule(va):
    # a workspace with room for the static layout only (a runner sized for
    # another shape) gives the static schedule: bitwise the explicit split
    pg = long_problem(seed=15)
    out, desc, plan = desc_plan(va, pg)
    assert plan.balance == 1
    _, sdesc, splan = desc_plan(va, pg, split_tokens=plan.split_tokens)
    small = torch.empty(splan.workspace_bytes, dtype=torch.uint8, device=dev())
    assert splan.workspace_bytes < plan.workspace_bytes
    got = run(va, pg, ws=small)
    want = run(va, pg, split_tokens=plan.split_tokens)
    assert torch.equal(got, want)
