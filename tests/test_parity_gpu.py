"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (tests/parity.py): elementwise |gpu - ref| <= atol + rtol*|ref| with
atol 2e-2 / rtol 1e-2 for a bf16 pool and atol 3e-2 / rtol 1e-2 for an fp8
pool -- the bounds the test file of the pages uses against its single-pass
baseline (test_verify_splitkv.py, ATOL/RTOL, ~10x over the ~2e-3 observed on
gfx950), widened for fp8 -- and a relative L2 error of at most 1e-2 over the
compared values, which is what still tells a right output from a wrong one at
long context, where every output value is ~1e-2.

Shapes: the five specified workloads at full size (every output value
compared, the 64k-prefix one included), the shape sweeps of
test_verify_splitkv.py, batches past the register-held range lookup, graph
replays with a capacity-sized kv_indices buffer, and edge cases.
"""
import math

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


def dev():
    return torch.device("cuda", 0)


def run_gpu(va, p: W.Problem, **kw):
    out = va.verify_attn_run(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr,
                             p.kv_indices, p.l_ext, p.sm_scale, p.k_scale, p.v_scale, **kw)
    torch.cuda.synchronize()
    return out


def oracle_of(p: W.Problem, select=None):
    return oracle.verify_attn(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr,
                              p.kv_indices, p.sm_scale, p.k_scale, p.v_scale, select=select)


def tol_of(p):
    return FP8_TOL if p.kv_fp8 else BF16_TOL


def check_full(va, p, **kw):
    pg = p.to(dev())
    out = run_gpu(va, pg, **kw)
    return assert_close(out, oracle_of(p), tol_of(p), p.name)


# ------------------------------------------------------- specified workloads ---
def test_tiny(va):
    check_full(va, W.config_tiny())


def test_b3_512(va):
    check_full(va, W.config_b3_512())


def test_b8_8k_full(va):
    # the headline workload at full size, in the launch configuration the
    # benchmark times (heuristic split); compared on every output value
    check_full(va, W.config_b8_8k())


def test_fp8_ragged_full(va):
    check_full(va, W.config_fp8_ragged())


def test_fp8_ragged_permuted_pool(va):
    check_full(va, W.config_fp8_ragged(permute=True))


def test_b4_64k_full(va):
    # the long-context workload at full size: every (sequence, head) pair,
    # every output value, against the oracle (about 30 s of host work)
    pg = W.config_b4_64k(device=dev())
    out = run_gpu(va, pg)
    cpu = pg.to("cpu")
    del pg
    torch.cuda.empty_cache()
    ref = oracle_of(cpu)
    assert_close(out, ref, BF16_TOL, "b4_64k")


# ------------------------------------------- shape sweeps of the pages' tests ---
@pytest.mark.parametrize("lens", [[512, 512, 512], [768, 1536, 3072], [4096, 8192]])
def test_head_dim_256(va, lens):
    check_full(va, W.make_problem(lens, 4, 16, 2, 256, seed=51, name="d256 %s" % lens))


def test_head_dim_128(va):
    check_full(va, W.make_problem([1024, 2048], 4, 16, 2, 128, seed=52, name="d128"))


@pytest.mark.parametrize("hq,hkv", [(16, 1), (8, 1), (8, 2), (8, 4), (8, 8)])
def test_gqa_ratios(va, hq, hkv):
    check_full(va, W.make_problem([1024, 2048], 4, hq, hkv, 256, seed=53, name="gqa %d/%d" % (hq, hkv)))


@pytest.mark.parametrize("l_ext", [1, 2, 4, 8, 12, 16])
def test_extend_lengths(va, l_ext):
    # l_ext > 8: draft rows past the combine pass's first load batch, and
    # (16 / 2 heads) 96 or 128 rows per KV head, i.e. two row chunks
    check_full(va, W.make_problem([1024, 1024], l_ext, 16, 2, 256, seed=54, name="l_ext %d" % l_ext))


@pytest.mark.parametrize("l_ext", [63, 64, 65, 100])
@pytest.mark.parametrize("kv_dtype", [torch.bfloat16, torch.float8_e4m3fn])
def test_long_draft_blocks(va, l_ext, kv_dtype):
    # the combine pass keeps the visible draft keys of a row as a 64-bit word:
    # rows 63 and 64 sit on its edge, rows past 64 take only the online loop;
    # 2 * l_ext query rows per KV head (up to 200: four row chunks, the last ragged)
    check_full(va, W.make_problem([300, 517], l_ext, 4, 2, 128, kv_dtype=kv_dtype, seed=55,
                                  name="l_ext %d %s" % (l_ext, kv_dtype)))


@pytest.mark.parametrize("kw", [dict(), dict(n_splits=4), dict(split_tokens=128)])
def test_many_sequences(va, kw):
    # more than 64 sequences: range lookups walk the index pointers in
    # chunks of 64 (prefix and combine passes); ragged, some prefixes empty
    g = torch.Generator().manual_seed(71)
    lens = torch.randint(0, 300, (150,), generator=g)
    lens[::17] = 0
    p = W.make_problem(lens.tolist(), 3, 8, 2, 128, pool_factor=2, permute=True, seed=72,
                       name="150 sequences %s" % kw)
    check_full(va, p, **kw)


def _hint_and_fit(va, p, num_kv_indices=None):
    """(the planner's range-size hint, the kernels' fitted size) in tokens."""
    out = torch.empty(p.q.shape[0], p.h_q, p.v_head_dim, dtype=torch.bfloat16, device="meta")
    idx = p.kv_indices if num_kv_indices is None else torch.empty(num_kv_indices, dtype=torch.int64,
                                                                  device="meta")
    plan = va.verify_attn_plan(va.make_desc(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, idx, out, p.bs),
                               p.l_ext)
    m = [-(-n // 64) for n in p.prefix_lens]
    nz = sum(1 for x in m if x > 0)
    if plan.mode == 3 and sum(m) > 0 and max(m) * nz <= sum(m) + sum(m) // 8:
        return plan.split_tokens, 64 * max(m)  # near-equal prefixes in rounds: whole sequences
    k = 1
    while sum(-(-x // k) for x in m) > plan.range_slots:
        k += 1
    return plan.split_tokens, 64 * k


@pytest.mark.parametrize("case", ["bf16 six", "bf16 100 sequences", "fp8 four"])
def test_fitted_range_size_differs_from_the_hint(va, case):
    # Ragged batches whose fitted range size is not the planner's hint: the
    # first range starts where the early index copies went, but its length
    # differs from what they cover, so the prefix pass must fetch its indices
    # again.
    if case == "bf16 six":
        p = W.make_problem([100, 1, 4097, 64, 0, 700], 4, 16, 2, 256, pool_factor=2, permute=True,
                           seed=81, name=case)
    elif case == "bf16 100 sequences":
        g = torch.Generator().manual_seed(82)
        lens = torch.randint(0, 2000, (100,), generator=g).tolist()
        p = W.make_problem(lens, 2, 8, 1, 256, pool_factor=2, permute=True, seed=83, name=case)
    else:
        p = W.make_problem([3000, 5, 129, 2049], 8, 8, 1, 128, kv_dtype=torch.float8_e4m3fn,
                           pool_factor=2, permute=True, seed=84, name=case)
    hint, fit = _hint_and_fit(va, p)
    assert hint != fit, "the case must make the kernels depart from the hint"
    check_full(va, p)


@pytest.mark.parametrize("bs,l_ext,hq,hkv,d,kv", [
    (512, 1, 16, 2, 256, "bf16"),   # decode batch: every sequence in the register-held lookup
    (600, 1, 8, 1, 128, "fp8"),     # past it: the lookups walk a second group of sequences
    (1100, 2, 4, 1, 64, "bf16"),    # three groups
])
def test_large_batches(va, bs, l_ext, hq, hkv, d, kv):
    # ragged prefixes 0..600 tokens (every 37th empty)
    g = torch.Generator().manual_seed(bs)
    lens = torch.randint(1, 600, (bs,), generator=g)
    lens[::37] = 0
    dt = torch.float8_e4m3fn if kv == "fp8" else torch.bfloat16
    p = W.make_problem(lens.tolist(), l_ext, hq, hkv, d, kv_dtype=dt, pool_factor=2, permute=True,
                       seed=bs + 1, name="bs %d" % bs)
    check_full(va, p)
    check_full(va, p, split_tokens=128)


@pytest.mark.parametrize("spread", [0, 200, 1800])
def test_batches_in_rounds_whole_or_split(va, spread):
    # 520 sequences (16/2 heads, D = 256, decode) of up to 2048 tokens: more
    # than the resident prefix workgroups, so the heuristic plans rounds and a
    # grid of about one range per MiB of K/V per KV head.  Prefixes within 1/8
    # of equal keep one range per sequence (the surplus slots hold none); a
    # wider spread is cut into ranges.
    g = torch.Generator().manual_seed(90 + spread)
    lens = (2048 - torch.randint(0, spread + 1, (520,), generator=g)).tolist()
    p = W.make_problem(lens, 1, 16, 2, 256, pool_factor=2, permute=True, seed=91, name="rounds")
    hint, fit = _hint_and_fit(va, p)
    if spread <= 200:
        assert fit == -(-max(lens) // 64) * 64
    else:
        assert fit < -(-max(lens) // 64) * 64
    check_full(va, p)


@pytest.mark.parametrize("case", ["600 decode bf16", "600 decode fp8", "8 x 8192"])
def test_capacity_buffer_splits_like_an_exact_one(va, case):
    # kv_indices at 4x the batch's tokens (a graph-capture buffer) plans a
    # larger grid, but the kernels fit the ranges to the tokens kv_indptr
    # holds, so the split and every rounding match the exact buffer's: the
    # outputs are bit-equal.  The 600-sequence batches run past the resident
    # workgroups (plan mode 3, round-sized ranges); 8 x 8192 is mode 0.
    g = torch.Generator().manual_seed(95)
    if case == "8 x 8192":
        p = W.make_problem([8192] * 8, 4, 16, 2, 256, k_scale=0.5, v_scale=0.25, pool_factor=2, permute=True,
                           seed=96, name=case)
    else:
        lens = torch.randint(256, 2049, (600,), generator=g).tolist()
        kv = torch.float8_e4m3fn if "fp8" in case else torch.bfloat16
        hq, hkv, d = (16, 2, 256) if kv == torch.bfloat16 else (8, 1, 128)
        p = W.make_problem(lens, 1, hq, hkv, d, kv_dtype=kv, pool_factor=2, permute=True, seed=97, name=case)
    pg = p.to(dev())
    cap = torch.zeros(4 * p.total_prefix, dtype=torch.int64, device=dev())
    cap[:p.total_prefix].copy_(pg.kv_indices)
    out_cap = torch.empty(pg.q.shape[0], p.h_q, p.v_head_dim, dtype=torch.bfloat16, device=dev())
    plans = [va.verify_attn_plan(va.make_desc(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, idx, out_cap, p.bs),
                                 p.l_ext) for idx in (pg.kv_indices, cap)]
    assert plans[0].mode == (0 if case == "8 x 8192" else 3)
    if plans[0].mode == 3:
        assert plans[1].prefix_blocks > plans[0].prefix_blocks
    else:  # mode 0 sizes its grid by the resident workgroups alone
        assert plans[1].prefix_blocks == plans[0].prefix_blocks
    exact = run_gpu(va, pg)
    va.verify_attn_run(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr, cap, p.l_ext,
                       p.sm_scale, p.k_scale, p.v_scale, out=out_cap)
    torch.cuda.synchronize()
    assert torch.equal(exact, out_cap), "a capacity-sized kv_indices changed the split"
    sel = [(b, h) for b in (0, p.bs // 2, p.bs - 1) for h in (0, p.h_q - 1)]
    rows = np.zeros(out_cap.shape, dtype=bool)
    for b, h in sel:
        rows[b * p.l_ext:(b + 1) * p.l_ext, h] = True
    assert_close(out_cap, oracle_of(p, select=sel), tol_of(p), case, mask=rows)


def test_one_long_sequence_among_short_ones(va):
    # 40 sequences whose grid averages under 8 ranges each, so the combine
    # pass preloads 8 partial rows at a time; the 20000-token sequence has
    # about 157 ranges, so its merge loops over batches of 8 and reloads the
    # range weights past every 64 ranges
    lens = [20000] + [10] * 39
    p = W.make_problem(lens, 4, 16, 2, 256, k_scale=0.5, v_scale=0.25, pool_factor=2, permute=True,
                       seed=85, name="one long")
    hint, fit = _hint_and_fit(va, p)
    assert -(-20000 // fit) > 64
    check_full(va, p)


def test_kv_scales(va):
    check_full(va, W.make_problem([1024, 2048], 4, 16, 2, 256, k_scale=0.5, v_scale=0.25, seed=55,
                                  name="scales"))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_fp8_head_dims(va, d):
    p = W.make_problem([300, 1000, 77], 4, 8, 2, d, kv_dtype=torch.float8_e4m3fn, pool_factor=2,
                       permute=True, seed=56, name="fp8 d%d" % d)
    p.q.mul_(5.0)  # exercise the query cast to E4M3FN
    check_full(va, p)


@pytest.mark.parametrize("rows", [16, 64])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_every_prefix_kernel_shape(va, kv, d, rows):
    # each (pool dtype, head dim, query blocks) instance of the prefix pass:
    # 16 query rows per KV head fill one 32-row block, 64 rows two; the
    # shapes whose tiles hold several 32-token sub-tiles merge per-wave
    # token shares at the end of a range
    hq, hkv, l_ext = (8, 2, 4) if rows == 16 else (8, 1, 8)
    dt = torch.float8_e4m3fn if kv == "fp8" else torch.bfloat16
    p = W.make_problem([300, 1000, 77], l_ext, hq, hkv, d, kv_dtype=dt, pool_factor=2, permute=True,
                       seed=58, name="%s d%d rows %d" % (kv, d, rows))
    check_full(va, p)


@pytest.mark.parametrize("rows", [16, 64])
@pytest.mark.parametrize("d,dv", [(64, 128), (128, 64), (128, 256), (256, 128)])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_value_head_dim_differs(va, kv, d, dv, rows):
    # the pages keep head_dim and v_head_dim apart (verify_splitkv.py,
    # _verify_prefix_stage1 BLOCK_DV; VerifySplitKV(..., head_dim,
    # v_head_dim, ...)): scores over D, values / output over Dv, for every
    # pair the kernels are built for and both prefix kernel shapes
    hq, hkv, l_ext = (8, 2, 4) if rows == 16 else (8, 1, 8)
    dt = torch.float8_e4m3fn if kv == "fp8" else torch.bfloat16
    p = W.make_problem([300, 1000, 77, 0], l_ext, hq, hkv, d, dv, kv_dtype=dt, k_scale=0.5, v_scale=0.25,
                       pool_factor=2, permute=True, seed=59, name="%s d%d dv%d rows %d" % (kv, d, dv, rows))
    check_full(va, p)


def test_value_head_dim_differs_long_and_split(va):
    # D=256 / Dv=128 at 2 x 8k with k/v scales, heuristic and explicit splits
    p = W.make_problem([8192, 5000], 4, 16, 2, 256, 128, k_scale=0.5, v_scale=0.25, pool_factor=2,
                       permute=True, seed=60, name="d256 dv128 long")
    check_full(va, p)
    check_full(va, p, n_splits=16)


def test_fixed_runner_with_value_head_dim_and_smaller_calls(va):
    # VerifyAttn sized once (6 sequences, 15000 indices, D = 128 / Dv = 256:
    # the partials it holds are sized by Dv) serves calls with fewer
    # sequences and fewer indices from the same workspace
    runner = va.VerifyAttn(8, 2, 128, 4, torch.bfloat16, max_bs=6, max_kv_indices=15000, device=dev(),
                           v_head_dim=256)
    ws = runner.workspace.data_ptr()
    for lens, seed in (([1000, 2000, 2000], 70), ([5000], 71), ([64, 0, 3000, 10, 700, 1200], 72)):
        p = W.make_problem(lens, 4, 8, 2, 128, 256, k_scale=0.5, v_scale=0.25, pool_factor=2, permute=True,
                           seed=seed, name="fixed runner, %d sequences" % len(lens))
        pg = p.to(dev())
        out = runner(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr, pg.kv_indices,
                     pg.sm_scale, k_scale=pg.k_scale, v_scale=pg.v_scale)
        torch.cuda.synchronize()
        assert runner.workspace.data_ptr() == ws
        assert_close(out, oracle_of(p), BF16_TOL, p.name)


def test_many_rows_two_row_chunks(va):
    # G=16, l_ext=8: 128 query rows per KV head -> two 64-row chunks
    check_full(va, W.make_problem([700, 1500], 8, 16, 1, 128, seed=57, name="128 rows"))


# ------------------------------------------------------------ split invariance ---
@pytest.mark.parametrize("kw", [dict(split_tokens=64), dict(split_tokens=192), dict(split_tokens=4096),
                                dict(n_splits=1), dict(n_splits=4), dict(n_splits=16),
                                dict(n_splits=64)])
def test_split_count_invariance(va, kw):
    p = W.make_problem([1000, 33, 4100, 640], 4, 16, 2, 256, k_scale=0.5, v_scale=0.25, pool_factor=2,
                       permute=True, seed=61, name="split %s" % kw)
    pg = p.to(dev())
    ref = oracle_of(p)
    base = run_gpu(va, pg)
    out = run_gpu(va, pg, **kw)
    assert_close(out, ref, BF16_TOL, p.name)
    # the split changes only rounding: outputs agree with each other too
    assert float((out.float() - base.float()).abs().max()) < 2e-2


def test_empty_splits_do_not_leak_stale_values(va):
    # n_splits = 64 with 100-token prefixes leaves most ranges empty; poison
    # the workspace with NaN first: the empty ranges must write 0 / -inf.
    p = W.make_problem([100, 5, 37], 4, 8, 1, 128, seed=62, name="empty splits")
    pg = p.to(dev())
    out = torch.empty(pg.q.shape[0], pg.h_q, pg.v_head_dim, dtype=torch.bfloat16, device=dev())
    desc = va.make_desc(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.kv_indices, out, pg.bs,
                        n_splits=64)
    ws = va.alloc_workspace(desc, pg.l_ext, dev())
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    out = run_gpu(va, pg, out=out, workspace=ws, n_splits=64)
    assert_close(out, oracle_of(p), BF16_TOL, p.name)


def test_kv_indices_permutation_invariance(va):
    p = W.make_problem([2000, 700], 4, 16, 2, 256, pool_factor=2, permute=True, seed=63, name="perm")
    a = run_gpu(va, p.to(dev()))
    g = torch.Generator().manual_seed(3)
    idx = p.kv_indices.clone()
    for b in range(p.bs):
        s, e = int(p.kv_indptr[b]), int(p.kv_indptr[b + 1])
        idx[s:e] = idx[s:e][torch.randperm(e - s, generator=g)]
    p.kv_indices = idx
    b_ = run_gpu(va, p.to(dev()))
    assert float((a.float() - b_.float()).abs().max()) < 2e-2
    assert_close(b_, oracle_of(p), BF16_TOL, "perm")


# ----------------------------------------------------------------- edge cases ---
def test_empty_and_short_prefixes(va):
    # n_b = 0 (draft-only softmax), n_b shorter than one tile, ragged tails
    check_full(va, W.make_problem([0, 1, 31, 33, 65, 0, 257], 4, 8, 2, 256, pool_factor=2, permute=True,
                                  seed=71, name="short"))


def test_all_prefixes_empty(va):
    check_full(va, W.make_problem([0, 0, 0], 3, 4, 2, 128, seed=72, name="all empty"))


def test_single_token_everything(va):
    check_full(va, W.make_problem([1], 1, 1, 1, 64, seed=73, name="single"))


def test_large_score_range(va):
    # queries scaled up: sharply peaked softmax over prefix and drafts
    p = W.make_problem([900, 400], 4, 8, 2, 128, seed=74, name="peaked")
    p.q.mul_(6.0)
    check_full(va, p)


def test_strided_views(va):
    # q / out as views with padded head strides; pool with padded row stride
    p = W.make_problem([300, 200], 4, 8, 2, 128, seed=75, name="strided")
    pg = p.to(dev())
    qbig = torch.zeros(pg.q.shape[0], pg.h_q, 192, dtype=torch.bfloat16, device=dev())
    qbig[:, :, :128] = pg.q
    kb = torch.zeros(pg.k_buf.shape[0], pg.h_kv + 1, 128, dtype=torch.bfloat16, device=dev())
    kb[:, :pg.h_kv] = pg.k_buf
    outbig = torch.full((pg.q.shape[0], pg.h_q, 160), 7.0, dtype=torch.bfloat16, device=dev())
    out = outbig[:, :, :128]
    va.verify_attn_run(qbig[:, :, :128], pg.k_ext, pg.v_ext, kb[:, :pg.h_kv], pg.v_buf, pg.qo_indptr,
                       pg.kv_indptr, pg.kv_indices, pg.l_ext, pg.sm_scale, out=out)
    torch.cuda.synchronize()
    assert_close(out, oracle_of(p), BF16_TOL, "strided")
    assert bool((outbig[:, :, 128:] == 7.0).all()), "wrote outside the output view"


# -------------------------------------------------------- structure / runtime ---
def test_deterministic(va):
    pg = W.make_problem([3000, 1000], 4, 16, 2, 256, seed=81).to(dev())
    a, b = run_gpu(va, pg), run_gpu(va, pg)
    assert torch.equal(a, b)


def test_two_passes_equal_run(va):
    pg = W.make_problem([1500, 900], 4, 16, 2, 256, k_scale=0.5, v_scale=2.0, seed=82).to(dev())
    full = run_gpu(va, pg)
    out = torch.empty_like(full)
    desc = va.make_desc(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.kv_indices, out, pg.bs)
    ws = va.alloc_workspace(desc, pg.l_ext, dev())
    va.verify_attn_prefix(pg.q, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr, pg.kv_indices,
                          pg.l_ext, pg.sm_scale, pg.k_scale, pg.v_scale, desc, ws)
    va.verify_attn_combine(pg.q, pg.k_ext, pg.v_ext, pg.qo_indptr, pg.kv_indptr, pg.l_ext,
                           pg.sm_scale, out, desc, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, full)


def test_runtime_errors_are_status_codes(va):
    pg = W.config_tiny(device=dev())
    with pytest.raises(va.VerifyAttnError):
        va.verify_attn_run(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr,
                           pg.kv_indices, pg.l_ext, pg.sm_scale, k_scale=float("nan"))
    small = torch.empty(16, dtype=torch.uint8, device=dev())
    with pytest.raises(va.VerifyAttnError):
        va.verify_attn_run(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr,
                           pg.kv_indices, pg.l_ext, pg.sm_scale, workspace=small[:1])


def test_graph_capture_replay(va):
    # capture one call with fixed buffers; refill the inputs in place between
    # replays (eager work and syncs in between) and check every replay
    p = W.make_problem([1200, 800, 64], 4, 16, 2, 256, pool_factor=2, permute=True, seed=91)
    pg = p.to(dev())
    runner = va.VerifyAttn(pg.h_q, pg.h_kv, pg.head_dim, pg.l_ext, pg.k_buf.dtype, max_bs=pg.bs,
                           max_kv_indices=pg.kv_indices.numel(), device=dev())
    out = torch.empty(pg.q.shape[0], pg.h_q, pg.v_head_dim, dtype=torch.bfloat16, device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        runner(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr,
               pg.kv_indices, pg.sm_scale, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        runner(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr,
               pg.kv_indices, pg.sm_scale, out=out)
    for rep in range(3):
        fresh = W.make_problem(p.prefix_lens, 4, 16, 2, 256, pool_factor=2, permute=True,
                               seed=100 + rep)
        for name in ("q", "k_ext", "v_ext", "k_buf", "v_buf", "kv_indices"):
            getattr(pg, name).copy_(getattr(fresh, name))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = run_gpu(va, pg)
        assert torch.equal(out, eager), "replay %d differs from eager" % rep
        assert_close(out, oracle_of(fresh), BF16_TOL, "graph replay %d" % rep)


GRAPH_CASES = {
    # name: (bs, l_ext, h_q, h_kv, D, pool dtype, lengths of the replays)
    "bf16 8x8k": (8, 4, 16, 2, 256, torch.bfloat16, [
        ("8 x 8192", [8192] * 8),
        ("ragged", [13000, 7, 9000, 700, 16000, 1, 4000, 15000]),
        ("shorter", [1000] * 8),
        ("one empty", [8192, 0, 4096, 8192, 100, 8192, 8192, 3000]),
    ]),
    "fp8 mqa": (16, 8, 8, 1, 128, torch.float8_e4m3fn, [
        ("ragged", [1024 + 613 * i for i in range(16)]),
        ("short", [64 * (i % 5) + 3 for i in range(16)]),
        ("two empty", [0, 9000] + [2000] * 13 + [0]),
    ]),
    # decode batch past the resident prefix workgroups (plan mode 3): ragged
    # lengths cut into round-sized ranges, near-equal ones kept whole
    "bf16 decode 600": (600, 1, 16, 2, 256, torch.bfloat16, [
        ("ragged", [256 + (i * 379) % 1793 for i in range(600)]),
        ("near-equal", [1500 - (i % 7) * 10 for i in range(600)]),
        ("some empty", [0 if i % 9 == 0 else 700 + (i * 131) % 900 for i in range(600)]),
    ]),
}


@pytest.mark.parametrize("geometry", list(GRAPH_CASES))
def test_graph_replay_with_capacity_kv_indices(va, geometry):
    # The pages' graph mode: one capture, kv_indices a buffer of fixed
    # capacity (aiter_backend.py, init_cuda_graph_state: cuda_graph_kv_indices
    # sized for max_bs full contexts; _apply_cuda_graph_metadata fills it in
    # place), then replays after kv_indptr, the indices and the pool were
    # refilled with other lengths (verify_splitkv.py: the split clamps each
    # range to the sequence's real length at replay).  The buffer is 4x the
    # longest batch replayed.  Every replay is compared bit for bit with an
    # eager call on the same buffers and with the oracle.
    bs, L, hq, hkv, D, kv_dtype, cases = GRAPH_CASES[geometry]
    longest = max(sum(lens) for _, lens in cases)
    cap_tokens = 4 * longest
    pool_rows = 2 * longest
    d = dev()
    bf = torch.bfloat16
    q = torch.zeros(bs * L, hq, D, dtype=bf, device=d)
    k_ext = torch.zeros(bs * L, hkv, D, dtype=bf, device=d)
    v_ext = torch.zeros(bs * L, hkv, D, dtype=bf, device=d)
    k_buf = torch.zeros(pool_rows, hkv, D, dtype=bf, device=d).to(kv_dtype)
    v_buf = torch.zeros(pool_rows, hkv, D, dtype=bf, device=d).to(kv_dtype)
    kv_indices = torch.zeros(cap_tokens, dtype=torch.int64, device=d)
    kv_indptr = torch.zeros(bs + 1, dtype=torch.int32, device=d)
    qo_indptr = torch.arange(0, bs * L + 1, L, dtype=torch.int32, device=d)
    out = torch.empty(bs * L, hq, D, dtype=bf, device=d)
    runner = va.VerifyAttn(hq, hkv, D, L, kv_dtype, max_bs=bs, max_kv_indices=cap_tokens, device=d)
    sm = 1.0 / math.sqrt(D)
    k_scale, v_scale = (0.5, 0.25) if kv_dtype == bf else (0.011, 0.009)

    def call():
        runner(q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, sm, k_scale=k_scale,
               v_scale=v_scale, out=out)

    def load(lens, seed):
        p = W.make_problem(lens, L, hq, hkv, D, kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale,
                           pool_factor=2, permute=True, seed=seed, name=geometry)
        # the pool holds codes; the scales are the captured ones
        p.k_scale, p.v_scale = k_scale, v_scale
        q.copy_(p.q)
        k_ext.copy_(p.k_ext)
        v_ext.copy_(p.v_ext)
        n = p.k_buf.shape[0]
        k_buf[:n].copy_(p.k_buf)
        v_buf[:n].copy_(p.v_buf)
        kv_indices.zero_()
        kv_indices[:p.total_prefix].copy_(p.kv_indices)
        kv_indptr.copy_(p.kv_indptr)
        return p

    load(cases[0][1], 400)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i, (name, lens) in enumerate(cases):
        p = load(lens, 500 + i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        out.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        assert torch.equal(got, out), "replay %s differs from the eager call" % name
        assert_close(got, oracle_of(p), tol_of(p), "%s capacity replay %s" % (geometry, name))
