"""verify_attn_run_noalloc (partials in the library's device array) against
verify_attn_run (partials in the caller's workspace), through the C ABI.

Two calls in a row on the same GPU array, the second with a smaller batch: each
output must equal verify_attn_run's bit for bit (same kernels, same plan) and
match the fp64 oracle within the parity bounds.  A call whose plan needs more
than the array holds is refused on the host with VA_ERR_WORKSPACE.
"""
import ctypes

import pytest
import torch

import oracle
from parity import BF16_TOL, FP8_TOL, assert_close
from speculative_decoding_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

VA_ERR_WORKSPACE = -9


@pytest.fixture(scope="module")
def va():
    from speculative_decoding_attention_amd import verify_attn
    return verify_attn


def _noalloc(va, p, out):
    desc = va.make_desc(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.kv_indices, out, p.bs)
    rc = va.lib().verify_attn_run_noalloc(
        p.q.data_ptr(), p.k_ext.data_ptr(), p.v_ext.data_ptr(), p.k_buf.data_ptr(), p.v_buf.data_ptr(),
        p.qo_indptr.data_ptr(), p.kv_indptr.data_ptr(), p.kv_indices.data_ptr(), p.l_ext,
        ctypes.c_float(p.sm_scale), ctypes.c_float(p.k_scale), ctypes.c_float(p.v_scale), out.data_ptr(),
        ctypes.byref(desc), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, va.lib().verify_attn_last_error().decode()


def test_noalloc_matches_the_workspace_entry_point(va):
    d = torch.device("cuda", 0)
    cases = [
        W.config_b8_8k(),  # 8.5 MB of partials
        W.make_problem([700, 33, 2048], 4, 16, 2, 256, k_scale=0.5, v_scale=0.25, pool_factor=2,
                       permute=True, seed=7, name="smaller"),
        W.make_problem([300, 1000, 77], 8, 8, 1, 128, kv_dtype=torch.float8_e4m3fn, pool_factor=2,
                       permute=True, seed=8, name="smaller fp8"),
    ]
    for p in cases:
        pg = p.to(d)
        out = torch.full((pg.q.shape[0], pg.h_q, pg.v_head_dim), float("nan"), dtype=torch.bfloat16, device=d)
        _noalloc(va, pg, out)
        torch.cuda.synchronize()
        ref_ws = va.verify_attn_run(pg.q, pg.k_ext, pg.v_ext, pg.k_buf, pg.v_buf, pg.qo_indptr, pg.kv_indptr,
                                    pg.kv_indices, pg.l_ext, pg.sm_scale, pg.k_scale, pg.v_scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_ws), "%s: noalloc output differs from verify_attn_run" % p.name
        ref = oracle.verify_attn(p.q, p.k_ext, p.v_ext, p.k_buf, p.v_buf, p.qo_indptr, p.kv_indptr,
                                 p.kv_indices, p.sm_scale, p.k_scale, p.v_scale)
        assert_close(out, ref, FP8_TOL if p.kv_fp8 else BF16_TOL, "noalloc " + p.name)


def test_noalloc_refuses_plans_beyond_its_array(va):
    # 4096 sequences x 8 KV heads x 32 rows x (2 * 256 + 4) bytes of partials
    # is far past the array: refused on the host before anything is launched
    # (the pointers below are never dereferenced).
    m = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device="meta")
    bs, L = 4096, 4
    desc = va.make_desc(m(bs * L, 64, 256), m(bs * L, 8, 256), m(bs * L, 8, 256), m(8, 8, 256), m(8, 8, 256),
                        m(bs * 64, dt=torch.int64), m(bs * L, 64, 256), bs)
    assert va.verify_attn_plan(desc, L).workspace_bytes > 32 << 20
    fake = ctypes.c_void_p(256)
    rc = va.lib().verify_attn_run_noalloc(fake, fake, fake, fake, fake, fake, fake, fake, L, ctypes.c_float(0.1),
                                          ctypes.c_float(1.0), ctypes.c_float(1.0), fake, ctypes.byref(desc),
                                          None)
    assert rc == VA_ERR_WORKSPACE
    assert "verify_attn_run_noalloc holds at most" in va.lib().verify_attn_last_error().decode()
