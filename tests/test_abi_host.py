"""Host-only tests of the C-ABI library: exports, validation, the static plan.

No test here launches a kernel; they run without a GPU.  Validation mirrors
can_handle() in sglang's verify_splitkv.py and its fallback tests in
test_verify_splitkv.py (non-causal / exotic features have no parameter in this
ABI; the ragged-extend case maps to q_rows != bs * l_ext).
"""
import ctypes
import math
import os
import re

import pytest
import torch

from speculative_decoding_attention_amd import verify_attn as va
from speculative_decoding_attention_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verify_attn.h")


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"VA_API\s+[\w\s\*]+?\b(verify_attn_\w+)\s*\(", text)


def test_header_declares_the_documented_entry_points():
    names = set(declared_symbols())
    assert {"verify_attn_run", "verify_attn_prefix", "verify_attn_combine", "verify_attn_check",
            "verify_attn_plan", "verify_attn_workspace_bytes", "verify_attn_strerror",
            "verify_attn_last_error", "verify_attn_version", "verify_attn_run_tree",
            "verify_attn_combine_tree", "verify_attn_append_kv", "verify_attn_build_kv_indices"} <= names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(va.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert va.lib().verify_attn_version() >= 100


def meta_problem(bs=3, l_ext=4, h_q=16, h_kv=2, d=256, n=512, kv_dtype=torch.bfloat16, **kw):
    m = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device="meta")
    q = m(bs * l_ext, h_q, d)
    return dict(q=q, k_ext=m(bs * l_ext, h_kv, d), v_ext=m(bs * l_ext, h_kv, d),
                k_buf=m(bs * n, h_kv, d, dt=kv_dtype), v_buf=m(bs * n, h_kv, d, dt=kv_dtype),
                kv_indices=m(bs * n, dt=torch.int64), out=m(bs * l_ext, h_q, d), bs=bs, **kw)


def desc_of(**kw):
    return va.make_desc(**meta_problem(**kw))


def test_valid_descriptor_passes():
    assert va.verify_attn_check(desc_of(), 4) == 0
    assert va.verify_attn_check(desc_of(kv_dtype=torch.float8_e4m3fn, d=128, h_q=8, h_kv=1), 4) == 0


@pytest.mark.parametrize("mutate,l_ext,code", [
    (lambda d: setattr(d, "bs", 0), 4, -2),
    (lambda d: setattr(d, "h_kv", 3), 4, -3),          # 16 % 3 != 0
    (lambda d: setattr(d, "h_kv", 0), 4, -3),
    (lambda d: setattr(d, "head_dim", 96), 4, -4),
    (lambda d: setattr(d, "v_head_dim", 64), 4, -4),   # Dv = D / 4
    (lambda d: setattr(d, "v_head_dim", 96), 4, -4),
    (lambda d: setattr(d, "kv_dtype", 7), 4, -5),
    (lambda d: None, 0, -6),                            # l_ext < 1
    (lambda d: None, 5, -6),                            # ragged: q_rows != bs * (mle + 1)
    (lambda d: d.q_stride.__setitem__(0, -1), 4, -7),
    (lambda d: d.kbuf_stride.__setitem__(0, 257), 4, -7),   # row start not 16-B aligned
    (lambda d: d.out_stride.__setitem__(1, 8), 4, -7),      # overlapping output rows
    (lambda d: setattr(d, "split_tokens", 100), 4, -10),    # not a multiple of 64
    (lambda d: (setattr(d, "split_tokens", 64), setattr(d, "n_splits", 4)), 4, -10),
    (lambda d: setattr(d, "num_kv_indices", -1), 4, -13),
])
def test_invalid_descriptors_are_rejected(mutate, l_ext, code):
    d = desc_of()
    mutate(d)
    assert va.verify_attn_check(d, l_ext) == code
    assert va.lib().verify_attn_last_error().decode() != ""
    assert va.lib().verify_attn_strerror(code).decode() not in ("", "unknown status")


@pytest.mark.parametrize("d,dv,ok", [(64, 128, True), (128, 64, True), (128, 256, True), (256, 128, True),
                                     (64, 256, False), (256, 64, False), (256, 96, False)])
def test_value_head_dim_pairs(d, dv, ok):
    # head_dim and v_head_dim are separate (the pages' VerifySplitKV takes
    # both); the kernels are built for equal dims and dims a factor 2 apart
    meta = meta_problem(d=d)
    meta["v_ext"] = torch.empty(12, 2, dv, dtype=torch.bfloat16, device="meta")
    meta["v_buf"] = torch.empty(3 * 512, 2, dv, dtype=torch.bfloat16, device="meta")
    meta["out"] = torch.empty(12, 16, dv, dtype=torch.bfloat16, device="meta")
    desc = va.make_desc(**meta)
    assert (va.verify_attn_check(desc, 4) == 0) == ok
    if ok:
        plan = va.verify_attn_plan(desc, 4, 256)
        assert plan.partial_bytes >= plan.range_slots * 2 * 32 * dv * 2
        assert plan.tile_tokens == 16384 // (2 * max(d, dv))


def test_null_descriptor():
    assert va.lib().verify_attn_check(None, 4) == -1


def test_plan_is_pure_given_cu_count():
    d = desc_of()
    a = va.verify_attn_plan(d, 4, 256).as_dict()
    b = va.verify_attn_plan(d, 4, 256).as_dict()
    assert a == b
    assert va.verify_attn_workspace_bytes(d, 4, 256) == a["workspace_bytes"]


def _plan_for(p: W.Problem, cus=256, **kw):
    desc = va.make_desc(p.q.to("meta"), p.k_ext.to("meta"), p.v_ext.to("meta"), p.k_buf[:1].to("meta"),
                        p.v_buf[:1].to("meta"), p.kv_indices.to("meta"), p.q.to("meta"), p.bs, **kw)
    return va.verify_attn_plan(desc, p.l_ext, cus)


def test_plan_headline_shapes():
    # B=8, 8k prefix, l_ext=4, 16/2 heads, D=256: 2 KV heads x 65536 tokens
    # shared over two resident workgroups per CU on 256 CUs -> 256-token ranges
    meta = meta_problem(bs=8, n=8192)
    plan = va.verify_attn_plan(va.make_desc(**meta), 4, 256)
    assert plan.mode == 0 and plan.split_tokens == 256
    assert plan.rows == 32 and plan.row_chunks == 1 and plan.tile_tokens == 32
    assert plan.range_slots >= 8 * 8192 // 256
    assert plan.workspace_bytes >= plan.range_slots * 2 * 32 * (256 * 2 + 4)


def _fitted_units(lens, cap, rounds=False):
    """The kernels' mode-0 range size in units of 64 tokens, by plain search:
    the smallest k >= 1 with sum_b ceil(ceil(n_b / 64) / k) <= cap.  In mode 3
    (rounds=True) a batch whose longest prefix is within 1/8 of the mean over
    its non-empty ones keeps whole sequences."""
    m = [-(-n // 64) for n in lens]
    nz = sum(1 for x in m if x > 0)
    if rounds and sum(m) > 0 and max(m) * nz <= sum(m) + sum(m) // 8:
        return max(m)
    k = 1
    while sum(-(-x // k) for x in m) > cap:
        k += 1
    return k


def _meta_with_indices(bs, T, **kw):
    meta = meta_problem(bs=bs, n=1, **kw)
    meta["kv_indices"] = torch.empty(T, dtype=torch.int64, device="meta")
    return meta


@pytest.mark.parametrize("seed", range(5))
def test_ragged_batches_fit_the_resident_workgroups(seed):
    # Mode 0 (heuristic): the grid holds one range per resident prefix
    # workgroup (two 4-wave workgroups per CU here), at least one per sequence
    # and at most ceil(T / 64) -- or, for a batch past the resident
    # workgroups, about one per MiB of K/V; the kernels fit the range size to
    # the lengths so that a ragged batch never needs more ranges than that.
    g = torch.Generator().manual_seed(seed)
    bs = int(torch.randint(1, 40, (1,), generator=g))
    lens = torch.randint(0, 5000, (bs,), generator=g).tolist()
    T = sum(lens)
    meta = _meta_with_indices(bs, T, l_ext=2, h_q=8, h_kv=1, d=128)
    for cus in (8, 80, 256):
        plan = va.verify_attn_plan(va.make_desc(**meta), 2, cus)
        assert plan.mode == (3 if bs > 2 * cus else 0)
        c = plan.split_tokens
        assert c % 64 == 0 and c >= 64
        cap = plan.prefix_blocks  # one KV head, one row chunk
        assert plan.range_slots == cap
        if T == 0:
            assert cap == 0
            continue
        expect = max(min(2 * cus, -(-T // 64)), bs)
        if bs > 2 * cus:  # rounds of workgroups: ~1 MiB of K/V (2048 tokens here) a range
            expect = max(expect, -(-T // 2048))
        assert cap == expect
        k = _fitted_units(lens, cap, rounds=plan.mode == 3)
        assert sum(-(-n // (64 * k)) for n in lens) <= cap
        assert k * 64 <= -(-max(lens) // 64) * 64  # never longer than one range per sequence


def test_capacity_sized_kv_indices_keep_the_grid():
    # Under graph capture kv_indices is a buffer sized for the largest batch
    # (aiter_backend.py, init_cuda_graph_state: cuda_graph_kv_indices).  The
    # headline batch (8 x 8192, 16/2 heads, D=256) with that buffer at 1x, 2x,
    # 4x and 8x its needed length keeps every range slot, and the kernels'
    # fitted size is the 256 tokens the exact buffer gives.
    base = None
    for factor in (1, 2, 4, 8):
        meta = _meta_with_indices(8, factor * 8 * 8192)
        plan = va.verify_attn_plan(va.make_desc(**meta), 4, 256)
        if base is None:
            base = plan
        assert plan.range_slots == base.range_slots == 256
        assert plan.prefix_blocks == base.prefix_blocks == 512
        assert plan.workspace_bytes == base.workspace_bytes
        assert _fitted_units([8192] * 8, plan.range_slots) == 4


@pytest.mark.parametrize("shape", [
    dict(l_ext=4, h_q=16, h_kv=2, d=256),
    dict(l_ext=8, h_q=8, h_kv=1, d=128, kv_dtype=torch.float8_e4m3fn),
    dict(l_ext=8, h_q=16, h_kv=1, d=64),          # two row chunks
    dict(l_ext=1, h_q=16, h_kv=2, d=256),         # decode
])
@pytest.mark.parametrize("split", [dict(), dict(split_tokens=128), dict(n_splits=8)])
def test_workspace_is_an_upper_bound_for_smaller_calls(shape, split):
    # A workspace sized once for (max_bs, T_max) must serve every call with
    # bs <= max_bs and T <= T_max (VerifySplitKV on page 1 sizes its scratch by
    # max_bs for the same reason): the size never decreases as T or bs grow.
    max_bs, t_max = 24, 200_000
    l_ext = shape["l_ext"]
    for cus in (256, 4):  # 4 CUs: batches past the resident workgroups, split for the rounds
        _check_workspace_monotone(shape, split, max_bs, t_max, l_ext, cus)


def _check_workspace_monotone(shape, split, max_bs, t_max, l_ext, cus):
    ts = sorted(set([0, 1, 63, 64, 65, 127, 129, 1000, 4095, 4097, 13423, 16423, 65536, t_max] +
                    list(range(0, t_max + 1, 997))))
    top = va.verify_attn_workspace_bytes(va.make_desc(**_meta_with_indices(max_bs, t_max, **shape), **split),
                                         l_ext, cus)
    for bs in (1, 2, 7, 8, 23, 24):
        prev = -1
        for T in ts:
            n = va.verify_attn_workspace_bytes(va.make_desc(**_meta_with_indices(bs, T, **shape), **split),
                                               l_ext, cus)
            assert n >= prev, (bs, T, n, prev)
            assert n <= top, (bs, T, n, top)
            prev = n
    for T in (0, 1000, 65536, t_max):
        prev = -1
        for bs in range(1, max_bs + 1):
            n = va.verify_attn_workspace_bytes(va.make_desc(**_meta_with_indices(bs, T, **shape), **split),
                                               l_ext, cus)
            assert n >= prev, (bs, T, n, prev)
            prev = n


def test_batches_past_the_resident_workgroups_get_round_sized_ranges():
    # 512 sequences, 16/2 heads, D=256 on 256 CUs: 256 ranges per KV head are
    # resident, so the grid runs in rounds; ranges of ~1 MiB of K/V per KV
    # head (1024 tokens) let a ragged batch balance instead of ending on its
    # longest sequences.  A batch within the resident workgroups keeps one
    # range per resident workgroup.
    T = 512 * 2560
    plan = va.verify_attn_plan(va.make_desc(**_meta_with_indices(512, T, l_ext=1, h_q=16, h_kv=2, d=256)), 1, 256)
    assert plan.mode == 3 and plan.range_slots == -(-T // 1024)
    # ragged: the kernels split the long sequences; near-equal: whole sequences
    g = torch.Generator().manual_seed(3)
    ragged = torch.randint(1024, 4097, (512,), generator=g).tolist()
    assert _fitted_units(ragged, plan.range_slots, rounds=True) < -(-max(ragged) // 64)
    equal = [2560] * 500 + [2400] * 12
    assert _fitted_units(equal, plan.range_slots, rounds=True) == 40
    plan = va.verify_attn_plan(va.make_desc(**_meta_with_indices(256, T, l_ext=1, h_q=16, h_kv=2, d=256)), 1, 256)
    assert plan.mode == 0 and plan.range_slots == 256
    # fp8, D = 128: 256 bytes a token -> 4096-token ranges
    plan = va.verify_attn_plan(va.make_desc(**_meta_with_indices(
        600, 600 * 3000, l_ext=1, h_q=8, h_kv=1, d=128, kv_dtype=torch.float8_e4m3fn)), 1, 256)
    assert plan.range_slots == max(600, -(-600 * 3000 // 4096))


def test_explicit_split_tokens_are_kept():
    # split_tokens given (mode 2): the grid bound covers every batch at exactly that size
    lens = [100, 1, 4097, 64, 0, 700]
    meta = _meta_with_indices(len(lens), sum(lens), l_ext=2, h_q=8, h_kv=1, d=128)
    plan = va.verify_attn_plan(va.make_desc(**meta, split_tokens=128), 2, 256)
    assert plan.mode == 2 and plan.split_tokens == 128
    assert sum(-(-n // 128) for n in lens) <= plan.range_slots


def test_pages_split_rule_mode():
    plan = va.verify_attn_plan(desc_of(n_splits=8), 4, 256)
    assert plan.mode == 1 and plan.n_splits == 8 and plan.range_slots == 3 * 8


def test_row_chunks_beyond_64_rows():
    plan = va.verify_attn_plan(desc_of(h_q=16, h_kv=1, l_ext=8), 8, 256)
    assert plan.rows == 128 and plan.row_chunks == 2


def test_run_rejects_bad_arguments_without_launching():
    # Null pointers / bad scales return an error code; nothing is launched.
    d = desc_of()
    rc = va.lib().verify_attn_run(None, None, None, None, None, None, None, None, 4,
                                  ctypes.c_float(0.1), ctypes.c_float(1.0), ctypes.c_float(1.0),
                                  None, ctypes.byref(d), None, 0, None)
    assert rc < 0


# ---------------------------------------------- tree / append / index build ---
def test_tree_entry_rejects_bad_mask_arguments():
    lib = va.lib()
    d = desc_of(l_ext=4)
    fake = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation first
    args = lambda mask, mi, l_ext, dd: (fake, fake, fake, fake, fake, fake, fake, fake, l_ext,
                                        ctypes.c_float(0.1), ctypes.c_float(1.0), ctypes.c_float(1.0),
                                        mask, mi, fake, ctypes.byref(dd), fake, 1 << 30, None)
    assert lib.verify_attn_run_tree(*args(None, fake, 4, d)) == -1
    assert lib.verify_attn_run_tree(*args(fake, None, 4, d)) == -1
    d65 = desc_of(l_ext=65)
    assert lib.verify_attn_run_tree(*args(fake, fake, 65, d65)) == -6


def _append_desc(kv_dtype=torch.bfloat16, d=128, h=2):
    m = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device="meta")
    return va.append_desc(m(8, h, d), m(8, h, d), m(100, h, d, dt=kv_dtype), m(100, h, d, dt=kv_dtype))


@pytest.mark.parametrize("mutate,n,scale,code", [
    (lambda d: setattr(d, "kv_dtype", 9), 8, 1.0, -5),
    (lambda d: setattr(d, "head_dim", 96), 8, 1.0, -4),
    (lambda d: setattr(d, "h_kv", 0), 8, 1.0, -3),
    (lambda d: d.kbuf_stride.__setitem__(0, 7), 8, 1.0, -7),
    (lambda d: None, -1, 1.0, -13),
])
def test_append_rejects_bad_arguments(mutate, n, scale, code):
    d = _append_desc()
    mutate(d)
    fake = ctypes.c_void_p(256)
    rc = va.lib().verify_attn_append_kv(fake, fake, fake, n, ctypes.c_float(scale), ctypes.c_float(scale),
                                        fake, fake, ctypes.byref(d), None)
    assert rc == code


def test_append_fp8_rejects_bad_scales_and_empty_is_a_no_op():
    d = _append_desc(torch.float8_e4m3fn)
    fake = ctypes.c_void_p(256)
    lib = va.lib()
    for ks in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.verify_attn_append_kv(fake, fake, fake, 8, ctypes.c_float(ks), ctypes.c_float(1.0),
                                         fake, fake, ctypes.byref(d), None) == -8
    assert lib.verify_attn_append_kv(None, None, None, 0, ctypes.c_float(1.0), ctypes.c_float(1.0),
                                     None, None, ctypes.byref(d), None) == 0


def test_build_kv_indices_rejects_bad_arguments():
    lib = va.lib()
    fake = ctypes.c_void_p(256)
    assert lib.verify_attn_build_kv_indices(fake, 10, fake, fake, None, 0, 10, fake, fake, None) == -2
    assert lib.verify_attn_build_kv_indices(fake, 10, fake, None, None, 2, 10, fake, fake, None) == -1
    assert lib.verify_attn_build_kv_indices(fake, -1, fake, fake, None, 2, 10, fake, fake, None) == -13


def test_paged_entry_rejects_bad_arguments():
    lib = va.lib()
    d = desc_of()
    fake = ctypes.c_void_p(256)
    call = lambda bt, stride, ps: lib.verify_attn_run_paged(
        fake, fake, fake, fake, fake, fake, fake, bt, stride, ps, 4, ctypes.c_float(0.1),
        ctypes.c_float(1.0), ctypes.c_float(1.0), fake, ctypes.byref(d), fake, 1 << 30, None)
    assert call(fake, 8, 0) == -13
    assert call(fake, -1, 16) == -7
    assert call(None, 8, 16) == -1


C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "verify_attn.h"

/* 8 sequences of 8192 tokens, l_ext 4, 16/2 heads, D = Dv = 256, bf16 pool */
int main(void)
{
    va_desc_t d;
    va_plan_t p;
    size_t ws = 0;
    int rc;
    memset(&d, 0, sizeof d);
    d.bs = 8; d.h_q = 16; d.h_kv = 2; d.head_dim = 256; d.v_head_dim = 256;
    d.kv_dtype = VA_DTYPE_BF16; d.q_rows = 32; d.num_kv_indices = 65536;
    d.q_stride[0] = 16 * 256; d.q_stride[1] = 256;
    d.out_stride[0] = 16 * 256; d.out_stride[1] = 256;
    d.kext_stride[0] = d.vext_stride[0] = d.kbuf_stride[0] = d.vbuf_stride[0] = 2 * 256;
    d.kext_stride[1] = d.vext_stride[1] = d.kbuf_stride[1] = d.vbuf_stride[1] = 256;
    rc = verify_attn_plan(&d, 4, 256, &p);
    if (rc == VA_OK)
        rc = verify_attn_workspace_bytes(&d, 4, 256, &ws);
    printf("%d %d %d %lld %lld %zu %zu %d\n", rc, p.mode, p.split_tokens, (long long)p.range_slots,
           (long long)p.prefix_blocks, p.workspace_bytes, ws, verify_attn_version());
    d.h_q = 15;  /* not a multiple of h_kv: rejected with a status, nothing launched */
    rc = verify_attn_check(&d, 4);
    printf("%d %s\n", rc, verify_attn_strerror(rc));
    return 0;
}
"""


def test_header_is_plain_c_and_links():
    # The boundary is a C ABI: the header compiles as strict C99 and a C
    # program links against the library and plans the headline shape
    # without Python (no device needed for planning).
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    pkg = os.path.dirname(va.LIB_PATH)
    with tempfile.TemporaryDirectory() as tmp:
        src, exe = os.path.join(tmp, "client.c"), os.path.join(tmp, "client")
        with open(src, "w") as f:
            f.write(C_CLIENT)
        include = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
        subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", include, src,
                        "-o", exe, "-L", pkg, "-lverify_attn", "-Wl,-rpath," + pkg], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split("\n")
    rc, mode, split, slots, blocks, ws_plan, ws, version = (int(x) for x in out[0].split())
    plan = va.verify_attn_plan(va.make_desc(**meta_problem(bs=8, n=8192)), 4, 256)
    assert rc == 0 and version == va.lib().verify_attn_version()
    assert (mode, split, slots, blocks, ws_plan) == (plan.mode, plan.split_tokens, plan.range_slots,
                                                      plan.prefix_blocks, plan.workspace_bytes)
    assert ws == ws_plan
    code, msg = out[1].split(" ", 1)
    assert int(code) == -3 and msg.strip()  # VA_ERR_HEADS
