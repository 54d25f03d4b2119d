"""Thin ctypes binding of ``libverify_attn.so`` (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only turns torch tensors into the pointers, shapes and strides the C ABI in
``include/verify_attn.h`` takes, and passes torch's current HIP stream.
Importing it loads the library and raises if it has not been built: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libverify_attn.so")

VA_DTYPE_BF16 = 0
VA_DTYPE_FP8_E4M3FN = 1

STATUS = {
    0: "VA_OK", -1: "VA_ERR_NULL_ARG", -2: "VA_ERR_BATCH", -3: "VA_ERR_HEADS",
    -4: "VA_ERR_HEAD_DIM", -5: "VA_ERR_DTYPE", -6: "VA_ERR_EXTEND", -7: "VA_ERR_STRIDE",
    -8: "VA_ERR_SCALE", -9: "VA_ERR_WORKSPACE", -10: "VA_ERR_SPLIT", -11: "VA_ERR_ALIGN",
    -12: "VA_ERR_DEVICE", -13: "VA_ERR_SIZE",
}


class VaDesc(ctypes.Structure):
    _fields_ = [
        ("bs", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("v_head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("q_rows", ctypes.c_int64), ("num_kv_indices", ctypes.c_int64),
        ("q_stride", ctypes.c_int64 * 2), ("kext_stride", ctypes.c_int64 * 2),
        ("vext_stride", ctypes.c_int64 * 2), ("kbuf_stride", ctypes.c_int64 * 2),
        ("vbuf_stride", ctypes.c_int64 * 2), ("out_stride", ctypes.c_int64 * 2),
        ("split_tokens", ctypes.c_int32), ("n_splits", ctypes.c_int32),
    ]


class VaPlan(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32), ("split_tokens", ctypes.c_int32), ("n_splits", ctypes.c_int32),
        ("rows", ctypes.c_int32), ("row_chunks", ctypes.c_int32), ("tile_tokens", ctypes.c_int32),
        ("range_slots", ctypes.c_int64), ("prefix_blocks", ctypes.c_int64),
        ("combine_blocks", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
        ("partial_bytes", ctypes.c_size_t), ("table_offset", ctypes.c_size_t),
    ]

    def as_dict(self):
        return {f[0]: getattr(self, f[0]) for f in self._fields_}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libverify_attn.so is not built (expected at %s); run "
            "`python -m speculative_decoding_attention_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    DP = ctypes.POINTER(VaDesc)
    lib.verify_attn_check.argtypes = [DP, I32]
    lib.verify_attn_plan.argtypes = [DP, I32, I32, ctypes.POINTER(VaPlan)]
    lib.verify_attn_workspace_bytes.argtypes = [DP, I32, I32, ctypes.POINTER(SZ)]
    lib.verify_attn_run.argtypes = [P, P, P, P, P, P, P, P, I32, F, F, F, P, DP, P, SZ, P]
    lib.verify_attn_run_noalloc.argtypes = [P, P, P, P, P, P, P, P, I32, F, F, F, P, DP, P]
    lib.verify_attn_prefix.argtypes = [P, P, P, P, P, P, I32, F, F, F, DP, P, SZ, P]
    lib.verify_attn_combine.argtypes = [P, P, P, P, P, I32, F, P, DP, P, SZ, P]
    lib.verify_attn_run_paged.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int64, I32, I32, F, F, F, P, DP,
                                          P, SZ, P]
    lib.verify_attn_prefix_paged.argtypes = [P, P, P, P, P, P, ctypes.c_int64, I32, I32, F, F, F, DP, P, SZ, P]
    lib.verify_attn_run_tree.argtypes = [P, P, P, P, P, P, P, P, I32, F, F, F, P, P, P, DP, P, SZ, P]
    lib.verify_attn_combine_tree.argtypes = [P, P, P, P, P, I32, F, P, P, P, DP, P, SZ, P]
    lib.verify_attn_append_kv.argtypes = [P, P, P, ctypes.c_int64, F, F, P, P, DP, P]
    lib.verify_attn_build_kv_indices.argtypes = [P, ctypes.c_int64, P, P, P, I32, ctypes.c_int64, P, P, P]
    for name in ("verify_attn_check", "verify_attn_plan", "verify_attn_workspace_bytes",
                 "verify_attn_run", "verify_attn_run_noalloc", "verify_attn_prefix", "verify_attn_combine",
                 "verify_attn_run_tree", "verify_attn_combine_tree", "verify_attn_append_kv",
                 "verify_attn_run_paged", "verify_attn_prefix_paged",
                 "verify_attn_build_kv_indices",
                 "verify_attn_version"):
        getattr(lib, name).restype = ctypes.c_int
    lib.verify_attn_strerror.argtypes = [ctypes.c_int]
    lib.verify_attn_strerror.restype = ctypes.c_char_p
    lib.verify_attn_last_error.argtypes = []
    lib.verify_attn_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


class VerifyAttnError(RuntimeError):
    def __init__(self, code, where):
        msg = _lib.verify_attn_last_error().decode() or _lib.verify_attn_strerror(code).decode()
        super().__init__("%s: %s (%s)" % (where, STATUS.get(code, code), msg))
        self.code = code


def _ok(code, where):
    if code != 0:
        raise VerifyAttnError(code, where)


def lib():
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return VA_DTYPE_BF16
    if t.dtype == torch.float8_e4m3fn:
        return VA_DTYPE_FP8_E4M3FN
    raise TypeError("pool dtype must be bfloat16 or float8_e4m3fn, got %s" % t.dtype)


def _strides(t: torch.Tensor, name: str):
    if t.dim() != 3:
        raise ValueError("%s must be 3-D, got shape %s" % (name, tuple(t.shape)))
    if t.stride(2) != 1:
        raise ValueError("%s: last dimension must be contiguous" % name)
    return (t.stride(0), t.stride(1))


def make_desc(q, k_ext, v_ext, k_buf, v_buf, kv_indices, out, bs: int,
              split_tokens: int = 0, n_splits: int = 0) -> VaDesc:
    """Descriptor of a problem from tensor shapes/strides (no device read)."""
    for name, t in (("q", q), ("k_ext", k_ext), ("v_ext", v_ext), ("out", out)):
        if t.dtype != torch.bfloat16:
            raise TypeError("%s must be bfloat16, got %s" % (name, t.dtype))
    if k_buf.dtype != v_buf.dtype:
        raise TypeError("k_buf and v_buf must share a dtype")
    if kv_indices.dtype != torch.int64:
        raise TypeError("kv_indices must be int64")
    d = VaDesc()
    d.bs = bs
    d.h_q, d.h_kv = q.shape[1], k_ext.shape[1]
    d.head_dim, d.v_head_dim = q.shape[2], v_ext.shape[2]
    d.kv_dtype = _dtype_code(k_buf)
    d.q_rows = q.shape[0]
    d.num_kv_indices = kv_indices.numel()
    d.q_stride[:] = _strides(q, "q")
    d.kext_stride[:] = _strides(k_ext, "k_ext")
    d.vext_stride[:] = _strides(v_ext, "v_ext")
    d.kbuf_stride[:] = _strides(k_buf, "k_buf")
    d.vbuf_stride[:] = _strides(v_buf, "v_buf")
    d.out_stride[:] = _strides(out, "out")
    d.split_tokens = int(split_tokens)
    d.n_splits = int(n_splits)
    return d


def verify_attn_check(desc: VaDesc, l_ext: int) -> int:
    return _lib.verify_attn_check(ctypes.byref(desc), int(l_ext))


def verify_attn_plan(desc: VaDesc, l_ext: int, num_cus: int = 0) -> VaPlan:
    plan = VaPlan()
    _ok(_lib.verify_attn_plan(ctypes.byref(desc), int(l_ext), int(num_cus), ctypes.byref(plan)),
        "verify_attn_plan")
    return plan


def verify_attn_workspace_bytes(desc: VaDesc, l_ext: int, num_cus: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _ok(_lib.verify_attn_workspace_bytes(ctypes.byref(desc), int(l_ext), int(num_cus), ctypes.byref(n)),
        "verify_attn_workspace_bytes")
    return n.value


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def alloc_workspace(desc: VaDesc, l_ext: int, device) -> torch.Tensor:
    n = verify_attn_workspace_bytes(desc, l_ext)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def verify_attn_run(q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, l_ext,
                    sm_scale=None, k_scale=1.0, v_scale=1.0, out=None, workspace=None,
                    split_tokens=0, n_splits=0, stream=None, desc=None):
    """Run both passes; returns ``out`` ([rows, H_Q, Dv] bf16).

    ``workspace`` (uint8 device tensor) may be given to keep a fixed address
    across calls (graph capture); otherwise one is allocated for the call.
    """
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if out is None:
        out = torch.empty(q.shape[0], q.shape[1], v_ext.shape[2], dtype=q.dtype, device=q.device)
    bs = qo_indptr.shape[0] - 1
    if desc is None:
        desc = make_desc(q, k_ext, v_ext, k_buf, v_buf, kv_indices, out, bs, split_tokens, n_splits)
    if workspace is None:
        workspace = alloc_workspace(desc, l_ext, q.device)
    rc = _lib.verify_attn_run(
        _ptr(q), _ptr(k_ext), _ptr(v_ext), _ptr(k_buf), _ptr(v_buf), _ptr(qo_indptr),
        _ptr(kv_indptr), _ptr(kv_indices) if kv_indices.numel() else 0, int(l_ext),
        float(sm_scale), float(k_scale), float(v_scale), _ptr(out), ctypes.byref(desc),
        _ptr(workspace), workspace.numel(), _stream(stream))
    _ok(rc, "verify_attn_run")
    return out


def verify_attn_run_noalloc(q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, l_ext,
                            sm_scale=None, k_scale=1.0, v_scale=1.0, out=None, split_tokens=0,
                            n_splits=0, stream=None, desc=None):
    """As verify_attn_run with the partials in the library's own device array
    (no workspace argument; the library allocates nothing).  ``out`` should be
    given by callers that cannot allocate."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if out is None:
        out = torch.empty(q.shape[0], q.shape[1], v_ext.shape[2], dtype=q.dtype, device=q.device)
    bs = qo_indptr.shape[0] - 1
    if desc is None:
        desc = make_desc(q, k_ext, v_ext, k_buf, v_buf, kv_indices, out, bs, split_tokens, n_splits)
    rc = _lib.verify_attn_run_noalloc(
        _ptr(q), _ptr(k_ext), _ptr(v_ext), _ptr(k_buf), _ptr(v_buf), _ptr(qo_indptr),
        _ptr(kv_indptr), _ptr(kv_indices) if kv_indices.numel() else 0, int(l_ext),
        float(sm_scale), float(k_scale), float(v_scale), _ptr(out), ctypes.byref(desc), _stream(stream))
    _ok(rc, "verify_attn_run_noalloc")
    return out


def verify_attn_prefix(q, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, l_ext, sm_scale,
                       k_scale, v_scale, desc, workspace, stream=None):
    rc = _lib.verify_attn_prefix(
        _ptr(q), _ptr(k_buf), _ptr(v_buf), _ptr(qo_indptr), _ptr(kv_indptr),
        _ptr(kv_indices) if kv_indices.numel() else 0, int(l_ext), float(sm_scale),
        float(k_scale), float(v_scale), ctypes.byref(desc), _ptr(workspace), workspace.numel(),
        _stream(stream))
    _ok(rc, "verify_attn_prefix")


def verify_attn_combine(q, k_ext, v_ext, qo_indptr, kv_indptr, l_ext, sm_scale, out, desc,
                        workspace, stream=None):
    rc = _lib.verify_attn_combine(
        _ptr(q), _ptr(k_ext), _ptr(v_ext), _ptr(qo_indptr), _ptr(kv_indptr), int(l_ext),
        float(sm_scale), _ptr(out), ctypes.byref(desc), _ptr(workspace), workspace.numel(),
        _stream(stream))
    _ok(rc, "verify_attn_combine")
    return out


def verify_attn_run_paged(q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, block_table, page_size,
                          l_ext, num_prefix_tokens, sm_scale=None, k_scale=1.0, v_scale=1.0, out=None,
                          workspace=None, split_tokens=0, n_splits=0, stream=None, desc=None):
    """Verify over a page-table prefix: token t of sequence b is pool row
    ``block_table[b, t // page_size] * page_size + t % page_size``
    (``block_table`` int32 [bs, max_pages]); ``num_prefix_tokens`` is the
    host-known total of the prefix lengths."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if out is None:
        out = torch.empty(q.shape[0], q.shape[1], v_ext.shape[2], dtype=q.dtype, device=q.device)
    bs = qo_indptr.shape[0] - 1
    if desc is None:
        desc = make_desc(q, k_ext, v_ext, k_buf, v_buf,
                         torch.empty(int(num_prefix_tokens), dtype=torch.int64, device="meta"),
                         out, bs, split_tokens, n_splits)
    if workspace is None:
        workspace = alloc_workspace(desc, l_ext, q.device)
    rc = _lib.verify_attn_run_paged(
        _ptr(q), _ptr(k_ext), _ptr(v_ext), _ptr(k_buf), _ptr(v_buf), _ptr(qo_indptr), _ptr(kv_indptr),
        _ptr(block_table), int(block_table.stride(0)), int(page_size), int(l_ext), float(sm_scale),
        float(k_scale), float(v_scale), _ptr(out), ctypes.byref(desc), _ptr(workspace), workspace.numel(),
        _stream(stream))
    _ok(rc, "verify_attn_run_paged")
    return out


def verify_attn_run_tree(q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices, l_ext,
                         custom_mask, mask_indptr, sm_scale=None, k_scale=1.0, v_scale=1.0, out=None,
                         workspace=None, split_tokens=0, n_splits=0, stream=None, desc=None):
    """Tree verify: as verify_attn_run with the draft block under ``custom_mask``
    (uint8/bool, per-sequence ``[l_ext, n_b + l_ext]`` row-major at
    ``mask_indptr[b]``, int64; prefix columns not read)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[2])
    if out is None:
        out = torch.empty(q.shape[0], q.shape[1], v_ext.shape[2], dtype=q.dtype, device=q.device)
    bs = qo_indptr.shape[0] - 1
    if desc is None:
        desc = make_desc(q, k_ext, v_ext, k_buf, v_buf, kv_indices, out, bs, split_tokens, n_splits)
    if workspace is None:
        workspace = alloc_workspace(desc, l_ext, q.device)
    rc = _lib.verify_attn_run_tree(
        _ptr(q), _ptr(k_ext), _ptr(v_ext), _ptr(k_buf), _ptr(v_buf), _ptr(qo_indptr),
        _ptr(kv_indptr), _ptr(kv_indices) if kv_indices.numel() else 0, int(l_ext),
        float(sm_scale), float(k_scale), float(v_scale), _ptr(custom_mask), _ptr(mask_indptr),
        _ptr(out), ctypes.byref(desc), _ptr(workspace), workspace.numel(), _stream(stream))
    _ok(rc, "verify_attn_run_tree")
    return out


def verify_attn_combine_tree(q, k_ext, v_ext, qo_indptr, kv_indptr, l_ext, sm_scale, custom_mask,
                             mask_indptr, out, desc, workspace, stream=None):
    rc = _lib.verify_attn_combine_tree(
        _ptr(q), _ptr(k_ext), _ptr(v_ext), _ptr(qo_indptr), _ptr(kv_indptr), int(l_ext),
        float(sm_scale), _ptr(custom_mask), _ptr(mask_indptr), _ptr(out), ctypes.byref(desc),
        _ptr(workspace), workspace.numel(), _stream(stream))
    _ok(rc, "verify_attn_combine_tree")
    return out


def append_desc(k, v, k_buf, v_buf) -> VaDesc:
    """Descriptor for verify_attn_append_kv (only head counts, dims, dtype and
    the four strides are read)."""
    d = VaDesc()
    d.bs = 1
    d.h_q = k.shape[1]
    d.h_kv = k.shape[1]
    d.head_dim = k.shape[2]
    d.v_head_dim = v.shape[2]
    d.kv_dtype = _dtype_code(k_buf)
    d.q_rows = k.shape[0]
    d.num_kv_indices = 0
    for field, t, name in (("kext_stride", k, "k"), ("vext_stride", v, "v"),
                           ("kbuf_stride", k_buf, "k_buf"), ("vbuf_stride", v_buf, "v_buf")):
        st = _strides(t, name)
        getattr(d, field)[0], getattr(d, field)[1] = st[0], st[1]
    return d


def verify_attn_append_kv(k, v, out_cache_loc, k_buf, v_buf, k_scale=1.0, v_scale=1.0, stream=None):
    """Write draft K/V rows into the pool at ``out_cache_loc`` (int64), casting
    to E4M3FN (x / scale, saturating) when the pool is fp8."""
    desc = append_desc(k, v, k_buf, v_buf)
    n = int(out_cache_loc.numel())
    rc = _lib.verify_attn_append_kv(_ptr(k) if n else 0, _ptr(v) if n else 0,
                                    _ptr(out_cache_loc) if n else 0, n, float(k_scale), float(v_scale),
                                    _ptr(k_buf), _ptr(v_buf), ctypes.byref(desc), _stream(stream))
    _ok(rc, "verify_attn_append_kv")


def verify_attn_build_kv_indices(req_to_token, req_pool_indices, seq_lens, kv_indptr, kv_indices,
                                 kv_start_idx=None, stream=None):
    """Fill ``kv_indptr`` (int32, bs + 1) and ``kv_indices`` (int64) from the
    request-to-token table (int32 [rows, stride])."""
    bs = int(seq_lens.numel())
    rc = _lib.verify_attn_build_kv_indices(
        _ptr(req_to_token), int(req_to_token.stride(0)), _ptr(req_pool_indices), _ptr(seq_lens),
        _ptr(kv_start_idx) if kv_start_idx is not None else 0, bs, int(kv_indices.numel()),
        _ptr(kv_indptr), _ptr(kv_indices) if kv_indices.numel() else 0, _stream(stream))
    _ok(rc, "verify_attn_build_kv_indices")


class VerifyAttn:
    """Fixed-address runner for one problem shape family.

    Holds a workspace sized once for the largest batch (``max_bs``) and the
    largest ``num_kv_indices`` (``max_kv_indices``) it will see, so its address
    never changes and calls can be captured in a HIP graph (the pages'
    VerifySplitKV caches its scratch per shape, sized by max_bs, for the same
    reason).  The library's workspace size never decreases as the batch or
    the index count grow, so every call with ``bs <= max_bs`` and
    ``len(kv_indices) <= max_kv_indices`` fits; ``kv_indices`` may be a buffer
    of fixed capacity whose used part ``kv_indptr`` delimits.  ``v_head_dim``
    (default ``head_dim``) is the value head dim the partials are sized by.
    """

    def __init__(self, h_q, h_kv, head_dim, l_ext, kv_dtype, max_bs, max_kv_indices, device,
                 split_tokens=0, n_splits=0, v_head_dim=None):
        self.l_ext = int(l_ext)
        self.device = torch.device(device)
        self.split_tokens, self.n_splits = int(split_tokens), int(n_splits)
        dv = int(head_dim if v_head_dim is None else v_head_dim)
        dummy = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="meta")
        d = make_desc(dummy(max_bs * l_ext, h_q, head_dim), dummy(max_bs * l_ext, h_kv, head_dim),
                      dummy(max_bs * l_ext, h_kv, dv),
                      torch.empty(1, h_kv, head_dim, dtype=kv_dtype, device="meta"),
                      torch.empty(1, h_kv, dv, dtype=kv_dtype, device="meta"),
                      torch.empty(max_kv_indices, dtype=torch.int64, device="meta"),
                      dummy(max_bs * l_ext, h_q, dv), max_bs, split_tokens, n_splits)
        with torch.cuda.device(self.device):
            self.workspace = alloc_workspace(d, l_ext, self.device)

    def __call__(self, q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices,
                 sm_scale=None, k_scale=1.0, v_scale=1.0, out=None, stream=None):
        return verify_attn_run(q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices,
                               self.l_ext, sm_scale, k_scale, v_scale, out, self.workspace,
                               self.split_tokens, self.n_splits, stream)
