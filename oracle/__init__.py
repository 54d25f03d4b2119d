"""fp64 CPU oracle for split-KV target-verify attention (topk = 1).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product (the HIP
library and its Python binding) never imports, links or calls it, and this
package imports nothing from the product.

The arithmetic lives in ``verify_attn_oracle.c`` (plain C, fp64, OpenMP over
(sequence, query-head) pairs).  This module only builds that file with gcc and
marshals numpy arrays into it.  What it computes is the single causal softmax
described in sglang's ``verify_splitkv.py`` (module docstring; kernels
``_verify_prefix_stage1`` and ``_verify_combine_stage2``): every draft query
sees the whole paged prefix (score scaled by ``sm_scale * k_scale``, value rows
by ``v_scale``, query rounded to the pool dtype) and the draft keys ``j <= i``
(score scaled by ``sm_scale`` only).

Pins (tests/test_oracle_pins.py): the fp8 decode table and the RNE encode
against torch's own float8_e4m3fn conversion; bf16 decode against torch;
closed forms (all keys zero gives the mean of the visible values, with
``v_scale`` on the prefix part only; equal-score constructions that check the
``k_scale`` placement; one-hot attention); torch's fp64
``scaled_dot_product_attention`` on an augmented-query construction that
reproduces the two score rules; ``l_ext = 1`` reducing to textbook
single-query attention; invariance to permuting ``kv_indices``, to relocating
pool rows, to power-of-two rescaling of the pool against the scales, to batch
order and to GQA -> MHA head expansion; and a numpy brute force on tiny
shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "verify_attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` with gcc + OpenMP."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path):
    lib = ctypes.CDLL(path)
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3fn_to_f64.restype = ctypes.c_double
    lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_f64_to_e4m3fn.restype = ctypes.c_uint8
    lib.oracle_f64_to_e4m3fn.argtypes = [ctypes.c_double]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_set_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_int64
    D = ctypes.c_double
    lib.oracle_verify_attn.restype = ctypes.c_int
    lib.oracle_verify_attn.argtypes = [
        I, I, I, I, I, I,
        P, L, L, P, L, L, P, L, L,
        P, L, L, P, L, L,
        P, P, P,
        D, D, D,
        I, P, P,
        P, L, L,
    ]
    lib.oracle_verify_attn_masked.restype = ctypes.c_int
    lib.oracle_verify_attn_masked.argtypes = [
        I, I, I, I, I, I,
        P, L, L, P, L, L, P, L, L,
        P, L, L, P, L, L,
        P, P, P,
        P, P,
        D, D, D,
        I, P, P,
        P, L, L,
    ]
    F = ctypes.c_float
    lib.oracle_append_kv.restype = ctypes.c_int
    lib.oracle_append_kv.argtypes = [L, I, I, I, I, P, L, L, P, L, L, P, F, F, P, L, L, P, L, L]
    lib.oracle_build_kv_indices.restype = ctypes.c_int
    lib.oracle_build_kv_indices.argtypes = [I, P, L, P, P, P, P, P]
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _bind(_LIB_PATH)
    return _lib


def load_variant(path):
    """Bind an alternative build of the oracle source (used by the mutation
    tests, which compile deliberately broken copies on the CPU)."""
    return _bind(path)


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits) & 0xFFFF)


def e4m3fn_to_f64(code: int) -> float:
    return _load().oracle_e4m3fn_to_f64(int(code) & 0xFF)


def f64_to_e4m3fn(x: float) -> int:
    return int(_load().oracle_f64_to_e4m3fn(float(x)))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> int:
    """OpenMP threads for later calls (n <= 0: all processors); returns the
    count in effect.  Changes only how long the oracle takes."""
    return int(_load().oracle_set_threads(int(n)))


def _bits16(a) -> np.ndarray:
    """bf16 tensor / uint16 array -> contiguous uint16 numpy array of bit patterns."""
    if hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch
        a = a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns (uint16), got %s" % a.dtype)
    return a


def _bits8(a) -> np.ndarray:
    if hasattr(a, "dtype") and str(a.dtype) == "torch.float8_e4m3fn":
        import torch
        a = a.detach().cpu().contiguous().view(torch.uint8).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError("expected e4m3fn codes (uint8), got %s" % a.dtype)
    return a


def _np(a, dtype):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def verify_attn(q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr, kv_indices,
                sm_scale, k_scale=1.0, v_scale=1.0, kv_fp8=None, select=None, lib=None,
                custom_mask=None, mask_indptr=None):
    """fp64 oracle output ``[rows, H_Q, Dv]`` (numpy float64).

    ``q [rows, H_Q, D]``, ``k_ext [rows, H_KV, D]``, ``v_ext [rows, H_KV, Dv]``
    are bf16 (torch tensors or uint16 bit arrays); ``k_buf [pool, H_KV, D]`` and
    ``v_buf [pool, H_KV, Dv]`` are bf16 or float8_e4m3fn (uint8 codes with
    ``kv_fp8=True``).  ``select`` is an optional list of (b, h) pairs; rows of
    other pairs come back as NaN.  ``custom_mask`` (bytes, nonzero = visible)
    with ``mask_indptr`` (int64, bs + 1) gives a tree mask over the draft keys:
    sequence b's mask is row-major ``[n_draft, n_b + n_draft]`` at
    ``mask_indptr[b]`` and only its draft columns are read.
    """
    lib = lib or _load()
    if kv_fp8 is None:
        kv_fp8 = hasattr(k_buf, "dtype") and str(k_buf.dtype) == "torch.float8_e4m3fn"
    qn, ken, ven = _bits16(q), _bits16(k_ext), _bits16(v_ext)
    if kv_fp8:
        kbn, vbn = _bits8(k_buf), _bits8(v_buf)
    else:
        kbn, vbn = _bits16(k_buf), _bits16(v_buf)
    qo = _np(qo_indptr, np.int32)
    kvp = _np(kv_indptr, np.int32)
    kvi = _np(kv_indices, np.int64)
    if kvi.size == 0:
        kvi = np.zeros(1, np.int64)
    rows, h_q, d = qn.shape
    h_kv = ken.shape[1]
    dv = ven.shape[2]
    bs = qo.shape[0] - 1
    out = np.full((rows, h_q, dv), np.nan, dtype=np.float64)
    if select:
        sel_b = np.ascontiguousarray([p[0] for p in select], dtype=np.int32)
        sel_h = np.ascontiguousarray([p[1] for p in select], dtype=np.int32)
        n_sel = len(select)
    else:
        sel_b = np.zeros(1, np.int32)
        sel_h = np.zeros(1, np.int32)
        n_sel = 0

    def ptr(a):
        return a.ctypes.data_as(ctypes.c_void_p)

    head = (
        bs, h_q, h_kv, d, dv, 1 if kv_fp8 else 0,
        ptr(qn), qn.strides[0] // qn.itemsize, qn.strides[1] // qn.itemsize,
        ptr(ken), ken.strides[0] // ken.itemsize, ken.strides[1] // ken.itemsize,
        ptr(ven), ven.strides[0] // ven.itemsize, ven.strides[1] // ven.itemsize,
        ptr(kbn), kbn.strides[0] // kbn.itemsize, kbn.strides[1] // kbn.itemsize,
        ptr(vbn), vbn.strides[0] // vbn.itemsize, vbn.strides[1] // vbn.itemsize,
        ptr(qo), ptr(kvp), ptr(kvi),
    )
    tail = (
        float(sm_scale), float(k_scale), float(v_scale),
        n_sel, ptr(sel_b), ptr(sel_h),
        ptr(out), out.strides[0] // 8, out.strides[1] // 8,
    )
    if custom_mask is None:
        rc = lib.oracle_verify_attn(*head, *tail)
    else:
        mk = _np(custom_mask, np.uint8)
        if mk.size == 0:
            mk = np.zeros(1, np.uint8)
        mi = _np(mask_indptr, np.int64)
        rc = lib.oracle_verify_attn_masked(*head, ptr(mk), ptr(mi), *tail)
    if rc != 0:
        raise RuntimeError("oracle_verify_attn failed (rc=%d)" % rc)
    return out


def append_kv(k, v, out_cache_loc, k_buf, v_buf, k_scale=1.0, v_scale=1.0, kv_fp8=None, lib=None):
    """Pool contents after the draft K/V append (copies; inputs untouched).

    ``k [n, H_KV, D]`` / ``v [n, H_KV, Dv]`` bf16; ``k_buf`` / ``v_buf`` bf16 or
    float8_e4m3fn pools.  Returns (k_bits, v_bits) as uint16 / uint8 arrays of
    the pool shape.
    """
    lib = lib or _load()
    if kv_fp8 is None:
        kv_fp8 = hasattr(k_buf, "dtype") and str(k_buf.dtype) == "torch.float8_e4m3fn"
    kn, vn = _bits16(k), _bits16(v)
    kb = (_bits8(k_buf) if kv_fp8 else _bits16(k_buf)).copy()
    vb = (_bits8(v_buf) if kv_fp8 else _bits16(v_buf)).copy()
    loc = _np(out_cache_loc, np.int64)
    if loc.size == 0:
        return kb, vb
    n, h_kv, d = kn.shape
    dv = vn.shape[2]

    def ptr(a):
        return a.ctypes.data_as(ctypes.c_void_p)

    lib.oracle_append_kv(
        n, h_kv, d, dv, 1 if kv_fp8 else 0,
        ptr(kn), kn.strides[0] // 2, kn.strides[1] // 2,
        ptr(vn), vn.strides[0] // 2, vn.strides[1] // 2,
        ptr(loc), float(k_scale), float(v_scale),
        ptr(kb), kb.strides[0] // kb.itemsize, kb.strides[1] // kb.itemsize,
        ptr(vb), vb.strides[0] // vb.itemsize, vb.strides[1] // vb.itemsize)
    return kb, vb


def build_kv_indices(req_to_token, req_pool_indices, seq_lens, kv_start_idx=None, lib=None):
    """(kv_indptr int32 [bs + 1], kv_indices int64 [sum seq_lens]) from the
    request-to-token table (int32 [rows, stride])."""
    lib = lib or _load()
    rt = _np(req_to_token, np.int32)
    rp = _np(req_pool_indices, np.int64)
    sl = _np(seq_lens, np.int32)
    st = None if kv_start_idx is None else _np(kv_start_idx, np.int32)
    bs = sl.shape[0]
    indptr = np.zeros(bs + 1, np.int32)
    indices = np.zeros(max(int(sl.sum()), 1), np.int64)

    def ptr(a):
        return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None

    lib.oracle_build_kv_indices(bs, ptr(rt), rt.strides[0] // 4, ptr(rp), ptr(sl), ptr(st),
                                ptr(indptr), ptr(indices))
    return indptr, indices[: int(sl.sum())]


def expand_block_table(block_table, kv_indptr, page_size):
    """Token rows of a page-table prefix: token t of sequence b lives in pool
    row block_table[b, t // page_size] * page_size + t % page_size (the
    unified-verify block table of aiter_backend.py, the pool viewed as
    [pages, page_size, H_KV, D]).  Returns int64 kv_indices over all prefix
    tokens in sequence order."""
    bt = _np(block_table, np.int64)
    kvp = _np(kv_indptr, np.int64)
    out = []
    for b in range(kvp.shape[0] - 1):
        t = np.arange(int(kvp[b + 1] - kvp[b]), dtype=np.int64)
        out.append(bt[b, t // page_size] * page_size + t % page_size)
    return np.concatenate(out) if out else np.zeros(0, np.int64)
