"""Seeded synthetic inputs for target-verify attention.

This module only *generates inputs*; it holds none of the attention
arithmetic.  Both the fp64 oracle (through the tests) and the HIP path read
the tensors it returns, so the two sides always see identical bits.

Shapes follow the problem statement in sglang's ``verify_splitkv.py``
(``_verify_prefix_stage1`` argument comments) and the builder in
``test_verify_splitkv.py`` (``_build_verify_inputs``):

* ``q``     ``[B*l_ext, H_Q, D]``  bf16, draft queries;
* ``k_ext`` ``[B*l_ext, H_KV, D]`` bf16, draft keys; ``v_ext`` likewise with Dv;
* ``k_buf`` ``[pool, H_KV, D]``   bf16 or float8_e4m3fn, paged prefix pool;
  ``v_buf`` likewise with Dv;
* ``qo_indptr`` ``arange(0, (B+1)*l_ext, l_ext)`` int32 (constant extend
  length, as at topk = 1);
* ``kv_indptr`` ``[B+1]`` int32 cumulative prefix lengths;
* ``kv_indices`` ``[sum n_b]`` int64 pool row per prefix token (page size 1).

Value distributions: N(0, 1) for every bf16 tensor.  For an fp8 pool the pool
is drawn N(0, 1) in fp32 and stored as ``x / scale`` in E4M3FN with the
per-tensor ``scale = absmax / 448`` (the scale is then the dequant multiplier
the kernel receives as ``k_scale`` / ``v_scale``).  Scattered pools hold twice
the needed rows and ``kv_indices`` is the first ``sum n_b`` entries of a seeded
random permutation of the pool rows (distinct single-token pages).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

FP8_E4M3_MAX = 448.0


@dataclasses.dataclass
class Problem:
    name: str
    q: torch.Tensor
    k_ext: torch.Tensor
    v_ext: torch.Tensor
    k_buf: torch.Tensor
    v_buf: torch.Tensor
    qo_indptr: torch.Tensor
    kv_indptr: torch.Tensor
    kv_indices: torch.Tensor
    l_ext: int
    sm_scale: float
    k_scale: float
    v_scale: float
    prefix_lens: List[int]

    @property
    def bs(self) -> int:
        return len(self.prefix_lens)

    @property
    def h_q(self) -> int:
        return self.q.shape[1]

    @property
    def h_kv(self) -> int:
        return self.k_ext.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q.shape[2]

    @property
    def v_head_dim(self) -> int:
        return self.v_ext.shape[2]

    @property
    def kv_fp8(self) -> bool:
        return self.k_buf.dtype == torch.float8_e4m3fn

    @property
    def total_prefix(self) -> int:
        return int(sum(self.prefix_lens))

    def kv_bytes(self) -> int:
        """Bytes of pool K and V rows the prefix pass must read once."""
        e = self.k_buf.element_size()
        return self.total_prefix * self.h_kv * (self.head_dim + self.v_head_dim) * e

    def to(self, device) -> "Problem":
        f = {}
        for fld in dataclasses.fields(self):
            v = getattr(self, fld.name)
            f[fld.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Problem(**f)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_problem(prefix_lens, l_ext, h_q, h_kv, head_dim, v_head_dim=None, *,
                 kv_dtype=torch.bfloat16, k_scale=1.0, v_scale=1.0,
                 pool_factor: Optional[int] = None, permute=False,
                 seed=0, device="cpu", sm_scale=None, name="custom") -> Problem:
    """Build one seeded verify problem.

    ``pool_factor=None`` gives a pool of exactly ``sum n_b`` rows with
    ``kv_indices = arange`` (the test-builder layout); ``pool_factor=k`` gives
    ``k * sum n_b`` rows.  ``permute=True`` draws ``kv_indices`` from a seeded
    random permutation of the pool rows.  For ``kv_dtype=float8_e4m3fn`` the
    ``k_scale``/``v_scale`` arguments are ignored and replaced by the
    per-tensor absmax/448 scales of the generated pool.
    """
    if v_head_dim is None:
        v_head_dim = head_dim
    prefix_lens = [int(n) for n in prefix_lens]
    bs = len(prefix_lens)
    total = sum(prefix_lens)
    pool = total if pool_factor is None else max(1, int(pool_factor) * total)
    pool = max(pool, 1)
    g = _gen(device, seed)
    n_ext = bs * l_ext
    bf = torch.bfloat16

    q = torch.randn(n_ext, h_q, head_dim, generator=g, device=device, dtype=torch.float32).to(bf)
    k_ext = torch.randn(n_ext, h_kv, head_dim, generator=g, device=device, dtype=torch.float32).to(bf)
    v_ext = torch.randn(n_ext, h_kv, v_head_dim, generator=g, device=device, dtype=torch.float32).to(bf)

    if kv_dtype == torch.float8_e4m3fn:
        kf = torch.randn(pool, h_kv, head_dim, generator=g, device=device, dtype=torch.float32)
        vf = torch.randn(pool, h_kv, v_head_dim, generator=g, device=device, dtype=torch.float32)
        k_scale = float(kf.abs().max()) / FP8_E4M3_MAX
        v_scale = float(vf.abs().max()) / FP8_E4M3_MAX
        k_buf = (kf / k_scale).clamp_(-FP8_E4M3_MAX, FP8_E4M3_MAX).to(torch.float8_e4m3fn)
        v_buf = (vf / v_scale).clamp_(-FP8_E4M3_MAX, FP8_E4M3_MAX).to(torch.float8_e4m3fn)
        del kf, vf
    elif kv_dtype == bf:
        k_buf = torch.randn(pool, h_kv, head_dim, generator=g, device=device, dtype=torch.float32).to(bf)
        v_buf = torch.randn(pool, h_kv, v_head_dim, generator=g, device=device, dtype=torch.float32).to(bf)
    else:
        raise ValueError("unsupported pool dtype %s" % kv_dtype)

    if permute:
        kv_indices = torch.randperm(pool, generator=g, device=device)[:total].to(torch.int64)
    else:
        kv_indices = torch.arange(total, dtype=torch.int64, device=device)
    lens = torch.tensor(prefix_lens, dtype=torch.int64)
    kv_indptr = torch.zeros(bs + 1, dtype=torch.int64)
    kv_indptr[1:] = torch.cumsum(lens, 0)
    kv_indptr = kv_indptr.to(torch.int32).to(device)
    qo_indptr = torch.arange(0, n_ext + 1, l_ext, dtype=torch.int32, device=device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    return Problem(name, q, k_ext, v_ext, k_buf, v_buf, qo_indptr, kv_indptr,
                   kv_indices, int(l_ext), float(sm_scale), float(k_scale),
                   float(v_scale), prefix_lens)


def make_paged_block_table(prefix_lens, page_size, pages, seed=0, device="cpu"):
    """Seeded page table for a pool of ``pages`` pages of ``page_size`` token
    rows: int32 [bs, max_pages], each sequence drawing distinct random page
    ids for its ceil(n_b / page_size) pages (unused entries 0).  A generator
    only: which pool row a token lands in is left to the code under test."""
    prefix_lens = [int(n) for n in prefix_lens]
    need = [(n + page_size - 1) // page_size for n in prefix_lens]
    if sum(need) > pages:
        raise ValueError("pool of %d pages too small for %d" % (pages, sum(need)))
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(pages, generator=g)
    width = max(1, max(need))
    table = torch.zeros(len(prefix_lens), width, dtype=torch.int32)
    pos = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[pos:pos + k].to(torch.int32)
        pos += k
    return table.to(device)


# The five workloads the path is specified on.  "tiny" finishes in the oracle
# in milliseconds; "b8_8k" is the headline throughput workload.
def config_tiny(device="cpu", seed=1):
    return make_problem([64], 2, 2, 1, 64, 64, seed=seed, device=device, name="tiny")


def config_b3_512(device="cpu", seed=2):
    return make_problem([512, 512, 512], 4, 16, 2, 256, 256, seed=seed,
                        device=device, name="b3_512")


def config_b8_8k(device="cpu", seed=3):
    return make_problem([8192] * 8, 4, 16, 2, 256, 256, k_scale=0.5, v_scale=0.25,
                        pool_factor=2, permute=True, seed=seed, device=device,
                        name="b8_8k")


def fp8_prefix_lens(seed=4, bs=16, lo=1024, hi=16384) -> List[int]:
    """Per-sequence prefix lengths uniform on [lo, hi] inclusive, seeded."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 1000)
    return [int(x) for x in torch.randint(lo, hi + 1, (bs,), generator=g)]


def config_fp8_ragged(device="cpu", seed=4, permute=False):
    return make_problem(fp8_prefix_lens(seed), 8, 8, 1, 128, 128,
                        kv_dtype=torch.float8_e4m3fn, permute=permute,
                        pool_factor=2 if permute else None, seed=seed,
                        device=device, name="fp8_ragged")


def config_b4_64k(device="cpu", seed=5):
    return make_problem([65536] * 4, 8, 32, 8, 256, 256, pool_factor=2, permute=True,
                        seed=seed, device=device, name="b4_64k")


# Reuse of the same entry point for other modes with a fixed extend length
# per request: plain decode (l_ext = 1) of a 64- and a 512-sequence batch, and
# the draft model's
# DRAFT_EXTEND_V2 step (num_draft_tokens new tokens per request over the
# draft-side prefix); both with the headline attention geometry (16/2 heads,
# D = 256, scattered pool) and seeded ragged prefixes.
def config_decode_b64(device="cpu", seed=6):
    return make_problem(fp8_prefix_lens(seed, bs=64, lo=2048, hi=6144), 1, 16, 2, 256, 256,
                        pool_factor=2, permute=True, seed=seed, device=device, name="decode_b64")


def config_decode_b512(device="cpu", seed=8):
    return make_problem(fp8_prefix_lens(seed, bs=512, lo=1024, hi=4096), 1, 16, 2, 256, 256,
                        pool_factor=2, permute=True, seed=seed, device=device, name="decode_b512")


def config_draft_extend_b16(device="cpu", seed=7):
    return make_problem(fp8_prefix_lens(seed, bs=16, lo=1024, hi=8192), 4, 16, 2, 256, 256,
                        pool_factor=2, permute=True, seed=seed, device=device,
                        name="draft_extend_b16")


CONFIGS = {
    "tiny": config_tiny,
    "b3_512": config_b3_512,
    "b8_8k": config_b8_8k,
    "fp8_ragged": config_fp8_ragged,
    "b4_64k": config_b4_64k,
    "decode_b64": config_decode_b64,
    "decode_b512": config_decode_b512,
    "draft_extend_b16": config_draft_extend_b16,
}
