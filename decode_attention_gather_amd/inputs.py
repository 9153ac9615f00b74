"""Seeded synthetic inputs for MLA decode over a paged FP8 E4M3 cache.

This module holds no attention arithmetic: it only draws random numbers (torch CPU
generator), casts them to E4M3 with torch's own conversion, and lays out a paged cache
with a random block table. Both the HIP path and the fp64 oracle are fed from here.

Workload shapes follow TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA decode slower after
#19338" (Setup: latent 512 + rope 64, page size 32, FP8 E4M3 q and KV, 12 heads per
rank, q = 1 and q = 8, KV 128K and 1M, batch 1-16; Repro 1: softmax_scale 0.0722,
output_scale 1.0, uniform split_kv per shape). The pages benchmark on the module's own
random tensors, not on a dataset, so N(0, 1) values stand in for real activations.

Recipe (fixed order of draws from one ``torch.Generator`` seeded with ``seed``):
  1. per-request KV lengths, when drawn (mixed batches): ``randint(lo, hi + 1, (B,))``;
  2. q ~ N(0, 1) of shape [B, q_len, H, 576], clamped to +-448, cast to float8_e4m3fn;
  3. a random permutation of the ``sum_b ceil(L_b / 32)`` pages the requests use;
     request b takes the next ceil(L_b / 32) entries of it as its block table;
  4. the cache ~ N(0, 1), [num_pages, 32, 576], drawn page-chunk by page-chunk, clamped
     and cast the same way.
One extra page (the last one) is filled with the E4M3 NaN code 0x7F; unused block-table
entries point at it, and the slots of each request's last page past its length are set
to 0x7F too (NaN poisoning: a kernel that reads a byte it should not turns the result
into NaN instead of silently passing).

BF16 variant (``kv_dtype="bf16"``, the BF16 kernel the same issue compares against): the
same draws, cast to bfloat16 by torch (round to nearest even) instead of E4M3, stored as
int16 bit patterns (q [B, q_len, H, 576], cache [num_pages, 32, 576]); the poison is the
BF16 NaN 0x7FC0.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

D_QK = 576
D_V = 512
PAGE = 32
E4M3_NAN = 0x7F
BF16_NAN = 0x7FC0
SOFTMAX_SCALE = 0.0722
OUTPUT_SCALE = 1.0
_CHUNK_PAGES = 2048


@dataclasses.dataclass
class Case:
    """One decode batch; tensors live on the CPU (uint8 E4M3 codes or int16 BF16 bit
    patterns, int32 indices)."""
    q: torch.Tensor            # uint8 / int16 [B, q_len, H, 576]
    kv: torch.Tensor           # uint8 / int16 [num_pages, 32, 576]
    block_table: torch.Tensor  # int32 [B, max_pages]
    kv_lens: torch.Tensor      # int32 [B]
    q_len: int
    num_heads: int
    softmax_scale: float = SOFTMAX_SCALE
    output_scale: float = OUTPUT_SCALE
    split_kv: int = 0          # 0: the planner decides; >0 uniform split count
    name: str = ""
    kv_dtype: str = "e4m3"     # "e4m3" or "bf16" (q has the cache's type)

    @property
    def batch(self) -> int:
        return int(self.kv_lens.numel())

    @property
    def rows(self) -> int:
        return self.batch * self.q_len * self.num_heads

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def kv_bytes(self) -> int:
        """Bytes of KV the method must read: every visible token's row once (576 bytes
        in E4M3, 1152 in BF16)."""
        return int(self.kv_lens.to(torch.int64).sum().item()) * D_QK * self.elem_bytes

    @property
    def elem_bytes(self) -> int:
        return 2 if self.kv_dtype == "bf16" else 1


def to_e4m3_codes(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> uint8 OCP E4M3FN codes via torch's cast (round to nearest even)."""
    return x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def to_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> int16 BF16 bit patterns via torch's cast (round to nearest even)."""
    return x.to(torch.bfloat16).view(torch.int16)


def make_case(kv_lens: Sequence[int] | None, *, num_heads: int, q_len: int, seed: int,
              batch: int | None = None, len_range: tuple[int, int] | None = None,
              split_kv: int = 0, softmax_scale: float = SOFTMAX_SCALE,
              output_scale: float = OUTPUT_SCALE, poison: bool = True,
              name: str = "", kv_dtype: str = "e4m3") -> Case:
    """Build a seeded case. Give ``kv_lens`` explicitly, or ``batch`` and ``len_range``
    (inclusive) to draw them uniformly. ``kv_dtype``: "e4m3" or "bf16"."""
    assert kv_dtype in ("e4m3", "bf16")
    bf16 = kv_dtype == "bf16"
    cast = to_bf16_bits if bf16 else to_e4m3_codes
    nan_code = BF16_NAN if bf16 else E4M3_NAN
    g = torch.Generator().manual_seed(int(seed))
    if kv_lens is None:
        assert batch is not None and len_range is not None
        lo, hi = len_range
        lens = torch.randint(int(lo), int(hi) + 1, (int(batch),), generator=g,
                             dtype=torch.int64)
    else:
        lens = torch.as_tensor(list(kv_lens), dtype=torch.int64)
    B = int(lens.numel())
    assert B >= 1 and int(lens.min()) >= q_len >= 1

    q = cast(torch.randn(B, q_len, num_heads, D_QK, generator=g))

    npages = [(int(L) + PAGE - 1) // PAGE for L in lens.tolist()]
    used = sum(npages)
    perm = torch.randperm(used, generator=g).to(torch.int32)
    poison_page = used
    num_pages = used + 1
    max_pages = max(npages)
    bt = torch.full((B, max_pages), poison_page, dtype=torch.int32)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[off:off + n]
        off += n

    kv = torch.empty((num_pages, PAGE, D_QK), dtype=torch.int16 if bf16 else torch.uint8)
    for p0 in range(0, used, _CHUNK_PAGES):
        p1 = min(used, p0 + _CHUNK_PAGES)
        kv[p0:p1] = cast(torch.randn(p1 - p0, PAGE, D_QK, generator=g))
    kv[poison_page].fill_(nan_code)
    if poison:
        for b, L in enumerate(lens.tolist()):
            tail = L % PAGE
            if tail:
                kv[int(bt[b, npages[b] - 1]), tail:, :] = nan_code
    return Case(q=q, kv=kv, block_table=bt, kv_lens=lens.to(torch.int32), q_len=q_len,
                num_heads=num_heads, softmax_scale=softmax_scale,
                output_scale=output_scale, split_kv=split_kv, name=name, kv_dtype=kv_dtype)


# The five workloads (seed = 20260 + index), plus the H12 q1 B16 128K shape that the
# headline metric names (the q = 1 sibling of workload 3).
CONFIGS = {
    "c1_b1_h12_q1_2k": dict(kv_lens=[2048], num_heads=12, q_len=1, split_kv=4, seed=20261),
    "c2_b4_h12_q1_128k": dict(kv_lens=[131072] * 4, num_heads=12, q_len=1, split_kv=25,
                              seed=20262),
    "c3_b16_h12_q8_128k": dict(kv_lens=[131072] * 16, num_heads=12, q_len=8, split_kv=6,
                               seed=20263),
    "c4_b1_h12_q1_1m": dict(kv_lens=[1048576], num_heads=12, q_len=1, split_kv=100,
                            seed=20264),
    "c5_b8_h96_q8_mixed": dict(kv_lens=None, batch=8, len_range=(4096, 131072),
                               num_heads=96, q_len=8, split_kv=0, seed=20265),
    "m_b16_h12_q1_128k": dict(kv_lens=[131072] * 16, num_heads=12, q_len=1, split_kv=6,
                              seed=20266),
    # skewed batch: one 1M-token request beside seven short ones, H12 q8 (split planning
    # matters most here)
    "s_b8_h12_q8_skewed": dict(kv_lens=[1048576] + [4096] * 7, num_heads=12, q_len=8,
                               split_kv=0, seed=20267),
    # the BF16 cache beside the FP8 one: B1 1M at H12 q8 (the setting of the BF16 figure
    # the same issue quotes), and the headline H12 q1 B16 128K shape
    "b_b1_h12_q8_1m_bf16": dict(kv_lens=[1048576], num_heads=12, q_len=8, split_kv=0,
                                seed=20268, kv_dtype="bf16"),
    "b_b16_h12_q1_128k_bf16": dict(kv_lens=[131072] * 16, num_heads=12, q_len=1, split_kv=6,
                                   seed=20269, kv_dtype="bf16"),
    # 32 rows per request (16 heads, 2 causal query tokens): the two-row-tile narrow kernel
    # at the headline's KV size
    "t_b16_h16_q2_128k": dict(kv_lens=[131072] * 16, num_heads=16, q_len=2, split_kv=0,
                              seed=20270),
}


def make_config(name: str, **overrides) -> Case:
    kw = dict(CONFIGS[name])
    kw.update(overrides)
    lens = kw.pop("kv_lens")
    return make_case(lens, name=name, **kw)


def sample_rows(case: Case, count: int, seed: int = 7) -> List[int]:
    """A seeded sample of flat row ids, always including the first and the last row."""
    g = torch.Generator().manual_seed(seed)
    n = case.rows
    if count >= n:
        return list(range(n))
    picks = set([0, n - 1])
    extra = torch.randperm(n, generator=g)[: count].tolist()
    for r in extra:
        if len(picks) >= count:
            break
        picks.add(int(r))
    return sorted(picks)


def sample_rows_per_tile(case: Case, count: int, seed: int = 7) -> List[int]:
    """sample_rows(case, count) plus one seeded row from every 16-row tile of every
    request, so that every row block a kernel launch forms is checked."""
    g = torch.Generator().manual_seed(seed + 1)
    rows_per_req = case.q_len * case.num_heads
    picks = set(sample_rows(case, count, seed))
    for b in range(len(case.kv_lens)):
        for t0 in range(0, rows_per_req, 16):
            n = min(16, rows_per_req - t0)
            picks.add(b * rows_per_req + t0 + int(torch.randint(n, (1,), generator=g)))
    return sorted(picks)
