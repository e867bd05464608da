"""Workload shapes.

Each workload is named by what it is.  The shapes follow the deployment the
pages describe: 64-token pages and a 576-byte fp8 latent per token per layer
(512 latent + 64 rope) from "Serving Macaron-V1 at Scale: Page-Level 2D KV
Resharding", section 5.3 (Table 3 caption); 4K-32K and 500K-1M token
requests from sections 1 and 5.3 of the same page; 48 sessions with a
100K-token context each from "SGLang's path" (the DCP paragraph).

Size readings (the pages are silent): 2K/4K/32K/128K are binary
(4K = 4096 tokens), 100K/500K/1M are decimal (100K = 100000 tokens); uniform
ranges are integers drawn inclusive of both ends.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

MLA_LATENT = 512
MLA_ROPE = 64
MLA_DIM = MLA_LATENT + MLA_ROPE  # 576 bytes of fp8 per token per layer


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    # request lengths: tuple of segments (count, lo, hi); lo == hi is a fixed length
    seq_segments: Tuple[Tuple[int, int, int], ...]
    page_size: int
    dcp_size: int            # N: DCP shards (page pools on one GPU)
    pool_pages: int          # M: local page slots per DCP pool per layer
    kv_dtype: str            # "f32" | "bf16" | "fp8"
    layout: str              # "split" ([K,V][Hkv][page][D]) | "mla" ([page][576] fp8)
    num_layers: int          # L: layers in each DCP pool
    num_q_heads: int = 0     # 0: no attention in this workload
    num_kv_heads: int = 1
    head_dim_qk: int = 0
    head_dim_v: int = 0
    q_len: int = 1
    q_dtype: str = "f32"     # "f32" | "bf16"
    # layer-split sources feeding the reshard (0: no reshard)
    num_sources: int = 0
    cached_frac: float = 0.0           # leading fraction of pages that are prefix-cached
    reshard_min_len: int = 0           # only requests with T >= this are resharded
    attn_layer: int = 0                # layer the decode attention runs on
    notes: str = ""

    # --- derived sizes -------------------------------------------------
    @property
    def num_requests(self) -> int:
        return sum(c for c, _, _ in self.seq_segments)

    @property
    def has_attention(self) -> bool:
        return self.num_q_heads > 0

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.kv_dtype]

    @property
    def page_bytes(self) -> int:
        if self.layout == "mla":
            return self.page_size * MLA_DIM
        return 2 * self.num_kv_heads * self.page_size * self.head_dim_qk * self.elem_bytes

    @property
    def has_scales(self) -> bool:
        return self.kv_dtype == "fp8"

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim_qk)

    def pages_for(self, tokens: int) -> int:
        return -(-tokens // self.page_size)


WORKLOADS = {
    # 1 request, 1 layer, 8 query heads / 1 KV head, head_dim 64, page 16,
    # 1000 tokens (63 pages, the last holding 8 tokens), N = 2, fp32.
    "tiny_fp32": Workload(
        name="tiny_fp32", seed=1001, seq_segments=((1, 1000, 1000),),
        page_size=16, dcp_size=2, pool_pages=64, kv_dtype="f32", layout="split",
        num_layers=1, num_q_heads=8, num_kv_heads=1, head_dim_qk=64, head_dim_v=64,
        q_len=1, q_dtype="f32", num_sources=1,
        notes="reshard from 1 layer-split source holding the 1 layer"),
    # GQA bf16 decode: 16 requests of U[4096, 32768] tokens, 32 q / 8 kv heads,
    # head_dim 128, page 64, N = 4, 2048 slots per pool, permuted free list.
    "gqa_bf16_16x4k-32k": Workload(
        name="gqa_bf16_16x4k-32k", seed=1002, seq_segments=((16, 4096, 32768),),
        page_size=64, dcp_size=4, pool_pages=2048, kv_dtype="bf16", layout="split",
        num_layers=1, num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
        q_len=1, q_dtype="bf16", num_sources=1,
        notes="the full path per step: reshard from one layer-split source, partial, merge"),
    # Page-level reshard only: 4 layer-split sources x 16 of 64 layers, one
    # 131072-token request (2048 pages), first 40% of pages prefix-cached,
    # fp8 latent pages of 36864 B, N = 8 destination pools of 512 slots.
    "reshard_mla_128k": Workload(
        name="reshard_mla_128k", seed=1003, seq_segments=((1, 131072, 131072),),
        page_size=64, dcp_size=8, pool_pages=512, kv_dtype="fp8", layout="mla",
        num_layers=64, num_sources=4, cached_frac=0.4),
    # MLA-style fp8 decode: 48 sessions x 100000 tokens, 128 q heads sharing
    # one latent KV, e4m3 with a bf16 scale per (layer, page), N = 8.
    "mla_fp8_48x100k": Workload(
        name="mla_fp8_48x100k", seed=1004, seq_segments=((48, 100000, 100000),),
        page_size=64, dcp_size=8, pool_pages=16384, kv_dtype="fp8", layout="mla",
        num_layers=1, num_q_heads=128, num_kv_heads=1, head_dim_qk=MLA_DIM,
        head_dim_v=MLA_LATENT, q_len=1, q_dtype="bf16"),
    # Long-context mix with speculative verify: 8 x U[500000, 1000000] + 40 x 2048,
    # q_len 4 causal drafts, 4 layers, the long requests resharded from 4
    # layer-split sources (one layer each), nothing cached.
    "mla_fp8_longmix_verify": Workload(
        name="mla_fp8_longmix_verify", seed=1005,
        seq_segments=((8, 500000, 1000000), (40, 2048, 2048)),
        page_size=64, dcp_size=8, pool_pages=32768, kv_dtype="fp8", layout="mla",
        num_layers=4, num_q_heads=128, num_kv_heads=1, head_dim_qk=MLA_DIM,
        head_dim_v=MLA_LATENT, q_len=4, q_dtype="bf16", num_sources=4,
        reshard_min_len=500000),
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def scaled(w: Workload, **overrides) -> Workload:
    """A copy of a workload with some fields replaced (small parity cases)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(overrides)
    return Workload(**d)
