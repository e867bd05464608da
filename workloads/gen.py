"""Seeded input draws.

Recipe (stated once here and in the design notes):
  * integer draws (request lengths, free-list order, source page order) come
    from numpy's PCG64 seeded with SeedSequence([workload.seed, tag]);
  * bulk values come from a torch.Generator on the device that will hold them,
    seeded from the same SeedSequence, drawn in fixed chunks of pages;
  * q, k, v and the latent are N(0, 1) in float32, then rounded
    to-nearest-even to the workload dtype;
  * fp8 pages: one bf16 scale per (layer, page) s = bf16(max|x| / 448)
    (1 if the page is all zero), codes = e4m3fn(clamp(x / s, +-448)).
    This quantiser exists only to make inputs; the method reads codes and
    scales as given.

Nothing here computes a step of the method.
"""

from __future__ import annotations

import numpy as np
import torch

from .configs import MLA_DIM, Workload

_TAGS = {"seq_lens": 1, "free": 2, "src_order": 3, "q": 4, "kv": 5, "pool": 6, "misc": 7, "src": 8}
FILL_CHUNK_PAGES = 2048


def np_rng(w: Workload, tag: str, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, _TAGS[tag], sub])))


def torch_gen(w: Workload, tag: str, device, sub: int = 0) -> torch.Generator:
    seed = int(np_rng(w, tag, sub).integers(0, 2**62))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw_seq_lens(w: Workload) -> np.ndarray:
    r = np_rng(w, "seq_lens")
    out = []
    for count, lo, hi in w.seq_segments:
        if lo == hi:
            out.extend([lo] * count)
        else:
            out.extend(int(x) for x in r.integers(lo, hi + 1, size=count))
    return np.asarray(out, dtype=np.int64)


def draw_free_order(w: Workload) -> np.ndarray:
    """A permutation of the virtual page ids [0, pool_pages): the free list."""
    return np_rng(w, "free").permutation(w.pool_pages).astype(np.int64)


def draw_src_order(w: Workload, n: int) -> np.ndarray:
    """A permutation of [0, n): where the prefill side keeps each page."""
    return np_rng(w, "src_order").permutation(n).astype(np.int64)


def draw_q(w: Workload, device="cpu") -> torch.Tensor:
    g = torch_gen(w, "q", device)
    q = torch.randn((w.num_requests, w.q_len, w.num_q_heads, w.head_dim_qk),
                    generator=g, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16) if w.q_dtype == "bf16" else q


def _fill_chunk(pages: torch.Tensor, scales: torch.Tensor | None, w: Workload, g: torch.Generator):
    n, page_bytes = pages.shape
    dev = pages.device
    if w.kv_dtype == "f32":
        x = torch.randn((n, page_bytes // 4), generator=g, device=dev, dtype=torch.float32)
        pages.copy_(x.view(torch.uint8).view(n, page_bytes))
    elif w.kv_dtype == "bf16":
        x = torch.randn((n, page_bytes // 2), generator=g, device=dev, dtype=torch.float32)
        pages.copy_(x.to(torch.bfloat16).view(torch.uint8).view(n, page_bytes))
    elif w.kv_dtype == "fp8":
        x = torch.randn((n, page_bytes), generator=g, device=dev, dtype=torch.float32)
        amax = x.abs().amax(dim=1)
        s = (amax / 448.0).to(torch.bfloat16)
        s = torch.where(s == 0, torch.ones_like(s), s)
        codes = (x / s.float()[:, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        pages.copy_(codes.view(torch.uint8))
        if scales is not None:
            scales.copy_(s.view(torch.int16))
    else:
        raise ValueError(w.kv_dtype)


def fill_pages_(pages: torch.Tensor, w: Workload, tag: str, sub: int = 0,
                scales: torch.Tensor | None = None) -> None:
    """Fill a [n, page_bytes] uint8 tensor with random page contents.

    For fp8 workloads ``scales`` (int16 bit patterns of bf16, shape [n]) receives
    the per-page scales.  Draws go in fixed chunks so a result depends only on
    (workload, tag, sub, n, device type).
    """
    assert pages.dtype == torch.uint8 and pages.dim() == 2
    n = pages.shape[0]
    g = torch_gen(w, tag, pages.device, sub)
    for a in range(0, n, FILL_CHUNK_PAGES):
        b = min(n, a + FILL_CHUNK_PAGES)
        _fill_chunk(pages[a:b], None if scales is None else scales[a:b], w, g)


def sentinel_fill_(t: torch.Tensor, byte: int) -> None:
    """Fill with one byte value (a recognisable pattern for untouched memory)."""
    t.view(torch.uint8).fill_(byte)


SRC_TRANSIENT_SENTINEL = 0x5A
DST_SENTINEL = 0xA5
SCALE_SENTINEL = 0x7F7F  # a bf16 bit pattern (about 3.39e38), never a drawn scale


def latent_dim() -> int:
    return MLA_DIM
