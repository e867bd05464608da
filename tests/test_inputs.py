"""The seeded input recipe: every draw repeats exactly for the same (workload, tag, sub),
differs between tags and subs, and has the shape, range and structure the workloads state
(lengths inside their segments, free lists that are permutations, fp8 pages whose codes
times their bf16 page scale give back the drawn N(0, 1) values to e4m3 precision)."""

import numpy as np
import torch

from workloads import gen
from workloads.configs import get_workload, scaled


def test_integer_draws_repeat_and_respect_their_ranges():
    for name in ("tiny_fp32", "gqa_bf16_16x4k-32k", "mla_fp8_48x100k", "mla_fp8_longmix_verify"):
        w = get_workload(name)
        a, b = gen.draw_seq_lens(w), gen.draw_seq_lens(w)
        assert np.array_equal(a, b) and len(a) == w.num_requests
        i = 0
        for count, lo, hi in w.seq_segments:
            assert ((a[i:i + count] >= lo) & (a[i:i + count] <= hi)).all()
            i += count
        f = gen.draw_free_order(w)
        assert np.array_equal(np.sort(f), np.arange(w.pool_pages)) and np.array_equal(f, gen.draw_free_order(w))
        s = gen.draw_src_order(w, 100)
        assert np.array_equal(np.sort(s), np.arange(100))
    w = get_workload("gqa_bf16_16x4k-32k")
    assert not np.array_equal(gen.draw_seq_lens(w), gen.draw_seq_lens(scaled(w, seed=w.seed + 1)))


def test_page_fills_repeat_per_tag_and_sub():
    w = scaled(get_workload("gqa_bf16_16x4k-32k"), page_size=4)
    pb = 2 * w.num_kv_heads * w.page_size * w.head_dim_qk * 2
    pages = [torch.empty((5, pb), dtype=torch.uint8) for _ in range(4)]
    gen.fill_pages_(pages[0], w, "pool", sub=1)
    gen.fill_pages_(pages[1], w, "pool", sub=1)
    gen.fill_pages_(pages[2], w, "pool", sub=2)
    gen.fill_pages_(pages[3], w, "src", sub=1)
    assert torch.equal(pages[0], pages[1])
    assert not torch.equal(pages[0], pages[2]) and not torch.equal(pages[0], pages[3])
    x = pages[0].view(torch.bfloat16).float()
    assert abs(float(x.mean())) < 0.05 and abs(float(x.std()) - 1.0) < 0.05


def test_fp8_pages_decode_to_the_drawn_values():
    w = scaled(get_workload("mla_fp8_48x100k"), page_size=64)
    pb = w.page_size * 576
    pages = torch.empty((6, pb), dtype=torch.uint8)
    scales = torch.empty((6,), dtype=torch.int16)
    gen.fill_pages_(pages, w, "pool", sub=0, scales=scales)
    # the same draw, regenerated: the generator is seeded per (workload, tag, sub)
    g = gen.torch_gen(w, "pool", "cpu", 0)
    x = torch.randn((6, pb), generator=g, dtype=torch.float32)
    s = scales.view(torch.bfloat16).float()
    assert (s > 0).all() and (scales != gen.SCALE_SENTINEL).all()
    assert torch.equal(s, (x.abs().amax(dim=1) / 448.0).to(torch.bfloat16).float())
    codes = pages.view(torch.float8_e4m3fn).float()
    assert codes.abs().max() <= 448.0 and torch.isfinite(codes).all()
    back = codes * s[:, None]
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 for normal codes, and an absolute
    # error of half the smallest subnormal step (2^-10 of the scale) below them
    err = (back - x).abs()
    assert (err <= x.abs() * 2.0 ** -4 + s[:, None] * 2.0 ** -10).all()


def test_queries_repeat_and_round_to_bf16():
    w = get_workload("gqa_bf16_16x4k-32k")
    a, b = gen.draw_q(w), gen.draw_q(w)
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)
    assert a.shape == (w.num_requests, w.q_len, w.num_q_heads, w.head_dim_qk)
