"""dcp_decode_partial_noalloc (the entry point for callers that cannot allocate device memory)
against dcp_decode_partial on the same inputs, through the C ABI: two calls in a row, the second
with a smaller input, so the second runs on what the first left in the library's scratch."""

import numpy as np
import pytest
import torch

import context_paged_kv_amd as K
from tests import harness as H
from workloads.configs import get_workload, scaled

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(case):
    """The workspace entry point's outputs, then the no-alloc entry point's into fresh buffers."""
    ref = H.run_decode(case, merge=False)
    got, _ = H.alloc_outputs(case)
    K.dcp_decode_partial_noalloc(H.attn_desc(case), q=case.q, kv_pools=case.pools, kv_scales=case.scales,
                                 block_tables=case.bt_dev, seq_lens=case.sl_dev, total_tokens=case.total_tokens,
                                 partial_out=got.partial_out, partial_lse=got.partial_lse)
    torch.cuda.synchronize()
    return ref, got


def _compare(case, ref, got, exact):
    w = case.w
    if exact:  # the same plan and kernels: the same bits
        assert torch.equal(got.partial_out, ref.partial_out) and torch.equal(got.partial_lse, ref.partial_lse)
        return
    tol_o, tol_l = H.tolerance(w)
    po_r, pl_r = ref.partial_out.double().cpu().numpy(), ref.partial_lse.double().cpu().numpy()
    po_g, pl_g = got.partial_out.cpu().numpy(), got.partial_lse.cpu().numpy()
    for d in range(w.dcp_size):
        for b in range(w.num_requests):
            H.check_rows(f"no-alloc vs workspace d={d} b={b}", po_g[d, b], pl_g[d, b], po_r[d, b], pl_r[d, b],
                         tol_o, tol_l)


def test_noalloc_matches_the_workspace_entry_point_twice():
    # first call: fp8 MLA verify (512 query rows per request): the split the planner wants holds
    # more chunk partials than the scratch, so the no-alloc call runs a coarser split
    base = get_workload("mla_fp8_longmix_verify")
    w1 = scaled(base, seed=base.seed + 700, seq_segments=((3, 8000, 9000), (2, 2048, 2048)), pool_pages=512,
                num_layers=1, attn_layer=0)
    c1 = H.make_decode_case(w1, DEV)
    desc1 = H.attn_desc(c1)
    assert K.dcp_decode_partial_workspace(desc1, c1.total_tokens) > K.NOALLOC_SCRATCH_BYTES
    H.log("no-alloc call 1: mla fp8 q_len 4, 5 requests, 128 heads, N=8 (coarser split)")
    ref1, got1 = _both(c1)
    _compare(c1, ref1, got1, exact=False)
    worst = H.check_decode(c1, H.DecodeOut(got1.partial_out, got1.partial_lse, got1.out, got1.lse),
                           requests=[0, 4], heads=[0, 63, 127], shards=list(range(w1.dcp_size)))
    H.log("  vs oracle: " + H.fmt_worst(worst))
    # second call, smaller: bf16 GQA; its whole split fits the scratch, so the plan and the bits
    # are those of the workspace call
    gb = get_workload("gqa_bf16_16x4k-32k")
    w2 = scaled(gb, seed=gb.seed + 700, seq_segments=((3, 70, 3000),), pool_pages=128)
    c2 = H.make_decode_case(w2, DEV)
    assert K.dcp_decode_partial_workspace(H.attn_desc(c2), c2.total_tokens) <= K.NOALLOC_SCRATCH_BYTES
    H.log("no-alloc call 2: gqa bf16, 3 requests, N=4 (same plan as the workspace call)")
    ref2, got2 = _both(c2)
    _compare(c2, ref2, got2, exact=True)


def test_noalloc_rejects_a_plan_beyond_its_scratch():
    """Far more (shard, request) pairs than the scratch can plan for: EINVAL before anything runs."""
    base = get_workload("gqa_bf16_16x4k-32k")
    w = scaled(base, seed=base.seed + 701, seq_segments=((2, 100, 200),), pool_pages=64)
    c = H.make_decode_case(w, DEV)
    outs, _ = H.alloc_outputs(c)
    big = H.attn_desc(c)
    big.batch = 1 << 21  # 2^21 requests x 4 shards: 8M pair plans of 16 bytes > 64 MiB
    with pytest.raises(K.DcpkvError) as e:
        K.dcp_decode_partial_noalloc(big, q=c.q, kv_pools=c.pools, kv_scales=c.scales, block_tables=c.bt_dev,
                                     seq_lens=c.sl_dev, total_tokens=0, partial_out=outs.partial_out,
                                     partial_lse=outs.partial_lse)
    assert e.value.code == K.DCPKV_EINVAL and "scratch" in str(e.value)
