"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times.  The reshard is checked completely and bit for bit against the
oracle's copy plan; attention element by element against the oracle on every
request: all heads of the GQA batch, sixteen seeded heads per request of the
128-head MLA workloads, every shard's partial and the merge, all draft
positions.  The oracle runs per request in worker processes."""

import numpy as np
import pytest
import torch

import context_paged_kv_amd as K
from tests import harness as H
from workloads.configs import get_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_full_reshard_mla_128k():
    w = get_workload("reshard_mla_128k")
    H.log("full reshard: 4 sources x 16 of 64 layers, 2048 pages, 40% cached, N=8")
    rc = H.make_reshard_case(w, DEV)
    assert rc.first_uncached == 819
    chk = [t.view(torch.int64).sum().item() for t in rc.src_pools]
    H.run_reshard(rc)
    torch.cuda.synchronize()
    n_copies = H.check_reshard_by_plan(rc)
    assert n_copies == 64 * (2048 - 819)
    assert chk == [t.view(torch.int64).sum().item() for t in rc.src_pools]  # sources untouched
    H.log(f"  {n_copies} page copies verified")


def test_full_gqa_reshard_16_requests():
    """The transfer the default bench times: every page of the 16 requests (4K-32K tokens, bf16
    GQA pages of 256 KiB) from the source into the N = 4 pools, bit for bit against the
    oracle's copy plan."""
    w = get_workload("gqa_bf16_16x4k-32k")
    H.log("full reshard: gqa bf16 16 x U[4K,32K], 256 KiB pages, N=4")
    sl = np.asarray(H.gen.draw_seq_lens(w))
    rc = H.make_reshard_case(w, DEV, seq_lens=sl, first_uncached=0)
    H.run_reshard(rc)
    torch.cuda.synchronize()
    n_copies = H.check_reshard_by_plan(rc)
    assert n_copies == len(rc.dst_ids)
    H.log(f"  {n_copies} page copies verified")


def seeded_heads(w, b, layer=0, count=16):
    """The query heads checked for request b: all of them up to `count`, else a seeded subset."""
    if w.num_q_heads <= count:
        return list(range(w.num_q_heads))
    rng = np.random.default_rng([w.seed, 77, layer, b])
    return sorted(int(h) for h in rng.choice(w.num_q_heads, size=count, replace=False))


@pytest.mark.timeout(600)
def test_full_gqa_bf16_16x4k_32k():
    w = get_workload("gqa_bf16_16x4k-32k")
    H.log("full decode: gqa bf16 16 x U[4K,32K], N=4: all 16 requests x 32 heads")
    case = H.make_decode_case(w, DEV)
    outs = H.run_decode(case)
    torch.cuda.synchronize()
    assert torch.isfinite(outs.out).all()
    worst = H.check_decode_parallel(case, outs, lambda b: range(w.num_q_heads))
    H.log("  " + H.fmt_worst(worst))


@pytest.mark.timeout(900)
def test_full_mla_fp8_48x100k():
    w = get_workload("mla_fp8_48x100k")
    H.log("full decode: mla fp8 48 x 100000, Hq=128, N=8: all 48 requests x 16 seeded heads")
    case = H.make_decode_case(w, DEV)
    outs = H.run_decode(case)
    torch.cuda.synchronize()
    assert torch.isfinite(outs.out).all()
    worst = H.check_decode_parallel(case, outs, lambda b: seeded_heads(w, b))
    H.log("  " + H.fmt_worst(worst))


def test_full_gqa_token_ownership_reshard_then_decode():
    """The token-ownership step the bench times: all 16 requests scattered from the source in one
    launch (offsets per request), then decode under token ownership; sampled rows of every shard
    and the merged output against the oracle's attention over the source pages."""
    w = get_workload("gqa_bf16_16x4k-32k")
    H.log("full token ownership: gqa bf16 16 x U[4K,32K], N=4, token reshard then decode")
    sl = np.asarray(H.gen.draw_seq_lens(w))
    case = H.make_decode_case(w, DEV, seq_lens=sl, own=K.OWN_TOKEN)
    rc = H.make_reshard_case(w, DEV, seq_lens=sl, first_uncached=0, dst_pools=case.pools, dst_scales=case.scales)
    offs = np.cumsum([0] + [len(p) for p in case.pages])
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.run_reshard_tokens(rc, bad=bad, request_offsets=offs)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    outs = H.run_decode(case)
    torch.cuda.synchronize()
    assert torch.isfinite(outs.out).all()

    def source_pages(b):  # the request's pages as the prefill side holds them, in sequence order
        sids = torch.from_numpy(rc.src_ids[offs[b]:offs[b + 1]]).to(DEV)
        return rc.src_pools[0][0].index_select(0, sids).cpu().numpy(), None

    worst = H.check_decode_parallel(case, outs, lambda b: range(w.num_q_heads), pages_of=source_pages)
    H.log("  all 16 requests x 32 heads match: " + H.fmt_worst(worst))


@pytest.mark.timeout(900)
def test_full_mla_fp8_48x100k_token_ownership():
    """The 48 x 100000 MLA decode under token ownership (token t on shard t mod N), as the bench
    times it with --own token; every request's 16 seeded heads, every shard and the merge."""
    w = get_workload("mla_fp8_48x100k")
    H.log("full decode, token ownership: mla fp8 48 x 100000, Hq=128, N=8: 48 requests x 16 seeded heads")
    case = H.make_decode_case(w, DEV, own=K.OWN_TOKEN)
    outs = H.run_decode(case)
    torch.cuda.synchronize()
    assert torch.isfinite(outs.out).all()
    worst = H.check_decode_parallel(case, outs, lambda b: seeded_heads(w, b, layer=1))
    H.log("  " + H.fmt_worst(worst))


@pytest.mark.timeout(1200)
def test_full_longmix_verify_pipeline():
    """Reshard of the long requests from 4 layer-split sources, then q_len 4
    causal verify attention on every layer, each layer's all 48 requests x 16
    seeded heads against the oracle computed from the inputs (source pages for
    long requests, pool pages for the short ones)."""
    w = get_workload("mla_fp8_longmix_verify")
    H.log("full pipeline: 8 x U[500K,1M] + 40 x 2048, q_len 4, 4 layers, N=8")
    sl = np.asarray(H.gen.draw_seq_lens(w))
    long_ids = [b for b in range(len(sl)) if sl[b] >= w.reshard_min_len]
    pools, scales = H.alloc_pools(w, DEV)  # random pages: what the short requests hold
    rc = H.make_reshard_case(w, DEV, seq_lens=sl, requests=long_ids, first_uncached=0, dst_pools=pools,
                             dst_scales=scales)
    H.run_reshard(rc)
    torch.cuda.synchronize()
    case = H.make_decode_case(w, DEV, seq_lens=sl, pools=pools, scales=scales)
    # logical KV of a long request comes from the SOURCE pages (the reshard's inputs), of a short
    # one from the pools (never overwritten)
    offs = {}
    off = 0
    for b in long_ids:
        offs[b] = off
        off += len(case.pages[b])
    for layer in range(w.num_layers):
        outs = H.run_decode(case, layer=layer)
        torch.cuda.synchronize()
        assert torch.isfinite(outs.out).all()
        r, first = next((r, a) for r in range(w.num_sources)
                        for a, bb in [H.K.cp_layersplit_layer_range(w.num_layers, w.num_sources, r)]
                        if a <= layer < bb)

        def pages_of(b, layer=layer, r=r, first=first):
            if b not in offs:
                return H.gather_request_pages(case.pools, case.scales, case.pages[b], w.dcp_size, layer)
            sids = torch.from_numpy(rc.src_ids[offs[b]:offs[b] + len(case.pages[b])]).to(DEV)
            pb = rc.src_pools[r][layer - first].index_select(0, sids).cpu().numpy()
            ps = rc.src_scales[r][layer - first].index_select(0, sids).cpu().numpy().astype(np.int64) & 0xFFFF
            return pb, ps

        # the long requests first (the slowest oracle tasks), at most 8 workers (each holds a
        # float64 copy of up to 1M x 576 latents)
        order = long_ids + [b for b in range(len(sl)) if b not in offs]
        worst = H.check_decode_parallel(case, outs, lambda b: seeded_heads(w, b, layer=layer), requests=order,
                                        layer=layer, pages_of=pages_of, workers=8, label=f"L{layer} ")
        H.log(f"  layer {layer}: all 48 requests x 16 heads match: " + H.fmt_worst(worst))


def test_full_path_pack_unpack_mla_128k():
    """The full 128K reshard done path by path through a 256-page (9 MiB) staging buffer, checked
    bit for bit against the oracle's copy plan like the direct reshard."""
    w = get_workload("reshard_mla_128k")
    H.log("full path pack/unpack: 4 sources x 16 of 64 layers, 2048 pages, 40% cached, N=8, 256-page windows")
    rc = H.make_reshard_case(w, DEV)
    chk = [t.view(torch.int64).sum().item() for t in rc.src_pools]
    moved = H.run_path_pack(rc, 256)
    torch.cuda.synchronize()
    assert moved == 64 * (2048 - 819)
    assert H.check_reshard_by_plan(rc) == 64 * (2048 - 819)
    assert chk == [t.view(torch.int64).sum().item() for t in rc.src_pools]
    H.log(f"  {moved} units verified")
