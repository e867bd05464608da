"""GPU parity of the HIP path against the float64 oracle at sizes the oracle
finishes in seconds: several tiles, ragged last pages, empty shards, causal
drafts.  Reshards must match bit for bit; attention within the stated
tolerance (1e-5 fp32, 2e-3 relative bf16/fp8)."""

import math

import numpy as np
import pytest
import torch

import context_paged_kv_amd as K
import oracle as O
from tests import harness as H
from workloads import gen
from workloads.configs import get_workload, scaled

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _sync():
    torch.cuda.synchronize()


# --------------------------------------------------------------------------- decode


def test_decode_tiny_fp32_full():
    w = get_workload("tiny_fp32")
    H.log("decode tiny_fp32: B=1 T=1000 page 16 N=2 fp32")
    case = H.make_decode_case(w, DEV)
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs)
    H.log("  " + H.fmt_worst(worst))


@pytest.mark.parametrize("seed_shift,q_len,split", [(0, 1, "even"), (1, 1, "even"), (2, 2, "even"), (3, 4, "even"),
                                                   (0, 1, "chunks"), (3, 4, "chunks")])
def test_decode_gqa_bf16_small(seed_shift, q_len, split, monkeypatch):
    # the GQA kernel under its even split (the default) and under the chunk plan it takes for
    # batches beyond the even planner's pairs
    base = get_workload("gqa_bf16_16x4k-32k")
    w = scaled(base, seed=base.seed + 100 + seed_shift, seq_segments=((5, 70, 3000),), pool_pages=256,
               q_len=q_len)
    H.log(f"decode gqa bf16 small seed {w.seed} q_len {q_len} split {split}")
    if split == "chunks":
        monkeypatch.setenv("DCPKV_GQA_SPLIT", "chunks")
    case = H.make_decode_case(w, DEV)
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs)
    H.log("  " + H.fmt_worst(worst))


def test_decode_gqa_bf16_generic_kernel(monkeypatch):
    # the generic VALU kernel on the same shape, selected through the library's switch
    base = get_workload("gqa_bf16_16x4k-32k")
    w = scaled(base, seed=base.seed + 150, seq_segments=((3, 70, 2000),), pool_pages=128)
    case = H.make_decode_case(w, DEV)
    monkeypatch.setenv("DCPKV_FORCE_GENERIC", "1")
    outs = H.run_decode(case)
    _sync()
    monkeypatch.delenv("DCPKV_FORCE_GENERIC")
    H.check_decode(case, outs)


def test_decode_mla_fp8_small():
    base = get_workload("mla_fp8_48x100k")
    w = scaled(base, seed=base.seed + 100, seq_segments=((3, 200, 5000),), pool_pages=512)
    H.log("decode mla fp8 small q_len 1")
    case = H.make_decode_case(w, DEV)
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs)
    H.log("  " + H.fmt_worst(worst))


def test_decode_mla_fp8_verify_small():
    base = get_workload("mla_fp8_longmix_verify")
    w = scaled(base, seed=base.seed + 100, seq_segments=((2, 3000, 9000), (3, 2048, 2048)),
               pool_pages=512, num_layers=2, attn_layer=1)
    H.log("decode mla fp8 small q_len 4 causal, layer 1 of 2")
    case = H.make_decode_case(w, DEV)
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs)
    H.log("  " + H.fmt_worst(worst))


# Every instantiation of the generic VALU kernel (KV kind x query dtype) against the oracle: the
# fast kernels take bf16 queries only, so an f32 query, an MLA page other than 64 tokens or the
# library's switch routes a call here.
_GENERIC_CASES = {
    "split f32 KV, bf16 q": ("tiny_fp32", dict(q_dtype="bf16"), False),
    "split bf16 KV, f32 q": ("gqa_bf16_16x4k-32k", dict(q_dtype="f32", seq_segments=((3, 70, 2000),),
                                                        pool_pages=128), False),
    "mla fp8, f32 q": ("mla_fp8_48x100k", dict(q_dtype="f32", seq_segments=((2, 100, 3000),), pool_pages=256),
                       False),
    "mla fp8, page 32": ("mla_fp8_48x100k", dict(page_size=32, seq_segments=((2, 100, 3000),), pool_pages=512),
                         False),
    "mla fp8, forced, q_len 1": ("mla_fp8_48x100k", dict(seq_segments=((2, 64 * 9 + 5, 3000), (1, 3, 3)),
                                                         pool_pages=256), True),
    "mla fp8, forced, q_len 4": ("mla_fp8_longmix_verify", dict(seq_segments=((2, 64 * 9 + 5, 3000), (1, 4, 4)),
                                                                pool_pages=256, num_layers=2, attn_layer=1), True),
}


@pytest.mark.parametrize("label", list(_GENERIC_CASES))
def test_decode_generic_kernel_instantiations(label, monkeypatch):
    name, over, force = _GENERIC_CASES[label]
    base = get_workload(name)
    w = scaled(base, seed=base.seed + 160 + list(_GENERIC_CASES).index(label), **over)
    H.log(f"decode generic kernel: {label}")
    case = H.make_decode_case(w, DEV)
    if force:
        monkeypatch.setenv("DCPKV_FORCE_GENERIC", "1")
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs, heads=list(range(min(w.num_q_heads, 16))))
    H.log("  " + H.fmt_worst(worst))


@pytest.mark.parametrize("q_len", [1, 4])
def test_decode_mla_fp8_outlier_queries(q_len):
    """Queries with outliers: three entries x 64 and about half of the entries at 2^-12 .. 2^-14
    of the row's largest.  The fp8 score instruction keeps about 2^-12 of the largest product of
    a block (measured), which is too coarse for such rows, so the kernel sends the wavefronts
    whose rows have an entry above 16x their root mean square down its exact (fp16) score path;
    the outputs must meet the bar against the oracle on the same bf16 queries."""
    base = get_workload("mla_fp8_longmix_verify" if q_len == 4 else "mla_fp8_48x100k")
    w = scaled(base, seed=base.seed + 500 + q_len, seq_segments=((3, 700, 4000),), pool_pages=256, num_layers=1,
               attn_layer=0, q_len=q_len)
    case = H.make_decode_case(w, DEV)
    g = torch.Generator().manual_seed(31 + q_len)
    q = case.q.float().cpu()
    big = torch.rand(q.shape, generator=g).argsort(dim=-1)[..., :3]
    q.scatter_(-1, big, q.gather(-1, big) * 64.0)
    rmax = q.abs().amax(dim=-1, keepdim=True)
    tiny = torch.rand(q.shape, generator=g) < 0.5
    tiny.scatter_(-1, big, False)
    mag = rmax * torch.exp2(-12.0 - 2.0 * torch.rand(q.shape, generator=g))
    sign = torch.where(torch.rand(q.shape, generator=g) < 0.5, -1.0, 1.0)
    q = torch.where(tiny, sign * mag, q)
    case.q.copy_(q.to(torch.bfloat16).to(DEV))
    H.log(f"decode mla fp8 outlier queries, q_len {q_len}")
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs, heads=list(range(0, w.num_q_heads, 4)))
    H.log("  " + H.fmt_worst(worst))


@pytest.mark.parametrize("mode,q_len", [("exact", 1), ("exact", 4), ("fp8", 1)])
def test_decode_mla_fp8_score_paths(mode, q_len, monkeypatch):
    """Each score path of the fp8 MLA kernel for every row (DCPKV_MLA_SCORES), on N(0,1) queries
    with ragged tails, against the oracle."""
    base = get_workload("mla_fp8_longmix_verify" if q_len == 4 else "mla_fp8_48x100k")
    w = scaled(base, seed=base.seed + 520 + q_len, seq_segments=((3, 64 * 7 + 9, 4000),), pool_pages=256,
               num_layers=1, attn_layer=0, q_len=q_len)
    case = H.make_decode_case(w, DEV)
    monkeypatch.setenv("DCPKV_MLA_SCORES", mode)
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs, heads=list(range(0, w.num_q_heads, 4)))
    H.log(f"  {mode} scores, q_len {q_len}: " + H.fmt_worst(worst))


def _rescale_pages(case, f_repr, f_value):
    """Page (d, slot) of the attention layer: scale x 2^(f_repr + f_value), codes re-encoded as
    value x 2^-f_repr (e4m3fn, rounded by torch).  f_repr changes only how the page is written,
    f_value changes its values."""
    for d, (pool, sc) in enumerate(zip(case.pools, case.scales)):
        fr = torch.from_numpy(np.exp2(-f_repr[d]).astype(np.float32)).to(pool.device)
        codes = pool[case.layer].view(torch.float8_e4m3fn).float() * fr[:, None]
        pool[case.layer].copy_(codes.to(torch.float8_e4m3fn).view(torch.uint8))
        bits = sc[case.layer].cpu().numpy().astype(np.uint16)
        vals = (bits.astype(np.uint32) << 16).view(np.float32) * np.exp2(f_repr[d] + f_value[d]).astype(np.float32)
        sc[case.layer].copy_(torch.from_numpy((vals.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)).to(sc.device))


@pytest.mark.parametrize("q_len", [1, 4])
def test_decode_mla_fp8_rescale_paths(q_len):
    # Both rare paths of the fp8 MLA kernel's online softmax, against the oracle:
    #  * every page is rewritten with scale x 2^f, f in {0..3}, and codes x 2^-f: the values (and
    #    the scores) stay N(0,1)-like, but neighbouring page scales differ by up to 8x, so the
    #    accumulator's reference scale has to move;
    #  * one page in the middle of request 0 gets its values x 4: its scores jump past the running
    #    row maximum by more than 2^8 in log2 units.
    base = get_workload("mla_fp8_longmix_verify" if q_len == 4 else "mla_fp8_48x100k")
    w = scaled(base, seed=base.seed + 400 + q_len, seq_segments=((2, 3000, 6000),), pool_pages=512,
               num_layers=1, attn_layer=0, q_len=q_len)
    case = H.make_decode_case(w, DEV)
    rng = np.random.default_rng(11 + q_len)
    f_repr = [rng.integers(0, 4, size=w.pool_pages).astype(np.float64) for _ in range(w.dcp_size)]
    f_value = [np.zeros(w.pool_pages) for _ in range(w.dcp_size)]
    mid = case.pages[0][len(case.pages[0]) // 2]
    f_value[mid % w.dcp_size][mid // w.dcp_size] = 2.0
    _rescale_pages(case, f_repr, f_value)
    H.log(f"decode mla fp8 q_len {q_len}: page scales x 2^U[0, 3] (codes / same), page {mid} values x 4")
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs)
    H.log("  " + H.fmt_worst(worst))


@pytest.mark.parametrize("name", ["tiny_fp32", "gqa_bf16_16x4k-32k", "mla_fp8_longmix_verify"])
def test_decode_edge_lengths(name):
    # T = q_len (only the drafts), T = 1 page + 1 token, lengths below N pages (empty shards)
    base = get_workload(name)
    ql = base.q_len
    lens = [ql, base.page_size + 1, 2 * base.page_size - 1, 3]
    lens = [max(ql, t) for t in lens]
    w = scaled(base, seed=base.seed + 200, seq_segments=tuple((1, t, t) for t in lens), pool_pages=64,
               num_layers=1, attn_layer=0)
    H.log(f"decode edge lengths {name}: {lens}")
    case = H.make_decode_case(w, DEV)
    outs = H.run_decode(case)
    _sync()
    H.check_decode(case, outs)
    # shards that own no page of a request give (0, -inf)
    for b, t in enumerate(lens):
        pages = -(-t // w.page_size)
        for d in range(pages, w.dcp_size):
            assert torch.isneginf(outs.partial_lse[d, b]).all()
            assert (outs.partial_out[d, b] == 0).all()


@pytest.mark.parametrize("name,force_generic", [("tiny_fp32", False), ("gqa_bf16_16x4k-32k", False),
                                                 ("gqa_bf16_16x4k-32k", True), ("mla_fp8_48x100k", False)])
def test_decode_out_of_range_table_entries(name, force_generic, monkeypatch):
    """A block-table entry outside [0, M) is a page of no tokens: the shard's partial leaves out
    exactly that page's tokens (first, middle and last local pages; negative and too-large
    entries), and the merge combines what is left."""
    base = get_workload(name)
    ps = base.page_size
    w = scaled(base, seed=base.seed + 210, seq_segments=((1, ps * 9 + 3, ps * 9 + 3), (1, ps * 14, ps * 14),
                                                        (1, ps * 5 + 1, ps * 5 + 1)), pool_pages=64, q_len=2,
               num_layers=1, attn_layer=0)
    n = w.dcp_size
    case = H.make_decode_case(w, DEV)
    tables = case.tables.copy()
    holes = {0: [(1 % n, 0, -1)], 1: [(2 % n, 1, w.pool_pages), (0, 0, -7)], 2: [(0, -(-6 // n) - 1, 1 << 30)]}
    for b, hs in holes.items():
        for d, j, v in hs:
            assert j < -(-(-(-int(case.seq_lens[b]) // ps) - d) // n)  # a page the shard holds
            tables[d, b, j] = v
    case.bt_dev.copy_(torch.from_numpy(tables))
    if force_generic:
        monkeypatch.setenv("DCPKV_FORCE_GENERIC", "1")
    outs = H.run_decode(case)
    _sync()
    _check_with_holes(case, outs, holes, heads=list(range(min(w.num_q_heads, 8))))


@pytest.mark.parametrize("name", ["tiny_fp32", "gqa_bf16_16x4k-32k", "mla_fp8_48x100k"])
@pytest.mark.parametrize("tokens_hint", ["one", "tenfold"])
def test_decode_split_does_not_change_results(name, tokens_hint):
    """total_tokens only sizes the split: far too small a figure forces one chunk per (shard,
    request) (the workspace cannot hold a split: the planner's fallback), far too large a one
    longer chunks; both give the oracle's partials and merge."""
    base = get_workload(name)
    ps = base.page_size
    w = scaled(base, seed=base.seed + 220, seq_segments=((2, ps * 40 + 5, ps * 90), (2, 3, ps * 3)),
               pool_pages=256, num_layers=1, attn_layer=0)
    case = H.make_decode_case(w, DEV)
    hint = 1 if tokens_hint == "one" else 10 * case.total_tokens
    desc = H.attn_desc(case)
    ws = torch.empty(K.dcp_decode_partial_workspace(desc, hint), dtype=torch.uint8, device=DEV)
    outs, _ = H.alloc_outputs(case)
    K.dcp_decode_partial(desc, q=case.q, kv_pools=case.pools, kv_scales=case.scales, block_tables=case.bt_dev,
                         seq_lens=case.sl_dev, total_tokens=hint, partial_out=outs.partial_out,
                         partial_lse=outs.partial_lse, workspace=ws)
    rows = w.num_requests * w.q_len * w.num_q_heads
    K.dcp_lse_merge(w.dcp_size, rows, w.head_dim_v, outs.partial_out, outs.partial_lse, outs.out, outs.lse)
    _sync()
    H.check_decode(case, outs, heads=list(range(min(w.num_q_heads, 16))))


def _read_plan(ws: torch.Tensor, pairs: int):
    """The planner's output in the workspace: the header's chunk count, the per-pair plans
    (chunk prefix, workspace slot, k, local pages) and the chunk entries (pair, first page,
    end page, output slot).  Layout: 64-byte header at 0, pair plans from byte 256, chunk
    entries from the next 256-byte boundary, 16 bytes each."""
    raw = ws.cpu().numpy().view(np.int32)
    total = int(raw[0])
    pp = raw[64: 64 + 4 * pairs].reshape(pairs, 4)
    c0 = ((256 + 16 * pairs + 255) // 256) * 256 // 4
    ch = raw[c0: c0 + 4 * (total + 1)].reshape(total + 1, 4)
    return total, pp, ch


def _check_plan(total, pp, ch, nl_expected):
    """Every pair's local pages are covered once, by its k chunks of sizes that differ by at
    most one, each written to its own output slot; the entries run longest first (to within
    one of the 64 size classes) and the entry after the last is empty."""
    assert ch[total, 0] == -1
    assert total == int(pp[:, 2].sum())
    seen = {}
    for pair, jb, je, out in ch[:total]:
        seen.setdefault(int(pair), []).append((int(jb), int(je), int(out)))
    for i, n_local in enumerate(nl_expected):
        k = int(pp[i, 2])
        assert int(pp[i, 3]) == n_local and k >= 1
        got = sorted(seen.get(i, []))
        assert len(got) == k
        assert [g[0] for g in got] == [0] + [g[1] for g in got[:-1]] and got[-1][1] == n_local
        sizes = [je - jb for jb, je, _ in got]
        assert max(sizes) - min(sizes) <= 1
        outs = [o for _, _, o in got]
        assert outs == ([-1] if k == 1 else list(range(int(pp[i, 1]), int(pp[i, 1]) + k)))
    sizes = (ch[:total, 2] - ch[:total, 1]).astype(np.int64)
    span = max(int(sizes.max()), 1)
    assert (np.diff(sizes) <= span // 64 + 1).all(), "chunks are not longest first"


def _local_pages(seq_lens, page_size, n):
    out = []
    for d in range(n):
        for t in seq_lens:
            p = -(-int(t) // page_size)
            out.append((p - 1 - d) // n + 1 if p > d else 0)
    return out


def test_decode_plan_splits_mixed_lengths_longest_first(monkeypatch):
    """Unequal pairs are split into chunks of at most C pages, emitted longest first (the
    GQA kernel under its chunk plan)."""
    monkeypatch.setenv("DCPKV_GQA_SPLIT", "chunks")
    base = get_workload("gqa_bf16_16x4k-32k")
    ps, n = base.page_size, base.dcp_size
    w = scaled(base, seed=base.seed + 240, seq_segments=((12, ps * n * 4, ps * n * 40), (2, 5, ps)),
               pool_pages=512, num_layers=1, attn_layer=0)
    H.log("plan: GQA bf16 B=14 mixed 5..10240 tokens, N=4")
    case = H.make_decode_case(w, DEV)
    outs, ws = H.alloc_outputs(case)
    H.run_decode(case, outs, ws)
    _sync()
    pairs = n * w.num_requests
    total, pp, ch = _read_plan(ws, pairs)
    nl = _local_pages(case.seq_lens, ps, n)
    _check_plan(total, pp, ch, nl)
    assert (pp[:, 2] >= 2).any(), "the long pairs were not split"
    H.check_decode(case, outs, heads=list(range(8)))


def test_decode_plan_keeps_equal_pairs_whole_when_they_fill_the_device(monkeypatch):
    """Equal-length pairs whose work items fill every workgroup slot in whole rounds keep one
    chunk each (GQA kernel under its chunk plan: four resident workgroups per compute unit,
    one per KV head and chunk); one pair shorter than the rest breaks the rule and the long
    pairs split again."""
    monkeypatch.setenv("DCPKV_GQA_SPLIT", "chunks")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    base = get_workload("gqa_bf16_16x4k-32k")
    ps, n = base.page_size, base.dcp_size
    b = cus * 4 // (n * base.num_kv_heads)  # pairs x KV heads = one round of slots
    t = ps * n * 20                        # 20 local pages per pair: above the chunk size
    for shorter in (False, True):
        segs = ((b, t, t),) if not shorter else ((b - 1, t, t), (1, t // 2, t // 2))
        w = scaled(base, seed=base.seed + 250, seq_segments=segs, pool_pages=24 * b, num_layers=1, attn_layer=0)
        H.log(f"plan: GQA bf16 B={b} x {t} tokens (one shorter: {shorter}), N={n}, {cus} CUs")
        case = H.make_decode_case(w, DEV)
        outs, ws = H.alloc_outputs(case)
        H.run_decode(case, outs, ws)
        _sync()
        pairs = n * b
        total, pp, ch = _read_plan(ws, pairs)
        _check_plan(total, pp, ch, _local_pages(case.seq_lens, ps, n))
        if shorter:
            assert (pp[:, 2] >= 2).any()
        else:
            assert total == pairs and (pp[:, 2] == 1).all()
        H.check_decode(case, outs, requests=[0, b - 1], heads=list(range(4)))


def _read_even_plan(ws: torch.Tensor, pairs: int, slots: int):
    """The even planner's output in the workspace: waves with work and page-items (header
    words 3 and 4-5), the pair entries from byte 256 (16 bytes: -, -, next pair with pages,
    local pages), the pairs' page prefix sums (int64) and the wave starts (32 bytes: pair,
    KV head, first page, count, local pages, next pair, request length, -), each from the
    next 256-byte boundary."""
    raw = ws.cpu().numpy()
    i32 = raw.view(np.int32)
    waves, total = int(i32[3]), int(raw[16:24].view(np.int64)[0])
    al = lambda x: (x + 255) // 256 * 256
    pp = i32[64:64 + 4 * pairs].reshape(pairs, 4)
    pfx_off = al(256 + 16 * pairs)
    pfx = raw[pfx_off:pfx_off + 8 * (pairs + 1)].view(np.int64)
    wst_off = al(pfx_off + 8 * (pairs + 1))
    wst = i32[wst_off // 4:wst_off // 4 + 8 * slots].reshape(slots, 8)
    return waves, total, pp, pfx, wst


@pytest.mark.parametrize("segs", [((14, 64 * 4 * 4, 64 * 4 * 40), (2, 5, 64)),  # mixed lengths
                                  ((3, 70, 300), (2, 10, 10), (2, 64 * 9, 64 * 9)),  # shards without pages
                                  ((60, 64 * 4 * 2, 64 * 4 * 6), (10, 10, 60), (10, 64 * 9, 64 * 9))])  # 320 pairs
def test_decode_gqa_even_plan_covers_every_page_item(segs):
    """The even split: the pairs' local pages, their prefix sums, the next pair with pages and
    the header (waves with work, page-items) the reduction reads.  Beyond 256 pairs, where the
    planner writes the wave starts: the waves' ranges tile the page-items of the (pair, KV
    head) segments in order, with counts that differ by at most one, and every start names
    the segment and page of its first item and carries that pair's length and the next pair
    with pages.  (Up to 256 pairs every wave plans its own range; the oracle comparison below
    covers it.)"""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    slots = cus * 4
    base = get_workload("gqa_bf16_16x4k-32k")
    ps, n, hkv = base.page_size, base.dcp_size, base.num_kv_heads
    w = scaled(base, seed=base.seed + 260, seq_segments=segs, pool_pages=512, num_layers=1, attn_layer=0)
    case = H.make_decode_case(w, DEV, seq_lens=np.concatenate(
        [np.linspace(lo, hi, k).astype(np.int64) for k, lo, hi in segs]))
    outs, ws = H.alloc_outputs(case)
    H.run_decode(case, outs, ws)
    _sync()
    pairs = n * w.num_requests
    waves, total, pp, pfx, wst = _read_even_plan(ws, pairs, slots)
    nl = np.array(_local_pages(case.seq_lens, ps, n), dtype=np.int64)
    assert (pp[:, 3] == nl).all()
    assert (pfx == np.concatenate([[0], np.cumsum(nl)])).all()
    P = int(nl.sum()) * hkv
    assert total == P and waves == min(slots, P)
    nxt = [next((j for j in range(i + 1, pairs) if nl[j] > 0), pairs) for i in range(pairs)]
    assert (pp[:, 2] == np.array(nxt)).all()
    if pairs <= 256:
        H.check_decode(case, outs, heads=list(range(8)))
        return
    x = 0
    for wv in range(slots):
        pair, hb, j0, cnt, nlw, nxw, slw, _ = (int(v) for v in wst[wv])
        if wv >= waves:
            assert cnt == 0
            continue
        assert x == wv * P // waves and cnt == (wv + 1) * P // waves - x
        assert pfx[pair] * hkv + hb * nl[pair] + j0 == x and 0 <= j0 < nl[pair] and 0 <= hb < hkv
        assert nlw == nl[pair] and nxw == nxt[pair] and slw == int(case.seq_lens[pair % w.num_requests])
        x += cnt
    assert x == P
    H.check_decode(case, outs, heads=list(range(8)))


def _check_with_holes(case, outs, holes, heads):
    """Partials and merge against the oracle with the table entries of `holes` ({request:
    [(shard, local page, value)]}) out of range: those pages' tokens take no part."""
    w = case.w
    n, ps = w.dcp_size, w.page_size
    tol_o, tol_l = H.tolerance(w)
    for b in range(w.num_requests):
        T = int(case.seq_lens[b])
        pb, psc = H.gather_request_pages(case.pools, case.scales, case.pages[b], n, case.layer)
        k, v = H.oracle_logical_kv(w, pb, psc, T)
        q = H.q_host(case, b)
        po, pl = [], []
        for d in range(n):
            mask = O.shard_token_mask(case.pages[b], ps, T, n, d)
            for dd, j, _ in holes.get(b, []):
                if dd == d:  # local page j of shard d is sequence page j*N + d
                    mask[(j * n + d) * ps:min(T, (j * n + d + 1) * ps)] = False
            o_, l_ = O.request_attention(q, k, v, T, w.softmax_scale, mask, heads)
            po.append(o_)
            pl.append(l_)
        po, pl = np.stack(po), np.stack(pl)
        uo, ul = O.lse_merge(po, pl)
        for d in range(n):
            H.check_rows(f"partial d={d} b={b}", outs.partial_out[d, b][:, heads].cpu().numpy(),
                         outs.partial_lse[d, b][:, heads].cpu().numpy(), po[d][:, heads], pl[d][:, heads],
                         tol_o, tol_l)
        H.check_rows(f"merged b={b}", outs.out[b][:, heads].cpu().numpy(), outs.lse[b][:, heads].cpu().numpy(),
                     uo[:, heads], ul[:, heads], tol_o, tol_l)


def test_decode_gqa_even_segments_without_valid_pages():
    """Even split, segments that span many waves (a few page-items per wave): a shard whose
    first 66 local pages are out of range (its first page with a slot lies past the first
    64-entry window), a shard with no page in range at all (its part is empty: O = 0,
    LSE = -inf), and out-of-range pages at the ends of wave ranges."""
    base = get_workload("gqa_bf16_16x4k-32k")
    ps, n = base.page_size, base.dcp_size
    long_t = ps * n * 70 + 17  # 71 local pages on shard 0, 70 on the others
    w = scaled(base, seed=base.seed + 270, seq_segments=((1, long_t, long_t), (1, ps * n * 12, ps * n * 12),
                                                        (1, 300, 300)), pool_pages=1024, q_len=2,
               num_layers=1, attn_layer=0)
    case = H.make_decode_case(w, DEV)
    tables = case.tables.copy()
    holes = {0: [(0, j, -1) for j in range(66)] + [(2, 30, w.pool_pages)],
             1: [(1, j, -3) for j in range(12)] + [(3, 11, 1 << 28)]}
    for b, hs in holes.items():
        for d, j, v in hs:
            tables[d, b, j] = v
    case.bt_dev.copy_(torch.from_numpy(tables))
    H.log("decode gqa even split: 71-page shard with 66 holes, an all-hole shard, B=3, N=4, q_len 2")
    outs = H.run_decode(case)
    _sync()
    assert torch.isneginf(outs.partial_lse[1, 1]).all() and (outs.partial_out[1, 1] == 0).all()
    _check_with_holes(case, outs, holes, heads=list(range(w.num_q_heads)))


def test_decode_gqa_many_pairs_take_the_chunk_plan():
    """More (shard, request) pairs than the even planner holds: the GQA kernel runs under the
    chunk plan; sampled requests against the oracle."""
    base = get_workload("gqa_bf16_16x4k-32k")
    B = 1100  # x 4 shards = 4400 pairs > 4096
    w = scaled(base, seed=base.seed + 280, seq_segments=((B, 20, 700),), pool_pages=4096, num_layers=1,
               attn_layer=0)
    case = H.make_decode_case(w, DEV)
    H.log(f"decode gqa bf16, B={B} x N={w.dcp_size} pairs: chunk plan")
    outs = H.run_decode(case)
    _sync()
    H.check_decode(case, outs, requests=[0, 1, 549, 1098, 1099], heads=list(range(8)))


def test_decode_shard_subset_calls():
    # partials computed one shard range at a time equal the all-shard call
    base = get_workload("gqa_bf16_16x4k-32k")
    w = scaled(base, seed=base.seed + 300, seq_segments=((3, 500, 2500),), pool_pages=128)
    case = H.make_decode_case(w, DEV)
    full = H.run_decode(case)
    part, ws = H.alloc_outputs(case)
    H.run_decode(case, part, ws, shard_begin=0, shard_count=1, merge=False)
    H.run_decode(case, part, ws, shard_begin=1, shard_count=3, merge=False)
    _sync()
    assert torch.equal(part.partial_out, full.partial_out)
    assert torch.equal(part.partial_lse, full.partial_lse)


# --------------------------------------------------------------------------- merge


@pytest.mark.parametrize("n,rows,dv", [(1, 7, 64), (2, 33, 128), (8, 100, 512), (5, 9, 10), (8, 17, 256),
                                      (3, 5, 4), (9, 6, 128)])
def test_lse_merge_vs_oracle(n, rows, dv):
    g = torch.Generator().manual_seed(n * 1000 + rows)
    po = torch.randn((n, rows, dv), generator=g)
    pl = torch.randn((n, rows), generator=g) * 5
    pl[0, : rows // 3] = float("-inf")          # some shards empty
    if n > 1:
        pl[:, rows - 1] = float("-inf")         # a row with nothing anywhere
        po[:, rows - 1] = 0
    out = torch.empty((rows, dv), device=DEV)
    lse = torch.empty((rows,), device=DEV)
    K.dcp_lse_merge(n, rows, dv, po.to(DEV), pl.to(DEV), out, lse)
    _sync()
    ro, rl = O.lse_merge(po.double().numpy(), pl.double().numpy())
    H.check_rows("merge", out.cpu().numpy(), lse.cpu().numpy(), ro, rl, 1e-6, 1e-6)
    if n > 1:
        assert torch.isneginf(lse[rows - 1]) and (out[rows - 1] == 0).all()


# --------------------------------------------------------------------------- reshard


def _host_pools(ts):
    return [t.cpu().numpy() for t in ts]


def test_reshard_tiny_fp32_full_oracle():
    w = get_workload("tiny_fp32")
    H.log("reshard tiny_fp32: 1 source, 1 layer, N=2")
    rc = H.make_reshard_case(w, DEV)
    src_before = [t.clone() for t in rc.src_pools]
    dst_host = _host_pools(rc.dst_pools)
    sent = O.reshard(_host_pools(rc.src_pools), dst_host, rc.num_layers, w.dcp_size, rc.src_ids, rc.dst_ids,
                     rc.first_uncached)
    H.run_reshard(rc)
    _sync()
    for d in range(w.dcp_size):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])
    for a, b in zip(src_before, rc.src_pools):
        assert torch.equal(a, b)
    assert sum(sent) == len(rc.dst_ids)


@pytest.mark.parametrize("cached,dst_filter", [(0, -1), (5, -1), (3, 2)])
def test_reshard_multi_source_scales(cached, dst_filter):
    base = get_workload("reshard_mla_128k")
    w = scaled(base, seed=base.seed + 100, seq_segments=((1, 64 * 37 + 13, 64 * 37 + 13),), num_layers=7,
               num_sources=3, pool_pages=16, dcp_size=4)
    H.log(f"reshard 3 sources x 7 layers N=4 cached={cached} filter={dst_filter}")
    rc = H.make_reshard_case(w, DEV, first_uncached=cached)
    src_before = [t.clone() for t in rc.src_pools]
    dst_host = _host_pools(rc.dst_pools)
    dsc_host = _host_pools(rc.dst_scales)
    sent = O.reshard(_host_pools(rc.src_pools), dst_host, rc.num_layers, w.dcp_size, rc.src_ids, rc.dst_ids,
                     rc.first_uncached, dst_filter, _host_pools(rc.src_scales), dsc_host)
    counts = torch.zeros(w.dcp_size, dtype=torch.int64, device=DEV)
    H.run_reshard(rc, dst_filter=dst_filter, pages_per_dst=counts)
    _sync()
    assert counts.cpu().tolist() == sent  # the per-destination page counts of the transfer
    for d in range(w.dcp_size):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])
        assert np.array_equal(rc.dst_scales[d].cpu().numpy(), dsc_host[d])
    for a, b in zip(src_before, rc.src_pools):
        assert torch.equal(a, b)
    H.check_reshard_by_plan(rc, dst_filter)


def test_reshard_pages_per_dst_full_transfer_log_line():
    """[2DR] section 6.3's transfer log at N = 4: 256 pages of a 16K-token request, 64 to each
    destination; the counts accumulate over calls and skip bad entries."""
    base = get_workload("gqa_bf16_16x4k-32k")
    w = scaled(base, seed=base.seed + 130, seq_segments=((1, 16384, 16384),), pool_pages=128)
    rc = H.make_reshard_case(w, DEV, first_uncached=0)
    assert len(rc.dst_ids) == 256
    counts = torch.zeros(4, dtype=torch.int64, device=DEV)
    H.run_reshard(rc, pages_per_dst=counts)
    _sync()
    assert counts.cpu().tolist() == [64, 64, 64, 64]
    dst = rc.dst_ids.copy()
    dst[[0, 5]] = -1  # two bad entries (owners 0 and 1) are not counted
    H.run_reshard(rc, pages_per_dst=counts, dst_ids=dst)
    _sync()
    assert counts.cpu().tolist() == [127, 127, 128, 128]
    H.check_reshard_by_plan(rc)


def test_reshard_precondition_check_refuses_repeated_pages(monkeypatch):
    """With DCPKV_CHECK_PRECONDITIONS=1 a destination page listed twice is refused before anything
    is written (page and token reshards); a list without repeats still moves as the oracle says."""
    base = get_workload("reshard_mla_128k")
    w = scaled(base, seed=base.seed + 103, seq_segments=((1, 64 * 12, 64 * 12),), num_layers=2, num_sources=1,
               pool_pages=8, dcp_size=2)
    rc = H.make_reshard_case(w, DEV, first_uncached=2)
    monkeypatch.setenv("DCPKV_CHECK_PRECONDITIONS", "1")
    dup = rc.dst_ids.copy()
    dup[9] = dup[4]
    before = [t.clone() for t in rc.dst_pools]
    with pytest.raises(K.DcpkvError) as e:
        H.run_reshard(rc, dst_ids=dup)
    assert e.value.code == K.DCPKV_EINVAL and "appears twice" in str(e.value)
    rc_tok = H.ReshardCase(**{**rc.__dict__, "dst_scales": None, "src_scales": None})
    with pytest.raises(K.DcpkvError):
        H.run_reshard_tokens(rc_tok, dst_ids=dup)
    _sync()
    for a, b in zip(before, rc.dst_pools):
        assert torch.equal(a, b)
    dup[0] = dup[4]  # a repeat of a cached entry's page is no repeat of the call
    dup[9] = rc.dst_ids[9]
    dst_host = _host_pools(rc.dst_pools)
    O.reshard(_host_pools(rc.src_pools), dst_host, 2, 2, rc.src_ids, dup, rc.first_uncached,
              -1, _host_pools(rc.src_scales), _host_pools(rc.dst_scales))
    H.run_reshard(rc, dst_ids=dup)
    _sync()
    for d in range(2):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])


def test_reshard_follows_destination_value_not_position():
    base = get_workload("reshard_mla_128k")
    w = scaled(base, seed=base.seed + 101, seq_segments=((1, 64 * 8, 64 * 8),), num_layers=2, num_sources=1,
               pool_pages=8, dcp_size=4)
    rc = H.make_reshard_case(w, DEV, first_uncached=0)
    # destination ids whose residues mod 4 do not follow their list positions
    rc.dst_ids = np.array([7, 2, 4, 13, 0, 9, 30, 17], dtype=np.int64)
    dst_host = _host_pools(rc.dst_pools)
    O.reshard(_host_pools(rc.src_pools), dst_host, 2, 4, rc.src_ids, rc.dst_ids, 0)
    H.run_reshard(rc)
    _sync()
    for d in range(4):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])


def test_reshard_out_of_range_entries_are_skipped_and_counted():
    base = get_workload("reshard_mla_128k")
    w = scaled(base, seed=base.seed + 102, seq_segments=((1, 64 * 6, 64 * 6),), num_layers=3, num_sources=2,
               pool_pages=4, dcp_size=2)
    rc = H.make_reshard_case(w, DEV, first_uncached=0)
    src = rc.src_ids.copy()
    dst = rc.dst_ids.copy()
    src[1] = rc.src_pages + 5       # source page out of range
    dst[4] = w.pool_pages * 2 + 3   # destination page out of range
    dst[5] = -1
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.run_reshard(rc, bad=bad, src_ids=src, dst_ids=dst)
    _sync()
    assert int(bad.item()) == 3 * w.num_layers
    keep = [i for i in range(len(dst)) if i not in (1, 4, 5)]
    dst_host = _host_pools([torch.full_like(t, gen.DST_SENTINEL) for t in rc.dst_pools])
    O.reshard(_host_pools(rc.src_pools), dst_host, 3, 2, src[keep], dst[keep], 0)
    for d in range(2):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])


# --------------------------------------------------------------------------- token ownership


_TOKEN_CASES = {
    "tiny_fp32": dict(seq_segments=((1, 1000, 1000),)),
    "gqa_bf16_16x4k-32k": dict(seq_segments=((5, 70, 3000),), pool_pages=256),
    "mla_fp8_48x100k": dict(seq_segments=((3, 200, 5000),), pool_pages=512),
    "mla_fp8_longmix_verify": dict(seq_segments=((2, 3000, 9000), (3, 2048, 2048)), pool_pages=512,
                                   num_layers=2, attn_layer=1),
}


@pytest.mark.parametrize("name", list(_TOKEN_CASES))
def test_decode_token_ownership(name):
    """Token t on shard t mod N ([SGL]): every kernel (generic fp32, bf16 GQA, fp8 MLA with q_len 1
    and causal q_len 4) against the oracle under token ownership."""
    base = get_workload(name)
    w = scaled(base, seed=base.seed + 300, **_TOKEN_CASES[name])
    H.log(f"decode token ownership {name}")
    case = H.make_decode_case(w, DEV, own=K.OWN_TOKEN)
    outs = H.run_decode(case)
    _sync()
    worst = H.check_decode(case, outs)
    H.log("  " + H.fmt_worst(worst))


def test_decode_token_ownership_generic_kernel(monkeypatch):
    base = get_workload("gqa_bf16_16x4k-32k")
    w = scaled(base, seed=base.seed + 301, seq_segments=((3, 70, 2000),), pool_pages=128, q_len=2)
    case = H.make_decode_case(w, DEV, own=K.OWN_TOKEN)
    monkeypatch.setenv("DCPKV_FORCE_GENERIC", "1")
    outs = H.run_decode(case)
    _sync()
    monkeypatch.delenv("DCPKV_FORCE_GENERIC")
    H.check_decode(case, outs)


@pytest.mark.parametrize("name", ["tiny_fp32", "gqa_bf16_16x4k-32k", "mla_fp8_longmix_verify"])
def test_decode_token_ownership_edge_lengths(name):
    """T = q_len, just over one page, and fewer tokens than shards: shards holding no token give
    (0, -inf); a shard whose page ownership would hold nothing now holds tokens."""
    base = get_workload(name)
    ql = base.q_len
    lens = [max(ql, t) for t in (ql, base.page_size + 1, 2 * base.page_size - 1, 3)]
    w = scaled(base, seed=base.seed + 302, seq_segments=tuple((1, t, t) for t in lens), pool_pages=64,
               num_layers=1, attn_layer=0)
    case = H.make_decode_case(w, DEV, own=K.OWN_TOKEN)
    outs = H.run_decode(case)
    _sync()
    H.check_decode(case, outs)
    for b, t in enumerate(lens):
        for d in range(w.dcp_size):
            empty = d >= t
            assert bool(torch.isneginf(outs.partial_lse[d, b]).all()) == empty


# --------------------------------------------------------------------------- bounded pack / unpack


@pytest.mark.parametrize("cap", [1, 3, 22, 4096])
def test_path_pack_unpack_windows_vs_oracle(cap):
    """Entries, every staging window (pages, scales, unit count) and the final destination pools
    of the path-by-path transfer, bit for bit against the oracle; the pools also equal what the
    oracle's reshard writes."""
    base = get_workload("reshard_mla_128k")
    w = scaled(base, seed=base.seed + 110, seq_segments=((1, 64 * 37 + 13, 64 * 37 + 13),), num_layers=7,
               num_sources=3, pool_pages=16, dcp_size=4)
    H.log(f"path pack/unpack 3 sources x 7 layers N=4 cached=5 cap={cap}")
    rc = H.make_reshard_case(w, DEV, first_uncached=5)
    src_host = _host_pools(rc.src_pools)
    ssc_host = _host_pools(rc.src_scales)
    dst_host = _host_pools(rc.dst_pools)
    dsc_host = _host_pools(rc.dst_scales)
    ref_dst = [a.copy() for a in dst_host]
    ref_dsc = [a.copy() for a in dsc_host]
    O.reshard(src_host, ref_dst, rc.num_layers, w.dcp_size, rc.src_ids, rc.dst_ids, 5, -1, ssc_host, ref_dsc)
    seen = []

    def check(d, r, u0, stg, stg_sc, n, pos, count):
        ent = O.path_entries(rc.src_ids, rc.dst_ids, 5, w.dcp_size, d, rc.src_pages, w.pool_pages)
        assert count == len(ent) and pos[:count].cpu().numpy().tolist() == ent
        ostg = np.full((cap, w.page_bytes), gen.DST_SENTINEL, dtype=np.uint8)
        osc = np.full(cap, gen.SCALE_SENTINEL, dtype=np.int16)
        k = O.pack_pages(src_host[r], ssc_host[r], rc.src_ids, rc.num_layers, rc.num_sources, r, ent, u0, cap,
                         ostg, osc)
        assert n == k
        assert np.array_equal(stg.cpu().numpy(), ostg) and np.array_equal(stg_sc.cpu().numpy(), osc)
        O.unpack_pages(dst_host[d], dsc_host[d], rc.dst_ids, rc.num_layers, rc.num_sources, r, w.dcp_size, ent,
                       u0, cap, ostg, osc)
        seen.append(k)

    moved = H.run_path_pack(rc, cap, check_windows=check)
    _sync()
    assert moved == sum(seen) == (len(rc.dst_ids) - 5) * rc.num_layers
    for d in range(w.dcp_size):
        got = rc.dst_pools[d].cpu().numpy()
        assert np.array_equal(got, dst_host[d]) and np.array_equal(got, ref_dst[d])
        got_sc = rc.dst_scales[d].cpu().numpy()
        assert np.array_equal(got_sc, dsc_host[d]) and np.array_equal(got_sc, ref_dsc[d])


def test_path_entries_value_owned_and_bad_ids_excluded():
    base = get_workload("reshard_mla_128k")
    w = scaled(base, seed=base.seed + 111, seq_segments=((1, 64 * 8, 64 * 8),), num_layers=2, num_sources=1,
               pool_pages=8, dcp_size=4)
    rc = H.make_reshard_case(w, DEV, first_uncached=0)
    rc.dst_ids = np.array([7, 2, 4, 13, 0, 9, 30, 17], dtype=np.int64)  # residues differ from positions
    src = rc.src_ids.copy()
    dst = rc.dst_ids.copy()
    src[1] = rc.src_pages + 5
    dst[4] = w.pool_pages * 4 + 3
    dst[5] = -1
    si = torch.from_numpy(src.astype(np.int32)).to(DEV)
    di = torch.from_numpy(dst).to(DEV)
    pos = torch.empty(8, dtype=torch.int32, device=DEV)
    cnt = torch.empty(1, dtype=torch.int64, device=DEV)
    for d in range(4):
        K.kv_path_entries(num_sources=1, num_layers=2, dcp_size=4, page_bytes=w.page_bytes, src_pages=rc.src_pages,
                          dst_pages=w.pool_pages, dest=d, src_page_ids=si, dst_global_pages=di, out_positions=pos,
                          out_count=cnt)
        _sync()
        want = O.path_entries(src, dst, 0, 4, d, rc.src_pages, w.pool_pages)
        assert pos[: int(cnt.item())].cpu().numpy().tolist() == want
    dst_host = _host_pools([torch.full_like(t, gen.DST_SENTINEL) for t in rc.dst_pools])
    keep = [i for i in range(8) if i not in (1, 4, 5)]
    O.reshard(_host_pools(rc.src_pools), dst_host, 2, 4, src[keep], dst[keep], 0)
    H.run_path_pack(rc, 3, src_ids=src, dst_ids=dst)
    _sync()
    for d in range(4):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])


# --------------------------------------------------------------------------- token scatter reshard


@pytest.mark.parametrize("name,n,cached", [("gqa_bf16_16x4k-32k", 4, 3), ("tiny_fp32", 2, 0),
                                           ("gqa_bf16_16x4k-32k", 3, 0), ("gqa_bf16_16x4k-32k", 1, 2)])
def test_reshard_tokens_vs_oracle(name, n, cached):
    """Layer-split sources into token-owned pools, bit for bit against the oracle (several sources
    and layers, cached pages, a partial last page, N that does not divide the page)."""
    base = get_workload(name)
    w = scaled(base, seed=base.seed + 120, seq_segments=((1, base.page_size * 23 + 5, base.page_size * 23 + 5),),
               num_layers=5, num_sources=2, pool_pages=32, dcp_size=n)
    H.log(f"token reshard {name} N={n} cached={cached}")
    rc = H.make_reshard_case(w, DEV, first_uncached=cached)
    dst_host = _host_pools(rc.dst_pools)
    R, rb = H.token_geometry(w)
    O.reshard_tokens(_host_pools(rc.src_pools), dst_host, rc.num_layers, n, w.page_size, R, rb, rc.src_ids,
                     rc.dst_ids, cached)
    H.run_reshard_tokens(rc)
    _sync()
    for d in range(n):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])


@pytest.mark.parametrize("name,n,cached", [("gqa_bf16_16x4k-32k", 4, 3), ("reshard_mla_128k", 8, 0),
                                           ("tiny_fp32", 3, 1)])
def test_reshard_tokens_batch_vs_oracle(name, n, cached):
    """Several requests in one launch, delimited by offsets: each request's tokens restart at
    position 0 and land in its own virtual pages (the MLA case: 576-byte rows over N = 8, the
    pools' scales not passed).  Bit for bit against the oracle."""
    base = get_workload(name)
    ps = base.page_size
    lens = (ps * 9 + 5, ps * 2, 3, ps * 13 + 1)
    w = scaled(base, seed=base.seed + 130, seq_segments=tuple((1, t, t) for t in lens), num_layers=3,
               num_sources=2, pool_pages=32, dcp_size=n)
    H.log(f"token reshard batch {name} N={n} cached={cached}")
    rc = H.make_reshard_case(w, DEV, seq_lens=lens, first_uncached=cached)
    offs = np.cumsum([0] + [-(-t // ps) for t in lens])
    assert offs[-1] == len(rc.dst_ids)
    dst_host = _host_pools(rc.dst_pools)
    R, rb = H.token_geometry(w)
    O.reshard_tokens(_host_pools(rc.src_pools), dst_host, 3, n, ps, R, rb, rc.src_ids, rc.dst_ids, cached,
                     request_offsets=offs)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.run_reshard_tokens(rc, bad=bad, request_offsets=offs)
    _sync()
    assert int(bad.item()) == 0
    for d in range(n):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])


def test_reshard_tokens_bad_request_offsets_skipped_and_counted():
    """Entries that no request of the offsets contains (a last offset past the list, a negative
    first offset) are skipped and counted once per layer; the rest move as for a good split."""
    base = get_workload("gqa_bf16_16x4k-32k")
    lens = (64 * 5 + 3, 64 * 4)
    w = scaled(base, seed=base.seed + 131, seq_segments=tuple((1, t, t) for t in lens), num_layers=2,
               num_sources=1, pool_pages=8, dcp_size=4)
    R, rb = H.token_geometry(w)
    for offs, keep in (([0, 6, 14], slice(0, 6)), ([-1, 6, 10], slice(6, 10))):
        rc = H.make_reshard_case(w, DEV, seq_lens=lens, first_uncached=0)
        dst_host = _host_pools(rc.dst_pools)
        bad = torch.zeros(1, dtype=torch.int32, device=DEV)
        H.run_reshard_tokens(rc, bad=bad, request_offsets=offs)
        _sync()
        assert int(bad.item()) == 2 * (10 - (keep.stop - keep.start))
        O.reshard_tokens(_host_pools(rc.src_pools), dst_host, 2, 4, w.page_size, R, rb, rc.src_ids[keep],
                         rc.dst_ids[keep], 0)
        for d in range(4):
            assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])


def test_reshard_tokens_bad_pages_skipped_and_counted():
    base = get_workload("gqa_bf16_16x4k-32k")
    w = scaled(base, seed=base.seed + 121, seq_segments=((1, 64 * 9, 64 * 9),), num_layers=2, num_sources=1,
               pool_pages=8, dcp_size=4)
    rc = H.make_reshard_case(w, DEV, first_uncached=0)
    src = rc.src_ids.copy()
    src[2] = rc.src_pages + 1  # page 2: source id out of range
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    H.run_reshard_tokens(rc, bad=bad, src_ids=src)
    _sync()
    assert int(bad.item()) == 2  # one per layer
    dst_host = _host_pools([torch.full_like(t, gen.DST_SENTINEL) for t in rc.dst_pools])
    R, rb = H.token_geometry(w)
    keep_src = src.copy()
    src_host = _host_pools(rc.src_pools)
    # the oracle moves every page; page 2's rows are then put back to the sentinel
    O.reshard_tokens(src_host, dst_host, 2, 4, w.page_size, R, rb, np.where(keep_src >= rc.src_pages, 0, keep_src),
                     rc.dst_ids, 0)
    for x in range(w.page_size):
        d, slot, y = O.token_place(2 * w.page_size + x, 4, w.page_size, rc.dst_ids)
        for layer in range(2):
            pg = dst_host[d][layer, slot].reshape(R, w.page_size, rb)
            pg[:, y, :] = gen.DST_SENTINEL
    for d in range(4):
        assert np.array_equal(rc.dst_pools[d].cpu().numpy(), dst_host[d])


@pytest.mark.parametrize("q_len", [1, 3])
def test_token_pipeline_reshard_then_decode(q_len):
    """Token reshard into token-owned pools, then decode under token ownership: every partial and
    the merged output against the oracle's attention over the source pages' logical sequence."""
    base = get_workload("gqa_bf16_16x4k-32k")
    lens = (64 * 20 + 7, 64 * 7 + 63)
    w = scaled(base, seed=base.seed + 122 + q_len, seq_segments=tuple((1, t, t) for t in lens), num_layers=1,
               num_sources=1, pool_pages=64, dcp_size=4, q_len=q_len)
    case = H.make_decode_case(w, DEV, seq_lens=lens, own=K.OWN_TOKEN)
    for b in range(len(lens)):
        rc = H.make_reshard_case(w, DEV, seq_lens=lens, requests=[b], first_uncached=0, dst_pools=case.pools,
                                 dst_scales=case.scales)
        H.run_reshard_tokens(rc)
        _sync()
        srcp = rc.src_pools[0][0].index_select(0, torch.from_numpy(rc.src_ids).to(DEV)).cpu().numpy()
        kv = H.oracle_logical_kv(w, srcp, None, lens[b])
        (po, pl), (uo, ul) = H.oracle_request(case, b, kv=kv)
        outs = H.run_decode(case)
        _sync()
        tol_o, tol_l = H.tolerance(w)
        for d in range(4):
            H.check_rows(f"partial d={d}", outs.partial_out[d, b].cpu().numpy(), outs.partial_lse[d, b].cpu().numpy(),
                         po[d], pl[d], tol_o, tol_l)
        H.check_rows("merged", outs.out[b].cpu().numpy(), outs.lse[b].cpu().numpy(), uo, ul, tol_o, tol_l)


# --------------------------------------------------------------------------- measurement aid


@pytest.mark.parametrize("kind,per_mfma", [(0, 2 * 16 * 16 * 32), (1, 2 * 16 * 16 * 128)])
def test_probe_mfma_counts_its_work(kind, per_mfma):
    """The MFMA rate probe reports the flops it issues (CUs x 8 wavefronts x iters x 8 MFMAs) and
    writes finite sums; its rate stays below the published dense peak."""
    sink = torch.full((K.PROBE_SINK_FLOATS,), float("nan"), dtype=torch.float32, device=DEV)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 500
    K.dcpkv_probe_mfma(kind, 10, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = K.dcpkv_probe_mfma(kind, iters, sink)
    e1.record()
    _sync()
    grid = min(cus, 1024)
    assert flops == grid * 8 * iters * 8 * per_mfma
    assert torch.isfinite(sink[:grid * 512]).all()
    rate = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    H.log(f"  probe kind {kind}: {rate:.0f} TFLOP/s")
    assert 0 < rate < (2600 if kind == 0 else 5200)


def test_probe_copy_pages_moves_listed_pages():
    """The page-list copy (the scattered-copy ceiling) moves page src_pages[i] to page
    dst_pages[i], skips entries outside either buffer, and touches nothing else."""
    for page_bytes, n_src, n_dst in ((256 * 1024, 40, 48), (36864, 70, 64), (48, 9, 9)):
        g = torch.Generator(device=DEV).manual_seed(page_bytes)
        src = torch.randint(0, 256, (n_src * page_bytes,), dtype=torch.uint8, device=DEV, generator=g)
        dst = torch.zeros(n_dst * page_bytes, dtype=torch.uint8, device=DEV)
        rng = np.random.default_rng(page_bytes)
        k = min(n_src, n_dst) - 2
        sp = rng.permutation(n_src)[:k].astype(np.int32)
        dp = rng.permutation(n_dst)[:k].astype(np.int32)
        sp[1], dp[2] = -1, n_dst  # skipped entries
        K.dcpkv_probe_copy_pages(src, dst, torch.from_numpy(sp).to(DEV), torch.from_numpy(dp).to(DEV), page_bytes)
        _sync()
        s2, d2 = src.view(n_src, page_bytes).cpu(), dst.view(n_dst, page_bytes).cpu()
        written = set()
        for i in range(k):
            if 0 <= sp[i] < n_src and 0 <= dp[i] < n_dst:
                assert torch.equal(d2[dp[i]], s2[sp[i]])
                written.add(int(dp[i]))
        for j in range(n_dst):
            if j not in written:
                assert (d2[j] == 0).all()


def test_probe_copy_copies_every_byte():
    """The streaming copy the reshard is read against moves its bytes exactly (odd sizes leave a
    short last segment; bytes past the end stay untouched)."""
    for nbytes in (16, 36864 * 3 + 48, (5 << 20) + 160):
        g = torch.Generator(device=DEV).manual_seed(nbytes)
        src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device=DEV, generator=g)
        dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
        K.dcpkv_probe_copy(src, dst, nbytes)
        _sync()
        assert torch.equal(dst[:nbytes], src[:nbytes]) and (dst[nbytes:] == 0).all()
