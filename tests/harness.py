"""Test harness: builds device inputs for a workload, runs the HIP path through
the C ABI and computes the oracle's expectation on the same inputs.

Inputs come from workloads.gen (seeded); the page map and block tables come
from the library (host code under test, checked against the oracle's own page
map); the oracle reads the inputs only (never a kernel output).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

import context_paged_kv_amd as K
import oracle as O
from workloads import gen
from workloads.configs import MLA_DIM, Workload


def kv_dtype_code(w: Workload) -> int:
    return {"f32": K.KV_F32, "bf16": K.KV_BF16, "fp8": K.KV_FP8E4M3}[w.kv_dtype]


def log(msg: str) -> None:
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# decode inputs
# ---------------------------------------------------------------------------


@dataclass
class DecodeCase:
    w: Workload
    seq_lens: np.ndarray
    pages: List[np.ndarray]            # global pages per request (library page map)
    max_local: int
    tables: np.ndarray                 # [N][B][max_local]
    pools: List[torch.Tensor]          # per shard uint8 [L][M][page_bytes]
    scales: Optional[List[torch.Tensor]]  # per shard int16 [L][M]
    q: torch.Tensor                    # [B][q_len][Hq][Dqk]
    bt_dev: torch.Tensor
    sl_dev: torch.Tensor
    layer: int = 0
    own: int = 0                       # K.OWN_PAGE or K.OWN_TOKEN

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.sum())


def page_map_pages(w: Workload, seq_lens: Sequence[int], check_oracle: bool = True) -> List[np.ndarray]:
    free = gen.draw_free_order(w)
    pm = K.PageMap(w.dcp_size, w.page_size, w.pool_pages, free)
    pages = [pm.alloc(int(t)) for t in seq_lens]
    pm.close()
    if check_oracle:  # host page map vs the oracle's, bit for bit
        opm = O.PageMap(w.dcp_size, w.page_size, w.pool_pages, free)
        for t, g in zip(seq_lens, pages):
            assert list(g) == opm.alloc(int(t))
    return pages


def alloc_pools(w: Workload, device, fill: str = "random", tag: str = "pool"):
    n, L, M, pb = w.dcp_size, w.num_layers, w.pool_pages, w.page_bytes
    pools, scales = [], [] if w.has_scales else None
    for d in range(n):
        p = torch.empty((L, M, pb), dtype=torch.uint8, device=device)
        s = torch.empty((L, M), dtype=torch.int16, device=device) if w.has_scales else None
        if fill == "random":
            gen.fill_pages_(p.view(L * M, pb), w, tag, sub=d, scales=None if s is None else s.view(-1))
        else:
            gen.sentinel_fill_(p, gen.DST_SENTINEL)
            if s is not None:
                s.fill_(gen.SCALE_SENTINEL)
        pools.append(p)
        if s is not None:
            scales.append(s)
    return pools, scales


def make_decode_case(w: Workload, device="cuda", seq_lens=None, pools=None, scales=None, own: int = 0) -> DecodeCase:
    sl = gen.draw_seq_lens(w) if seq_lens is None else np.asarray(seq_lens, dtype=np.int64)
    assert len(sl) == w.num_requests
    pages = page_map_pages(w, sl)
    max_local = max(1, max(-(-len(p) // w.dcp_size) for p in pages))
    tables, counts = K.dcp_build_block_tables(w.dcp_size, pages, max_local, token_interleave=own)
    if pools is None:
        pools, scales = alloc_pools(w, device)
    q = gen.draw_q(w, device)
    return DecodeCase(w=w, seq_lens=sl, pages=pages, max_local=max_local, tables=tables, pools=pools,
                      scales=scales, q=q, bt_dev=torch.from_numpy(tables).to(device),
                      sl_dev=torch.from_numpy(sl.astype(np.int32)).to(device), layer=w.attn_layer, own=own)


def attn_desc(case: DecodeCase, layer: Optional[int] = None):
    w = case.w
    return K.make_attn_desc(
        kv_dtype=kv_dtype_code(w), kv_layout=K.LAYOUT_MLA if w.layout == "mla" else K.LAYOUT_SPLIT,
        q_dtype=K.Q_BF16 if w.q_dtype == "bf16" else K.Q_F32, num_q_heads=w.num_q_heads,
        num_kv_heads=w.num_kv_heads, head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v,
        page_size=w.page_size, dcp_size=w.dcp_size, batch=w.num_requests, q_len=w.q_len,
        max_local_pages=case.max_local, layer=case.layer if layer is None else layer, num_layers=w.num_layers,
        pages_per_layer=w.pool_pages, softmax_scale=w.softmax_scale, token_interleave=case.own)


@dataclass
class DecodeOut:
    partial_out: torch.Tensor
    partial_lse: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor


def alloc_outputs(case: DecodeCase):
    w = case.w
    dev = case.q.device
    B, ql, hq, dv, n = w.num_requests, w.q_len, w.num_q_heads, w.head_dim_v, w.dcp_size
    desc = attn_desc(case)
    ws = torch.empty(K.dcp_decode_partial_workspace(desc, case.total_tokens), dtype=torch.uint8, device=dev)
    return DecodeOut(
        partial_out=torch.full((n, B, ql, hq, dv), float("nan"), dtype=torch.float32, device=dev),
        partial_lse=torch.full((n, B, ql, hq), float("nan"), dtype=torch.float32, device=dev),
        out=torch.full((B, ql, hq, dv), float("nan"), dtype=torch.float32, device=dev),
        lse=torch.full((B, ql, hq), float("nan"), dtype=torch.float32, device=dev)), ws


def run_decode(case: DecodeCase, outs: Optional[DecodeOut] = None, ws=None, layer=None,
               shard_begin=0, shard_count=None, merge=True) -> DecodeOut:
    w = case.w
    if outs is None:
        outs, ws = alloc_outputs(case)
    desc = attn_desc(case, layer)
    K.dcp_decode_partial(desc, q=case.q, kv_pools=case.pools, kv_scales=case.scales, block_tables=case.bt_dev,
                         seq_lens=case.sl_dev, total_tokens=case.total_tokens, partial_out=outs.partial_out,
                         partial_lse=outs.partial_lse, workspace=ws, shard_begin=shard_begin,
                         shard_count=shard_count)
    if merge:
        rows = w.num_requests * w.q_len * w.num_q_heads
        K.dcp_lse_merge(w.dcp_size, rows, w.head_dim_v, outs.partial_out, outs.partial_lse, outs.out, outs.lse)
    return outs


# ---------------------------------------------------------------------------
# oracle side
# ---------------------------------------------------------------------------


def gather_request_pages(pools, scales, pages, n: int, layer: int):
    """Host copies of one request's pages (and scales) in sequence order."""
    dev = pools[0].device
    owners = np.array([O.dcp_owner(int(g), n) for g in pages])
    slots = np.array([O.dcp_local_slot(int(g), n) for g in pages])
    pb = pools[0].shape[-1]
    out = np.empty((len(pages), pb), dtype=np.uint8)
    sc = np.empty(len(pages), dtype=np.int64) if scales is not None else None
    for d in range(n):
        idx = np.nonzero(owners == d)[0]
        if idx.size == 0:
            continue
        sl = torch.from_numpy(slots[idx]).to(dev)
        out[idx] = pools[d][layer].index_select(0, sl).cpu().numpy()
        if scales is not None:
            sc[idx] = scales[d][layer].index_select(0, sl).cpu().numpy().astype(np.int64) & 0xFFFF
    return out, sc


def oracle_logical_kv(w: Workload, page_bytes: np.ndarray, page_scales, seq_len: int):
    """Logical K, V of one request from its pages (host bytes, sequence order), decoded by the oracle."""
    if w.layout == "mla":
        lat = np.concatenate([O.decode_mla_page(page_bytes[i], int(page_scales[i]), w.page_size)
                              for i in range(len(page_bytes))], axis=0)[:seq_len]
        return lat[None], lat[None, :, :w.head_dim_v]
    ks, vs = zip(*[O.decode_split_page(page_bytes[i], w.kv_dtype, w.num_kv_heads, w.page_size, w.head_dim_qk)
                   for i in range(len(page_bytes))])
    return np.concatenate(ks, axis=1)[:, :seq_len], np.concatenate(vs, axis=1)[:, :seq_len]


def gather_token_layout_kv(case: DecodeCase, b: int, layer: int):
    """Logical K, V of request b under token ownership: host copies of every shard's pages at the
    request's virtual slots, read back token by token by the oracle."""
    w = case.w
    n = w.dcp_size
    pages = case.pages[b]
    vslots = [O.dcp_local_slot(int(pages[j]), n) for j in range(0, len(pages), n)]
    sl = torch.tensor(vslots, dtype=torch.int64, device=case.pools[0].device)
    host = {}
    for d in range(n):
        pb = case.pools[d][layer].index_select(0, sl).cpu().numpy()
        sc = (case.scales[d][layer].index_select(0, sl).cpu().numpy().astype(np.int64) & 0xFFFF
              if case.scales is not None else None)
        for i, s_ in enumerate(vslots):
            host[(d, s_)] = (pb[i], None if sc is None else int(sc[i]))
    T = int(case.seq_lens[b])
    if w.layout == "mla":
        return O.logical_kv_mla_tokens(lambda d, s_: host[(d, s_)], pages, n, w.page_size, T, w.head_dim_v)
    return O.logical_kv_split_tokens(lambda d, s_: host[(d, s_)][0], pages, n, w.kv_dtype, w.num_kv_heads,
                                     w.page_size, w.head_dim_qk, T)


def q_host(case: DecodeCase, b: int) -> np.ndarray:
    return case.q[b].float().cpu().numpy().astype(np.float64)


def oracle_request(case: DecodeCase, b: int, heads=None, kv=None, layer=None):
    """(partials O [N][q_len][Hq][Dv], LSE [N][q_len][Hq]), (unsharded O, LSE) for request b."""
    w = case.w
    lay = case.layer if layer is None else layer
    if kv is None and case.own:
        kv = gather_token_layout_kv(case, b, lay)
    if kv is None:
        pb, ps = gather_request_pages(case.pools, case.scales, case.pages[b], w.dcp_size, lay)
        kv = oracle_logical_kv(w, pb, ps, int(case.seq_lens[b]))
    k, v = kv
    q = q_host(case, b)
    T = int(case.seq_lens[b])
    po, pl = O.request_partials(q, k, v, T, w.softmax_scale, case.pages[b], w.page_size, w.dcp_size, heads,
                                own="token" if case.own else "page")
    uo, ul = O.request_attention(q, k, v, T, w.softmax_scale, None, heads)
    return (po, pl), (uo, ul)


def rel_row_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-row relative L2 error ||got - ref|| / ||ref|| over the last axis (0 when both are 0)."""
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def lse_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    both_inf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):
        return np.where(both_inf, 0.0, np.abs(got - ref))


def elem_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-element error |got_i - ref_i| / max_j |ref_j| over each row (the last axis); rows
    whose reference is all zero give the plain absolute error."""
    den = np.abs(ref).max(axis=-1, keepdims=True)
    return np.abs(got - ref) / np.where(den > 0, den, 1.0)


def check_rows(name, got_o, got_l, ref_o, ref_l, tol_o, tol_l):
    """Rows of outputs (last axis) and their LSEs against the oracle: every element within
    tol_o of its row's largest reference magnitude, every row's relative L2 error within
    tol_o, every |LSE error| within tol_l.  Returns the worst (row L2, LSE, element) errors."""
    got_o = np.asarray(got_o, np.float64)
    eo = rel_row_err(got_o, ref_o)
    el = lse_err(np.asarray(got_l, np.float64), ref_l)
    ee = elem_err(got_o, ref_o)
    assert np.isfinite(eo).all() and np.isfinite(ee).all(), f"{name}: non-finite output error"
    if ee.size and ee.max() > tol_o:
        at = np.unravel_index(int(np.argmax(ee)), ee.shape)
        raise AssertionError(f"{name}: element {at} off by {ee.max():.3e} of its row's largest value > {tol_o}")
    assert eo.size == 0 or eo.max() <= tol_o, f"{name}: max relative row error {eo.max():.3e} > {tol_o}"
    assert el.size == 0 or el.max() <= tol_l, f"{name}: max |LSE error| {el.max():.3e} > {tol_l}"
    return (float(eo.max()) if eo.size else 0.0, float(el.max()) if el.size else 0.0,
            float(ee.max()) if ee.size else 0.0)


def tolerance(w: Workload):
    # the stated bars: 1e-5 for fp32, 2e-3 relative for bf16 / fp8
    return (1e-5, 1e-5) if w.kv_dtype == "f32" else (2e-3, 2e-3)


def check_decode(case: DecodeCase, outs: DecodeOut, requests=None, heads=None, shards=None):
    """Compare partials, merged output and LSE with the oracle for the listed requests/heads."""
    w = case.w
    tol_o, tol_l = tolerance(w)
    n = w.dcp_size
    shards = range(n) if shards is None else shards
    hs = list(range(w.num_q_heads)) if heads is None else list(heads)
    worst = [0.0, 0.0, 0.0]
    for b in (range(w.num_requests) if requests is None else requests):
        (po, pl), (uo, ul) = oracle_request(case, b, heads=hs)
        for d in shards:
            e = check_rows(f"partial d={d} b={b}", outs.partial_out[d, b][:, hs].cpu().numpy(),
                           outs.partial_lse[d, b][:, hs].cpu().numpy(), po[d][:, hs], pl[d][:, hs], tol_o, tol_l)
            worst = [max(x, y) for x, y in zip(worst, e)]
        if shards == range(n):
            e = check_rows(f"merged b={b}", outs.out[b][:, hs].cpu().numpy(), outs.lse[b][:, hs].cpu().numpy(),
                           uo[:, hs], ul[:, hs], tol_o, tol_l)
            worst = [max(x, y) for x, y in zip(worst, e)]
    return worst


def fmt_worst(worst) -> str:
    return f"worst rel row {worst[0]:.2e}, lse {worst[1]:.2e}, element {worst[2]:.2e}"


def request_geo(case: DecodeCase) -> dict:
    w = case.w
    return {"layout": w.layout, "kv_dtype": w.kv_dtype, "num_kv_heads": w.num_kv_heads,
            "head_dim_qk": w.head_dim_qk, "head_dim_v": w.head_dim_v, "page_size": w.page_size,
            "dcp_size": w.dcp_size, "num_q_heads": w.num_q_heads, "q_len": w.q_len,
            "softmax_scale": w.softmax_scale, "own": "token" if case.own else "page"}


def check_decode_parallel(case: DecodeCase, outs: DecodeOut, heads_of, requests=None, layer=None, workers=None,
                          pages_of=None, label=""):
    """check_decode at full size: the oracle runs per request in spawned worker processes (numpy
    and the oracle only, one BLAS thread each), fed with host copies of the request's pages that
    this process gathers; heads_of(b) lists the query heads checked for request b.  pages_of(b),
    if given, returns (page bytes, page scales) of request b in sequence order instead of the
    pools' (e.g. the source pages of a reshard).  Every shard's partial and the merged output
    of those rows are compared element by element.  Returns the worst errors."""
    import multiprocessing as mp
    import os
    from tests import oracle_workers as OW

    w = case.w
    lay = case.layer if layer is None else layer
    tol_o, tol_l = tolerance(w)
    reqs = list(range(w.num_requests) if requests is None else requests)
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    got_po = outs.partial_out.cpu().numpy()
    got_pl = outs.partial_lse.cpu().numpy()
    got_o = outs.out.cpu().numpy()
    got_l = outs.lse.cpu().numpy()
    geo = request_geo(case)
    worst = [0.0, 0.0, 0.0]
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"

    def task(b):
        hs = list(heads_of(b))
        pages = case.pages[b]
        pages_h = scales_h = by_slot = None
        if pages_of is not None:
            pages_h, scales_h = pages_of(b)
        elif case.own:
            n = w.dcp_size
            vslots = [O.dcp_local_slot(int(pages[j]), n) for j in range(0, len(pages), n)]
            sl = torch.tensor(vslots, dtype=torch.int64, device=case.pools[0].device)
            by_slot = {}
            for d in range(n):
                pb = case.pools[d][lay].index_select(0, sl).cpu().numpy()
                sc = (case.scales[d][lay].index_select(0, sl).cpu().numpy().astype(np.int64) & 0xFFFF
                      if case.scales is not None else None)
                for i, s_ in enumerate(vslots):
                    by_slot[(d, s_)] = (pb[i], None if sc is None else int(sc[i]))
        else:
            pages_h, scales_h = gather_request_pages(case.pools, case.scales, pages, w.dcp_size, lay)
        return (geo, pages_h, scales_h, by_slot, pages, int(case.seq_lens[b]), q_host(case, b), hs), hs

    def compare(b, hs, res):
        nonlocal worst
        po, pl, uo, ul = res
        for d in range(w.dcp_size):
            e = check_rows(f"{label}partial d={d} b={b}", got_po[d, b][:, hs], got_pl[d, b][:, hs], po[d], pl[d],
                           tol_o, tol_l)
            worst = [max(x, y) for x, y in zip(worst, e)]
        e = check_rows(f"{label}merged b={b}", got_o[b][:, hs], got_l[b][:, hs], uo, ul, tol_o, tol_l)
        worst = [max(x, y) for x, y in zip(worst, e)]

    try:
        with mp.get_context("spawn").Pool(workers) as pool:
            pending = []
            done = 0
            for b in reqs:
                args, hs = task(b)
                pending.append((b, hs, pool.apply_async(OW.oracle_request_rows, (args,))))
                while len(pending) > workers:  # bounded host memory: one task queued per worker
                    b0, hs0, r0 = pending.pop(0)
                    compare(b0, hs0, r0.get())
                    done += 1
                    if done % 8 == 0:
                        log(f"  {label}{done} of {len(reqs)} requests match the oracle ({fmt_worst(worst)})")
            for b0, hs0, r0 in pending:
                compare(b0, hs0, r0.get())
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return worst


# ---------------------------------------------------------------------------
# reshard inputs
# ---------------------------------------------------------------------------


@dataclass
class ReshardCase:
    w: Workload
    num_layers: int
    num_sources: int
    src_pools: List[torch.Tensor]            # [|L_r|+1][S][pb]
    src_scales: Optional[List[torch.Tensor]]  # [|L_r|+1][S]
    dst_pools: List[torch.Tensor]            # [L][M][pb]
    dst_scales: Optional[List[torch.Tensor]]
    src_ids: np.ndarray                      # per entry
    dst_ids: np.ndarray                      # per entry (global pages)
    first_uncached: int
    src_pages: int


def make_source_pools(w: Workload, num_sources: int, S: int, device, tag="src"):
    pools, scales = [], [] if w.has_scales else None
    pb = w.page_bytes
    for r in range(num_sources):
        a, b = K.cp_layersplit_layer_range(w.num_layers, num_sources, r)
        slots = (b - a) + 1
        p = torch.empty((slots, S, pb), dtype=torch.uint8, device=device)
        s = torch.empty((slots, S), dtype=torch.int16, device=device) if w.has_scales else None
        gen.fill_pages_(p[:-1].reshape((slots - 1) * S, pb), w, tag, sub=r,
                        scales=None if s is None else s[:-1].reshape(-1))
        gen.sentinel_fill_(p[-1], gen.SRC_TRANSIENT_SENTINEL)  # transient slot: never read
        if s is not None:
            s[-1].fill_(gen.SCALE_SENTINEL)
        pools.append(p)
        if s is not None:
            scales.append(s)
    return pools, scales


def make_reshard_case(w: Workload, device="cuda", seq_lens=None, requests=None, first_uncached=None,
                      dst_pools=None, dst_scales=None) -> ReshardCase:
    """One transfer: the listed requests' pages (concatenated) from the layer-split sources."""
    sl = gen.draw_seq_lens(w) if seq_lens is None else np.asarray(seq_lens, dtype=np.int64)
    pages = page_map_pages(w, sl)
    reqs = range(len(sl)) if requests is None else requests
    dst_ids = np.concatenate([pages[b] for b in reqs]).astype(np.int64)
    P = len(dst_ids)
    S = P
    src_ids = gen.draw_src_order(w, S)[:P].astype(np.int64)
    src_pools, src_scales = make_source_pools(w, w.num_sources, S, device)
    if dst_pools is None:
        dst_pools, dst_scales = alloc_pools(w, device, fill="sentinel")
    c = int(math.floor(w.cached_frac * P)) if first_uncached is None else first_uncached
    return ReshardCase(w=w, num_layers=w.num_layers, num_sources=w.num_sources, src_pools=src_pools,
                       src_scales=src_scales, dst_pools=dst_pools, dst_scales=dst_scales, src_ids=src_ids,
                       dst_ids=dst_ids, first_uncached=c, src_pages=S)


def run_reshard(rc: ReshardCase, dst_filter=-1, bad=None, src_ids=None, dst_ids=None, stream=None,
                pages_per_dst=None):
    w = rc.w
    dev = rc.src_pools[0].device
    si = torch.from_numpy((rc.src_ids if src_ids is None else src_ids).astype(np.int32)).to(dev)
    di = torch.from_numpy((rc.dst_ids if dst_ids is None else dst_ids).astype(np.int64)).to(dev)
    K.kv_reshard_pages(num_layers=rc.num_layers, dcp_size=w.dcp_size, page_bytes=w.page_bytes,
                       src_pages=rc.src_pages, dst_pages=w.pool_pages, src_pools=rc.src_pools,
                       dst_pools=rc.dst_pools, src_page_ids=si, dst_global_pages=di,
                       first_uncached=rc.first_uncached, dst_filter=dst_filter, src_scales=rc.src_scales,
                       dst_scales=rc.dst_scales, bad_entries=bad, pages_per_dst=pages_per_dst, stream=stream)
    return si, di


def run_path_pack(rc: ReshardCase, cap_units: int, stream=None, src_ids=None, dst_ids=None, check_windows=None):
    """The reshard done path by path through a staging buffer of cap_units pages: for every
    destination d, kv_path_entries, then for every source r the windows of kv_pack_pages /
    kv_unpack_pages.  check_windows(d, r, u0, staging, staging_scales, n) is called after each
    pack (synchronised).  Returns the number of units moved."""
    w = rc.w
    dev = rc.src_pools[0].device
    si = torch.from_numpy((rc.src_ids if src_ids is None else src_ids).astype(np.int32)).to(dev)
    di = torch.from_numpy((rc.dst_ids if dst_ids is None else dst_ids).astype(np.int64)).to(dev)
    P = si.numel()
    geo = dict(num_sources=rc.num_sources, num_layers=rc.num_layers, dcp_size=w.dcp_size, page_bytes=w.page_bytes,
               src_pages=rc.src_pages, dst_pages=w.pool_pages)
    pos = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    cnt = torch.empty(1, dtype=torch.int64, device=dev)
    nout = torch.empty(1, dtype=torch.int64, device=dev)
    stg = torch.empty((cap_units, w.page_bytes), dtype=torch.uint8, device=dev)
    stg_sc = torch.empty(cap_units, dtype=torch.int16, device=dev) if rc.src_scales is not None else None
    moved = 0
    for d in range(w.dcp_size):
        K.kv_path_entries(dest=d, src_page_ids=si, dst_global_pages=di, out_positions=pos, out_count=cnt,
                          first_uncached=rc.first_uncached, stream=stream, **geo)
        count = int(cnt.item())
        for r in range(rc.num_sources):
            a, b = K.cp_layersplit_layer_range(rc.num_layers, rc.num_sources, r)
            total = count * (b - a)
            for u0 in range(0, total, cap_units):
                if check_windows is not None:
                    gen.sentinel_fill_(stg, gen.DST_SENTINEL)
                    if stg_sc is not None:
                        stg_sc.fill_(gen.SCALE_SENTINEL)
                K.kv_pack_pages(source=r, src_pool=rc.src_pools[r], src_page_ids=si, positions=pos, count=cnt,
                                unit_begin=u0, cap_units=cap_units, staging=stg,
                                src_scales=None if rc.src_scales is None else rc.src_scales[r],
                                staging_scales=stg_sc, out_units=nout, stream=stream, **geo)
                if check_windows is not None:
                    torch.cuda.synchronize()
                    check_windows(d, r, u0, stg, stg_sc, int(nout.item()), pos, count)
                K.kv_unpack_pages(source=r, dest=d, dst_pool=rc.dst_pools[d], dst_global_pages=di, positions=pos,
                                  count=cnt, unit_begin=u0, cap_units=cap_units, staging=stg,
                                  dst_scales=None if rc.dst_scales is None else rc.dst_scales[d],
                                  staging_scales=stg_sc, stream=stream, **geo)
                moved += min(cap_units, total - u0)
    return moved


def token_geometry(w: Workload):
    """(token_rows, row_bytes) of the workload's page layout for the token reshard."""
    if w.layout == "mla":
        return 1, 576
    return 2 * w.num_kv_heads, w.head_dim_qk * w.elem_bytes


def run_reshard_tokens(rc: ReshardCase, bad=None, src_ids=None, dst_ids=None, request_offsets=None, stream=None):
    """kv_reshard_tokens over the case's lists; request_offsets (host ints, B + 1) splits them into
    requests, None passes one request."""
    w = rc.w
    dev = rc.src_pools[0].device
    si = torch.from_numpy((rc.src_ids if src_ids is None else src_ids).astype(np.int32)).to(dev)
    di = torch.from_numpy((rc.dst_ids if dst_ids is None else dst_ids).astype(np.int64)).to(dev)
    ro = (torch.tensor(np.asarray(request_offsets, dtype=np.int64), device=dev)
          if request_offsets is not None else None)
    R, rb = token_geometry(w)
    K.kv_reshard_tokens(num_layers=rc.num_layers, dcp_size=w.dcp_size, page_size=w.page_size, token_rows=R,
                        row_bytes=rb, src_pages=rc.src_pages, dst_pages=w.pool_pages, src_pools=rc.src_pools,
                        dst_pools=rc.dst_pools, src_page_ids=si, dst_global_pages=di,
                        first_uncached=rc.first_uncached, request_offsets=ro, bad_entries=bad, stream=stream)
    return si, di


def check_reshard_by_plan(rc: ReshardCase, dst_filter=-1, sentinel=gen.DST_SENTINEL):
    """Bit-exact check of every destination page against the oracle's copy plan.

    The plan (which source page lands where) is the oracle's; the byte compare
    runs on the device with torch indexing.  Pages outside the plan must still
    hold the sentinel; sources must be unchanged (checked by the caller)."""
    w = rc.w
    n, L, M = w.dcp_size, rc.num_layers, w.pool_pages
    plan = O.reshard_plan(L, rc.num_sources, n, rc.src_ids, rc.dst_ids, rc.first_uncached, dst_filter)
    dev = rc.dst_pools[0].device
    arr = np.asarray(plan, dtype=np.int64).reshape(-1, 6)
    touched = [np.zeros((L, M), dtype=bool) for _ in range(n)]
    for d in range(n):
        sel = arr[arr[:, 3] == d]
        touched[d][sel[:, 4], sel[:, 5]] = True
        for r in range(rc.num_sources):
            s2 = sel[sel[:, 0] == r]
            if s2.size == 0:
                continue
            for start in range(0, len(s2), 4096):
                blk = s2[start:start + 4096]
                src_flat = rc.src_pools[r].view(-1, w.page_bytes)
                dst_flat = rc.dst_pools[d].view(-1, w.page_bytes)
                si = torch.from_numpy(blk[:, 1] * rc.src_pages + blk[:, 2]).to(dev)
                di = torch.from_numpy(blk[:, 4] * M + blk[:, 5]).to(dev)
                want = src_flat.index_select(0, si)
                got = dst_flat.index_select(0, di)
                assert torch.equal(got, want), f"page bytes differ (d={d}, source {r})"
                if rc.src_scales is not None:
                    assert torch.equal(rc.dst_scales[d].view(-1).index_select(0, di),
                                       rc.src_scales[r].view(-1).index_select(0, si)), "scales differ"
        for layer in range(L):
            mask = torch.from_numpy(~touched[d][layer]).to(dev)
            rest = rc.dst_pools[d][layer][mask]
            assert bool((rest == sentinel).all()), f"untouched pages of d={d} layer={layer} changed"
            if rc.dst_scales is not None:
                assert bool((rc.dst_scales[d][layer][mask] == gen.SCALE_SENTINEL).all())
    return len(plan)
