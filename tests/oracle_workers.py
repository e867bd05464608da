"""Worker-process side of the bench's CPU baseline: the float64 oracle on host copies
of the inputs, one unit of work per call.  Imports numpy and the oracle only (never
torch), so spawned workers start quickly and never touch a GPU."""

from __future__ import annotations

import time

import numpy as np

import oracle as O


def reshard_sample(args):
    """Scalar reshard passes until the deadline over this worker's own page set: the sample pages
    (one layer per source) tiled into about target_bytes of distinct source pages per source, moved
    into N pools of their own.  Returns (bytes read + written, pages per source)."""
    sample, page_bytes, dcp_size, own, page_size, rows, row_bytes, target_bytes, deadline = args
    n_src = len(sample)
    pages = max(1, int(target_bytes // (page_bytes * n_src)))
    src_h = []
    for r in range(n_src):
        t = np.empty((2, pages, page_bytes), np.uint8)  # one layer + the transient slot
        t[0] = np.resize(sample[r], (pages, page_bytes))
        t[1] = 0x5A
        src_h.append(t)
    m = -(-pages // dcp_size)
    dst_h = [np.zeros((n_src, m, page_bytes), np.uint8) for _ in range(dcp_size)]
    ids = np.arange(pages)
    moved = 0
    while time.time() < deadline:
        if own:
            O.reshard_tokens(src_h, dst_h, n_src, dcp_size, page_size, rows, row_bytes, ids, ids, 0)
        else:
            O.reshard(src_h, dst_h, n_src, dcp_size, ids, ids, 0)
        moved += 2 * pages * n_src * page_bytes
    return moved, pages


def _logical_kv(geo: dict, pages_h, scales_h, host_by_slot, global_pages, seq_len: int):
    """Logical K, V of one request from host page bytes: in sequence order (page ownership) or
    by (shard, slot) (token ownership)."""
    n, ps = geo["dcp_size"], geo["page_size"]
    if host_by_slot is not None:
        if geo["layout"] == "mla":
            return O.logical_kv_mla_tokens(lambda d, s: host_by_slot[(d, s)], global_pages, n, ps, seq_len,
                                           geo["head_dim_v"])
        return O.logical_kv_split_tokens(lambda d, s: host_by_slot[(d, s)][0], global_pages, n, geo["kv_dtype"],
                                         geo["num_kv_heads"], ps, geo["head_dim_qk"], seq_len)
    if geo["layout"] == "mla":
        lat = np.concatenate([O.decode_mla_page(pages_h[i], int(scales_h[i]), ps) for i in range(len(pages_h))],
                             axis=0)[:seq_len]
        return lat[None], lat[None, :, :geo["head_dim_v"]]
    ks, vs = zip(*[O.decode_split_page(pages_h[i], geo["kv_dtype"], geo["num_kv_heads"], ps, geo["head_dim_qk"])
                   for i in range(len(pages_h))])
    return np.concatenate(ks, axis=1)[:, :seq_len], np.concatenate(vs, axis=1)[:, :seq_len]


def request_rows(args):
    """Decode one request's pages, then its per-shard partials and their merge head by head until
    the deadline.  Returns (decode seconds, tokens decoded, head seconds, (token, query, head)
    triples done, heads done)."""
    geo, pages_h, scales_h, host_by_slot, global_pages, seq_len, q, deadline = args
    if time.time() >= deadline:
        return 0.0, 0, 0.0, 0, 0
    t0 = time.perf_counter()
    k, v = _logical_kv(geo, pages_h, scales_h, host_by_slot, global_pages, seq_len)
    t1 = time.perf_counter()
    heads = 0
    for h in range(geo["num_q_heads"]):
        po, pl = O.request_partials(q, k, v, seq_len, geo["softmax_scale"], global_pages, geo["page_size"],
                                    geo["dcp_size"], heads=[h], own=geo["own"])
        O.lse_merge(po[:, :, [h]], pl[:, :, [h]])
        heads += 1
        if time.time() >= deadline:
            break
    t2 = time.perf_counter()
    return t1 - t0, seq_len, t2 - t1, heads * seq_len * geo["q_len"], heads


def oracle_request_rows(args):
    """The oracle's per-shard partials and unsharded attention of one request, for the listed
    heads only: (partial O [N][q_len][H'][Dv], partial LSE [N][q_len][H'], O [q_len][H'][Dv],
    LSE [q_len][H'])."""
    geo, pages_h, scales_h, host_by_slot, global_pages, seq_len, q, heads = args
    k, v = _logical_kv(geo, pages_h, scales_h, host_by_slot, global_pages, seq_len)
    po, pl = O.request_partials(q, k, v, seq_len, geo["softmax_scale"], global_pages, geo["page_size"],
                                geo["dcp_size"], heads=heads, own=geo["own"])
    uo, ul = O.request_attention(q, k, v, seq_len, geo["softmax_scale"], None, heads)
    return po[:, :, heads], pl[:, :, heads], uo[:, heads], ul[:, heads]


def warm(_):
    """No work: lets the pool start its processes before the timed region."""
    return 0
