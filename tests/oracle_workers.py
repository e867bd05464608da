"""Worker-process side of the bench's CPU baseline: the float64 oracle on host copies
of the inputs, one unit of work per call.  Imports numpy and the oracle only (never
torch), so spawned workers start quickly and never touch a GPU."""

from __future__ import annotations

import time

import numpy as np

import oracle as O


def reshard_passes(args) -> int:
    """Scalar reshard passes over a host sample until the deadline; returns the pass count."""
    src_h, n_dst, shape, num_layers, dcp_size, own, page_size, rows, row_bytes, g2, deadline = args
    dst_h = [np.zeros(shape, np.uint8) for _ in range(n_dst)]
    n = shape[1]
    reps = 0
    while time.time() < deadline:
        if own:
            O.reshard_tokens(src_h, dst_h, num_layers, dcp_size, page_size, rows, row_bytes, np.arange(n),
                             np.arange(n), 0)
        else:
            O.reshard(src_h, dst_h, num_layers, dcp_size, np.arange(n), g2, 0)
        reps += 1
    return reps


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
    """Decode one request's pages, then its per-shard partials and their merge head by head
    until the deadline; returns (rows done, query-token pairs done)."""
    geo, pages_h, scales_h, host_by_slot, global_pages, seq_len, q, deadline = args
    if time.time() >= deadline:
        return 0, 0
    k, v = _logical_kv(geo, pages_h, scales_h, host_by_slot, global_pages, seq_len)
    rows = done = 0
    for h in range(geo["num_q_heads"]):
        po, pl = O.request_partials(q, k, v, seq_len, geo["softmax_scale"], global_pages, geo["page_size"],
                                    geo["dcp_size"], heads=[h], own=geo["own"])
        O.lse_merge(po[:, :, [h]], pl[:, :, [h]])
        rows += 1
        done += seq_len * geo["q_len"]
        if time.time() >= deadline:
            break
    return rows, done


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
