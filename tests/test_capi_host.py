"""C-ABI library on the CPU: exported symbols, host logic against the oracle,
and argument errors that return before anything reaches a GPU."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import context_paged_kv_amd as K
import oracle as O
from context_paged_kv_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dcpkv.h")
# under DCPKV_HOST_ONLY=1 the binding loads the host part alone (the sanitizer build): the tests
# of device entry points' argument checks need the whole library
device_symbols = pytest.mark.skipif(L.HOST_ONLY, reason="host-only build of the library")


def declared_symbols():
    txt = open(HEADER).read()
    return re.findall(r"^DCPKV_API[^;(]*?\b(\w+)\s*\(", txt, flags=re.M)


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 14
    lib = C.CDLL(L.LIB_PATH)
    for n in (L.HOST_SYMBOLS if L.HOST_ONLY else names):
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)
    assert set(L.HOST_SYMBOLS) <= set(names)
    assert K.dcpkv_abi_version() == 7 == L.ABI_VERSION


@device_symbols
def test_graft_build_entry_accepts_the_built_library(monkeypatch):
    """build() compiles and then checks the library's ABI; with the compile step stubbed the
    check runs against the library already built."""
    import __graft_entry__ as G
    from context_paged_kv_amd import build as B

    monkeypatch.setattr(B, "build", lambda *a, **k: None)
    G.build()


@pytest.mark.parametrize("L_,n", [(78, 8), (64, 4), (4, 4), (17, 5), (1, 1), (100, 7)])
def test_layer_range_matches_oracle(L_, n):
    for r in range(n):
        assert K.cp_layersplit_layer_range(L_, n, r) == O.layer_range(L_, n, r)


def test_layer_range_errors():
    for args in [(3, 8, 0), (8, 0, 0), (8, 4, 4), (8, 4, -1)]:
        with pytest.raises(L.DcpkvError) as e:
            K.cp_layersplit_layer_range(*args)
        assert e.value.code == L.DCPKV_EINVAL


def test_filter_matches_oracle():
    rng = np.random.default_rng(2)
    idx = rng.permutation(500)[:300]
    for n in (1, 2, 4, 8):
        for d in range(n):
            assert list(K.dcp_filter_kv_indices(idx, n, d)) == O.filter_kv_indices_for_dcp_rank(idx, n, d)
    assert len(K.dcp_filter_kv_indices(range(256), 4, 3)) == 64
    with pytest.raises(L.DcpkvError):
        K.dcp_filter_kv_indices([1, -2], 4, 0)
    with pytest.raises(L.DcpkvError):
        K.dcp_filter_kv_indices([1, 2], 4, 4)


@pytest.mark.parametrize("n,page,M", [(1, 16, 40), (2, 16, 64), (4, 64, 97), (8, 64, 300)])
def test_pagemap_matches_oracle(n, page, M):
    rng = np.random.default_rng(n * 1000 + M)
    free = rng.permutation(M)
    pm = K.PageMap(n, page, M, free)
    om = O.PageMap(n, page, M, free)
    live = []
    for step in range(60):
        if live and rng.random() < 0.35:
            g = live.pop(int(rng.integers(len(live))))
            rel = [int(x) for x in rng.permutation(np.asarray(g))] + [int(x) for x in g[:2]]  # shuffled, repeats
            pm.release(rel)
            om.release(rel)
        else:
            T = int(rng.integers(1, page * n * 6))
            try:
                want = om.alloc(T)
            except MemoryError:
                with pytest.raises(L.DcpkvError) as e:
                    pm.alloc(T)
                assert e.value.code == L.DCPKV_ENOSPC
                continue
            got = pm.alloc(T)
            assert list(got) == want
            live.append(got)
        assert pm.num_free() == len(om.free)


def test_pagemap_errors():
    with pytest.raises(L.DcpkvError):
        K.PageMap(0, 64, 10)
    with pytest.raises(L.DcpkvError):
        K.PageMap(4, 64, 3, [0, 0, 1])
    pm = K.PageMap(2, 4, 4)
    g = pm.alloc(9)
    pm.release(g)
    with pytest.raises(L.DcpkvError):  # double free
        pm.release(g)
    with pytest.raises(L.DcpkvError):
        pm.release([10**6])
    with pytest.raises(L.DcpkvError):
        pm.alloc(0)


@pytest.mark.parametrize("own", [0, 1])
def test_block_tables_match_oracle(own):
    rng = np.random.default_rng(5)
    n, page, M = 4, 16, 200
    om = O.PageMap(n, page, M, rng.permutation(M))
    pages = [om.alloc(int(t)) for t in rng.integers(1, 600, size=9)]
    mx = max(-(-len(p) // n) for p in pages) + 2
    tables, counts = K.dcp_build_block_tables(n, pages, mx, token_interleave=own)
    want = O.block_tables(pages, n, "token" if own else "page")
    for d in range(n):
        for b in range(len(pages)):
            c = counts[d, b]
            assert list(tables[d, b, :c]) == want[d][b]
            assert (tables[d, b, c:] == -1).all()
    # placement where sequence page i is not on rank i mod N is rejected
    with pytest.raises(L.DcpkvError):
        K.dcp_build_block_tables(4, [[1, 0, 2, 3]], 4)
    with pytest.raises(L.DcpkvError):  # too narrow
        K.dcp_build_block_tables(n, pages, 1, token_interleave=own)
    with pytest.raises(L.DcpkvError):  # unknown ownership mode
        K.dcp_build_block_tables(n, pages, mx, token_interleave=2)


def test_token_block_tables_need_one_slot_per_virtual_page():
    """Under token ownership every shard reads virtual page j at one slot: pages with the right
    residues but in different slots are rejected (page ownership does not care)."""
    n = 4
    ok = [0 * n + 0, 0 * n + 1, 0 * n + 2, 0 * n + 3, 7 * n + 0, 7 * n + 1]
    mixed = [0 * n + 0, 0 * n + 1, 5 * n + 2, 0 * n + 3, 7 * n + 0, 7 * n + 1]  # page 2 in slot 5
    tail = [0 * n + 0, 0 * n + 1, 0 * n + 2, 0 * n + 3, 7 * n + 0, 8 * n + 1]   # page 5 in slot 8
    tables, _ = K.dcp_build_block_tables(n, [ok], 2, token_interleave=1)
    assert [list(tables[d, 0]) for d in range(n)] == [[0, 7]] * n
    for bad in (mixed, tail):
        with pytest.raises(L.DcpkvError) as e:
            K.dcp_build_block_tables(n, [bad], 2, token_interleave=1)
        assert e.value.code == L.DCPKV_EINVAL and "slot of virtual page" in str(e.value)
        K.dcp_build_block_tables(n, [bad], 2, token_interleave=0)  # page ownership: valid


def test_check_unique_pages():
    """The reshard's one-writer precondition: repeats among the uncached entries are found and
    the first list position that repeats is reported; cached entries do not count."""
    rng = np.random.default_rng(11)
    g = rng.permutation(10_000)[:3000]
    assert K.kv_check_unique_pages(g) == -1
    for first, at in ((0, 2999), (0, 1), (0, 1500), (100, 101)):
        h = g.copy()
        h[at] = h[first if first < at - 1 else at - 1]
        with pytest.raises(L.DcpkvError) as e:
            K.kv_check_unique_pages(h)
        assert e.value.code == L.DCPKV_EINVAL and e.value.first_duplicate == at
    h = g.copy()
    h[5] = h[2]            # a repeat whose first copy is cached is no repeat of the call
    assert K.kv_check_unique_pages(h, first_uncached=3) == -1
    with pytest.raises(L.DcpkvError) as e:
        K.kv_check_unique_pages(h, first_uncached=2)
    assert e.value.first_duplicate == 5
    h = np.array([4, 9, 4, 9, 4])
    with pytest.raises(L.DcpkvError) as e:
        K.kv_check_unique_pages(h)
    assert e.value.first_duplicate == 2
    assert K.kv_check_unique_pages([]) == -1
    assert L._lib.kv_check_unique_pages(None, 4, 0, None) == L.DCPKV_EINVAL
    assert L._lib.kv_check_unique_pages(None, 4, 5, None) == L.DCPKV_EINVAL


@device_symbols
def test_device_entry_points_reject_bad_arguments_on_host():
    d = L.kv_reshard_desc(1, 1, 2, -1, 100, 4, 4)  # page_bytes not a multiple of 16
    p = (C.c_void_p * 2)(16, 16)
    rc = L._lib.kv_reshard_pages(C.byref(d), p, p, None, None, C.c_void_p(16), C.c_void_p(16), 4, 0, None, None, None)
    assert rc == L.DCPKV_EINVAL and "page_bytes" in K.dcpkv_last_error()
    d = L.kv_reshard_desc(2, 1, 2, -1, 64, 4, 4)  # fewer layers than sources
    assert L._lib.kv_reshard_pages(C.byref(d), p, p, None, None, None, None, 4, 0, None, None, None) == L.DCPKV_EINVAL
    d = L.kv_reshard_desc(1, 1, 2, -1, 64, 4, 4)
    assert L._lib.kv_reshard_pages(C.byref(d), p, p, None, None, None, None, 4, 5, None, None, None) == L.DCPKV_EINVAL
    # nothing to copy is a no-op success even without a GPU
    assert L._lib.kv_reshard_pages(C.byref(d), p, p, None, None, None, None, 4, 4, None, None, None) == 0
    assert L._lib.dcp_lse_merge(0, 4, 4, None, None, None, None, None) == L.DCPKV_EINVAL
    assert L._lib.dcp_lse_merge(2, 0, 4, None, None, None, None, None) == 0
    good = K.make_attn_desc(kv_dtype=K.KV_BF16, kv_layout=K.LAYOUT_SPLIT, q_dtype=K.Q_BF16, num_q_heads=32,
                            num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64, dcp_size=4, batch=2,
                            q_len=1, max_local_pages=4, layer=0, num_layers=1, pages_per_layer=16, softmax_scale=0.1)
    assert K.dcp_decode_partial_workspace(good, 1000) > 0
    bad = K.make_attn_desc(kv_dtype=K.KV_FP8E4M3, kv_layout=K.LAYOUT_SPLIT, q_dtype=K.Q_BF16, num_q_heads=32,
                           num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64, dcp_size=4, batch=2,
                           q_len=1, max_local_pages=4, layer=0, num_layers=1, pages_per_layer=16, softmax_scale=0.1)
    assert L._lib.dcp_decode_partial_workspace(C.byref(bad), 1000) == 0
    # the chunk reduction launches one block per 4 query rows, at most 65535 of them
    edge = dict(kv_dtype=K.KV_F32, kv_layout=K.LAYOUT_SPLIT, q_dtype=K.Q_F32, num_q_heads=4, num_kv_heads=4,
                head_dim_qk=64, head_dim_v=64, page_size=16, dcp_size=2, batch=1, max_local_pages=4, layer=0,
                num_layers=1, pages_per_layer=16, softmax_scale=0.1)
    assert K.dcp_decode_partial_workspace(K.make_attn_desc(q_len=65535, **edge), 1000) > 0
    big = K.make_attn_desc(q_len=65536, **edge)
    assert L._lib.dcp_decode_partial_workspace(C.byref(big), 1000) == 0
    rc = L._lib.dcp_decode_partial(C.byref(big), C.c_void_p(256), p, None, C.c_void_p(256), C.c_void_p(256), 0,
                                   0, 2, C.c_void_p(256), C.c_void_p(256), C.c_void_p(256), 1 << 30, None)
    assert rc == L.DCPKV_EINVAL and "limit" in K.dcpkv_last_error()
    rc = L._lib.dcp_decode_partial(C.byref(good), None, None, None, None, None, 0, 0, 4, None, None, None, 0, None)
    assert rc == L.DCPKV_EINVAL
    rc = L._lib.dcp_decode_partial(C.byref(good), C.c_void_p(256), p, None, C.c_void_p(256), C.c_void_p(256), 0,
                                   2, 3, C.c_void_p(256), C.c_void_p(256), C.c_void_p(256), 1 << 30, None)
    assert rc == L.DCPKV_EINVAL and "shard range" in K.dcpkv_last_error()
    # a misaligned per-destination count array, query or output is refused before any launch
    d = L.kv_reshard_desc(1, 1, 2, -1, 64, 4, 4)
    rc = L._lib.kv_reshard_pages(C.byref(d), p, p, None, None, C.c_void_p(256), C.c_void_p(256), 4, 0, None,
                                 C.c_void_p(260), None)
    assert rc == L.DCPKV_EINVAL and "pages_per_dst" in K.dcpkv_last_error()
    q4 = (C.c_void_p * 4)(256, 256, 256, 256)
    for q, po in ((264, 256), (256, 260)):
        rc = L._lib.dcp_decode_partial(C.byref(good), C.c_void_p(q), q4, None, C.c_void_p(256), C.c_void_p(256),
                                       0, 0, 4, C.c_void_p(po), C.c_void_p(256), C.c_void_p(256), 1 << 30, None)
        assert rc == L.DCPKV_EINVAL and "aligned" in K.dcpkv_last_error()
    q4m = (C.c_void_p * 4)(256, 264, 256, 256)
    rc = L._lib.dcp_decode_partial(C.byref(good), C.c_void_p(256), q4m, None, C.c_void_p(256), C.c_void_p(256),
                                   0, 0, 4, C.c_void_p(256), C.c_void_p(256), C.c_void_p(256), 1 << 30, None)
    assert rc == L.DCPKV_EINVAL and "pool 1" in K.dcpkv_last_error()
    assert L._lib.dcp_lse_merge(2, 4, 4, C.c_void_p(264), C.c_void_p(256), C.c_void_p(256), None,
                                None) == L.DCPKV_EINVAL
    # the softmax scale must be positive and finite
    for sc in (0.0, -0.1, float("inf"), float("nan")):
        bad_sc = K.make_attn_desc(kv_dtype=K.KV_BF16, kv_layout=K.LAYOUT_SPLIT, q_dtype=K.Q_BF16, num_q_heads=32,
                                  num_kv_heads=8, head_dim_qk=128, head_dim_v=128, page_size=64, dcp_size=4,
                                  batch=2, q_len=1, max_local_pages=4, layer=0, num_layers=1, pages_per_layer=16,
                                  softmax_scale=sc)
        assert L._lib.dcp_decode_partial_workspace(C.byref(bad_sc), 1000) == 0
        rc = L._lib.dcp_decode_partial(C.byref(bad_sc), C.c_void_p(256), q4, None, C.c_void_p(256),
                                       C.c_void_p(256), 0, 0, 4, C.c_void_p(256), C.c_void_p(256), C.c_void_p(256),
                                       1 << 30, None)
        assert rc == L.DCPKV_EINVAL and "softmax_scale" in K.dcpkv_last_error()


@device_symbols
def test_path_entry_points_reject_bad_arguments_on_host():
    """The bounded-pack calls check their arguments before anything is enqueued."""
    v = C.c_void_p(256)
    good = L.kv_reshard_desc(2, 4, 2, -1, 64, 8, 8)
    odd = L.kv_reshard_desc(2, 4, 2, -1, 72, 8, 8)  # page_bytes not a multiple of 16
    E = L.DCPKV_EINVAL
    assert L._lib.kv_path_entries(None, 0, v, v, 4, 0, v, v, None) == E
    assert L._lib.kv_path_entries(C.byref(good), 2, v, v, 4, 0, v, v, None) == E  # dest outside [0, N)
    assert L._lib.kv_path_entries(C.byref(good), 0, v, v, 4, 5, v, v, None) == E  # first_uncached > num_pages
    assert L._lib.kv_path_entries(C.byref(good), 0, v, v, 4, 0, None, v, None) == E
    assert L._lib.kv_path_entries(C.byref(good), 0, v, v, 1 << 31, 0, v, v, None) == E
    assert L._lib.kv_pack_pages(C.byref(odd), 0, v, None, v, v, v, 0, 4, v, None, None, None) == E
    assert L._lib.kv_pack_pages(C.byref(good), 2, v, None, v, v, v, 0, 4, v, None, None, None) == E  # source
    assert L._lib.kv_pack_pages(C.byref(good), 0, v, None, v, v, v, 0, 0, v, None, None, None) == E  # cap 0
    assert L._lib.kv_pack_pages(C.byref(good), 0, v, None, v, v, v, -1, 4, v, None, None, None) == E
    assert L._lib.kv_pack_pages(C.byref(good), 0, v, v, v, v, v, 0, 4, v, None, None, None) == E  # one scale side
    rc = L._lib.kv_pack_pages(C.byref(good), 0, C.c_void_p(264), None, v, v, v, 0, 4, v, None, None, None)
    assert rc == E and "aligned" in K.dcpkv_last_error()
    assert L._lib.kv_unpack_pages(C.byref(good), 0, 2, v, None, v, v, v, 0, 4, v, None, None) == E  # dest
    assert L._lib.kv_unpack_pages(C.byref(good), 0, 0, v, v, v, v, v, 0, 4, v, None, None) == E  # one scale side
    assert L._lib.kv_unpack_pages(C.byref(good), 0, 0, None, None, v, v, v, 0, 4, v, None, None) == E


@device_symbols
def test_token_reshard_rejects_bad_arguments_on_host():
    p = (C.c_void_p * 4)(256, 256, 256, 256)
    v = C.c_void_p(256)
    E = L.DCPKV_EINVAL
    call = L._lib.kv_reshard_tokens
    bad_rows = L.kv_token_reshard_desc(1, 2, 2, 64, 2, 72, 8, 8)     # row_bytes not a multiple of 16
    assert call(C.byref(bad_rows), p, p, v, v, 4, None, 1, 0, None, None) == E
    few_layers = L.kv_token_reshard_desc(2, 1, 2, 64, 1, 576, 8, 8)  # fewer layers than sources
    assert call(C.byref(few_layers), p, p, v, v, 4, None, 1, 0, None, None) == E
    good = L.kv_token_reshard_desc(1, 2, 2, 64, 1, 576, 8, 8)
    assert call(C.byref(good), p, p, v, v, 4, None, 1, 5, None, None) == E  # first_uncached
    assert call(C.byref(good), p, p, None, None, 4, None, 1, 0, None, None) == E
    assert call(C.byref(good), p, p, None, None, 4, None, 1, 4, None, None) == 0  # nothing to move
    assert call(C.byref(good), p, p, v, v, 4, None, 2, 0, None, None) == E  # two requests, no offsets
    assert call(C.byref(good), p, p, v, v, 4, v, 0, 0, None, None) == E     # offsets, no request
    assert call(C.byref(good), p, p, v, v, 4, None, -1, 0, None, None) == E
    mis = (C.c_void_p * 2)(264, 256)
    assert call(C.byref(good), mis, p, v, v, 4, None, 1, 0, None, None) == E


@device_symbols
def test_probe_rejects_bad_arguments_on_host():
    v = C.c_void_p(256)
    flops = C.c_int64(0)
    E = L.DCPKV_EINVAL
    assert L._lib.dcpkv_probe_mfma(2, 10, v, L.PROBE_SINK_FLOATS, C.byref(flops), None) == E  # kind
    assert L._lib.dcpkv_probe_mfma(0, 0, v, L.PROBE_SINK_FLOATS, C.byref(flops), None) == E   # iters
    assert L._lib.dcpkv_probe_mfma(0, 10, v, L.PROBE_SINK_FLOATS - 1, C.byref(flops), None) == E
    assert L._lib.dcpkv_probe_mfma(0, 10, None, L.PROBE_SINK_FLOATS, C.byref(flops), None) == E
    assert L._lib.dcpkv_probe_mfma(1, 10, v, L.PROBE_SINK_FLOATS, None, None) == E
    assert L._lib.dcpkv_probe_copy(v, C.c_void_p(1 << 20), 100, None) == E          # not a multiple of 16
    assert L._lib.dcpkv_probe_copy(C.c_void_p(264), C.c_void_p(1 << 20), 64, None) == E  # misaligned
    assert L._lib.dcpkv_probe_copy(v, C.c_void_p(512), 1024, None) == E            # overlapping
    assert L._lib.dcpkv_probe_copy(None, v, 64, None) == E
    P = C.c_void_p
    a, b, ids = P(1 << 20), P(1 << 30), P(4096)
    cp = L._lib.dcpkv_probe_copy_pages
    assert cp(a, b, ids, ids, 4, 8, 8, 100, None) == E                    # page not a multiple of 16
    assert cp(a, b, ids, ids, -1, 8, 8, 4096, None) == E                  # negative count
    assert cp(a, b, ids, ids, 4, 0, 8, 4096, None) == E                   # no source pages
    assert cp(a, P((1 << 20) + 4096), ids, ids, 4, 8, 8, 4096, None) == E  # overlapping buffers
    assert cp(P((1 << 20) + 8), b, ids, ids, 4, 8, 8, 4096, None) == E    # misaligned
    assert cp(a, b, None, ids, 4, 8, 8, 4096, None) == E
    assert cp(a, b, ids, P(4098), 4, 8, 8, 4096, None) == E               # misaligned list
    assert cp(None, None, None, None, 0, 8, 8, 4096, None) == L.DCPKV_OK  # nothing to copy
