"""Pins of the float64 oracle to things other than itself.

Each test ties an oracle function to a value the pages print (fixtures under
tests/golden/, each citing its passage), a closed form, an invariant the pages
state, a library routine (torch SDPA, torch's fp8/bf16 conversions, logsumexp)
or brute force on tiny inputs.  CPU only.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# --------------------------------------------------------------------------- layer split


def test_layer_split_worked_example():
    rows = _rows("layer_split_78_over_8.txt")
    assert len(rows) == 8
    for r, a, b in rows:
        assert O.layer_range(78, 8, int(r)) == (int(a), int(b))
    # section 6.5: first 6 ranks 10 layers, last 2 get 9
    sizes = [b - a for a, b in (O.layer_range(78, 8, r) for r in range(8))]
    assert sizes == [10] * 6 + [9] * 2


@pytest.mark.parametrize("L", [1, 4, 7, 64, 78, 100])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 12])
def test_layer_split_partition(L, n):
    if n > L:
        return
    ranges = [O.layer_range(L, n, r) for r in range(n)]
    # contiguous cover of [0, L)
    assert ranges[0][0] == 0 and ranges[-1][1] == L
    for (a0, b0), (a1, b1) in zip(ranges, ranges[1:]):
        assert b0 == a1
    sizes = [b - a for a, b in ranges]
    assert all(s in (L // n, L // n + 1) for s in sizes)
    assert sizes == sorted(sizes, reverse=True)
    assert sum(s == L // n + 1 for s in sizes) == (L % n if L % n else 0) or L % n == 0
    for layer in range(L):
        r = O.layer_owner(L, n, layer)
        a, b = ranges[r]
        assert a <= layer < b
    assert O.local_layer_count(L, n, 0) == sizes[0] + 1


def test_layer_split_64_over_4():
    assert [O.layer_range(64, 4, r) for r in range(4)] == [(0, 16), (16, 32), (32, 48), (48, 64)]
    assert O.local_layer_count(64, 4, 2) == 17


# --------------------------------------------------------------------------- round robin, filter


def test_round_robin_animation():
    for p, d, s in _rows("round_robin_16_over_4.txt"):
        assert O.dcp_owner(int(p), 4) == int(d)
        assert O.dcp_local_slot(int(p), 4) == int(s)


@pytest.mark.parametrize("n,m", [(1, 5), (2, 7), (4, 16), (8, 9)])
def test_owner_slot_bijection(n, m):
    seen = set()
    for p in range(n * m):
        d, s = O.dcp_owner(p, n), O.dcp_local_slot(p, n)
        assert 0 <= d < n and 0 <= s < m
        assert s * n + d == p
        seen.add((d, s))
    assert len(seen) == n * m


def test_filter_log_line_256_to_64():
    t = {k: v for k, v in _rows("transfer_volume.txt")}
    full = int(t["log_pages_full"])
    pages = list(range(full))
    for d in range(4):
        kept = O.filter_kv_indices_for_dcp_rank(pages, 4, d)
        assert len(kept) == int(t["log_pages_per_rank"])
        assert kept == list(range(64))
    # N <= 1 passes the list unchanged
    assert O.filter_kv_indices_for_dcp_rank([5, 3, 9], 1, 0) == [5, 3, 9]


def test_filter_reconstructs_full_set():
    rng = np.random.default_rng(0)
    idx = rng.permutation(200)[:77].tolist()
    back = set()
    for d in range(8):
        for s in O.filter_kv_indices_for_dcp_rank(idx, 8, d):
            back.add(s * 8 + d)
    assert back == set(idx)


def test_ownership_by_value_not_position():
    # destination values whose residues mod N differ from their list positions:
    # the filter and the plan must follow the VALUE (section 6.3; reading R6)
    dst = [7, 2, 4, 13, 0, 9]
    src = [100, 101, 102, 103, 104, 105]
    plan = O.reshard_plan(1, 1, 4, src, dst, 0)
    got = {(d, s): sp for (_, _, sp, d, _, s) in plan}
    assert got == {(3, 1): 100, (2, 0): 101, (0, 1): 102, (1, 3): 103, (0, 0): 104, (1, 2): 105}
    for d in range(4):
        assert sorted(O.filter_kv_indices_for_dcp_rank(dst, 4, d)) == sorted(s for (dd, s) in got if dd == d)


# --------------------------------------------------------------------------- volumes


def test_transfer_volume_bytes():
    t = {k: v for k, v in _rows("transfer_volume.txt")}
    L, B, T = int(t["layers"]), int(t["bytes_per_token_per_layer"]), int(t["tokens_32k"])
    page = 64
    pages = T // page
    n = 4
    pm = O.PageMap(n, page, pages)
    g = pm.alloc(T)
    plan = O.reshard_plan(L, 8, n, list(range(pages)), g, 0)
    page_bytes = page * B
    per_dst = [0] * n
    paths = set()
    for (r, _, _, d, _, _) in plan:
        per_dst[d] += page_bytes
        paths.add((r, d))
    total = sum(per_dst)
    assert total == L * B * T == 1_472_200_704
    assert abs(total / 1e9 - float(t["total_kv_bytes_approx_gb"])) < 0.005
    assert all(x == total // n for x in per_dst)
    assert abs(per_dst[0] / 1e6 - float(t["per_rank_bytes_approx_mb"])) < 0.5
    naive = n * total  # every rank receives the whole sequence (section 6.1)
    assert abs(naive / 1e9 - float(t["naive_total_approx_gb"])) < 0.01
    assert abs((naive - total) / 1e9 - float(t["naive_discarded_approx_gb"])) < 0.01
    assert (naive - total) / naive == float(t["naive_discarded_frac"])
    assert len(paths) == int(t["paths"])
    assert abs(-(-int(t["tokens_500k"]) // page) / 1000 - float(t["pages_500k_approx_k"])) < 0.05


def test_reshard_paths_cover_2d_target():
    # section 2: each path (r, d) carries exactly L_r x P_d
    L, ncp, n, pages = 11, 3, 4, 23
    rng = np.random.default_rng(1)
    pm = O.PageMap(n, 16, 40, rng.permutation(40))
    g = pm.alloc(pages * 16)
    src = rng.permutation(60)[:pages]
    plan = O.reshard_plan(L, ncp, n, src, g, 0)
    for r in range(ncp):
        a, b = O.layer_range(L, ncp, r)
        for d in range(n):
            got = {(ls + a, sp) for (rr, ls, sp, dd, _, _) in plan if rr == r and dd == d}
            want = {(layer, int(src[i])) for layer in range(a, b) for i in range(pages) if g[i] % n == d}
            assert got == want


# --------------------------------------------------------------------------- reshard brute force


def _tagged_sources(L, ncp, S, page_bytes):
    pools = []
    for r in range(ncp):
        n_slots = O.local_layer_count(L, ncp, r)
        p = np.zeros((n_slots, S, page_bytes), dtype=np.uint8)
        for ls in range(n_slots):
            for sp in range(S):
                tag = np.frombuffer(np.array([r, ls, sp, 0xC0FFEE], dtype=np.int32).tobytes(), dtype=np.uint8)
                p[ls, sp] = np.resize(tag, page_bytes)
        p[-1] = 0xEE  # transient slot: must never appear in a destination
        pools.append(p)
    return pools


@pytest.mark.parametrize("n,cached,dst_filter", [(1, 0, -1), (2, 0, -1), (4, 3, -1), (3, 5, -1), (4, 2, 1)])
def test_reshard_bruteforce_tags(n, cached, dst_filter):
    L, ncp, S, M, psz, page_bytes = 7, 3, 30, 20, 16, 32
    rng = np.random.default_rng(7 + n)
    pm = O.PageMap(n, psz, M, rng.permutation(M))
    T = 19 * psz - 5
    g = pm.alloc(T)
    P = len(g)
    src = rng.permutation(S)[:P]
    srcp = _tagged_sources(L, ncp, S, page_bytes)
    dst = [np.full((L, M, page_bytes), 0xA5, dtype=np.uint8) for _ in range(n)]
    sent = O.reshard(srcp, dst, L, n, src, g, cached, dst_filter)
    # pull view: for every destination page decide independently what must be there
    where = {int(gg): i for i, gg in enumerate(g)}
    for d in range(n):
        for layer in range(L):
            owner = next(r for r in range(ncp) if O.layer_range(L, ncp, r)[0] <= layer < O.layer_range(L, ncp, r)[1])
            for s in range(M):
                gg = s * n + d
                i = where.get(gg)
                page = dst[d][layer, s]
                if i is None or i < cached or (dst_filter >= 0 and d != dst_filter):
                    assert (page == 0xA5).all()
                else:
                    tag = page[:16].view(np.int32)
                    assert tag.tolist() == [owner, layer - O.layer_range(L, ncp, owner)[0], int(src[i]), 0xC0FFEE]
                assert not (page == 0xEE).all()
    for d in range(n):
        want = sum(1 for i in range(cached, P) if g[i] % n == d) if (dst_filter < 0 or dst_filter == d) else 0
        assert sent[d] == want


def test_reshard_moves_scales():
    L, n, M, S = 2, 2, 4, 6
    src = [np.arange(3 * S * 8, dtype=np.uint8).reshape(3, S, 8)]
    ssc = [np.arange(3 * S, dtype=np.uint16).reshape(3, S) + 1000]
    dst = [np.zeros((L, M, 8), np.uint8) for _ in range(n)]
    dsc = [np.zeros((L, M), np.uint16) for _ in range(n)]
    g = [4, 1, 2, 7]
    sp = [5, 0, 3, 2]
    O.reshard(src, dst, L, n, sp, g, 0, src_scales=ssc, dst_scales=dsc)
    for i, gg in enumerate(g):
        for layer in range(L):
            assert dsc[gg % n][layer, gg // n] == ssc[0][layer, sp[i]]
            assert (dst[gg % n][layer, gg // n] == src[0][layer, sp[i]]).all()


# --------------------------------------------------------------------------- token ownership


def test_token_ownership_fixture():
    """[SGL]: token t lives on rank t mod N (tests/golden/token_ownership_10_over_4.txt)."""
    for row in _rows("token_ownership_10_over_4.txt"):
        d, toks = int(row[0]), [int(x) for x in row[1:]]
        mask = O.shard_token_mask([0, 1, 2, 3], 16, 10, 4, d, own="token")
        assert np.nonzero(mask)[0].tolist() == toks
        assert all(O.token_owner(t, 4) == d for t in toks)


@pytest.mark.parametrize("own", ["page", "token"])
@pytest.mark.parametrize("n,T", [(1, 37), (2, 65), (4, 65), (4, 300), (3, 7), (8, 1000)])
def test_shard_masks_partition_the_sequence(own, n, T):
    pm = O.PageMap(n, 16, 64, list(range(64)))
    g = pm.alloc(T)
    masks = np.stack([O.shard_token_mask(g, 16, T, n, d, own) for d in range(n)])
    assert (masks.sum(axis=0) == 1).all()


def test_token_layout_hand_example():
    """N = 2, page 4, T = 11 tokens on virtual pages 5 and 9 (global pages 10, 11, 18), worked by
    hand: rank 0 holds tokens 0, 2, 4, 6 in rows 0-3 of slot 5 and 8, 10 in rows 0-1 of slot 9;
    rank 1 holds 1, 3, 5, 7 in slot 5 and 9 in row 0 of slot 9.  Block tables: page ownership
    gives rank 0 slots [5, 9] and rank 1 [5]; token ownership gives both [5, 9]."""
    g = [10, 11, 18]
    want = {0: (0, 5, 0), 2: (0, 5, 1), 4: (0, 5, 2), 6: (0, 5, 3), 8: (0, 9, 0), 10: (0, 9, 1),
            1: (1, 5, 0), 3: (1, 5, 1), 5: (1, 5, 2), 7: (1, 5, 3), 9: (1, 9, 0)}
    for t, place in want.items():
        assert O.token_place(t, 2, 4, g) == place
    assert O.block_tables([g], 2, "page") == [[[5, 9]], [[5]]]
    assert O.block_tables([g], 2, "token") == [[[5, 9]], [[5, 9]]]


@pytest.mark.parametrize("n,T,psz", [(2, 11, 4), (4, 65, 16), (4, 301, 16), (3, 50, 8), (8, 129, 4)])
def test_token_layout_places_every_token_once_within_its_table(n, T, psz):
    """Every token gets its own (shard, slot, row); each slot is in its shard's token block-table
    row; rows fill local pages in order; a shard holds ceil((T - d) / N) tokens."""
    M = 4 * (T // (psz * n) + 2)
    pm = O.PageMap(n, psz, M, list(reversed(range(M))))
    g = pm.alloc(T)
    places = [O.token_place(t, n, psz, g) for t in range(T)]
    assert len(set(places)) == T
    tab = O.block_tables([g], n, "token")
    for d in range(n):
        mine = [p for p in places if p[0] == d]
        assert len(mine) == max(0, -(-(T - d) // n))
        for u, (_, slot, row) in enumerate(mine):
            assert tab[d][0][u // psz] == slot and row == u % psz


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
def test_merge_equals_unsharded_token_ownership(n):
    """Any partition of the tokens merges back exactly ([SGL]: exact across ranks); here the
    token-residue partition."""
    rng = np.random.default_rng(40 + n)
    T, q_len, hq, hkv, d_ = 301, 2, 4, 2, 8
    q, k, v = _rand_req(rng, T, q_len, hq, hkv, d_, d_)
    pm = O.PageMap(n, 16, 64, list(range(64)))
    g = pm.alloc(T)
    po, pl = O.request_partials(q, k, v, T, 0.3, g, 16, n, own="token")
    mo, ml = O.lse_merge(po, pl)
    uo, ul = O.request_attention(q, k, v, T, 0.3, None)
    assert np.allclose(mo, uo, rtol=1e-12, atol=1e-12) and np.allclose(ml, ul, rtol=1e-12, atol=1e-12)


def test_logical_kv_gather_token_ownership():
    """Pools written token by token under token ownership (tagged rows) read back into the logical
    sequence, for the split and the latent layouts."""
    n, psz, T, hkv, D = 4, 8, 70, 2, 4
    M = 16
    pm = O.PageMap(n, psz, M, list(range(M)))
    g = pm.alloc(T)
    pools = np.zeros((n, M, 2, hkv, psz, D), dtype=np.float32)
    for t in range(T):
        d, slot, row = O.token_place(t, n, psz, g)
        pools[d, slot, 0, :, row, :] = t + 0.25
        pools[d, slot, 1, :, row, :] = -t
    k, v = O.logical_kv_split_tokens(lambda d, s: pools[d, s].reshape(-1).view(np.uint8), g, n, "f32", hkv, psz,
                                     D, T)
    assert (k[:, :, 0] == np.arange(T) + 0.25).all() and (v[:, :, 0] == -np.arange(T)).all()
    lat = np.zeros((n, M, psz, 576), dtype=np.uint8)
    for t in range(T):
        d, slot, row = O.token_place(t, n, psz, g)
        lat[d, slot, row, :] = 0x38  # e4m3 1.0
        lat[d, slot, row, 0] = 0x38 + (t % 8)  # 1.0 .. 1.875
    kk, vv = O.logical_kv_mla_tokens(lambda d, s: (lat[d, s].reshape(-1), 0x4000), g, n, psz, T)  # scale 2.0
    assert np.allclose(kk[0, :, 0], 2.0 * (1.0 + (np.arange(T) % 8) / 8.0)) and vv.shape == (1, T, 512)


def _token_tagged_sources(L, ncp, S, R, psz, rb):
    """Sources whose every row carries (source, layer slot, page, block, row) as int32s."""
    pools = []
    for r in range(ncp):
        n_slots = O.local_layer_count(L, ncp, r)
        p = np.zeros((n_slots + 1, S, R, psz, rb), dtype=np.uint8)
        for ls in range(n_slots):
            for sp in range(S):
                for blk in range(R):
                    for x in range(psz):
                        tag = np.array([r, ls, sp, blk, x, 0x70C], dtype=np.int32).view(np.uint8)
                        p[ls, sp, blk, x] = np.resize(tag, rb)
        p[-1] = 0xEE
        pools.append(p.reshape(n_slots + 1, S, R * psz * rb))
    return pools


@pytest.mark.parametrize("n,cached,T", [(1, 0, 70), (2, 0, 70), (4, 1, 150), (3, 2, 130), (8, 0, 64)])
def test_reshard_tokens_pull_view(n, cached, T):
    """Every destination row, checked from its tag: under token ownership row y of shard d's local
    page j (slot of virtual page j) holds token t = (j * page + y) * N + d of the sequence, from
    the source owning the layer; rows of cached or missing tokens keep the sentinel."""
    L, ncp, psz, R, rb, M = 5, 2, 8, 2, 32, 12
    rng = np.random.default_rng(60 + n)
    pm = O.PageMap(n, psz, M, rng.permutation(M))
    g = pm.alloc(T)
    P = len(g)
    S = P + 3
    src = rng.permutation(S)[:P]
    srcp = _token_tagged_sources(L, ncp, S, R, psz, rb)
    dst = [np.full((L, M, R * psz * rb), 0xA5, dtype=np.uint8) for _ in range(n)]
    moved = O.reshard_tokens(srcp, dst, L, n, psz, R, rb, src, g, cached)
    assert moved == L * (P - cached) * psz
    vslot = {j: O.dcp_local_slot(int(g[j * n]), n) for j in range(-(-P // n))}
    for d in range(n):
        for layer in range(L):
            owner = next(r for r in range(ncp) if O.layer_range(L, ncp, r)[0] <= layer < O.layer_range(L, ncp, r)[1])
            for s_ in range(M):
                page = dst[d][layer, s_].reshape(R, psz, rb)
                js = [j for j, v in vslot.items() if v == s_]
                for y in range(psz):
                    t = (js[0] * psz + y) * n + d if js else None
                    for blk in range(R):
                        row = page[blk, y]
                        if t is None or t // psz >= P or t // psz < cached:
                            assert (row == 0xA5).all()
                        else:
                            want = [owner, layer - O.layer_range(L, ncp, owner)[0], int(src[t // psz]), blk,
                                    t % psz, 0x70C]
                            assert row[:24].view(np.int32).tolist() == want


@pytest.mark.parametrize("n,cached,lens", [(4, 0, (70, 9, 33)), (3, 5, (20, 64, 1)), (2, 0, (8, 8))])
def test_reshard_tokens_pull_view_batch(n, cached, lens):
    """Several requests in one list, delimited by offsets: each request's tokens restart at
    position 0 and land in its own virtual pages; rows are checked from their tags as above."""
    L, ncp, psz, R, rb, M = 3, 2, 8, 1, 32, 24
    rng = np.random.default_rng(90 + n)
    pm = O.PageMap(n, psz, M, rng.permutation(M))
    reqs = [pm.alloc(T) for T in lens]
    offs = np.cumsum([0] + [len(g) for g in reqs])
    g_all = np.concatenate(reqs)
    P = len(g_all)
    S = P + 2
    src = rng.permutation(S)[:P]
    srcp = _token_tagged_sources(L, ncp, S, R, psz, rb)
    dst = [np.full((L, M, R * psz * rb), 0xA5, dtype=np.uint8) for _ in range(n)]
    moved = O.reshard_tokens(srcp, dst, L, n, psz, R, rb, src, g_all, cached, request_offsets=offs)
    assert moved == L * (P - cached) * psz
    owner_slot = {}  # slot -> (request, virtual page)
    for q, g in enumerate(reqs):
        for j in range(-(-len(g) // n)):
            owner_slot[O.dcp_local_slot(int(g[j * n]), n)] = (q, j)
    for d in range(n):
        for layer in range(L):
            owner = next(r for r in range(ncp) if O.layer_range(L, ncp, r)[0] <= layer < O.layer_range(L, ncp, r)[1])
            for s_ in range(M):
                page = dst[d][layer, s_].reshape(R, psz, rb)
                for y in range(psz):
                    row = page[0, y]
                    if s_ not in owner_slot:
                        assert (row == 0xA5).all()
                        continue
                    q, j = owner_slot[s_]
                    t = (j * psz + y) * n + d
                    e = offs[q] + t // psz  # list entry of the token's source page
                    if t // psz >= len(reqs[q]) or e < cached:
                        assert (row == 0xA5).all()
                    else:
                        want = [owner, layer - O.layer_range(L, ncp, owner)[0], int(src[e]), 0, t % psz, 0x70C]
                        assert row[:24].view(np.int32).tolist() == want


def test_reshard_tokens_one_shard_is_the_page_reshard():
    """With N = 1 token and page ownership coincide: the token reshard writes what the page
    reshard writes."""
    L, ncp, psz, R, rb, M = 4, 2, 8, 2, 16, 6
    rng = np.random.default_rng(70)
    pm = O.PageMap(1, psz, M, rng.permutation(M))
    g = pm.alloc(37)
    src = rng.permutation(len(g) + 2)[:len(g)]
    srcp = _token_tagged_sources(L, ncp, len(g) + 2, R, psz, rb)
    a = [np.full((L, M, R * psz * rb), 0xA5, dtype=np.uint8)]
    b = [np.full((L, M, R * psz * rb), 0xA5, dtype=np.uint8)]
    O.reshard_tokens(srcp, a, L, 1, psz, R, rb, src, g, 1)
    O.reshard(srcp, b, L, 1, src, g, 1)
    assert np.array_equal(a[0], b[0])


def test_reshard_tokens_gives_the_page_reshards_logical_sequence():
    """Same sources, either ownership: the token reshard read back under token ownership gives
    the same logical K/V as the page reshard read back under page ownership."""
    n, psz, hkv, D, T, M = 4, 8, 2, 4, 70, 16
    rng = np.random.default_rng(80)
    pm = O.PageMap(n, psz, M, rng.permutation(M))
    g = pm.alloc(T)
    P = len(g)
    src_ids = rng.permutation(P)
    pb = 2 * hkv * psz * D * 4
    srcp = [np.concatenate([rng.standard_normal((1, P, pb // 4)).astype(np.float32).view(np.uint8),
                            np.zeros((1, P, pb), np.uint8)])]
    dp = [np.zeros((1, M, pb), np.uint8) for _ in range(n)]
    dt = [np.zeros((1, M, pb), np.uint8) for _ in range(n)]
    O.reshard(srcp, dp, 1, n, src_ids, g, 0)
    O.reshard_tokens(srcp, dt, 1, n, psz, 2 * hkv, D * 4, src_ids, g, 0)
    kp, vp = O.logical_kv_split(lambda d, s_: dp[d][0, s_], g, n, "f32", hkv, psz, D, T)
    kt, vt = O.logical_kv_split_tokens(lambda d, s_: dt[d][0, s_], g, n, "f32", hkv, psz, D, T)
    assert np.array_equal(kp, kt) and np.array_equal(vp, vt)


# --------------------------------------------------------------------------- bounded pack / unpack


def _pack_all(srcp, ssc, src_ids, g, L, n, cached, S, M, cap, page_bytes, dst, dsc=None):
    """Every path (r, d), window after window through a staging buffer of `cap` pages."""
    ncp = len(srcp)
    packed = 0
    for d in range(n):
        ent = O.path_entries(src_ids, g, cached, n, d, S, M)
        for r in range(ncp):
            u0 = 0
            while True:
                stg = np.full((cap, page_bytes), 0x5A, dtype=np.uint8)
                stg_sc = np.zeros(cap, np.uint16) if ssc is not None else None
                k = O.pack_pages(srcp[r], None if ssc is None else ssc[r], src_ids, L, ncp, r, ent, u0, cap, stg,
                                 stg_sc)
                if k == 0:
                    break
                O.unpack_pages(dst[d], None if dsc is None else dsc[d], g, L, ncp, r, n, ent, u0, cap, stg, stg_sc)
                packed += k
                u0 += k
    return packed


@pytest.mark.parametrize("n,cached,cap", [(1, 0, 1), (2, 0, 3), (4, 3, 2), (3, 5, 7), (4, 2, 1000)])
def test_pack_unpack_round_trip_pull_view(n, cached, cap):
    """Window after window, pack + unpack over every path leaves each destination page exactly
    what the 2D target says ([2DR] section 2; ownership by value, section 6.3), checked page by
    page from the tags, and exactly what the reshard writes."""
    L, ncp, S, M, psz, page_bytes = 7, 3, 30, 20, 16, 32
    rng = np.random.default_rng(11 + n)
    pm = O.PageMap(n, psz, M, rng.permutation(M))
    g = pm.alloc(19 * psz - 5)
    P = len(g)
    src = rng.permutation(S)[:P]
    srcp = _tagged_sources(L, ncp, S, page_bytes)
    dst = [np.full((L, M, page_bytes), 0xA5, dtype=np.uint8) for _ in range(n)]
    packed = _pack_all(srcp, None, src, g, L, n, cached, S, M, cap, page_bytes, dst)
    assert packed == (P - cached) * L  # the same pages move, only in windows
    where = {int(gg): i for i, gg in enumerate(g)}
    for d in range(n):
        for layer in range(L):
            owner = next(r for r in range(ncp) if O.layer_range(L, ncp, r)[0] <= layer < O.layer_range(L, ncp, r)[1])
            for s_ in range(M):
                i = where.get(s_ * n + d)
                page = dst[d][layer, s_]
                if i is None or i < cached:
                    assert (page == 0xA5).all()
                else:
                    tag = page[:16].view(np.int32)
                    assert tag.tolist() == [owner, layer - O.layer_range(L, ncp, owner)[0], int(src[i]), 0xC0FFEE]
    ref = [np.full((L, M, page_bytes), 0xA5, dtype=np.uint8) for _ in range(n)]
    O.reshard(srcp, ref, L, n, src, g, cached)
    for d in range(n):
        assert np.array_equal(dst[d], ref[d])


def test_pack_windows_hand_example():
    """A window layout worked by hand from the definition: L = 4 over 2 sources (layers 0-1, 2-3),
    N = 2, g = [5, 2, 3, 0, 6], one cached page.  Path to d = 0 takes positions 1, 3, 4 (values
    2, 0, 6); source 1's units are (1,2) (1,3) (3,2) (3,3) (4,2) (4,3); four-page windows."""
    L, ncp, n, S, M, pb = 4, 2, 2, 16, 8, 16
    g = [5, 2, 3, 0, 6]
    src = [10, 11, 12, 13, 14]
    ent = O.path_entries(src, g, 1, n, 0, S, M)
    assert ent == [1, 3, 4]
    assert O.path_entries(src, g, 1, n, 1, S, M) == [2]
    assert O.path_units(L, ncp, 1, ent) == [(1, 2), (1, 3), (3, 2), (3, 3), (4, 2), (4, 3)]
    pool = np.zeros((3, S, pb), dtype=np.uint8)
    for ls in range(3):
        for sp in range(S):
            pool[ls, sp] = 16 * ls + sp
    stg = np.zeros((4, pb), dtype=np.uint8)
    assert O.pack_pages(pool, None, src, L, ncp, 1, ent, 0, 4, stg) == 4
    assert stg[:, 0].tolist() == [11, 16 + 11, 13, 16 + 13]
    stg[:] = 0
    assert O.pack_pages(pool, None, src, L, ncp, 1, ent, 4, 4, stg) == 2
    assert stg[:, 0].tolist() == [14, 16 + 14, 0, 0]
    assert O.pack_pages(pool, None, src, L, ncp, 1, ent, 6, 4, stg) == 0
    dst = np.zeros((L, M, pb), dtype=np.uint8)
    stg[:] = 0
    O.pack_pages(pool, None, src, L, ncp, 1, ent, 0, 4, stg)
    assert O.unpack_pages(dst, None, g, L, ncp, 1, n, ent, 0, 4, stg) == 4
    # value 2 -> slot 1, value 0 -> slot 0, layers 2 and 3
    assert dst[2, 1, 0] == 11 and dst[3, 1, 0] == 16 + 11 and dst[2, 0, 0] == 13 and dst[3, 0, 0] == 16 + 13
    assert int(dst.astype(np.int64).sum()) == pb * (11 + 27 + 13 + 29)


def test_pack_excludes_bad_ids_and_scales_ride_along():
    """Entries whose ids fall outside the pools carry nothing (the reshard skips them too); page
    scales travel with their pages through the staging buffer."""
    L, ncp, n, S, M, pb = 2, 1, 2, 6, 4, 8
    g = [4, 1, 9, 2, -3, 7]   # 9 >= M*N and -3 are out of range
    src = [5, 0, 3, 6, 1, 2]  # 6 >= S is out of range
    assert O.path_entries(src, g, 0, n, 0, S, M) == [0]
    assert O.path_entries(src, g, 0, n, 1, S, M) == [1, 5]
    pool = np.arange(3 * S * pb, dtype=np.uint8).reshape(3, S, pb)
    ssc = [np.arange(3 * S, dtype=np.uint16).reshape(3, S) + 1000]
    dst = [np.zeros((L, M, pb), np.uint8) for _ in range(n)]
    dsc = [np.zeros((L, M), np.uint16) for _ in range(n)]
    _pack_all([pool], ssc, src, g, L, n, 0, S, M, 3, pb, dst, dsc)
    ref = [np.zeros((L, M, pb), np.uint8) for _ in range(n)]
    rsc = [np.zeros((L, M), np.uint16) for _ in range(n)]
    keep = [i for i in range(len(g)) if 0 <= g[i] < M * n and 0 <= src[i] < S]
    O.reshard([pool], ref, L, n, [src[i] for i in keep], [g[i] for i in keep], 0, src_scales=ssc, dst_scales=rsc)
    for d in range(n):
        assert np.array_equal(dst[d], ref[d]) and np.array_equal(dsc[d], rsc[d])
    assert dsc[1][0, 0] == ssc[0][0, 0] and dsc[1][1, 3] == ssc[0][1, 2]  # values 1 and 7 -> slots 0 and 3


# --------------------------------------------------------------------------- page map


def test_pagemap_canonical_and_log_line():
    n, page = 4, 64
    pm = O.PageMap(n, page, 100, np.random.default_rng(3).permutation(100))
    g = pm.alloc(16384)  # 16K tokens -> 256 pages, 64 per rank (section 6.3 log line)
    assert len(g) == 256 and len(set(g)) == 256
    for i, gg in enumerate(g):
        assert gg % n == i % n  # page p lands on rank p mod N
        assert 0 <= gg // n < 100
    assert sum(1 for gg in g if gg % n == 2) == 64
    # one virtual page = N physical pages, one per rank, same local slot (section 6.4)
    for v in range(64):
        assert len({g[v * n + k] // n for k in range(n)}) == 1


def test_pagemap_partial_last_virtual_page_and_exhaustion():
    pm = O.PageMap(4, 16, 3, [2, 0, 1])
    g = pm.alloc(16 * 5 + 1)  # 6 pages -> 2 virtual pages
    assert g == [8, 9, 10, 11, 0, 1]
    with pytest.raises(MemoryError):
        pm.alloc(16 * 4 * 2)
    pm.release(g)
    assert list(pm.free) == [1, 2, 0]  # FIFO reuse (reading R12)
    with pytest.raises(ValueError):
        pm.release(g)
    with pytest.raises(ValueError):
        pm.alloc(0)


# --------------------------------------------------------------------------- number formats


def test_e4m3fn_table_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        if c in (0x7F, 0xFF):
            assert math.isnan(O.E4M3FN_TABLE[c]) and math.isnan(ref[c])
        else:
            assert O.E4M3FN_TABLE[c] == ref[c], c
    assert O.e4m3fn_value(0x7E) == 448.0
    assert O.e4m3fn_value(0x01) == 2.0 ** -9
    assert O.e4m3fn_value(0x08) == 2.0 ** -6
    assert O.e4m3fn_value(0x38) == 1.0
    assert math.copysign(1.0, O.e4m3fn_value(0x80)) == -1.0


def test_bf16_decode_vs_torch():
    bits = torch.randint(-32768, 32767, (4096,), dtype=torch.int16, generator=torch.Generator().manual_seed(0))
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_bits_to_f64(bits.numpy())
    ok = ~np.isnan(ref)
    assert (got[ok] == ref[ok]).all() and np.isnan(got[~ok]).all()


def test_fp8_times_bf16_scale_exact_in_f32():
    # dequant in float32 (code * scale) equals the float64 product: 4 x 8 significant bits
    rng = np.random.default_rng(5)
    scales = rng.integers(0x3000, 0x4400, size=64).astype(np.uint16)
    sv = O.bf16_bits_to_f64(scales)
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        x64 = O.E4M3FN_TABLE[c] * sv
        x32 = (np.float32(O.E4M3FN_TABLE[c]) * sv.astype(np.float32)).astype(np.float64)
        assert (x32 == x64).all()


def test_decode_pages_vs_torch():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, size=(16, 576), dtype=np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    sbits = int(torch.tensor([0.0123], dtype=torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    got = O.decode_mla_page(codes, sbits, 16)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64) * float(
        torch.tensor([sbits], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).item())
    assert np.array_equal(got, ref.numpy())
    x = torch.randn(2, 3, 4, 8, dtype=torch.float32)
    k, v = O.decode_split_page(x.numpy().view(np.uint8).reshape(-1), "f32", 3, 4, 8)
    assert np.array_equal(k, x[0].double().numpy()) and np.array_equal(v, x[1].double().numpy())
    xb = x.to(torch.bfloat16)
    k, v = O.decode_split_page(xb.view(torch.int16).numpy().view(np.uint8).reshape(-1), "bf16", 3, 4, 8)
    assert np.array_equal(k, xb[0].double().numpy()) and np.array_equal(v, xb[1].double().numpy())


# --------------------------------------------------------------------------- attention


def _rand_req(rng, T, q_len, hq, hkv, dqk, dv):
    q = rng.standard_normal((q_len, hq, dqk))
    k = rng.standard_normal((hkv, T, dqk))
    v = rng.standard_normal((hkv, T, dv))
    return q, k, v


@pytest.mark.parametrize("T,q_len,hq,hkv", [(37, 1, 4, 1), (50, 3, 8, 2), (9, 4, 6, 3)])
def test_attention_vs_torch_sdpa(T, q_len, hq, hkv):
    rng = np.random.default_rng(T)
    dqk, dv = 12, 10
    q, k, v = _rand_req(rng, T, q_len, hq, hkv, dqk, dv)
    scale = 1 / math.sqrt(dqk)
    out, lse = O.request_attention(q, k, v, T, scale)
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq][q_len][D]
    grp = hq // hkv
    kt = torch.from_numpy(k).repeat_interleave(grp, dim=0)  # head h reads kv head h // grp
    vt = torch.from_numpy(v).repeat_interleave(grp, dim=0)
    pos = torch.tensor([T - q_len + t for t in range(q_len)])
    mask = torch.arange(T)[None, :] <= pos[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)
    s = scale * (qt @ kt.transpose(-1, -2))
    ref_lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    assert np.allclose(lse, ref_lse.T.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_head_mapping_is_contiguous_groups():
    # kv head 0 all zeros, kv head 1 all ones: heads 0..1 must see zeros, heads 2..3 ones
    T = 5
    q = np.ones((1, 4, 3))
    k = np.zeros((2, T, 3))
    v = np.stack([np.zeros((T, 2)), np.ones((T, 2))])
    out, _ = O.request_attention(q, k, v, T, 1.0)
    assert (out[0, :2] == 0).all() and (out[0, 2:] == 1).all()


def test_attention_special_cases():
    rng = np.random.default_rng(11)
    q, k, v = _rand_req(rng, 1, 1, 2, 1, 6, 5)
    out, lse = O.request_attention(q, k, v, 1, 0.5)
    assert np.allclose(out[0, 0], v[0, 0]) and np.isclose(lse[0, 0], 0.5 * q[0, 0] @ k[0, 0])
    # equal scores: O = mean of visible v, LSE = log(n)
    T = 13
    q = np.zeros((2, 1, 4))
    _, k, v = _rand_req(rng, T, 2, 1, 1, 4, 3)
    out, lse = O.request_attention(q, k, v, T, 1.0)
    assert np.allclose(out[0, 0], v[0, :T - 1].mean(0)) and np.isclose(lse[0, 0], math.log(T - 1))
    assert np.allclose(out[1, 0], v[0, :T].mean(0)) and np.isclose(lse[1, 0], math.log(T))
    # a constant added to every score shifts LSE by it and leaves O unchanged
    q, k, v = _rand_req(rng, 20, 1, 1, 1, 4, 3)
    o1, l1 = O.request_attention(q, k, v, 20, 1.0)
    c = 2.75
    q2 = np.concatenate([q, np.full((1, 1, 1), c)], axis=2)
    k2 = np.concatenate([k, np.ones((1, 20, 1))], axis=2)
    o2, l2 = O.request_attention(q2, k2, v, 20, 1.0)
    assert np.allclose(o1, o2, rtol=1e-13) and np.isclose(l2[0, 0], l1[0, 0] + c, rtol=1e-13)


def test_attention_bruteforce_fsum():
    rng = np.random.default_rng(12)
    T, dqk, dv = 7, 3, 2
    q, k, v = _rand_req(rng, T, 2, 2, 1, dqk, dv)
    out, lse = O.request_attention(q, k, v, T, 0.7)
    for t in range(2):
        pos = T - 2 + t
        for h in range(2):
            s = [0.7 * math.fsum(q[t, h, i] * k[0, j, i] for i in range(dqk)) for j in range(pos + 1)]
            z = math.fsum(math.exp(x) for x in s)
            assert math.isclose(lse[t, h], math.log(z), rel_tol=1e-13)
            for c in range(dv):
                want = math.fsum(math.exp(s[j]) / z * v[0, j, c] for j in range(pos + 1))
                assert math.isclose(out[t, h, c], want, rel_tol=1e-12, abs_tol=1e-14)


# --------------------------------------------------------------------------- partials + merge


def _sharded_case(seed, n, T=301, page=16, q_len=2, hq=4, hkv=2, d=8):
    rng = np.random.default_rng(seed)
    q, k, v = _rand_req(rng, T, q_len, hq, hkv, d, d)
    pm = O.PageMap(n, page, 64, rng.permutation(64))
    g = pm.alloc(T)
    return q, k, v, g, T, page


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8])
def test_merge_equals_unsharded(n):
    q, k, v, g, T, page = _sharded_case(n, n)
    ref_o, ref_l = O.request_attention(q, k, v, T, 0.3)
    po, pl = O.request_partials(q, k, v, T, 0.3, g, page, n)
    mo, ml = O.lse_merge(po, pl)
    assert np.allclose(mo, ref_o, rtol=1e-12, atol=1e-13)
    assert np.allclose(ml, ref_l, rtol=1e-12, atol=1e-13)
    if n == 1:
        assert np.allclose(po[0], ref_o, rtol=0, atol=0) and np.allclose(pl[0], ref_l, rtol=0, atol=0)


def test_merge_order_independent_and_associative():
    q, k, v, g, T, page = _sharded_case(21, 4)
    po, pl = O.request_partials(q, k, v, T, 0.3, g, page, 4)
    a = O.lse_merge(po, pl)
    perm = [2, 0, 3, 1]
    b = O.lse_merge(po[perm], pl[perm])
    assert np.allclose(a[0], b[0], rtol=1e-13) and np.allclose(a[1], b[1], rtol=1e-13)
    # merge pairs first, then merge the two results
    m01 = O.lse_merge(po[:2], pl[:2])
    m23 = O.lse_merge(po[2:], pl[2:])
    c = O.lse_merge(np.stack([m01[0], m23[0]]), np.stack([m01[1], m23[1]]))
    assert np.allclose(a[0], c[0], rtol=1e-13) and np.allclose(a[1], c[1], rtol=1e-13)


def test_merge_split_shard_further():
    # splitting a shard's tokens in two and merging gives that shard's partial
    q, k, v, g, T, page = _sharded_case(22, 2)
    mask = O.shard_token_mask(g, page, T, 2, 1)
    idx = np.nonzero(mask)[0]
    half = np.zeros(T, bool)
    half[idx[: len(idx) // 2]] = True
    o_full, l_full = O.request_attention(q, k, v, T, 0.3, mask)
    o_a, l_a = O.request_attention(q, k, v, T, 0.3, mask & half)
    o_b, l_b = O.request_attention(q, k, v, T, 0.3, mask & ~half)
    mo, ml = O.lse_merge(np.stack([o_a, o_b]), np.stack([l_a, l_b]))
    assert np.allclose(mo, o_full, rtol=1e-12, atol=1e-13) and np.allclose(ml, l_full, rtol=1e-12)


def test_merge_empty_shard_and_all_empty():
    o = np.random.default_rng(0).standard_normal((3, 5, 4))
    l = np.array([[0.5, -1.0, 2.0, 0.1, 3.0], [-np.inf] * 5, [1.0, 1.0, 1.0, 1.0, 1.0]])
    mo, ml = O.lse_merge(o, l)
    mo2, ml2 = O.lse_merge(o[[0, 2]], l[[0, 2]])
    assert np.allclose(mo, mo2) and np.allclose(ml, ml2)
    mo3, ml3 = O.lse_merge(o, np.full((3, 5), -np.inf))
    assert (mo3 == 0).all() and np.isneginf(ml3).all()
    # a shard that holds nothing visible yields (0, -inf)
    q, k, v = _rand_req(np.random.default_rng(1), 10, 1, 2, 1, 4, 4)
    oo, ll = O.request_attention(q, k, v, 10, 1.0, np.zeros(10, bool))
    assert (oo == 0).all() and np.isneginf(ll).all()


def test_logical_kv_gather_from_pools():
    # pages placed by the page map's owner/slot are read back in sequence order
    n, page, hkv, dd, M = 2, 4, 1, 3, 6
    rng = np.random.default_rng(4)
    pm = O.PageMap(n, page, M, rng.permutation(M))
    T = 17
    g = pm.alloc(T)
    k = rng.standard_normal((hkv, len(g) * page, dd)).astype(np.float32)
    v = rng.standard_normal((hkv, len(g) * page, dd)).astype(np.float32)
    pools = np.zeros((n, M, 2, hkv, page, dd), np.float32)
    for i, gg in enumerate(g):
        pools[gg % n, gg // n, 0] = k[:, i * page:(i + 1) * page]
        pools[gg % n, gg // n, 1] = v[:, i * page:(i + 1) * page]
    kk, vv = O.logical_kv_split(lambda d, s: pools[d, s].reshape(-1).view(np.uint8), g, n, "f32", hkv, page, dd, T)
    assert np.array_equal(kk, k[:, :T].astype(np.float64)) and np.array_equal(vv, v[:, :T].astype(np.float64))


def test_block_tables_worked_example():
    # [2DR] section 5.1 with N = 2: pages 6, 7, 2, 3, 10 -> rank 0 holds 6, 2, 10 at slots 3, 1, 5;
    # rank 1 holds 7, 3 at slots 3, 1 (slots written out by hand from p div N)
    got = O.block_tables([[6, 7, 2, 3, 10], [1]], 2)
    assert got == [[[3, 1, 5], []], [[3, 1], [0]]]


def test_logical_kv_mla_vs_torch():
    rng = np.random.default_rng(13)
    n, page, M = 4, 8, 6
    pm = O.PageMap(n, page, M, rng.permutation(M))
    T = 29
    g = pm.alloc(T)
    codes = rng.integers(0, 0x7E, size=(n, M, page, 576), dtype=np.uint8)
    sbits = (torch.tensor(rng.uniform(0.001, 0.1, size=(n, M)), dtype=torch.bfloat16)
             .view(torch.int16).numpy().astype(np.int64) & 0xFFFF)
    k, v = O.logical_kv_mla(lambda d, s: (codes[d, s], sbits[d, s]), g, n, page, T)
    ref = []
    for gg in g:
        d, s = gg % n, gg // n
        sc = torch.tensor([int(sbits[d, s])], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).double()
        ref.append(torch.from_numpy(codes[d, s]).view(torch.float8_e4m3fn).double() * sc)
    ref = torch.cat(ref)[:T].numpy()
    assert k.shape == (1, T, 576) and v.shape == (1, T, 512)
    assert np.array_equal(k[0], ref) and np.array_equal(v[0], ref[:, :512])


def test_softmax_rows_mixed_visibility_bruteforce_fsum():
    """Rows with different visible sets (runs of equal sets, an empty row, a set that differs
    from its neighbours) each match a math.fsum brute force of the definition; rows that share
    a visible set are computed together, so a mix-up between them would show here."""
    rng = np.random.default_rng(13)
    T, dqk, dv, R = 9, 4, 3, 7
    q = rng.standard_normal((R, dqk))
    k = rng.standard_normal((T, dqk))
    v = rng.standard_normal((T, dv))
    vis = np.zeros((R, T), dtype=bool)
    vis[0:3, :6] = True      # three rows, one set
    vis[3, [1, 4, 8]] = True  # its own set
    vis[5:7, 2:] = True      # row 4 sees nothing; rows 5-6 share a set
    out, lse = O.softmax_rows(q, k, v, vis, 0.9)
    for r in range(R):
        js = [j for j in range(T) if vis[r, j]]
        if not js:
            assert lse[r] == float("-inf") and (out[r] == 0).all()
            continue
        s = {j: 0.9 * math.fsum(q[r, i] * k[j, i] for i in range(dqk)) for j in js}
        z = math.fsum(math.exp(x) for x in s.values())
        assert math.isclose(lse[r], math.log(z), rel_tol=1e-13)
        for c in range(dv):
            want = math.fsum(math.exp(s[j]) / z * v[j, c] for j in js)
            assert math.isclose(out[r, c], want, rel_tol=1e-12, abs_tol=1e-14)


def test_attention_gqa_head_subset_bruteforce_fsum():
    """A subset of query heads spread over several KV heads (groups of 3): each listed head
    matches the brute force with its own KV head; unlisted heads stay (0, -inf)."""
    rng = np.random.default_rng(14)
    T, dqk, dv, hq, hkv = 6, 3, 2, 6, 2
    q, k, v = _rand_req(rng, T, 2, hq, hkv, dqk, dv)
    heads = [0, 2, 4, 5]
    out, lse = O.request_attention(q, k, v, T, 0.5, None, heads)
    for t in range(2):
        pos = T - 2 + t
        for h in range(hq):
            if h not in heads:
                assert lse[t, h] == float("-inf") and (out[t, h] == 0).all()
                continue
            kh = h // 3
            s = [0.5 * math.fsum(q[t, h, i] * k[kh, j, i] for i in range(dqk)) for j in range(pos + 1)]
            z = math.fsum(math.exp(x) for x in s)
            assert math.isclose(lse[t, h], math.log(z), rel_tol=1e-13)
            for c in range(dv):
                want = math.fsum(math.exp(s[j]) / z * v[kh, j, c] for j in range(pos + 1))
                assert math.isclose(out[t, h, c], want, rel_tol=1e-12, abs_tol=1e-14)
