"""Float64 CPU oracle for Decode Context Parallelism over a paged KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline leg may import or run this module.  The product path (the HIP library
and its Python binding) never imports it, and it imports nothing from them.

It is written to be read against the pages, not to be fast: plain loops, numpy
float64, a library matmul or log/exp where a step is a plain sum.

Sources (cited by short name below):
  [2DR]  "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding" (macaron.im)
  [SGL]  "SGLang's path" (serving-k3, module 05; the DCP paragraph)
  [PR28] the fivechenxi/sglang pull request #28 thread (address-translation
         review comment; the review of the bounded-pack commit)

Readings where the pages are silent or garbled (each one is listed in the
design notes as well):
  R1  A shard's partial output is normalised by the shard's own softmax
      denominator: O_d = sum_{j in d} exp(s_j - LSE_d) v_j.  The raw weighted
      sum [SGL] describes is exp(LSE_d) * O_d; both carry the same
      information, the raw one overflows float32.
  R2  Partials are combined as O = sum_d exp(LSE_d - LSE) O_d with LSE the
      [2DR] section 5.2 merge; the page's annotation of the all-gather of O as a
      concatenation along the sequence is not a combination rule.
  R3  Logs are natural; the softmax scale is applied inside the scores.
  R4  Absorbed MLA: q is 576-d per head, K is the whole 576-d latent, V is its
      first 512 entries, one latent shared by all query heads.
  R5  fp8 is OCP e4m3fn (bias 7, max 448, codes 0x7F/0xFF are NaN, no inf),
      one bf16 scale per (layer, page); value = code * scale.
  R6  Ownership is decided by the destination global page VALUE (g mod N), as
      [2DR] section 6.3 states; the [PR28] review warns against using the
      residue of a position in the source page list.
  R7  Prefix-cached pages are the leading whole pages [0, c): never read,
      never written.
  R8  The reshard copies whole pages, tail bytes of a partial last page
      included; attention masks positions >= T.
  R9  Causal drafts: T includes the q_len draft positions; query t sits at
      position T - q_len + t and sees positions <= its own.  Every shard
      serves all q_len queries.
  R10 GQA: query head h reads KV head h // (Hq / Hkv).
  R11 An empty shard yields (O, LSE) = (0, -inf) and gets zero weight.
  R12 The free list is a FIFO: allocation pops from the front, freeing
      appends to the back.
  R17 Bounded pack: a path's pages are packed entry-major (one page's layers in
      a row) into a staging buffer of a fixed number of pages, window after
      window; the pages give the idea (a fixed pre-registered buffer reused in
      chunks, the same bytes moved), not a layout, so the order is ours.
  R18 Token ownership ([SGL]: token t lives on rank t mod N): token t is the
      (t div N)-th token of shard t mod N; shard d's local page j holds its
      tokens j*page_size .. j*page_size + page_size - 1 and sits at the slot of
      the request's j-th virtual page (the allocator's unit of N pages), the
      same slot page ownership gives it.
  R19 Per-page fp8 scales under token ownership: a destination page gathers
      tokens of N source pages, each quantised with its own page's scale, so a
      byte copy cannot keep one scale per page; the token reshard moves only
      pools without scales.

Parity pins live in tests/test_oracle_pins.py; every function here has one.
"""

from __future__ import annotations

import math
from collections import deque
from typing import List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")

# --------------------------------------------------------------------------
# Layer split on the prefill side  ([2DR] section 4.1)
# --------------------------------------------------------------------------


def layer_range(num_layers: int, num_sources: int, r: int) -> Tuple[int, int]:
    """Half-open layer range owned by layer-split source r.

    [2DR] section 4.1, the layer-assignment equation: contiguous ranges of
    floor(L / N_cp) layers, the first (L mod N_cp) ranks taking one extra.
    """
    if num_sources <= 0 or not (0 <= r < num_sources) or num_layers < 0:
        raise ValueError("bad layer split")
    base, extra = divmod(num_layers, num_sources)
    start = r * base + min(r, extra)
    end = (r + 1) * base + min(r + 1, extra)
    return start, end


def local_layer_count(num_layers: int, num_sources: int, r: int) -> int:
    """Layer slots in source r's pool: owned layers plus one transient slot.

    [2DR] section 4.1 (KV pool of per+1 slots per rank).  The transient slot
    holds broadcast prefix KV of other owners and is never read by the reshard.
    """
    a, b = layer_range(num_layers, num_sources, r)
    return (b - a) + 1


def layer_owner(num_layers: int, num_sources: int, layer: int) -> int:
    """The source that owns a layer: the inverse of layer_range ([2DR] 4.2)."""
    for r in range(num_sources):
        a, b = layer_range(num_layers, num_sources, r)
        if a <= layer < b:
            return r
    raise ValueError("layer out of range")


# --------------------------------------------------------------------------
# DCP page round robin  ([2DR] sections 5.1, 6.2)
# --------------------------------------------------------------------------


def dcp_owner(p: int, n: int) -> int:
    """owner(p) = p mod N  ([2DR] section 5.1)."""
    return p % n


def dcp_local_slot(p: int, n: int) -> int:
    """slot_local(p) = floor(p / N)  ([2DR] section 5.1)."""
    return p // n


def filter_kv_indices_for_dcp_rank(kv_indices: Sequence[int], n: int, d: int) -> List[int]:
    """Pages of the full list owned by DCP rank d, compressed to local slots.

    [2DR] section 6.2: keep p with p mod N = d and map it to floor(p / N);
    with N <= 1 the list passes unchanged.
    """
    if n <= 1:
        return [int(p) for p in kv_indices]
    return [int(p) // n for p in kv_indices if int(p) % n == d]


class PageMap:
    """DCP page allocator ([2DR] sections 5.1 and 6.4).

    The allocator hands out virtual pages of page_size * N tokens; virtual page
    v is the N physical pages with global ids v*N .. v*N + N-1, i.e. local slot
    v on every rank.  Sequence page i of a request therefore gets global page
    v[i // N] * N + (i mod N).  The free list order is an input (reading R12).
    """

    def __init__(self, dcp_size: int, page_size: int, num_virtual_pages: int,
                 free_order: Optional[Sequence[int]] = None):
        if dcp_size <= 0 or page_size <= 0 or num_virtual_pages <= 0:
            raise ValueError("bad page map geometry")
        self.n = dcp_size
        self.page_size = page_size
        self.m = num_virtual_pages
        order = list(range(num_virtual_pages)) if free_order is None else [int(v) for v in free_order]
        if sorted(order) != list(range(num_virtual_pages)):
            raise ValueError("free order is not a permutation")
        self.free = deque(order)
        self.used = set()

    def alloc(self, num_tokens: int) -> List[int]:
        if num_tokens <= 0:
            raise ValueError("empty request")
        pages = -(-num_tokens // self.page_size)
        virt = -(-pages // self.n)
        if virt > len(self.free):
            raise MemoryError("page map exhausted")
        vs = [self.free.popleft() for _ in range(virt)]
        self.used.update(vs)
        return [vs[i // self.n] * self.n + (i % self.n) for i in range(pages)]

    def release(self, global_pages: Sequence[int]) -> None:
        vs = []
        for g in global_pages:
            v = int(g) // self.n
            if v not in vs:
                vs.append(v)
        for v in vs:
            if v not in self.used:
                raise ValueError("double free")
        for v in vs:
            self.used.remove(v)
            self.free.append(v)


def block_tables(global_pages: Sequence[Sequence[int]], n: int, own: str = "page") -> List[List[List[int]]]:
    """Per shard d and request b: the slots of d's local pages, in order.

    own == "page": the pages d owns, in sequence order ([2DR] section 5.1).
    own == "token" (reading R18): local page j of every shard holds that shard's
    tokens of the request's j-th virtual page, whose slot is g_{jN} div N.
    """
    out = [[[] for _ in global_pages] for _ in range(n)]
    for b, pages in enumerate(global_pages):
        if own == "token":
            for j in range(0, len(pages), n):
                for d in range(n):
                    out[d][b].append(dcp_local_slot(int(pages[j]), n))
            continue
        for g in pages:
            out[dcp_owner(int(g), n)][b].append(dcp_local_slot(int(g), n))
    return out


def token_owner(t: int, n: int) -> int:
    """[SGL]: token t of the sequence lives on rank t mod N."""
    return t % n


def token_place(t: int, n: int, page_size: int, global_pages: Sequence[int]) -> Tuple[int, int, int]:
    """(shard, slot, row) of token t under token ownership (reading R18): shard t mod N holds it
    as its (t div N)-th token, row (t div N) mod page_size of its local page (t div N) div page_size,
    which sits at the slot of the request's virtual page of that index."""
    d = token_owner(t, n)
    u = t // n
    j = u // page_size
    return d, dcp_local_slot(int(global_pages[j * n]), n), u % page_size


# --------------------------------------------------------------------------
# Page-level 2D reshard  ([2DR] sections 2, 6.2-6.6)
# --------------------------------------------------------------------------


def reshard_plan(num_layers: int, num_sources: int, dcp_size: int,
                 src_page_ids: Sequence[int], dst_global_pages: Sequence[int],
                 first_uncached: int, dst_filter: int = -1):
    """Every page copy the reshard performs, as (r, src_layer_slot, src_page, d, layer, dst_slot).

    [2DR] section 2: for each path (r, d) transfer L_r x P_d.  Section 6.3:
    within one transfer, source and destination lists pair by position, and
    ownership is the destination page value's residue mod N (reading R6).
    Section 6.6: no CP-side index filtering under layer split.  Pages before
    first_uncached are prefix-cached and skipped (reading R7).
    """
    plan = []
    for r in range(num_sources):
        a, b = layer_range(num_layers, num_sources, r)
        for layer in range(a, b):
            for i in range(first_uncached, len(dst_global_pages)):
                g = int(dst_global_pages[i])
                if dcp_size > 1:
                    d, s = dcp_owner(g, dcp_size), dcp_local_slot(g, dcp_size)
                else:
                    d, s = 0, g
                if dst_filter >= 0 and d != dst_filter:
                    continue
                plan.append((r, layer - a, int(src_page_ids[i]), d, layer, s))
    return plan


def reshard(src_pools: Sequence[np.ndarray], dst_pools: Sequence[np.ndarray],
            num_layers: int, dcp_size: int, src_page_ids, dst_global_pages,
            first_uncached: int, dst_filter: int = -1,
            src_scales=None, dst_scales=None) -> List[int]:
    """Scalar page-map reshard on byte arrays; returns pages sent per destination.

    src_pools[r]: uint8 [|L_r|+1][S][page_bytes]; dst_pools[d]: uint8 [L][M][page_bytes]
    (modified in place).  Optional scales: src_scales[r] [|L_r|+1][S], dst_scales[d]
    [L][M] (uint16 bf16 bit patterns), moved like their pages.
    """
    num_sources = len(src_pools)
    sent = [0] * dcp_size
    for (r, ls, sp, d, layer, s) in reshard_plan(num_layers, num_sources, dcp_size, src_page_ids,
                                                 dst_global_pages, first_uncached, dst_filter):
        dst_pools[d][layer, s, :] = src_pools[r][ls, sp, :]
        if src_scales is not None and dst_scales is not None:
            dst_scales[d][layer, s] = src_scales[r][ls, sp]
        if r == 0 and ls == 0:
            sent[d] += 1
    return sent


# --------------------------------------------------------------------------
# Token scatter reshard under token ownership (readings R18, R19)
# --------------------------------------------------------------------------


def reshard_tokens(src_pools: Sequence[np.ndarray], dst_pools: Sequence[np.ndarray], num_layers: int,
                   dcp_size: int, page_size: int, token_rows: int, row_bytes: int, src_page_ids,
                   dst_global_pages, first_uncached: int, request_offsets=None) -> int:
    """Token-granular version of the 2D reshard for pools under token ownership; returns rows moved.

    [2DR] section 2 moves L_r x P_d per path; with token ownership ([SGL]) a
    source page's tokens land on every rank (reading R18: token t is row
    (t div N) mod page_size of local page (t div N) div page_size of shard t mod N,
    at the slot of that virtual page).  A page holds token_rows blocks of
    page_size rows of row_bytes bytes; token x of a page is row x of every block.
    Whole uncached source pages move, tail rows included (reading R8).  The
    lists concatenate requests: request b holds entries [o_b, o_{b+1}) of
    request_offsets (None: one request), and its entry i is its sequence page
    i - o_b.  first_uncached counts list entries.  Pools are uint8
    [.][S or M][page_bytes].
    """
    num_sources = len(src_pools)
    offs = [0, len(dst_global_pages)] if request_offsets is None else [int(o) for o in request_offsets]
    moved = 0
    for r in range(num_sources):
        a, b = layer_range(num_layers, num_sources, r)
        for layer in range(a, b):
            for i in range(first_uncached, len(dst_global_pages)):
                q = max(k for k in range(len(offs) - 1) if offs[k] <= i < offs[k + 1])
                req_pages = dst_global_pages[offs[q]:offs[q + 1]]
                src = src_pools[r][layer - a, int(src_page_ids[i])].reshape(token_rows, page_size, row_bytes)
                for x in range(page_size):
                    d, slot, y = token_place((i - offs[q]) * page_size + x, dcp_size, page_size, req_pages)
                    dst = dst_pools[d][layer, slot].reshape(token_rows, page_size, row_bytes)
                    dst[:, y, :] = src[:, x, :]
                    moved += 1
    return moved


# --------------------------------------------------------------------------
# Bounded pack / unpack of one (source, destination) path (reading R17)
# --------------------------------------------------------------------------


def path_entries(src_page_ids, dst_global_pages, first_uncached: int, dcp_size: int, dest: int,
                 src_pages: int, dst_pages: int) -> List[int]:
    """List positions the path to `dest` carries, in list order.

    [2DR] section 2: a path moves P_d pages; section 6.3: ownership by the
    destination page value (reading R6); reading R7: entries before
    first_uncached are cached.  Entries with ids out of range carry nothing
    (the reshard skips them too).
    """
    out = []
    for i in range(first_uncached, len(dst_global_pages)):
        g, sp = int(dst_global_pages[i]), int(src_page_ids[i])
        if dcp_size > 1:
            d, s = dcp_owner(g, dcp_size) if g >= 0 else -1, g // dcp_size if g >= 0 else -1
        else:
            d, s = 0, g
        if g < 0 or s >= dst_pages or not (0 <= sp < src_pages):
            continue
        if d == dest:
            out.append(i)
    return out


def path_units(num_layers: int, num_sources: int, r: int, entries: Sequence[int]) -> List[Tuple[int, int]]:
    """Units (list position, layer) of path (r, .), entry-major: one page's |L_r| layers in a row
    ([2DR] section 2: the path carries L_r x P_d pages)."""
    a, b = layer_range(num_layers, num_sources, r)
    return [(i, layer) for i in entries for layer in range(a, b)]


def pack_pages(src_pool: np.ndarray, src_scale, src_page_ids, num_layers: int, num_sources: int, r: int,
               entries: Sequence[int], unit_begin: int, cap_units: int, staging: np.ndarray,
               staging_scales=None) -> int:
    """Copy the window of units [unit_begin, unit_begin + n) of path (r, .) into staging (in place).

    [PR28] bounded pack: a fixed buffer of cap_units pages is filled window by
    window; n = min(cap_units, units - unit_begin), none past the end.
    staging[k] = src_pool[layer - begin_r][src page of the entry], k = u - unit_begin.
    """
    units = path_units(num_layers, num_sources, r, entries)
    a, _ = layer_range(num_layers, num_sources, r)
    n = max(0, min(cap_units, len(units) - unit_begin))
    for k in range(n):
        i, layer = units[unit_begin + k]
        sp = int(src_page_ids[i])
        staging[k, :] = src_pool[layer - a, sp, :]
        if src_scale is not None and staging_scales is not None:
            staging_scales[k] = src_scale[layer - a, sp]
    return n


def unpack_pages(dst_pool: np.ndarray, dst_scale, dst_global_pages, num_layers: int, num_sources: int, r: int,
                 dcp_size: int, entries: Sequence[int], unit_begin: int, cap_units: int, staging: np.ndarray,
                 staging_scales=None) -> int:
    """Scatter the same window from staging into the destination pool (in place):
    dst_pool[layer][g div N] = staging[k] (N == 1: slot g), section 6.3's value-owned slot."""
    units = path_units(num_layers, num_sources, r, entries)
    n = max(0, min(cap_units, len(units) - unit_begin))
    for k in range(n):
        i, layer = units[unit_begin + k]
        g = int(dst_global_pages[i])
        s = dcp_local_slot(g, dcp_size) if dcp_size > 1 else g
        dst_pool[layer, s, :] = staging[k, :]
        if dst_scale is not None and staging_scales is not None:
            dst_scale[layer, s] = staging_scales[k]
    return n


# --------------------------------------------------------------------------
# Number formats (readings R5)
# --------------------------------------------------------------------------


def e4m3fn_value(code: int) -> float:
    """Value of an OCP fp8 e4m3fn code: 1 sign, 4 exponent (bias 7), 3 mantissa bits."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16 / int16) to float64: the top half of a float32."""
    b = (np.asarray(bits).astype(np.int64) & 0xFFFF).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_split_page(page: np.ndarray, dtype: str, num_kv_heads: int, page_size: int, head_dim: int):
    """A split-layout page [K,V][Hkv][page_size][D] to float64 (K, V), each [Hkv][page_size][D]."""
    raw = np.ascontiguousarray(page)
    if dtype == "f32":
        x = raw.view(np.float32).astype(np.float64)
    elif dtype == "bf16":
        x = bf16_bits_to_f64(raw.view(np.uint16))
    else:
        raise ValueError(dtype)
    x = x.reshape(2, num_kv_heads, page_size, head_dim)
    return x[0], x[1]


def decode_mla_page(page: np.ndarray, scale_bits: int, page_size: int, dim: int = 576) -> np.ndarray:
    """An fp8 latent page [page_size][576] with its bf16 scale to float64 [page_size][576]."""
    codes = np.ascontiguousarray(page).reshape(page_size, dim)
    scale = float(bf16_bits_to_f64(np.array([int(scale_bits)]))[0])
    return E4M3FN_TABLE[codes] * scale


# --------------------------------------------------------------------------
# Attention  ([2DR] section 5.2; [SGL] DCP paragraph)
# --------------------------------------------------------------------------


def softmax_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray, scale: float):
    """Softmax attention of rows q [R][Dqk] over keys k [T][Dqk], values v [T][Dv].

    visible: bool [R][T].  Returns (O [R][Dv], LSE [R]) with
    s_j = scale * q . k_j,  LSE = log sum_j exp(s_j),  O = sum_j exp(s_j - LSE) v_j
    over visible j; a row with nothing visible gives (0, -inf) (reading R11).
    Consecutive rows that see the same tokens share one gather of those keys and
    values and one matmul for their scores (column c of S holds row r0 + c's).
    """
    r_rows = q.shape[0]
    out = np.zeros((r_rows, v.shape[1]), dtype=np.float64)
    lse = np.full((r_rows,), NEG_INF, dtype=np.float64)
    r0 = 0
    while r0 < r_rows:
        r1 = r0 + 1
        while r1 < r_rows and np.array_equal(visible[r1], visible[r0]):
            r1 += 1
        idx = np.nonzero(visible[r0])[0]
        if idx.size:
            s = scale * (k[idx] @ q[r0:r1].T)       # [visible tokens][rows]
            m = s.max(axis=0)
            lse[r0:r1] = m + np.log(np.exp(s - m).sum(axis=0))
            out[r0:r1] = np.exp(s - lse[r0:r1]).T @ v[idx]
        r0 = r1
    return out, lse


def query_positions(seq_len: int, q_len: int) -> List[int]:
    """Position of each of the q_len queries (reading R9)."""
    return [seq_len - q_len + t for t in range(q_len)]


def request_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, seq_len: int, scale: float,
                      token_mask: Optional[np.ndarray] = None, heads: Optional[Sequence[int]] = None):
    """Attention of one request, all queries, all heads (or the listed ones).

    q: [q_len][Hq][Dqk]; k: [Hkv][T][Dqk]; v: [Hkv][T][Dv] (logical token order).
    token_mask: optional bool [T]: tokens this shard holds (None = all).
    heads: optional subset of query heads to compute (others are left 0 / -inf).
    Returns O [q_len][Hq][Dv], LSE [q_len][Hq].
    """
    q_len, hq, _ = q.shape
    hkv = k.shape[0]
    group = hq // hkv
    t_all = np.arange(seq_len)
    out = np.zeros((q_len, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((q_len, hq), NEG_INF, dtype=np.float64)
    hs = list(range(hq) if heads is None else heads)
    for t, pos in enumerate(query_positions(seq_len, q_len)):
        vis = t_all <= pos
        if token_mask is not None:
            vis = vis & token_mask[:seq_len]
        for kh in range(hkv):
            rows = [h for h in hs if h // group == kh]  # reading R10: query head h reads KV head h // group
            if not rows:
                continue
            o, l = softmax_rows(q[t, rows], k[kh, :seq_len], v[kh, :seq_len],
                                np.broadcast_to(vis, (len(rows), seq_len)), scale)
            out[t, rows], lse[t, rows] = o, l
    return out, lse


def shard_token_mask(global_pages: Sequence[int], page_size: int, seq_len: int, n: int, d: int,
                     own: str = "page") -> np.ndarray:
    """Tokens held by shard d: those whose page's global id is owned by d ([2DR] 5.1), or, with
    own == "token", those with t mod N == d ([SGL])."""
    mask = np.zeros(seq_len, dtype=bool)
    if own == "token":
        for t in range(seq_len):
            mask[t] = token_owner(t, n) == d
        return mask
    for i, g in enumerate(global_pages):
        if dcp_owner(int(g), n) == d:
            mask[i * page_size:min(seq_len, (i + 1) * page_size)] = True
    return mask


def request_partials(q, k, v, seq_len, scale, global_pages, page_size, n, heads=None, own="page"):
    """Per-shard partials of one request: O [N][q_len][Hq][Dv], LSE [N][q_len][Hq]."""
    outs, lses = [], []
    for d in range(n):
        o, l = request_attention(q, k, v, seq_len, scale,
                                 shard_token_mask(global_pages, page_size, seq_len, n, d, own), heads)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def lse_merge(partial_out: np.ndarray, partial_lse: np.ndarray):
    """Exact merge of N partials ([2DR] section 5.2; [SGL]; readings R2, R11).

    partial_out [N][..][Dv], partial_lse [N][..] -> (O [..][Dv], LSE [..]):
    LSE = m + log sum_d exp(LSE_d - m), m = max_d LSE_d;  O = sum_d exp(LSE_d - LSE) O_d.
    """
    m = partial_lse.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(finite[None], np.exp(partial_lse - m_safe[None]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), NEG_INF)
    wn = np.where(finite[None], w / np.where(finite, tot, 1.0)[None], 0.0)
    out = (wn[..., None] * partial_out).sum(axis=0)
    return out, lse


# --------------------------------------------------------------------------
# Gathering a request's logical KV from paged pools (addressing of [2DR] 5.1)
# --------------------------------------------------------------------------


def logical_kv_split(pool_pages_of, global_pages, n, dtype, num_kv_heads, page_size, head_dim, seq_len):
    """Logical (K, V) [Hkv][T][D] of one request from split-layout DCP pools.

    pool_pages_of(d, slot) returns the raw page bytes held by shard d at local slot.
    """
    ks, vs = [], []
    for g in global_pages:
        k, v = decode_split_page(pool_pages_of(dcp_owner(int(g), n), dcp_local_slot(int(g), n)),
                                 dtype, num_kv_heads, page_size, head_dim)
        ks.append(k)
        vs.append(v)
    k = np.concatenate(ks, axis=1)[:, :seq_len]
    v = np.concatenate(vs, axis=1)[:, :seq_len]
    return k, v


def logical_kv_mla(page_and_scale_of, global_pages, n, page_size, seq_len, dv=512):
    """Logical (K, V) [1][T][576], [1][T][512] of one request from fp8 latent pools (reading R4)."""
    lat = []
    for g in global_pages:
        page, sbits = page_and_scale_of(dcp_owner(int(g), n), dcp_local_slot(int(g), n))
        lat.append(decode_mla_page(page, sbits, page_size))
    x = np.concatenate(lat, axis=0)[:seq_len]
    return x[None], x[None, :, :dv]


def logical_kv_split_tokens(pool_pages_of, global_pages, n, dtype, num_kv_heads, page_size, head_dim, seq_len):
    """Logical (K, V) [Hkv][T][D] of one request from split-layout pools under token ownership."""
    cache = {}
    k = np.zeros((num_kv_heads, seq_len, head_dim))
    v = np.zeros((num_kv_heads, seq_len, head_dim))
    for t in range(seq_len):
        d, slot, row = token_place(t, n, page_size, global_pages)
        if (d, slot) not in cache:
            cache[(d, slot)] = decode_split_page(pool_pages_of(d, slot), dtype, num_kv_heads, page_size, head_dim)
        pk, pv = cache[(d, slot)]
        k[:, t] = pk[:, row]
        v[:, t] = pv[:, row]
    return k, v


def logical_kv_mla_tokens(page_and_scale_of, global_pages, n, page_size, seq_len, dv=512):
    """Logical (K, V) [1][T][576], [1][T][512] from fp8 latent pools under token ownership; each
    token is dequantised with the scale of the page that holds it."""
    cache = {}
    x = np.zeros((seq_len, 576))
    for t in range(seq_len):
        d, slot, row = token_place(t, n, page_size, global_pages)
        if (d, slot) not in cache:
            page, sbits = page_and_scale_of(d, slot)
            cache[(d, slot)] = decode_mla_page(page, sbits, page_size)
        x[t] = cache[(d, slot)][row]
    return x[None], x[None, :, :dv]
