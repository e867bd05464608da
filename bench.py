"""Benchmark of the DCP hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. page-level 2D reshard of the transferred requests' pages from the
     layer-split sources into the N DCP pools (kv_reshard_pages),
  2. per-shard partial decode attention over the N pools (dcp_decode_partial),
  3. exact LSE merge of the N partials (dcp_lse_merge).

With no arguments the bench runs the four full-size workloads one after the
other in one process (each with its own inputs resident in HBM before its timed
region) and prints ONE JSON line.  The headline (`config.workload`, `value`,
`roofline`, `cpu_baseline`) is the largest single-GPU workload, the long-context
mix with speculative verify; every workload's own figures, roofline and CPU
oracle baseline are under `parts.workloads`.

    python bench.py [--steps K] [--warmup W] [--workload all|NAME] [--gpus 1]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 matrix peak
ROOT = os.path.dirname(os.path.abspath(__file__))
WORKLOADS = ("gqa_bf16_16x4k-32k", "reshard_mla_128k", "mla_fp8_48x100k", "mla_fp8_longmix_verify")
HEADLINE = "mla_fp8_longmix_verify"
# sources behind each timed call (a stored counter figure is used only while they are unchanged)
CALL_SOURCES = {"reshard_kernel": ["reshard.hip", "common.h"],
                "reshard_tokens_kernel": ["reshard.hip", "common.h"],
                "dcp_decode_partial": ["attention.hip", "attn_common.h", "attn_kernels.h", "dispatch.hip",
                                       "gqa_bf16.hip", "mla_fp8.hip"]}
# kernels of each timed call, as rocprofv3 names them; the first one that appears counts launches
CALL_KERNELS = {"reshard_kernel": ("reshard_kernel",), "reshard_tokens_kernel": ("reshard_tokens_kernel",),
                "dcp_decode_partial": ("gqa_bf16_even_kernel", "gqa_bf16_kernel", "mla_fp8_kernel",
                                       "partial_generic_kernel", "plan_kernel", "plan_even_kernel",
                                       "chunk_reduce_kernel", "even_reduce_kernel")}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", help="'all' (the four full-size workloads) or one name")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="budget of the CPU oracle sample per workload (half reshard, half attention)")
    ap.add_argument("--own", choices=["page", "token"], default="page",
                    help="DCP ownership: page p on shard p mod N (default) or token t on shard t mod N")
    ap.add_argument("--pack-cap-mib", type=int, default=64,
                    help="staging buffer of the path-by-path (bounded pack/unpack) transfer timed after the "
                         "steps; 0 skips it")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain copy of this many MiB (torch bitwise_not, int32) before timing: a "
                         "known-size kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--pmc-summarize", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "BENCH_JSON"),
                    help="no GPU run: turn the counter_collection.csv files of a FETCH_SIZE pass and a "
                         "WRITE_SIZE pass of this bench (one workload, run with --calib-copy-mib) plus the JSON "
                         "line that run printed into HBM bytes per launch of each timed call, stored in "
                         "profiles/pmc_traffic.json")
    return ap.parse_args(argv)


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "context_paged_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_DB = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def load_traffic(kernel_key: str, src_hash: str, launches_bytes: float = 0.0, path: str = TRAFFIC_DB):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(path) as f:
            d = json.load(f)
        e = d[kernel_key]
        if e.get("source_hash") != src_hash:
            return None
        return float(e["hbm_bytes_per_launch"])
    except Exception:
        return None


def device_telemetry():
    """What distinguishes one box from another: memory clock, partition modes and a hash of the
    device's unique id, read from sysfs (nothing is changed; missing entries are left out)."""
    out = {}
    try:
        import glob
        cards = sorted(glob.glob("/sys/class/drm/card*/device/current_compute_partition"))
        base = os.path.dirname(cards[0]) if cards else None
        if base is None:
            for c in sorted(glob.glob("/sys/class/drm/card*/device")):
                if os.path.exists(os.path.join(c, "pp_dpm_mclk")):
                    base = c
                    break
        if base is None:
            return out

        def rd(name):
            try:
                with open(os.path.join(base, name)) as f:
                    return f.read().strip()
            except OSError:
                return None

        for key, name in (("compute_partition", "current_compute_partition"),
                          ("memory_partition", "current_memory_partition")):
            v = rd(name)
            if v:
                out[key] = v
        mclk = rd("pp_dpm_mclk")
        if mclk:
            cur = [ln for ln in mclk.splitlines() if ln.strip().endswith("*")]
            out["memory_clock"] = (cur[0] if cur else mclk.splitlines()[-1]).split(":", 1)[-1].strip(" *")
        sclk = rd("pp_dpm_sclk")
        if sclk:
            cur = [ln for ln in sclk.splitlines() if ln.strip().endswith("*")]
            if cur:
                out["shader_clock"] = cur[0].split(":", 1)[-1].strip(" *")
        uid = rd("unique_id")
        if uid:
            out["unique_id_hash"] = hashlib.sha256(uid.encode()).hexdigest()[:12]
    except Exception:
        pass
    return out


class Step:
    """Device state of one workload: inputs, outputs and the three calls."""

    def __init__(self, w, dev, own: str = "page"):
        import torch
        import context_paged_kv_amd as K
        from workloads import gen

        self.w, self.dev, self.K = w, dev, K
        self.own = 1 if own == "token" else 0
        N, M, pb = w.dcp_size, w.pool_pages, w.page_bytes
        self.seq_lens = gen.draw_seq_lens(w)
        self.total_tokens = int(self.seq_lens.sum())
        pm = K.PageMap(N, w.page_size, M, gen.draw_free_order(w))
        self.pages = [pm.alloc(int(t)) for t in self.seq_lens]
        pm.close()
        self.max_local = max(-(-len(p) // N) for p in self.pages)
        tables, _ = K.dcp_build_block_tables(N, self.pages, self.max_local, token_interleave=self.own)
        # the transfer: every request's pages (or only the long ones), from the layer-split sources
        self.has_reshard = w.num_sources > 0
        self.has_attention = w.has_attention
        self.reshard_reqs = ([b for b in range(w.num_requests) if self.seq_lens[b] >= w.reshard_min_len]
                             if self.has_reshard else [])
        self.num_pages = sum(len(self.pages[b]) for b in self.reshard_reqs)
        S = max(1, self.num_pages)
        self.src_pages = S
        self.src, self.src_scales = [], ([] if w.has_scales else None)
        for r in range(w.num_sources):
            a, b = K.cp_layersplit_layer_range(w.num_layers, w.num_sources, r)
            t = torch.empty((b - a + 1, S, pb), dtype=torch.uint8, device=dev)
            sc = torch.empty((b - a + 1, S), dtype=torch.int16, device=dev) if w.has_scales else None
            gen.fill_pages_(t[:-1].reshape(-1, pb), w, "src", sub=r, scales=None if sc is None else sc[:-1].reshape(-1))
            t[-1].fill_(gen.SRC_TRANSIENT_SENTINEL)
            self.src.append(t)
            if sc is not None:
                sc[-1].fill_(gen.SCALE_SENTINEL)
                self.src_scales.append(sc)
            print(f"[bench] {w.name}: source {r + 1} of {w.num_sources} filled", file=sys.stderr, flush=True)
        # pools: random pages where requests are not transferred in the step, else a sentinel
        fill_random = self.has_attention and len(self.reshard_reqs) < w.num_requests
        self.pools, self.scales = [], ([] if w.has_scales else None)
        for d in range(N):
            t = torch.empty((w.num_layers, M, pb), dtype=torch.uint8, device=dev)
            sc = torch.empty((w.num_layers, M), dtype=torch.int16, device=dev) if w.has_scales else None
            if fill_random:
                gen.fill_pages_(t.view(-1, pb), w, "pool", sub=d, scales=None if sc is None else sc.view(-1))
            else:
                t.fill_(gen.DST_SENTINEL)
                if sc is not None:
                    sc.fill_(gen.SCALE_SENTINEL)
            self.pools.append(t)
            if sc is not None:
                self.scales.append(sc)
            print(f"[bench] {w.name}: pool {d + 1} of {N} filled", file=sys.stderr, flush=True)
        self.src_ids = torch.from_numpy(gen.draw_src_order(w, S)[: self.num_pages].astype(np.int32)).to(dev)
        self.dst_ids = torch.from_numpy(np.concatenate([self.pages[b] for b in self.reshard_reqs] or [np.zeros(0)])
                                        .astype(np.int64)).to(dev)
        self.first_uncached = int(np.floor(w.cached_frac * self.num_pages)) if self.has_reshard else 0
        # where each request's entries start in the lists (the token reshard restarts positions there)
        self.req_offsets = torch.from_numpy(np.cumsum([0] + [len(self.pages[b]) for b in self.reshard_reqs])
                                            .astype(np.int64)).to(dev)
        if not self.has_attention:
            return
        self.q = gen.draw_q(w, dev)
        self.bt = torch.from_numpy(tables).to(dev)
        self.sl = torch.from_numpy(self.seq_lens.astype(np.int32)).to(dev)
        B, ql, hq, dv = w.num_requests, w.q_len, w.num_q_heads, w.head_dim_v
        self.rows = B * ql * hq
        self.desc = K.make_attn_desc(
            kv_dtype={"f32": K.KV_F32, "bf16": K.KV_BF16, "fp8": K.KV_FP8E4M3}[w.kv_dtype],
            kv_layout=K.LAYOUT_MLA if w.layout == "mla" else K.LAYOUT_SPLIT,
            q_dtype=K.Q_BF16 if w.q_dtype == "bf16" else K.Q_F32, num_q_heads=hq, num_kv_heads=w.num_kv_heads,
            head_dim_qk=w.head_dim_qk, head_dim_v=dv, page_size=w.page_size, dcp_size=N, batch=B, q_len=ql,
            max_local_pages=self.max_local, layer=w.attn_layer, num_layers=w.num_layers, pages_per_layer=M,
            softmax_scale=w.softmax_scale, token_interleave=self.own)
        self.ws = torch.empty(K.dcp_decode_partial_workspace(self.desc, self.total_tokens), dtype=torch.uint8,
                              device=dev)
        self.po = torch.empty((N, B, ql, hq, dv), dtype=torch.float32, device=dev)
        self.pl = torch.empty((N, B, ql, hq), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, ql, hq, dv), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, ql, hq), dtype=torch.float32, device=dev)

    # --- the three calls ---------------------------------------------------
    def reshard(self):
        if not self.has_reshard:
            return
        w = self.w
        if self.own:  # token ownership: the token scatter (pools without page scales)
            rows, row_bytes = (1, 576) if w.layout == "mla" else (2 * w.num_kv_heads, w.head_dim_qk * w.elem_bytes)
            self.K.kv_reshard_tokens(num_layers=w.num_layers, dcp_size=w.dcp_size, page_size=w.page_size,
                                     token_rows=rows, row_bytes=row_bytes, src_pages=self.src_pages,
                                     dst_pages=w.pool_pages, src_pools=self.src, dst_pools=self.pools,
                                     src_page_ids=self.src_ids, dst_global_pages=self.dst_ids,
                                     request_offsets=self.req_offsets, first_uncached=self.first_uncached)
            return
        self.K.kv_reshard_pages(num_layers=w.num_layers, dcp_size=w.dcp_size, page_bytes=w.page_bytes,
                                src_pages=self.src_pages, dst_pages=w.pool_pages, src_pools=self.src,
                                dst_pools=self.pools, src_page_ids=self.src_ids, dst_global_pages=self.dst_ids,
                                first_uncached=self.first_uncached, src_scales=self.src_scales,
                                dst_scales=self.scales)

    def prepare_paths(self, cap_pages: int):
        """Entry lists of every destination's path (device) and their sizes (read back once), and a
        staging buffer of cap_pages pages, for the path-by-path transfer."""
        import torch
        w, K = self.w, self.K
        self.geo = dict(num_sources=w.num_sources, num_layers=w.num_layers, dcp_size=w.dcp_size,
                        page_bytes=w.page_bytes, src_pages=self.src_pages, dst_pages=w.pool_pages)
        self.cap = cap_pages
        self.pos, self.cnt = [], []
        for d in range(w.dcp_size):
            pos = torch.empty(max(1, self.num_pages), dtype=torch.int32, device=self.dev)
            cnt = torch.empty(1, dtype=torch.int64, device=self.dev)
            K.kv_path_entries(dest=d, src_page_ids=self.src_ids, dst_global_pages=self.dst_ids, out_positions=pos,
                              out_count=cnt, first_uncached=self.first_uncached, **self.geo)
            self.pos.append(pos)
            self.cnt.append(cnt)
        self.counts = [int(c.item()) for c in self.cnt]
        self.stg = torch.empty((cap_pages, w.page_bytes), dtype=torch.uint8, device=self.dev)
        self.stg_sc = torch.empty(cap_pages, dtype=torch.int16, device=self.dev) if w.has_scales else None
        self.windows = 0
        for d in range(w.dcp_size):
            for r in range(w.num_sources):
                a, b = K.cp_layersplit_layer_range(w.num_layers, w.num_sources, r)
                self.windows += -(-self.counts[d] * (b - a) // cap_pages)

    def path_transfer(self):
        """The reshard done path by path through the staging buffer (pack, then unpack, per window)."""
        w, K = self.w, self.K
        for d in range(w.dcp_size):
            for r in range(w.num_sources):
                a, b = K.cp_layersplit_layer_range(w.num_layers, w.num_sources, r)
                for u0 in range(0, self.counts[d] * (b - a), self.cap):
                    K.kv_pack_pages(source=r, src_pool=self.src[r], src_page_ids=self.src_ids, positions=self.pos[d],
                                    count=self.cnt[d], unit_begin=u0, cap_units=self.cap, staging=self.stg,
                                    src_scales=None if self.src_scales is None else self.src_scales[r],
                                    staging_scales=self.stg_sc, **self.geo)
                    K.kv_unpack_pages(source=r, dest=d, dst_pool=self.pools[d], dst_global_pages=self.dst_ids,
                                      positions=self.pos[d], count=self.cnt[d], unit_begin=u0, cap_units=self.cap,
                                      staging=self.stg, dst_scales=None if self.scales is None else self.scales[d],
                                      staging_scales=self.stg_sc, **self.geo)

    def partial(self):
        if not self.has_attention:
            return
        self.K.dcp_decode_partial(self.desc, q=self.q, kv_pools=self.pools, kv_scales=self.scales,
                                  block_tables=self.bt, seq_lens=self.sl, total_tokens=self.total_tokens,
                                  partial_out=self.po, partial_lse=self.pl, workspace=self.ws)

    def merge(self):
        if not self.has_attention:
            return
        self.K.dcp_lse_merge(self.w.dcp_size, self.rows, self.w.head_dim_v, self.po, self.pl, self.out, self.lse)

    # --- algorithmic bytes ---------------------------------------------------
    def bytes_reshard(self):
        w = self.w
        moved_pages = self.num_pages - self.first_uncached
        moved = moved_pages * w.num_layers * w.page_bytes
        scales = moved_pages * w.num_layers * 2 * 2 if w.has_scales else 0
        ids = moved_pages * (4 + 8)
        return 2 * moved + scales + ids  # read + write

    def flops_attn(self):
        w = self.w
        if not self.has_attention:
            return 0
        # visible (query, key) pairs x heads x (Dqk + Dv) x 2
        pairs = sum(int(t) * w.q_len - w.q_len * (w.q_len - 1) // 2 for t in self.seq_lens)
        return 2.0 * pairs * w.num_q_heads * (w.head_dim_qk + w.head_dim_v)

    def bytes_kv(self):
        """KV bytes the attention must read: every token once (tail of the last page excluded)."""
        w = self.w
        if not self.has_attention:
            return 0
        if w.layout == "mla":
            per_tok = 576
            scales = sum(len(p) for p in self.pages) * 2
        else:
            per_tok = 2 * w.num_kv_heads * w.head_dim_qk * w.elem_bytes
            scales = 0
        return self.total_tokens * per_tok + scales

    def bytes_partial_call(self):
        """Algorithmic HBM bytes of one dcp_decode_partial call: the KV, the query and the
        partials written once."""
        if not self.has_attention:
            return 0
        return self.bytes_kv() + self.q.numel() * self.q.element_size() + (self.po.numel() + self.pl.numel()) * 4

    def bytes_attn_other(self):
        w = self.w
        if not self.has_attention:
            return 0
        qb = self.q.numel() * self.q.element_size()
        partial = self.po.numel() * 4 + self.pl.numel() * 4
        out = self.out.numel() * 4 + self.lse.numel() * 4
        return qb + 2 * partial + out  # partials written once and read once by the merge


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_workers() -> int:
    """Worker processes of the CPU baseline: every core this process may run on, capped at 16,
    the host-core share one GPU of the bench box is given."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(st, budget_s: float):
    """The float64 oracle on the host, timed on a bounded sample of the same workload and
    scaled to the full step.  Units of work run on a pool of worker processes, each with one
    BLAS thread: reshard passes over each worker's own page set (distinct memory, 128 MiB of
    source pages per worker, so the sample streams from DRAM rather than cache), and requests
    of the attention, whose pages are decoded once and whose heads then run one at a time.
    Page bytes are copied from the GPU by this process; the workers never touch it."""
    import multiprocessing as mp
    import oracle as O
    from tests import harness as Hn  # oracle-side page gathering shared with the tests
    from tests import oracle_workers as OW

    w = st.w
    workers = cpu_workers()
    budget = budget_s / (2 if (st.has_reshard and st.has_attention) else 1)
    notes, extra = [], {}
    rs_wall_full = at_wall_full = None
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        with mp.get_context("spawn").Pool(workers) as pool:
            pool.map(OW.warm, range(workers))  # processes up before anything is timed
            if st.has_reshard and st.num_pages > st.first_uncached:
                # real source bytes of up to 16 uncached pages (one layer per source); each worker
                # tiles them into its own 128 MiB source set
                n = min(len(st.dst_ids) - st.first_uncached, 16)
                sids = st.src_ids[st.first_uncached:st.first_uncached + n]
                sample = [st.src[r][0].index_select(0, sids.long()).cpu().numpy() for r in range(w.num_sources)]
                rows, row_bytes = ((1, 576) if w.layout == "mla" else
                                   (2 * w.num_kv_heads, w.head_dim_qk * w.elem_bytes))
                target = 128 << 20
                deadline = time.time() + budget
                t0 = time.perf_counter()
                task = (sample, w.page_bytes, w.dcp_size, st.own, w.page_size, rows, row_bytes, target, deadline)
                res = pool.map(OW.reshard_sample, [task] * workers)
                t_rs = time.perf_counter() - t0
                moved = sum(m for m, _ in res)
                pages = res[0][1]
                rate = moved / t_rs  # bytes read + written per second over all workers
                rs_wall_full = st.bytes_reshard() / rate
                extra["reshard_GBps"] = round(rate / 1e9, 4)
                kind = "token scatter" if st.own else "page"
                notes.append(f"scalar {kind} reshard passes over {pages} distinct pages x {w.num_sources} source(s) "
                             f"({pages * w.page_bytes * w.num_sources >> 20} MiB of source per worker) on {workers} "
                             f"processes, {moved / 1e9:.2f} GB moved in {t_rs:.1f}s")
            if st.has_attention:
                geo = {"layout": w.layout, "kv_dtype": w.kv_dtype, "num_kv_heads": w.num_kv_heads,
                       "head_dim_qk": w.head_dim_qk, "head_dim_v": w.head_dim_v, "page_size": w.page_size,
                       "dcp_size": w.dcp_size, "num_q_heads": w.num_q_heads, "q_len": w.q_len,
                       "softmax_scale": w.softmax_scale, "own": "token" if st.own else "page"}
                n_sh, lay = w.dcp_size, w.attn_layer
                deadline = time.time() + budget
                t0 = time.perf_counter()
                # the requests the sample reaches, shortest first within a bounded set: one task per
                # worker at a time (the longest requests take the oracle tens of seconds to decode)
                order = sorted(range(w.num_requests), key=lambda b: int(st.seq_lens[b]))
                pending, results = [], []
                for b in order[: 2 * workers]:
                    if time.time() >= deadline:
                        break
                    pages = st.pages[b]
                    pages_h = scales_h = by_slot = None
                    if st.own:
                        import torch
                        vslots = [O.dcp_local_slot(int(pages[j]), n_sh) for j in range(0, len(pages), n_sh)]
                        sl = torch.tensor(vslots, dtype=torch.int64, device=st.pools[0].device)
                        by_slot = {}
                        for d in range(n_sh):
                            pb = st.pools[d][lay].index_select(0, sl).cpu().numpy()
                            sc = (st.scales[d][lay].index_select(0, sl).cpu().numpy().astype(np.int64) & 0xFFFF
                                  if st.scales is not None else None)
                            for i, s_ in enumerate(vslots):
                                by_slot[(d, s_)] = (pb[i], None if sc is None else int(sc[i]))
                    else:
                        pages_h, scales_h = Hn.gather_request_pages(st.pools, st.scales, pages, n_sh, lay)
                    q = st.q[b].float().cpu().numpy().astype(np.float64)
                    pending.append(pool.apply_async(OW.request_rows, ((geo, pages_h, scales_h, by_slot, pages,
                                                                       int(st.seq_lens[b]), q, deadline),)))
                    while len(pending) > workers:
                        results.append(pending.pop(0).get())
                results += [r.get() for r in pending]
                t_at = time.perf_counter() - t0
                dec_s = sum(r[0] for r in results)
                dec_tok = sum(r[1] for r in results)
                head_s = sum(r[2] for r in results)
                head_units = sum(r[3] for r in results)  # (token, query, head) triples
                heads = sum(r[4] for r in results)
                if dec_tok and head_units:
                    cpu_s = (st.total_tokens / (dec_tok / dec_s) +
                             st.total_tokens * w.q_len * w.num_q_heads / (head_units / head_s))
                    at_wall_full = cpu_s / workers
                notes.append(f"attention of {len(results)} requests ({dec_tok} tokens decoded, {heads} (request, head) "
                             f"rows of partials + merge) on {workers} processes in {t_at:.1f}s; page decode and "
                             f"per-head work extrapolated separately to all {st.total_tokens} tokens x "
                             f"{w.num_q_heads} heads")
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    if st.has_attention:
        if at_wall_full is None:
            return None
        value = st.bytes_kv() / at_wall_full / 1e9
        unit_note = "attention KV GB/s (partials + merge)"
    else:
        if rs_wall_full is None:
            return None
        value = st.bytes_reshard() / rs_wall_full / 1e9
        unit_note = "reshard GB/s (read + write)"
    out = {"value": round(value, 6), "unit": "GB/s", "cores": workers, "kind": "oracle",
           "sample": f"float64 numpy oracle, {unit_note}, on {workers} worker processes ({_cpu_model()}), one BLAS "
                     "thread each: " + "; ".join(notes) + "; scaled linearly to the full step"}
    out.update(extra)
    return out


def copy_ceiling_gbps(torch, K, dev, nbytes: int, reps: int = 5) -> float:
    """Read + write GB/s of the library's streaming copy (the reshard's own copy loop over one
    contiguous range) over about `nbytes` (capped at 4 GiB), timed with events."""
    n = max(1 << 20, min(int(nbytes), 4 << 30)) // 16 * 16
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    stream = torch.cuda.current_stream()
    K.dcpkv_probe_copy(a, b)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        K.dcpkv_probe_copy(a, b)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del a, b
    return 2 * n / float(np.median(ts)) / 1e9


def scatter_ceiling_gbps(torch, K, dev, page_bytes: int, nbytes: int, reps: int = 5, seed: int = 7) -> float:
    """Read + write GB/s of the library's page-list copy (the same loop over a page list) moving
    about `nbytes` (capped at 4 GiB) in pages of page_bytes between two buffers, source and
    destination pages each in an independent seeded random order: the copy rate this memory
    system gives a page scatter like the reshard's (random page maps on both sides)."""
    pages = max(1, min(int(nbytes), 4 << 30) // page_bytes)
    a = torch.empty(pages * page_bytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    rng = np.random.default_rng(seed)
    sp = torch.from_numpy(rng.permutation(pages).astype(np.int32)).to(dev)
    dp = torch.from_numpy(rng.permutation(pages).astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream()
    K.dcpkv_probe_copy_pages(a, b, sp, dp, page_bytes)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        K.dcpkv_probe_copy_pages(a, b, sp, dp, page_bytes)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del a, b
    return 2 * pages * page_bytes / float(np.median(ts)) / 1e9


def mfma_probe_tflops(torch, K, dev, kind: int, iters: int = 4000, reps: int = 3) -> float:
    """Median TFLOP/s of the library's MFMA rate probe (kind 0: fp16 16x16x32, 1: fp8 16x16x128)."""
    sink = torch.empty(K.PROBE_SINK_FLOATS, dtype=torch.float32, device=dev)
    K.dcpkv_probe_mfma(kind, 100, sink)  # warm-up
    stream = torch.cuda.current_stream()
    rates = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        flops = K.dcpkv_probe_mfma(kind, iters, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        rates.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return float(np.median(rates))


def pmc_summarize(fetch_csv: str, write_csv: str, bench_json: str, calib_mib: int, path: str = TRAFFIC_DB) -> dict:
    """Scale the FETCH_SIZE / WRITE_SIZE readings (KiB per dispatch) of each timed call's kernels by
    what the same counters read for the calibration copy, and store HBM bytes per launch per call."""
    import csv
    import re

    line = None
    with open(bench_json) as f:
        for ln in f:
            ln = ln.strip()
            if ln.startswith("{") and '"roofline"' in ln:
                line = json.loads(ln)
    if line is None:
        sys.exit(f"no bench JSON line in {bench_json}")
    wl = line["config"]["workload"]
    calls = line["parts"]["workloads"][wl]["calls"]
    own = ":token" if line["config"].get("ownership") == "token" else ""

    def per_dispatch(path_, counter):
        rows = {}
        with open(path_) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                rows.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])[1] += float(r["Counter_Value"])
        return [rows[k] for k in sorted(rows)]

    ds = {c: per_dispatch(p, c) for c, p in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv))}
    scale = {}
    for counter, rows in ds.items():
        calib = [v for k, v in rows if "bitwise_not" in k]
        if len(calib) != 1:
            sys.exit(f"{counter}: expected one calibration copy dispatch, found {len(calib)}")
        scale[counter] = calib_mib * (1 << 20) / (calib[0] * 1024.0)  # true bytes per counted byte
    try:
        with open(path) as f:
            db = json.load(f)
    except FileNotFoundError:
        db = {}
    stored = {}
    for call, info in calls.items():
        names = CALL_KERNELS[call]
        out = {}
        for counter, rows in ds.items():
            mine = [(k, v) for k, v in rows if any(re.search(r"\b" + n + r"\b", k) for n in names)]
            main = [n for n in names if any(re.search(r"\b" + n + r"\b", k) for k, _ in mine)]
            if not main:
                break
            launches = sum(1 for k, _ in mine if re.search(r"\b" + main[0] + r"\b", k))
            out[counter] = {"kib_per_launch": sum(v for _, v in mine) / launches, "launches": launches}
        if len(out) != 2:
            continue
        hbm = sum(out[c]["kib_per_launch"] * 1024.0 * scale[c] for c in out)
        key = f"{wl}:{call}{own}"
        db[key] = {"source_hash": info["source_hash"], "hbm_bytes_per_launch": round(hbm),
                   "fetch_kib_per_launch": round(out["FETCH_SIZE"]["kib_per_launch"], 1),
                   "write_kib_per_launch": round(out["WRITE_SIZE"]["kib_per_launch"], 1),
                   "scale_fetch": round(scale["FETCH_SIZE"], 4), "scale_write": round(scale["WRITE_SIZE"], 4),
                   "calib_copy_mib": calib_mib, "launches": out["FETCH_SIZE"]["launches"],
                   "algorithmic_bytes_per_launch": info.get("algorithmic_bytes")}
        stored[key] = db[key]
    if not stored:
        sys.exit("no timed call's kernels in the counter files")
    with open(path, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(stored))
    return stored


def measure(w, dev, a, probes):
    """Inputs of workload w in HBM, W warm-up steps, K timed steps; returns its part of the line."""
    import torch
    K = probes["K"]
    print(f"[bench] building inputs for {w.name}", file=sys.stderr, flush=True)
    st = Step(w, dev, a.own)
    torch.cuda.synchronize()
    if a.calib_copy_mib:  # one elementwise kernel reading and writing exactly this many bytes
        n = a.calib_copy_mib * (1 << 20) // 4
        src_c = torch.ones(n, dtype=torch.int32, device=dev)
        dst_c = torch.empty_like(src_c)
        torch.bitwise_not(src_c, out=dst_c)
        torch.cuda.synchronize()
        del src_c, dst_c
    for _ in range(a.warmup):
        st.reshard()
        st.partial()
        st.merge()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    print(f"[bench] {w.name}: timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        e = evs[i]
        e[0].record(stream)
        st.reshard()
        e[1].record(stream)
        st.partial()
        e[2].record(stream)
        st.merge()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_rs = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    t_pa = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    t_mg = np.array([e[2].elapsed_time(e[3]) for e in evs]) * 1e-3
    t_step = np.array([e[0].elapsed_time(e[3]) for e in evs]) * 1e-3
    if st.has_attention:
        assert torch.isfinite(st.out).all() and torch.isfinite(st.lse).all(), "non-finite attention output"
    b_rs, b_kv, b_other = st.bytes_reshard(), st.bytes_kv(), st.bytes_attn_other()
    part = {"requests": w.num_requests, "total_tokens": st.total_tokens, "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads, "head_dim": w.head_dim_qk, "page_size": w.page_size, "dcp_size": w.dcp_size,
            "q_len": w.q_len, "layers": w.num_layers, "dtype": w.kv_dtype,
            "step": " + ".join(x for x, on in (("reshard", st.has_reshard), ("partial attention", st.has_attention),
                                               ("LSE merge", st.has_attention)) if on),
            "ms_per_step": round(wall / a.steps * 1e3, 4), "step_event_us": round(t_step.mean() * 1e6, 2),
            "bytes": {"reshard_rw": b_rs, "kv": b_kv, "attn_other": b_other}, "calls": {}}
    calls = part["calls"]
    own = ":token" if st.own else ""
    if st.has_reshard:
        rs_gbps = b_rs / t_rs.mean() / 1e9
        name = "reshard_tokens_kernel" if st.own else "reshard_kernel"
        h = kernel_source_hash(CALL_SOURCES[name])
        ceil = copy_ceiling_gbps(torch, K, dev, b_rs // 2)
        sceil = scatter_ceiling_gbps(torch, K, dev, w.page_bytes, b_rs // 2)
        calls[name] = {"us": round(t_rs.mean() * 1e6, 2), "algorithmic_bytes": int(b_rs), "source_hash": h,
                       "traffic": load_traffic(f"{w.name}:{name}{own}", h)}
        part.update({"reshard_GBps": round(rs_gbps, 1), "reshard_frac_hbm": round(rs_gbps / HBM_PEAK_GBPS, 4),
                     "reshard_us": round(t_rs.mean() * 1e6, 2), "copy_ceiling_GBps": round(ceil, 1),
                     "reshard_frac_of_copy_ceiling": round(rs_gbps / ceil, 4),
                     "scatter_copy_ceiling_GBps": round(sceil, 1),
                     "reshard_frac_of_scatter_ceiling": round(rs_gbps / sceil, 4)})
        if a.pack_cap_mib > 0 and not st.own and st.num_pages > st.first_uncached:
            # the same pages path by path through a fixed staging buffer: every page is read and
            # written twice (source -> staging -> pool)
            cap = max(1, (a.pack_cap_mib << 20) // w.page_bytes)
            st.prepare_paths(cap)
            st.path_transfer()
            ts = []
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                st.path_transfer()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            t_pk = float(np.median(ts))
            pk_gbps = 2 * b_rs / t_pk / 1e9
            part.update({"pack_cap_pages": cap, "pack_windows": st.windows, "pack_unpack_us": round(t_pk * 1e6, 2),
                         "pack_unpack_GBps": round(pk_gbps, 1), "pack_unpack_frac_hbm": round(pk_gbps / HBM_PEAK_GBPS, 4),
                         "pack_unpack_time_vs_reshard": round(t_pk / t_rs.mean(), 3)})
    if st.has_attention:
        t_attn = t_pa.mean() + t_mg.mean()
        kv_gbps = b_kv / t_attn / 1e9
        h = kernel_source_hash(CALL_SOURCES["dcp_decode_partial"])
        calls["dcp_decode_partial"] = {"us": round(t_pa.mean() * 1e6, 2), "algorithmic_bytes": int(st.bytes_partial_call()),
                                       "source_hash": h,
                                       "traffic": load_traffic(f"{w.name}:dcp_decode_partial{own}", h)}
        part.update({"attn_kv_GBps": round(kv_gbps, 1), "attn_kv_frac_hbm": round(kv_gbps / HBM_PEAK_GBPS, 4),
                     "attn_all_bytes_GBps": round((b_kv + b_other) / t_attn / 1e9, 1),
                     "attn_TFLOPs": round(st.flops_attn() / t_pa.mean() / 1e12, 1),
                     "partial_us": round(t_pa.mean() * 1e6, 2), "merge_us": round(t_mg.mean() * 1e6, 2),
                     "decode_tokens_per_s": round(w.num_requests * w.q_len / t_attn, 1)})
        if w.layout == "mla":
            # what this device's matrix cores deliver on back-to-back MFMAs of the two kinds the
            # kernel issues, and the MFMA time of its instructions at those rates (latent scores:
            # two fp8 products per score, the query's hi and lo terms; rope and PV: fp16)
            r16, r8 = probes["mfma_f16"], probes["mfma_fp8"]
            pairs = st.flops_attn() / (2.0 * w.num_q_heads * (w.head_dim_qk + w.head_dim_v))
            f8 = 2.0 * pairs * w.num_q_heads * w.head_dim_v * 2
            f16 = 2.0 * pairs * w.num_q_heads * ((w.head_dim_qk - w.head_dim_v) + w.head_dim_v)
            t_mfma = f8 / (r8 * 1e12) + f16 / (r16 * 1e12)
            part.update({"attn_frac_mfma_peak": round(st.flops_attn() / t_pa.mean() / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                         "partial_mfma_us_at_probe_rates": round(t_mfma * 1e6, 2),
                         "partial_frac_of_probe_rates": round(t_mfma / t_pa.mean(), 4)})
    # roofline of the dominant call of the step
    if st.has_reshard and (not st.has_attention or t_rs.mean() >= t_pa.mean()):
        name = "reshard_tokens_kernel" if st.own else "reshard_kernel"
        achieved = b_rs / t_rs.mean() / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    else:
        name = "dcp_decode_partial"
        if w.layout == "mla":  # 128 heads share one latent: the matrix cores bind, fp16 MFMA peak
            achieved = st.flops_attn() / t_pa.mean() / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4)}
        else:
            achieved = st.bytes_partial_call() / t_pa.mean() / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    c = calls[name]
    roof.update({"traffic": c["traffic"], "kernel": name + (" (plan + partial + chunk-reduce kernels)"
                                                            if name == "dcp_decode_partial" else ""),
                 "algorithmic_bytes": c["algorithmic_bytes"], "launch_us": c["us"], "source_hash": c["source_hash"]})
    part["roofline"] = roof
    # the workload's own rate of the metric: attention KV GB/s where there is attention, else the
    # reshard's read + write GB/s
    part["value"] = part["attn_kv_GBps"] if st.has_attention else part["reshard_GBps"]
    part["value_is"] = ("attention KV GB/s (partial + merge)" if st.has_attention
                        else "reshard GB/s (read + write)")
    part["cpu_baseline"] = None
    if not a.no_cpu_baseline:
        print(f"[bench] {w.name}: timing the CPU oracle sample", file=sys.stderr, flush=True)
        part["cpu_baseline"] = cpu_baseline(st, a.cpu_seconds)
    del st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return part


def main():
    a = parse()
    if a.pmc_summarize:
        pmc_summarize(*a.pmc_summarize, a.calib_copy_mib or sys.exit("--pmc-summarize needs --calib-copy-mib"))
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the multi-GPU design "
              "is described in the design notes but not built", file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads.configs import get_workload

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(1)
    names = list(WORKLOADS) if a.workload == "all" else [a.workload]
    ws = [get_workload(n) for n in names]
    if a.own == "token":
        bad = [w.name for w in ws if w.has_scales and w.num_sources > 0]
        if bad:
            print(f"{bad}: their pools carry per-page fp8 scales, which the token reshard does not move",
                  file=sys.stderr)
            sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    import context_paged_kv_amd as K

    probes = {"K": K}
    if any(w.layout == "mla" and w.has_attention for w in ws):
        probes["mfma_f16"] = mfma_probe_tflops(torch, K, dev, 0)
        probes["mfma_fp8"] = mfma_probe_tflops(torch, K, dev, 1)
    parts = {}
    for w in ws:
        parts[w.name] = measure(w, dev, a, probes)
    head_name = HEADLINE if HEADLINE in parts else names[-1]
    head = parts[head_name]
    hw = get_workload(head_name)
    line = {
        "metric": "DCP decode attention KV GB/s (% HBM peak) + reshard GB/s, 1 MI355X",
        "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": hw.kv_dtype, "data": "synthetic (seeded N(0,1) KV, random page maps)",
        "config": {"workload": head_name, "requests": head["requests"], "total_tokens": head["total_tokens"],
                   "q_heads": head["q_heads"], "kv_heads": head["kv_heads"], "head_dim": head["head_dim"],
                   "page_size": head["page_size"], "dcp_size": head["dcp_size"], "q_len": head["q_len"],
                   "layers": head["layers"], "ownership": a.own, "step": head["step"]},
        "parts": {"value_is": head["value_is"] + " of the headline workload",
                  "headline_reshard_GBps": head.get("reshard_GBps"),
                  "headline_reshard_frac_hbm": head.get("reshard_frac_hbm"),
                  "device": device_telemetry(),
                  "mfma_probe_f16_TFLOPs": round(probes["mfma_f16"], 1) if "mfma_f16" in probes else None,
                  "mfma_probe_fp8_TFLOPs": round(probes["mfma_fp8"], 1) if "mfma_fp8" in probes else None,
                  "workloads": parts},
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
