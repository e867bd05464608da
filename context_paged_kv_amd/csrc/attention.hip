// Per-shard partial decode attention and the exact LSE merge.
//
// [2DR] = "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding"
//         (section 5.2: DCP attention, LSE merge; section 8: verify under DCP
//         with several draft tokens per request);
// [SGL] = "SGLang's path" (serving-k3, module 05): each rank produces a
//         partial (weighted sum + log-sum-exp) and the recombination is exact.
//
// This file holds the launch planning shared by every partial kernel, the
// generic VALU kernel (every dtype and layout; the reference path for odd
// shapes), the chunk reduction and dcp_lse_merge.  The MFMA kernels for the
// bf16 GQA and fp8 MLA shapes live in their own files and plug in through
// launch_fast_partial().

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "attn_common.h"
#include "attn_kernels.h"

namespace dcpkv {

// ---------------------------------------------------------------------------
// Plan: chunks per (shard, request) pair and workspace slots (one workgroup)
// ---------------------------------------------------------------------------

constexpr int kPlanThreads = 64;  // one wavefront: shuffles instead of barriers

// Size class of a chunk of `size` pages, 0 for the longest (size >= range), up to 63 for empty
// ones: 64 (range - size) / (range + 1), with rs = 64 / (range + 1) computed once (an ordering
// key only, so the float product needs no exact division; clamped into the 64 classes).
__device__ __forceinline__ int size_key(int size, int range, float rs) {
  const int k = (int)((float)(range - min(size, range)) * rs);
  return min(max(k, 0), 63);
}

// Inclusive prefix sum over the wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

constexpr int kPlanLdsPairs = 4096;  // pairs whose plan entries the planner keeps in LDS

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(AttnParams p) {
  const int lane = threadIdx.x;
  const int num_pairs = p.shard_count * p.batch;
  // One wavefront runs the plan, so its time is the latency of its dependent steps (integer
  // divisions, cross-lane shuffles): every pair's local pages are computed once into LDS
  // (eight request lengths in flight per lane), up to kPlanLdsPairs pairs.
  __shared__ int32_t s_nl[kPlanLdsPairs];
  __shared__ int32_t s_wsb[kPlanLdsPairs];  // each pair's first workspace slot, for the last pass
  auto pages_of = [&](int i, int32_t len) {
    const int d = p.shard_begin + i / p.batch;
    return local_pages_of(len, p.page_size, p.n, d, p.max_local, p.tok_il);
  };
  const bool staged = num_pairs <= kPlanLdsPairs;
  if (staged) {
    for (int i0 = 0; i0 < num_pairs; i0 += 8 * 64) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p.seq_lens[min(i0 + 64 * u + lane, num_pairs - 1) % p.batch];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + 64 * u + lane < num_pairs) s_nl[i0 + 64 * u + lane] = pages_of(i0 + 64 * u + lane, v[u]);
    }
    __syncthreads();
  }
  auto pair_pages = [&](int i) { return staged ? s_nl[i] : pages_of(i, p.seq_lens[i % p.batch]); };
  // Pairs of (nearly) equal length whose work items fill the device's workgroup slots in
  // whole rounds are already balanced: splitting them would only add the chunk round trip
  // and its reduction, so they keep one chunk each.  Equal: longest <= 17/16 of the
  // shortest non-empty pair; whole rounds: at most 1/32 of the slots of the last round idle.
  // In the same pass, the chunk totals of the split at C = chunk_pages: one chunk per pair
  // when the split would not fit the workspace or the launched grid.
  int ne = 0, lo = INT32_MAX, hi = 0;
  long long need = 0, need_all = 0;
  const int Cs = p.chunk_pages;
  for (int i = lane; i < num_pairs; i += 64) {
    const int nl = pair_pages(i);
    if (nl > 0) {
      ++ne;
      lo = min(lo, nl);
      hi = max(hi, nl);
    }
    const int k = nl > Cs ? (nl + Cs - 1) / Cs : 1;
    if (k >= 2) need += k;
    need_all += k;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {  // five independent reductions, their latencies overlapped
    const int ne2 = __shfl_xor(ne, off, 64), lo2 = __shfl_xor(lo, off, 64), hi2 = __shfl_xor(hi, off, 64);
    const long long nd2 = __shfl_xor(need, off, 64), na2 = __shfl_xor(need_all, off, 64);
    ne += ne2;
    lo = min(lo, lo2);
    hi = max(hi, hi2);
    need += nd2;
    need_all += na2;
  }
  const long long items1 = (long long)ne * p.hb_count, slots = p.slots;
  const long long rounds1 = slots > 0 ? (items1 + slots - 1) / slots : 0;
  const bool whole = ne > 0 && (long long)hi * 16 <= (long long)lo * 17 && items1 >= slots && slots > 0 &&
                     (rounds1 * slots - items1) * 32 <= rounds1 * slots;
  const int C = whole ? INT32_MAX : Cs;
  if (whole) {
    need = 0;
    need_all = num_pairs;
  }
  const int fallback = (need > (long long)p.ws_cap || need_all > (long long)p.max_chunks) ? 1 : 0;
  // size classes of the longest-first order: chunk sizes run up to C pages (a pair's whole
  // length when it is not split)
  __shared__ int s_cnt[64];
  s_cnt[lane] = 0;
  __syncthreads();
  const int range = (C == INT32_MAX || fallback) ? max(hi, 1) : C;
  const float rs = 64.f / ((float)range + 1.f);
  // then exclusive prefix sums of the chunks and of the workspace slots, 64 pairs at a time
  int carry_k = 0, carry_w = 0;
  for (int base = 0; base < num_pairs; base += 64) {
    const int i = base + lane;
    int k = 0, kw = 0, nl = 0;
    if (i < num_pairs) {
      nl = pair_pages(i);
      k = (!fallback && nl > C) ? (nl + C - 1) / C : 1;
      kw = k >= 2 ? k : 0;
    }
    const int sk = wave_incl_scan(k), sw = wave_incl_scan(kw);
    if (i < num_pairs) {
      PairPlan pp;
      pp.chunk_begin = carry_k + sk - k;
      pp.ws_begin = kw ? carry_w + sw - kw : -1;
      pp.k = k;
      pp.n_local = nl;
      p.pairs[i] = pp;
      if (staged) s_wsb[i] = pp.ws_begin;
      // a pair's chunks have at most two sizes: `extra` of base + 1 pages, then k - extra of base
      const int base_sz = nl / k, extra = nl - base_sz * k;
      if (extra) atomicAdd(&s_cnt[size_key(base_sz + 1, range, rs)], extra);
      if (k > extra) atomicAdd(&s_cnt[size_key(base_sz, range, rs)], k - extra);
    }
    carry_k += __shfl(sk, 63, 64);
    carry_w += __shfl(sw, 63, 64);
  }
  // Chunks go out longest first (a counting sort over 64 size classes), so the work items
  // the hardware dispatches last are the short ones and the tail of the grid stays short.
  // The order changes no result: a chunk's output slot is fixed by its pair and index.
  __syncthreads();
  {
    const int n_in = s_cnt[lane];
    s_cnt[lane] = wave_incl_scan(n_in) - n_in;
  }
  __syncthreads();
  for (int i = lane; i < num_pairs; i += 64) {
    PairPlan pp;
    if (staged) {  // from LDS (the entry of a pair is written by the same lane above)
      pp.n_local = s_nl[i];
      pp.k = (!fallback && pp.n_local > C) ? (pp.n_local + C - 1) / C : 1;
      pp.ws_begin = s_wsb[i];
    } else {
      pp = p.pairs[i];
    }
    const int base_sz = pp.n_local / pp.k, extra = pp.n_local - base_sz * pp.k;
    const int at_hi = extra ? atomicAdd(&s_cnt[size_key(base_sz + 1, range, rs)], extra) : 0;
    const int at_lo = pp.k > extra ? atomicAdd(&s_cnt[size_key(base_sz, range, rs)], pp.k - extra) : 0;
    for (int c = 0; c < pp.k; ++c) {
      int jb, je;
      chunk_range(pp, c, jb, je);
      p.chunks[c < extra ? at_hi + c : at_lo + (c - extra)] =
          ChunkPlan{i, jb, je, pp.ws_begin >= 0 ? pp.ws_begin + c : -1};
    }
  }
  for (int64_t c = carry_k + lane; c < p.max_chunks; c += 64) p.chunks[c] = ChunkPlan{-1, 0, 0, -1};
  if (lane == 0) {
    p.hdr->total_chunks = carry_k;
    p.hdr->ws_chunks = carry_w;
    p.hdr->fallback = fallback;
  }
}

// ---------------------------------------------------------------------------
// Even split plan (GQA kernel): page prefix sums and where each wave starts
// ---------------------------------------------------------------------------

constexpr int kEvenPlanThreads = 256;

__global__ __launch_bounds__(kEvenPlanThreads) void plan_even_kernel(AttnParams p) {
  __shared__ int64_t s_pfx[kEvenMaxPairs + 1];
  __shared__ int64_t s_wsum[kEvenPlanThreads / 64];
  __shared__ int32_t s_first[kEvenPlanThreads];
  __shared__ int32_t s_next[kEvenMaxPairs];
  const int tid = threadIdx.x;
  const int num_pairs = p.shard_count * p.batch;  // <= kEvenMaxPairs (the host checks)
  for (int i = tid; i < num_pairs; i += kEvenPlanThreads) {
    const int d = p.shard_begin + i / p.batch, b = i % p.batch;
    s_pfx[i + 1] = local_pages_of(p.seq_lens[b], p.page_size, p.n, d, p.max_local, p.tok_il);
  }
  if (tid == 0) s_pfx[0] = 0;
  __syncthreads();
  // inclusive prefix sums over s_pfx[1 .. num_pairs]: each thread a block of pairs, then a
  // scan of the block sums
  const int per = (num_pairs + kEvenPlanThreads - 1) / kEvenPlanThreads;
  const int lo = min(num_pairs, tid * per), hi = min(num_pairs, lo + per);
  int64_t sum = 0;
  int first = num_pairs;  // first pair with local pages in this thread's block
  for (int i = hi - 1; i >= lo; --i) {
    sum += s_pfx[i + 1];
    if (s_pfx[i + 1] > 0) first = i;
  }
  int64_t incl = sum;
  const int lane = tid & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t u = __shfl_up(incl, off, 64);
    if (lane >= off) incl += u;
  }
  if (lane == 63) s_wsum[tid >> 6] = incl;
  s_first[tid] = first;
  __syncthreads();
  int64_t run = incl - sum;
  for (int k = 0; k < (tid >> 6); ++k) run += s_wsum[k];
  // the next pair with pages after this block: the first later block that has one
  int after = num_pairs;
  for (int t = tid + 1; t < kEvenPlanThreads; ++t)
    if (s_first[t] < num_pairs) {
      after = s_first[t];
      break;
    }
  // pair entries (k = next pair with pages), written back to front within the block
  for (int i = hi - 1; i >= lo; --i) {
    const int nl = (int)s_pfx[i + 1];
    p.pairs[i] = PairPlan{0, -1, after, nl};
    s_next[i] = after;
    if (nl > 0) after = i;
  }
  for (int i = lo; i < hi; ++i) {
    run += s_pfx[i + 1];
    s_pfx[i + 1] = run;
  }
  __syncthreads();
  for (int i = tid; i <= num_pairs; i += kEvenPlanThreads) p.pair_pfx[i] = s_pfx[i];
  const int64_t P = s_pfx[num_pairs] * p.hkv;
  const int G = (int)min<int64_t>(p.slots, P);
  for (int w = tid; w < p.slots; w += kEvenPlanThreads) {
    WaveStart ws = {0, 0, 0, 0, 0, num_pairs, 0, 0};
    if (w < G) {
      const int64_t x0 = (int64_t)w * P / G, x1 = (int64_t)(w + 1) * P / G;
      // the pair holding item x0: the last one whose first item is <= x0 (it has pages)
      int a = 0, z = num_pairs - 1;
      while (a < z) {
        const int mid = (a + z + 1) >> 1;
        if (s_pfx[mid] * p.hkv <= x0) a = mid; else z = mid - 1;
      }
      const int64_t nl = s_pfx[a + 1] - s_pfx[a];
      const int64_t off = x0 - s_pfx[a] * p.hkv;
      ws.pair = a;
      ws.hb = (int)(off / nl);
      ws.j0 = (int)(off % nl);
      ws.count = (int)(x1 - x0);
      ws.n_local = (int)nl;
      ws.next_pair = s_next[a];
      ws.seq_len = p.seq_lens[a % p.batch];
    }
    p.wstarts[w] = ws;
  }
  if (tid == 0) {
    p.hdr->total_chunks = 0;
    p.hdr->ws_chunks = 0;
    p.hdr->fallback = 0;
    p.hdr->waves = G;
    p.hdr->total_work = P;
  }
}

// ---------------------------------------------------------------------------
// Generic VALU partial kernel
// ---------------------------------------------------------------------------

constexpr int kGenThreads = 256;
constexpr int kGenTT = 16;  // tokens per tile

template <int KIND>
struct GenCfg;
template <>
struct GenCfg<0> {  // split f32
  static constexpr int RB = 16;
};
template <>
struct GenCfg<1> {  // split bf16
  static constexpr int RB = 16;
};
template <>
struct GenCfg<2> {  // mla fp8
  static constexpr int RB = 8;
};

size_t generic_lds_bytes(int kind, int dqk, int dv) {
  const int RB = kind == 2 ? 8 : 16;
  size_t f = (size_t)RB * (dqk + 1) + (size_t)kGenTT * (dqk + 1);
  if (kind != 2) f += (size_t)kGenTT * (dv + 1);
  f += (size_t)RB * kGenTT + 3 * RB;
  return f * sizeof(float);
}

template <typename QT>
__device__ __forceinline__ float load_q(const QT* q, int64_t i);
template <>
__device__ __forceinline__ float load_q<float>(const float* q, int64_t i) {
  return q[i];
}
template <>
__device__ __forceinline__ float load_q<uint16_t>(const uint16_t* q, int64_t i) {
  return bf16_to_float(q[i]);
}

template <int KIND, typename QT>
__global__ __launch_bounds__(kGenThreads) void partial_generic_kernel(AttnParams p) {
  constexpr int RB = GenCfg<KIND>::RB;
  constexpr int TT = kGenTT;
  constexpr int KMAX = RB * 512 / kGenThreads;
  extern __shared__ float smem[];
  const int DQ = p.dqk, DV = p.dv;
  float* sQ = smem;
  float* sK = sQ + RB * (DQ + 1);
  float* sV = KIND == 2 ? sK : sK + TT * (DQ + 1);
  const int vstride = KIND == 2 ? DQ + 1 : DV + 1;
  float* sP = KIND == 2 ? sK + TT * (DQ + 1) : sV + TT * (DV + 1);
  float* sM = sP + RB * TT;
  float* sL = sM + RB;
  float* sA = sL + RB;
  const int tid = threadIdx.x;
  const QT* q = static_cast<const QT*>(p.q);
  const int total = p.hdr->total_chunks * p.hb_count;
  const int rg_rows = p.group * p.q_len;  // rows sharing one KV head

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int hb = w % p.hb_count;
    const ChunkPlan cp = load_chunk(p, w / p.hb_count);  // w < total: a planned chunk
    const int pair = cp.pair;
    const int d = p.shard_begin + pair / p.batch, b = pair % p.batch;
    const int hk = hb / p.rb_per_head;
    const int r0 = (hb % p.rb_per_head) * RB;
    const int nrows = min(RB, rg_rows - r0);
    const int T = p.seq_lens[b];
    __syncthreads();  // previous item done with shared memory
    for (int e = tid; e < RB * DQ; e += kGenThreads) {
      const int r = e / DQ, k = e - r * DQ;
      float v = 0.f;
      if (r < nrows) {
        const int rr = r0 + r, t = rr / p.group, h = hk * p.group + (rr % p.group);
        v = load_q<QT>(q, (((int64_t)b * p.q_len + t) * p.hq + h) * DQ + k);
      }
      sQ[r * (DQ + 1) + k] = v;
    }
    if (tid < RB) {
      sM[tid] = kNegInf;
      sL[tid] = 0.f;
    }
    float acc[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) acc[k] = 0.f;

    const int32_t* bt = p.block_tables + ((int64_t)d * p.batch + b) * p.max_local;
    for (int jj = cp.j_begin; jj < cp.j_end; ++jj) {
      const int32_t slot = bt[jj];
      if (slot < 0 || slot >= p.pages_per_layer) continue;
      const uint8_t* page =
          p.pools[d] + ((int64_t)p.layer * p.pages_per_layer + slot) * p.page_bytes;
      float pscale = 1.f;
      if (KIND == 2) pscale = bf16_to_float(p.scales[d][(int64_t)p.layer * p.pages_per_layer + slot]);
      for (int off = 0; off < p.page_size; off += TT) {
        const int ntok = min(TT, p.page_size - off);
        __syncthreads();  // previous tile consumed
        for (int e = tid; e < TT * DQ; e += kGenThreads) {
          const int j = e / DQ, k = e - j * DQ;
          float kv = 0.f;
          if (j < ntok && token_position(jj, off + j, p.page_size, p.n, d, p.tok_il) < T) {
            const int tok = off + j;
            if (KIND == 2) {
              kv = e4m3fn_to_float(page[(int64_t)tok * 576 + k]) * pscale;
            } else if (KIND == 1) {
              const uint16_t* kp = reinterpret_cast<const uint16_t*>(page);
              kv = bf16_to_float(kp[((int64_t)hk * p.page_size + tok) * DQ + k]);
            } else {
              const float* kp = reinterpret_cast<const float*>(page);
              kv = kp[((int64_t)hk * p.page_size + tok) * DQ + k];
            }
          }
          sK[j * (DQ + 1) + k] = kv;
        }
        if (KIND != 2) {
          for (int e = tid; e < TT * DV; e += kGenThreads) {
            const int j = e / DV, c = e - j * DV;
            float vv = 0.f;
            if (j < ntok && token_position(jj, off + j, p.page_size, p.n, d, p.tok_il) < T) {
              const int tok = off + j;
              const int64_t vi = (((int64_t)p.hkv + hk) * p.page_size + tok) * DV + c;
              if (KIND == 1)
                vv = bf16_to_float(reinterpret_cast<const uint16_t*>(page)[vi]);
              else
                vv = reinterpret_cast<const float*>(page)[vi];
            }
            sV[j * (DV + 1) + c] = vv;
          }
        }
        __syncthreads();
        // scores and online-softmax bookkeeping: thread (row r, token j)
        {
          const int r = tid / TT, j = tid % TT;
          float s = kNegInf;
          if (r < RB) {
            const int rr = r0 + r;
            const int t = rr / p.group;
            const int64_t pos = token_position(jj, off + j, p.page_size, p.n, d, p.tok_il);
            if (r < nrows && j < ntok && pos < T && pos <= (int64_t)T - p.q_len + t) {
              float dot = 0.f;
              const float* qr = sQ + r * (DQ + 1);
              const float* kr = sK + j * (DQ + 1);
              for (int k = 0; k < DQ; ++k) dot += qr[k] * kr[k];
              s = dot * p.scale;
            }
          }
          float mx = s;
#pragma unroll
          for (int o = TT / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, TT));
          float m_old = r < RB ? sM[r] : kNegInf;
          const float m_new = fmaxf(m_old, mx);
          const float pj = (s == kNegInf) ? 0.f : expf(s - m_new);
          float ps = pj;
#pragma unroll
          for (int o = TT / 2; o > 0; o >>= 1) ps += __shfl_xor(ps, o, TT);
          if (r < RB) {
            sP[r * TT + j] = pj;
            if (j == 0) {
              const float alpha = (m_old == kNegInf) ? 0.f : expf(m_old - m_new);
              sA[r] = alpha;
              sL[r] = sL[r] * alpha + ps;
              sM[r] = m_new;
            }
          }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int idx = tid + k * kGenThreads;
          if (idx < nrows * DV) {
            const int r = idx / DV, c = idx - r * DV;
            float a = acc[k] * sA[r];
            const float* pr = sP + r * TT;
            for (int j = 0; j < TT; ++j) a += pr[j] * sV[j * vstride + c];
            acc[k] = a;
          }
        }
      }
    }
    __syncthreads();
    // write the (chunk) partial
    const bool direct = cp.out < 0;
    const int64_t pair_row0 = ((int64_t)d * p.batch + b) * p.rows;
    const int64_t ws_row0 = direct ? 0 : (int64_t)cp.out * p.rows;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int idx = tid + k * kGenThreads;
      if (idx < nrows * DV) {
        const int r = idx / DV, c = idx - r * DV;
        const int rr = r0 + r, t = rr / p.group, h = hk * p.group + (rr % p.group);
        const int row = t * p.hq + h;
        const float l = sL[r];
        const float o = l > 0.f ? acc[k] / l : 0.f;
        if (direct)
          p.partial_out[(pair_row0 + row) * DV + c] = o;
        else
          p.ws_o[(ws_row0 + row) * DV + c] = o;
      }
    }
    if (tid < nrows) {
      const int rr = r0 + tid, t = rr / p.group, h = hk * p.group + (rr % p.group);
      const int row = t * p.hq + h;
      const float l = sL[tid];
      const float lse = l > 0.f ? sM[tid] + logf(l) : kNegInf;
      if (direct)
        p.partial_lse[pair_row0 + row] = lse;
      else
        p.ws_lse[ws_row0 + row] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// Chunk reduction: pairs split into k >= 2 chunks
// ---------------------------------------------------------------------------

constexpr int kRowsPerMergeBlock = 4;

__global__ __launch_bounds__(256) void chunk_reduce_kernel(AttnParams p) {
  const int pair = blockIdx.x;
  const PairPlan pp = p.pairs[pair];
  if (pp.k < 2) return;
  const int row = blockIdx.y * kRowsPerMergeBlock + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int d = p.shard_begin + pair / p.batch, b = pair % p.batch;
  const int64_t out_row = ((int64_t)d * p.batch + b) * p.rows + row;
  const int64_t ws_row = (int64_t)pp.ws_begin * p.rows + row;
  wave_merge_row(pp.k, p.ws_lse + ws_row, p.rows, p.ws_o + ws_row * p.dv, (int64_t)p.rows * p.dv,
                 p.dv, p.partial_out + out_row * p.dv, p.partial_lse + out_row);
}

// Even split: merge the parts of every segment that spans several waves (the same LSE
// algebra as the cross-shard merge, accumulated part by part), and write the rows of
// pairs without local pages (O = 0, LSE = -inf).  One workgroup per (pair, KV head):
// thread (row r, dims 8 (tid mod 16) .. + 8).
__global__ __launch_bounds__(256) void even_reduce_kernel(AttnParams p) {
  const int pair = blockIdx.x, hb = blockIdx.y;
  const int tid = threadIdx.x, r = tid >> 4, c8 = (tid & 15) * 8;
  const int rows = p.group * p.q_len;
  if (r >= rows || c8 >= p.dv) return;
  const int d = p.shard_begin + pair / p.batch, b = pair % p.batch;
  const int t = r / p.group, h = hb * p.group + r % p.group;
  const int64_t out_row = ((int64_t)d * p.batch + b) * p.rows + (int64_t)t * p.hq + h;
  float* out = p.partial_out + out_row * p.dv + c8;
  const int nl = p.pairs[pair].n_local;
  if (nl == 0) {
    *reinterpret_cast<float4*>(out) = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(out + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    if ((tid & 15) == 0) p.partial_lse[out_row] = kNegInf;
    return;
  }
  const int64_t P = p.hdr->total_work;
  const int G = p.hdr->waves;
  const int64_t X = p.pair_pfx[pair] * p.hkv + (int64_t)hb * nl;
  const int w0 = even_wave_of(X, P, G), w1 = even_wave_of(X + nl - 1, P, G);
  if (w0 == w1) return;  // one wave held the whole segment and wrote it
  // wave w0's part is its first segment's (slot 2 w0) when its range starts here, else its
  // last one's (2 w0 + 1); the waves after it start inside the segment (slot 2 w)
  const int64_t first_slot = ((int64_t)w0 * P / G == X) ? 2 * (int64_t)w0 : 2 * (int64_t)w0 + 1;
  const int K = w1 - w0 + 1;
  float m = kNegInf, sum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < K; i0 += 4) {
    float lv[4];
    float4 xa[4], xb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // all loads of four parts at once
      const int i = min(i0 + u, K - 1);
      const int64_t row = (i == 0 ? first_slot : 2 * ((int64_t)w0 + i)) * kEvenRows + r;
      lv[u] = p.ws_lse[row];
      xa[u] = *reinterpret_cast<const float4*>(p.ws_o + row * p.dv + c8);
      xb[u] = *reinterpret_cast<const float4*>(p.ws_o + row * p.dv + c8 + 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (i0 + u >= K || lv[u] == kNegInf) continue;  // an empty part's O may hold anything
      if (lv[u] > m) {
        const float sc = m == kNegInf ? 0.f : expf(m - lv[u]);
        sum *= sc;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] *= sc;
        m = lv[u];
      }
      const float wgt = expf(lv[u] - m);
      sum += wgt;
      acc[0] += wgt * xa[u].x;
      acc[1] += wgt * xa[u].y;
      acc[2] += wgt * xa[u].z;
      acc[3] += wgt * xa[u].w;
      acc[4] += wgt * xb[u].x;
      acc[5] += wgt * xb[u].y;
      acc[6] += wgt * xb[u].z;
      acc[7] += wgt * xb[u].w;
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  *reinterpret_cast<float4*>(out) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if ((tid & 15) == 0) p.partial_lse[out_row] = sum > 0.f ? m + logf(sum) : kNegInf;
}

// ---------------------------------------------------------------------------
// Cross-shard merge (dcp_lse_merge)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void lse_merge_kernel(int n, int64_t rows, int dv,
                                                         const float* __restrict__ po,
                                                         const float* __restrict__ pl,
                                                         float* __restrict__ out,
                                                         float* __restrict__ out_lse) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerMergeBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  wave_merge_row(n, pl + row, rows, po + row * dv, rows * dv, dv, out + row * dv,
                 out_lse ? out_lse + row : nullptr);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

static int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (!cache[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// DCPKV_MLA_SCORES selects the fp8 MLA kernel's score path: "auto" (default: exact fp16 scores
// for the rows whose query has outliers, fp8 for the rest), "fp8" or "exact" for every row.
static int mla_score_mode() {
  const char* e = std::getenv("DCPKV_MLA_SCORES");
  if (!e || !e[0] || !std::strcmp(e, "auto")) return 0;
  return !std::strcmp(e, "fp8") ? 1 : (!std::strcmp(e, "exact") ? 2 : 0);
}

// DCPKV_GQA_SPLIT=chunks gives the GQA kernel the chunk plan (the one it takes beyond
// kEvenMaxPairs pairs) at any batch; the default is the even split.
static bool gqa_force_chunks() {
  const char* e = std::getenv("DCPKV_GQA_SPLIT");
  return e && !std::strcmp(e, "chunks");
}

static int validate(const dcp_attn_desc& D) {
  const bool split = D.kv_layout == DCPKV_LAYOUT_SPLIT, mla = D.kv_layout == DCPKV_LAYOUT_MLA;
  if (!split && !mla) return set_error(DCPKV_EINVAL, "attn: unknown kv_layout %d", D.kv_layout);
  if (split && D.kv_dtype != DCPKV_KV_F32 && D.kv_dtype != DCPKV_KV_BF16)
    return set_error(DCPKV_EINVAL, "attn: split layout needs f32 or bf16 KV");
  if (mla && D.kv_dtype != DCPKV_KV_FP8E4M3)
    return set_error(DCPKV_EINVAL, "attn: MLA layout needs fp8 e4m3 KV");
  if (D.q_dtype != DCPKV_Q_F32 && D.q_dtype != DCPKV_Q_BF16)
    return set_error(DCPKV_EINVAL, "attn: unknown q_dtype %d", D.q_dtype);
  if (D.num_q_heads < 1 || D.num_kv_heads < 1 || D.num_q_heads % D.num_kv_heads)
    return set_error(DCPKV_EINVAL, "attn: Hq=%d must be a positive multiple of Hkv=%d",
                     D.num_q_heads, D.num_kv_heads);
  if (split && (D.head_dim_qk != D.head_dim_v || D.head_dim_qk < 1 || D.head_dim_qk > 256))
    return set_error(DCPKV_EINVAL, "attn: split layout needs head_dim_qk == head_dim_v in [1, 256]");
  if (mla && (D.head_dim_qk != 576 || D.head_dim_v != 512 || D.num_kv_heads != 1))
    return set_error(DCPKV_EINVAL, "attn: MLA layout needs Dqk=576, Dv=512, one KV head");
  if (D.page_size < 1 || D.dcp_size < 1 || D.dcp_size > kMaxShards || D.batch < 1 ||
      D.q_len < 1 || D.max_local_pages < 1 || D.layer < 0 || D.layer >= D.num_layers ||
      D.pages_per_layer < 1)
    return set_error(DCPKV_EINVAL, "attn: bad geometry");
  if (!(D.softmax_scale > 0.f) || !std::isfinite(D.softmax_scale))
    return set_error(DCPKV_EINVAL, "attn: softmax_scale %g must be positive and finite", (double)D.softmax_scale);
  if (D.token_interleave != DCPKV_OWN_PAGE && D.token_interleave != DCPKV_OWN_TOKEN)
    return set_error(DCPKV_EINVAL, "attn: token_interleave must be %d or %d", DCPKV_OWN_PAGE, DCPKV_OWN_TOKEN);
  // the chunk reduction's grid is (pairs, row blocks): at most 65535 row blocks
  if ((int64_t)D.q_len * D.num_q_heads > 65535LL * kRowsPerMergeBlock || (int64_t)D.batch * D.dcp_size > (1 << 24))
    return set_error(DCPKV_EINVAL, "attn: q_len * Hq = %lld rows (limit %d) or B * N = %lld (limit %d) too large",
                     (long long)D.q_len * D.num_q_heads, 65535 * kRowsPerMergeBlock,
                     (long long)D.batch * D.dcp_size, 1 << 24);
  return DCPKV_OK;
}

static int64_t page_bytes_of(const dcp_attn_desc& D) {
  if (D.kv_layout == DCPKV_LAYOUT_MLA) return (int64_t)D.page_size * 576;
  const int64_t elem = D.kv_dtype == DCPKV_KV_F32 ? 4 : 2;
  return 2 * (int64_t)D.num_kv_heads * D.page_size * D.head_dim_qk * elem;
}

struct Geometry {
  int kind;          // KernelKind
  int rb_rows, rb_per_head, hb_count, rows, chunk_pages;
  bool even;         // even split plan (GQA kernel) instead of chunks
  int slots;         // even split: waves launched
  int64_t ws_cap;
  size_t hdr_off, pairs_off, chunks_off, pfx_off, wst_off, o_off, lse_off, bytes;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static void plan_geometry(const dcp_attn_desc& D, int64_t total_tokens, int cus, Geometry& g) {
  g = Geometry{};
  g.kind = choose_kernel(D);
  g.rb_rows = kernel_rows_per_block(g.kind, D);
  const int rg_rows = (D.num_q_heads / D.num_kv_heads) * D.q_len;
  g.rb_per_head = (rg_rows + g.rb_rows - 1) / g.rb_rows;
  g.hb_count = D.num_kv_heads * g.rb_per_head;
  g.rows = D.q_len * D.num_q_heads;
  const int64_t tot = std::max<int64_t>(total_tokens, 0);
  // >= the local pages over all shards: sum of ceil(T_b / page) (page ownership), at most
  // T_b / page + N per request (token ownership: every shard may end on a partial page)
  const int64_t est_pages = tot / D.page_size + (int64_t)D.batch * (D.token_interleave ? D.dcp_size : 1);
  const int64_t target_items = (int64_t)cus * kernel_items_per_cu(g.kind);
  int64_t c = (est_pages * g.hb_count + target_items - 1) / std::max<int64_t>(target_items, 1);
  c = std::max<int64_t>(c, kernel_min_chunk_pages(g.kind, D));
  c = std::min<int64_t>(c, 1 << 20);
  g.chunk_pages = (int)c;
  // pairs with k >= 2 chunks hold at most 2 * (their local pages) / C chunks
  g.ws_cap = 2 * est_pages / c + 1;
  const int64_t pairs = (int64_t)D.dcp_size * D.batch;
  g.hdr_off = 0;
  g.pairs_off = align256(sizeof(PlanHeader));
  g.chunks_off = align256(g.pairs_off + (size_t)pairs * sizeof(PairPlan));
  // chunk plans: as many as the grid of any shard range covers (pairs + local pages / C + 1)
  g.o_off = align256(g.chunks_off + (size_t)(pairs + est_pages / c + 1) * sizeof(ChunkPlan));
  g.lse_off = align256(g.o_off + (size_t)g.ws_cap * g.rows * D.head_dim_v * sizeof(float));
  g.bytes = align256(g.lse_off + (size_t)g.ws_cap * g.rows * sizeof(float));
  // The GQA kernel splits evenly when the plan's pairs fit the planner's LDS and the
  // page-items of one wave fit 32 bits: pair prefix sums, one start per wave and two
  // part slots of kEvenRows rows per wave.
  g.slots = (int)std::min<int64_t>((int64_t)cus * kernel_resident_per_cu(g.kind), 1 << 20);
  if (g.kind == KK_GQA_BF16 && pairs <= kEvenMaxPairs && est_pages * D.num_kv_heads < (1LL << 31) &&
      !gqa_force_chunks()) {
    g.even = true;
    g.pfx_off = align256(g.pairs_off + (size_t)pairs * sizeof(PairPlan));
    g.wst_off = align256(g.pfx_off + (size_t)(pairs + 1) * sizeof(int64_t));
    g.o_off = align256(g.wst_off + (size_t)g.slots * sizeof(WaveStart));
    g.ws_cap = 2 * (int64_t)g.slots;
    g.lse_off = align256(g.o_off + (size_t)g.ws_cap * kEvenRows * D.head_dim_v * sizeof(float));
    g.bytes = align256(g.lse_off + (size_t)g.ws_cap * kEvenRows * sizeof(float));
  }
}

// Fit the geometry into `cap` bytes by holding fewer chunk partials (a coarser split: the
// planner keeps one chunk per pair when the split it wants does not fit).  False when even the
// plan without chunk partials does not fit.
static bool cap_geometry(const dcp_attn_desc& D, size_t cap, Geometry& g) {
  if (g.bytes <= cap) return true;
  if (g.even) return false;  // its size is fixed by the device (two part slots per wave)
  if (g.o_off + 512 > cap) return false;
  const size_t per_slot = (size_t)g.rows * (D.head_dim_v + 1) * sizeof(float);
  const int64_t fit = (int64_t)((cap - g.o_off - 512) / per_slot);
  g.ws_cap = std::min<int64_t>(g.ws_cap, fit);
  g.lse_off = align256(g.o_off + (size_t)g.ws_cap * g.rows * D.head_dim_v * sizeof(float));
  g.bytes = align256(g.lse_off + (size_t)g.ws_cap * g.rows * sizeof(float));
  return g.bytes <= cap;
}

// Scratch of dcp_decode_partial_noalloc: one array per device, held until the process ends.
// Host code uses only the device address hipGetSymbolAddress returns for it.
static __device__ __attribute__((aligned(256))) uint8_t scratch[DCPKV_NOALLOC_SCRATCH_BYTES];

static int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return set_error(DCPKV_EDEVICE, "attn: no current device");
  if (dev < 0 || dev >= 64) return set_error(DCPKV_EDEVICE, "attn: device %d beyond the 64 this build tracks", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return set_error(DCPKV_EDEVICE, "attn: scratch address on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return DCPKV_OK;
}

}  // namespace dcpkv

using namespace dcpkv;

extern "C" size_t dcp_decode_partial_workspace(const dcp_attn_desc* desc, int64_t total_tokens) {
  if (!desc || validate(*desc) != DCPKV_OK) return 0;
  Geometry g;
  plan_geometry(*desc, total_tokens, device_cus(), g);
  return g.bytes;
}

// Both entry points: with fit_scratch the workspace is the no-alloc scratch and the split is
// made as coarse as it must be to fit.
static int decode_partial(const dcp_attn_desc* desc, const void* q, const void* const* kv_pools,
                          const void* const* kv_scales, const int32_t* block_tables, const int32_t* seq_lens,
                          int64_t total_tokens, int32_t shard_begin, int32_t shard_count, float* partial_out,
                          float* partial_lse, void* workspace, size_t workspace_bytes, bool fit_scratch,
                          void* stream) {
  if (!desc) return set_error(DCPKV_EINVAL, "attn: NULL descriptor");
  const dcp_attn_desc& D = *desc;
  int rc = validate(D);
  if (rc) return rc;
  if (shard_begin < 0 || shard_count < 1 || shard_begin + shard_count > D.dcp_size)
    return set_error(DCPKV_EINVAL, "attn: shard range [%d, %d) outside [0, %d)", shard_begin,
                     shard_begin + shard_count, D.dcp_size);
  if (!q || !kv_pools || !block_tables || !seq_lens || !partial_out || !partial_lse || !workspace)
    return set_error(DCPKV_EINVAL, "attn: NULL pointer argument");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return set_error(DCPKV_EINVAL, "attn: workspace must be 256-byte aligned");
  if (!aligned16(q) || !aligned16(partial_out) || (reinterpret_cast<uintptr_t>(partial_lse) & 3u))
    return set_error(DCPKV_EINVAL, "attn: q and partial_out must be 16-byte aligned, partial_lse 4-byte aligned");
  if (D.kv_layout == DCPKV_LAYOUT_MLA && !kv_scales)
    return set_error(DCPKV_EINVAL, "attn: MLA fp8 needs per-page scales");
  Geometry g;
  plan_geometry(D, total_tokens, device_cus(), g);
  if (fit_scratch && !cap_geometry(D, workspace_bytes, g))
    return set_error(DCPKV_EINVAL,
                     "attn (no-alloc): the plan of %lld (shard, request) pairs needs %zu bytes, more than the "
                     "%zu-byte scratch", (long long)D.dcp_size * D.batch, g.o_off + 512, workspace_bytes);
  if (workspace_bytes < g.bytes)
    return set_error(DCPKV_EINVAL, "attn: workspace %zu bytes < %zu needed", workspace_bytes,
                     g.bytes);
  AttnParams p = {};
  p.q = q;
  for (int d = shard_begin; d < shard_begin + shard_count; ++d) {
    if (!kv_pools[d] || !aligned16(kv_pools[d]))
      return set_error(DCPKV_EINVAL, "attn: pool %d is NULL or not 16-byte aligned", d);
    p.pools[d] = static_cast<const uint8_t*>(kv_pools[d]);
    if (D.kv_layout == DCPKV_LAYOUT_MLA) {
      if (!kv_scales[d] || (reinterpret_cast<uintptr_t>(kv_scales[d]) & 3u))
        return set_error(DCPKV_EINVAL, "attn: scale array %d is NULL or not 4-byte aligned", d);
      p.scales[d] = static_cast<const uint16_t*>(kv_scales[d]);
    }
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.partial_out = partial_out;
  p.partial_lse = partial_lse;
  p.hdr = reinterpret_cast<PlanHeader*>(ws + g.hdr_off);
  p.pairs = reinterpret_cast<PairPlan*>(ws + g.pairs_off);
  p.chunks = reinterpret_cast<ChunkPlan*>(ws + g.chunks_off);
  p.pair_pfx = g.even ? reinterpret_cast<int64_t*>(ws + g.pfx_off) : nullptr;
  p.wstarts = g.even ? reinterpret_cast<WaveStart*>(ws + g.wst_off) : nullptr;
  // even split: up to 64 x 4 pairs every wave plans its own range (no planner launch)
  p.even = g.even ? ((int64_t)shard_count * D.batch <= 256 ? 2 : 1) : 0;
  p.ws_o = reinterpret_cast<float*>(ws + g.o_off);
  p.ws_lse = reinterpret_cast<float*>(ws + g.lse_off);
  p.ws_cap = g.ws_cap;
  p.pages_per_layer = D.pages_per_layer;
  p.page_bytes = page_bytes_of(D);
  p.kv_dtype = D.kv_dtype;
  p.layout = D.kv_layout;
  p.q_dtype = D.q_dtype;
  p.hq = D.num_q_heads;
  p.hkv = D.num_kv_heads;
  p.dqk = D.head_dim_qk;
  p.dv = D.head_dim_v;
  p.page_size = D.page_size;
  p.n = D.dcp_size;
  p.batch = D.batch;
  p.q_len = D.q_len;
  p.max_local = D.max_local_pages;
  p.layer = D.layer;
  p.shard_begin = shard_begin;
  p.shard_count = shard_count;
  p.chunk_pages = g.chunk_pages;
  p.slots = g.even ? g.slots
                   : (int32_t)std::min<int64_t>((int64_t)device_cus() * kernel_resident_per_cu(g.kind), INT32_MAX);
  p.group = D.num_q_heads / D.num_kv_heads;
  p.rows = g.rows;
  p.hb_count = g.hb_count;
  p.rb_rows = g.rb_rows;
  p.rb_per_head = g.rb_per_head;
  p.scale = D.softmax_scale;
  p.tok_il = D.token_interleave;
  p.mla_scores = mla_score_mode();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int cus = device_cus();

  // items: at most (pairs + local pages / C) chunks per head block; the grid covers
  // max_chunks chunks and the planner never produces more (it falls back to one
  // chunk per pair, which pairs <= max_chunks always allows)
  const int64_t pairs = (int64_t)shard_count * D.batch;
  const int64_t est_pages = std::max<int64_t>(total_tokens, 0) / D.page_size +
                            (int64_t)D.batch * (D.token_interleave ? D.dcp_size : 1);
  p.max_chunks = pairs + est_pages / g.chunk_pages + 1;
  const int64_t item_bound = p.max_chunks * g.hb_count;
  if (p.even == 1)
    hipLaunchKernelGGL(plan_even_kernel, dim3(1), dim3(kEvenPlanThreads), 0, st, p);
  else if (!p.even)
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "attn: plan launch: %s", hipGetErrorString(e));
  rc = launch_partial(g.kind, p, D, cus, item_bound, st);
  if (rc) return rc;

  if (g.even)
    hipLaunchKernelGGL(even_reduce_kernel, dim3((unsigned)pairs, (unsigned)D.num_kv_heads), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(chunk_reduce_kernel,
                       dim3((unsigned)pairs, (unsigned)((g.rows + kRowsPerMergeBlock - 1) / kRowsPerMergeBlock)),
                       dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "attn: reduce launch: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

extern "C" int dcp_decode_partial(const dcp_attn_desc* desc, const void* q,
                                  const void* const* kv_pools, const void* const* kv_scales,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  int64_t total_tokens, int32_t shard_begin, int32_t shard_count,
                                  float* partial_out, float* partial_lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_partial(desc, q, kv_pools, kv_scales, block_tables, seq_lens, total_tokens, shard_begin,
                        shard_count, partial_out, partial_lse, workspace, workspace_bytes, false, stream);
}

extern "C" int dcp_decode_partial_noalloc(const dcp_attn_desc* desc, const void* q,
                                          const void* const* kv_pools, const void* const* kv_scales,
                                          const int32_t* block_tables, const int32_t* seq_lens,
                                          int64_t total_tokens, int32_t shard_begin, int32_t shard_count,
                                          float* partial_out, float* partial_lse, void* stream) {
  if (!desc) return set_error(DCPKV_EINVAL, "attn: NULL descriptor");
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return decode_partial(desc, q, kv_pools, kv_scales, block_tables, seq_lens, total_tokens, shard_begin,
                        shard_count, partial_out, partial_lse, ws, DCPKV_NOALLOC_SCRATCH_BYTES, true, stream);
}

// Launch the generic kernel for this call (also the path for shapes the fast
// kernels do not take).
int dcpkv::launch_generic(const AttnParams& p, const dcp_attn_desc& D, int cus, int64_t item_bound,
                          hipStream_t st) {
  const int kind = D.kv_layout == DCPKV_LAYOUT_MLA ? 2 : (D.kv_dtype == DCPKV_KV_BF16 ? 1 : 0);
  const size_t lds = generic_lds_bytes(kind, D.head_dim_qk, D.head_dim_v);
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(item_bound, (int64_t)cus * 2));
  const bool qbf = D.q_dtype == DCPKV_Q_BF16;
#define DCPKV_GEN(K, QT)                                                                        \
  hipLaunchKernelGGL((partial_generic_kernel<K, QT>), dim3((unsigned)grid), dim3(kGenThreads), \
                     lds, st, p)
  if (kind == 0) {
    if (qbf) DCPKV_GEN(0, uint16_t); else DCPKV_GEN(0, float);
  } else if (kind == 1) {
    if (qbf) DCPKV_GEN(1, uint16_t); else DCPKV_GEN(1, float);
  } else {
    if (qbf) DCPKV_GEN(2, uint16_t); else DCPKV_GEN(2, float);
  }
#undef DCPKV_GEN
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(DCPKV_EDEVICE, "attn: generic launch: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

extern "C" int dcp_lse_merge(int32_t dcp_size, int64_t rows, int32_t head_dim_v,
                             const float* partial_out, const float* partial_lse, float* out,
                             float* out_lse, void* stream) {
  if (dcp_size < 1 || rows < 0 || head_dim_v < 1 || (rows > 0 && (!partial_out || !partial_lse || !out)))
    return set_error(DCPKV_EINVAL, "merge: bad arguments (N=%d rows=%lld Dv=%d)", dcp_size,
                     (long long)rows, head_dim_v);
  if (rows == 0) return DCPKV_OK;
  if (!aligned16(partial_out) || !aligned16(out) || (reinterpret_cast<uintptr_t>(partial_lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(out_lse) & 3u))
    return set_error(DCPKV_EINVAL, "merge: partial_out and out must be 16-byte aligned, the LSE arrays 4-byte aligned");
  const int64_t blocks = (rows + kRowsPerMergeBlock - 1) / kRowsPerMergeBlock;
  if (blocks > INT32_MAX / 256) return set_error(DCPKV_EINVAL, "merge: too many rows");
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), dcp_size, rows, head_dim_v, partial_out,
                     partial_lse, out, out_lse);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "merge: launch failed: %s", hipGetErrorString(e));
  return DCPKV_OK;
}
