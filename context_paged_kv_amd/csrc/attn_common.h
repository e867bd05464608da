// Device-side pieces shared by the partial-attention kernels, the chunk
// reduction and the cross-shard LSE merge.
//
// [2DR] = "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding";
// [SGL] = "SGLang's path" (serving-k3, module 05).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"

namespace dcpkv {

constexpr float kNegInf = -INFINITY;

// Work decomposition of one dcp_decode_partial call.
//   pair  = (shard d, request b); its local pages are split into k chunks of
//           at most chunk_pages pages (k = 1 when it fits or for empty pairs);
//   item  = (pair, chunk, head block); a head block is a set of query rows
//           that read the same KV head.
// Pairs with k == 1 write their partial straight to partial_out; pairs with
// k >= 2 write chunk partials to the workspace and a reduction kernel merges
// them with the same LSE algebra as the cross-shard merge ([SGL]: the
// combination is exact across tiles as across ranks).
struct PairPlan {
  int32_t chunk_begin;  // exclusive prefix sum of k over pairs
  int32_t ws_begin;     // first workspace chunk slot (k >= 2), else -1
  int32_t k;            // chunks of this pair; even split: the next pair with local pages (pairs if none)
  int32_t n_local;      // local pages of this pair
};

// One chunk of the split, written by the planner so that a work item finds its pair, its
// pages and its output with a single 16-byte load.  pair < 0 past the planned chunks.
struct alignas(16) ChunkPlan {
  int32_t pair;     // pair index (shard - shard_begin) * batch + request
  int32_t j_begin;  // local pages [j_begin, j_end) of the pair
  int32_t j_end;
  int32_t out;      // -1: the partial goes straight to partial_out; else its workspace slot
};

struct PlanHeader {
  int32_t total_chunks;
  int32_t ws_chunks;
  int32_t fallback;     // 1 when the workspace could not hold the split and k = 1 was used
  int32_t waves;        // even split: waves with work (G)
  int64_t total_work;   // even split: page-items over all (pair, KV head) segments (P)
  int32_t pad[10];
};

// Even split (the GQA kernel's plan).  The work is the sequence of page-items
// (pair, KV head, local page) in that order, split into P pages of segments
// (pair, KV head) of n_local pages each.  Wave w of the grid takes items
// [floor(w P / G), floor((w + 1) P / G)), so every wave streams the same number
// of pages (to one) and no wave waits on another.  A segment inside one wave's
// range is written straight to partial_out; the parts of a segment that spans
// several waves go to workspace slots (a wave's first segment to slot 2w, its
// last to 2w + 1) and the reduction merges them.  This is where wave w starts.
struct alignas(16) WaveStart {
  int32_t pair;       // pair of the first segment
  int32_t hb;         // KV head of the first segment
  int32_t j0;         // first local page
  int32_t count;      // page-items of the wave (0: no work)
  int32_t n_local;    // local pages of the pair
  int32_t next_pair;  // the next pair with local pages (pairs if none)
  int32_t seq_len;    // the pair's request length
  int32_t pad;
};

constexpr int kEvenRows = 16;        // query rows of one segment (group x q_len <= 16)
constexpr int kEvenMaxPairs = 4096;  // pairs the even planner holds in LDS

// Wave whose range holds page-item x of the even split (G waves over P items).
__device__ __forceinline__ int even_wave_of(int64_t x, int64_t P, int G) {
  return (int)(((x + 1) * G - 1) / P);
}

struct AttnParams {
  const void* q;
  const uint8_t* pools[kMaxShards];
  const uint16_t* scales[kMaxShards];
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* partial_out;
  float* partial_lse;
  PlanHeader* hdr;
  PairPlan* pairs;
  ChunkPlan* chunks;        // [max_chunks]
  int64_t* pair_pfx;        // even split: local pages of pairs before each pair, [pairs + 1]
  WaveStart* wstarts;       // even split: [slots]
  float* ws_o;
  float* ws_lse;
  int64_t ws_cap;           // chunk partial slots in the workspace
  int64_t max_chunks;       // chunks the launched grid covers
  int64_t pages_per_layer;  // M
  int64_t page_bytes;
  int32_t kv_dtype, layout, q_dtype;
  int32_t hq, hkv, dqk, dv, page_size, n, batch, q_len, max_local, layer;
  int32_t shard_begin, shard_count;
  int32_t chunk_pages;  // C
  int32_t slots;        // workgroups of the partial kernel the device runs at once
  int32_t group;        // Hq / Hkv
  int32_t rows;         // q_len * Hq: query rows per pair
  int32_t hb_count;     // head blocks per chunk
  int32_t rb_rows;      // rows per head block
  int32_t rb_per_head;  // head blocks per KV head
  float scale;
  int32_t tok_il;       // 1: token t on shard t mod N; 0: page ownership
  int32_t mla_scores;   // fp8 MLA kernel: 0 exact scores for rows with outliers, 1 fp8 always, 2 exact always
  int32_t even;         // 0: chunk plan; even split (GQA kernel): 1 from the planner, 2 planned by every wave
};

// Tokens of (request with seq_len tokens) held by shard d, and its local pages.
// Page ownership ([2DR] section 5.1): sequence page i on shard i mod N.  Token
// ownership ([SGL]): token t on shard t mod N, local token t div N.
__device__ __forceinline__ int32_t local_pages_of(int32_t seq_len, int32_t page_size, int32_t n,
                                                  int32_t d, int32_t max_local, int32_t tok_il) {
  int32_t nl;
  if (tok_il) {
    const int32_t toks = seq_len > d ? (seq_len - 1 - d) / n + 1 : 0;
    nl = (toks + page_size - 1) / page_size;
  } else {
    const int32_t pages = (seq_len + page_size - 1) / page_size;
    nl = pages > d ? (pages - 1 - d) / n + 1 : 0;
  }
  return nl < max_local ? nl : max_local;
}

// Position of token x of shard d's local page j.
__device__ __forceinline__ int64_t token_position(int32_t j, int32_t x, int32_t page_size, int32_t n, int32_t d,
                                                  int32_t tok_il) {
  return tok_il ? ((int64_t)j * page_size + x) * n + d : ((int64_t)j * n + d) * page_size + x;
}

// Largest x whose token_position(j, x) <= pos (pos >= -1); tokens of local page j
// past it are later than pos.  Page ownership: pos - first position of the page;
// token ownership: the local index of the last position <= pos, minus j * page_size.
__device__ __forceinline__ int64_t local_limit(int64_t pos, int32_t j, int32_t page_size, int32_t n, int32_t d,
                                               int32_t tok_il) {
  if (tok_il) return (pos >= d ? (pos - d) / n : -1) - (int64_t)j * page_size;
  return pos - ((int64_t)j * n + d) * page_size;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One wavefront merges `count` partials of one row:
//   m = max_i L_i, LSE = m + log sum_i exp(L_i - m), out = sum_i exp(L_i - LSE) O_i
// ([2DR] section 5.2 for LSE; the O rule is the exact recombination of [SGL]).
// Partial i's LSE is at lse[i * lse_stride], its output at o + i * o_stride.
// Partials with LSE = -inf (no visible token) take no part, whatever their O holds.
// Up to eight partials of at most 256 dims (a multiple of four), every load is
// issued before the first use: one memory round trip.  Up to 64 partials, lane
// i holds L_i and its weight, and the O loads of four partials are in flight
// together, so a row costs two memory round trips.
__device__ inline void wave_merge_row(int count, const float* __restrict__ lse, int64_t lse_stride,
                                      const float* __restrict__ o, int64_t o_stride, int dv,
                                      float* __restrict__ out, float* __restrict__ out_lse) {
  const int lane = threadIdx.x & 63;
  if (count <= 8 && (dv & 3) == 0 && dv <= 256 && (o_stride & 3) == 0) {
    // up to eight partials of up to 256 dims: every load (clamped into range, so none is
    // predicated) goes out before the first use, one memory round trip in all
    const int c = min(lane * 4, dv - 4);
    float4 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = *reinterpret_cast<const float4*>(o + min(i, count - 1) * o_stride + c);
    const float lraw = lse[min(lane, count - 1) * lse_stride];
    const float l = lane < count ? lraw : kNegInf;
    const float m = wave_max(l);
    if (m == kNegInf) {
      if (lane * 4 < dv) *reinterpret_cast<float4*>(out + c) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (lane == 0 && out_lse) *out_lse = kNegInf;
      return;
    }
    const float tot = m + logf(wave_sum(l == kNegInf ? 0.f : expf(l - m)));
    if (lane == 0 && out_lse) *out_lse = tot;
    const float w = l == kNegInf ? 0.f : expf(l - tot);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float wi = __shfl(w, i, 64);
      if (i >= count || wi == 0.f) continue;  // an empty partial's O may hold anything
      acc.x += wi * x[i].x;
      acc.y += wi * x[i].y;
      acc.z += wi * x[i].z;
      acc.w += wi * x[i].w;
    }
    if (lane * 4 < dv) *reinterpret_cast<float4*>(out + c) = acc;
    return;
  }
  if (count <= 64) {
    const float l = lane < count ? lse[lane * lse_stride] : kNegInf;
    const float m = wave_max(l);
    if (m == kNegInf) {
      for (int c = lane; c < dv; c += 64) out[c] = 0.f;
      if (lane == 0 && out_lse) *out_lse = kNegInf;
      return;
    }
    const float tot = m + logf(wave_sum(l == kNegInf ? 0.f : expf(l - m)));
    if (lane == 0 && out_lse) *out_lse = tot;
    const float w = l == kNegInf ? 0.f : expf(l - tot);
    if ((dv & 3) == 0 && (o_stride & 3) == 0) {
      for (int c = lane * 4; c < dv; c += 256) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int i0 = 0; i0 < count; i0 += 4) {
          float4 x[4];
          float wi[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = min(i0 + u, count - 1);
            wi[u] = i0 + u < count ? __shfl(w, i, 64) : 0.f;
            x[u] = *reinterpret_cast<const float4*>(o + i * o_stride + c);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (wi[u] == 0.f) continue;  // an empty partial's O may hold anything
            acc.x += wi[u] * x[u].x;
            acc.y += wi[u] * x[u].y;
            acc.z += wi[u] * x[u].z;
            acc.w += wi[u] * x[u].w;
          }
        }
        *reinterpret_cast<float4*>(out + c) = acc;
      }
    } else {
      for (int c = lane; c < dv; c += 64) {
        float acc = 0.f;
        for (int i = 0; i < count; ++i) {
          const float wi = __shfl(w, i, 64);
          if (wi != 0.f) acc += wi * o[i * o_stride + c];
        }
        out[c] = acc;
      }
    }
    return;
  }
  float m = kNegInf;
  for (int i = lane; i < count; i += 64) m = fmaxf(m, lse[i * lse_stride]);
  m = wave_max(m);
  if (m == kNegInf) {
    for (int c = lane; c < dv; c += 64) out[c] = 0.f;
    if (lane == 0 && out_lse) *out_lse = kNegInf;
    return;
  }
  float s = 0.f;
  for (int i = lane; i < count; i += 64) {
    const float l = lse[i * lse_stride];
    s += (l == kNegInf) ? 0.f : expf(l - m);
  }
  s = wave_sum(s);
  const float tot = m + logf(s);
  if (lane == 0 && out_lse) *out_lse = tot;
  if ((dv & 3) == 0 && (o_stride & 3) == 0) {
    for (int c = lane * 4; c < dv; c += 256) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int i = 0; i < count; ++i) {
        const float l = lse[i * lse_stride];
        if (l == kNegInf) continue;
        const float w = expf(l - tot);
        const float4 x = *reinterpret_cast<const float4*>(o + i * o_stride + c);
        acc.x += w * x.x;
        acc.y += w * x.y;
        acc.z += w * x.z;
        acc.w += w * x.w;
      }
      *reinterpret_cast<float4*>(out + c) = acc;
    }
  } else {
    for (int c = lane; c < dv; c += 64) {
      float acc = 0.f;
      for (int i = 0; i < count; ++i) {
        const float l = lse[i * lse_stride];
        if (l == kNegInf) continue;
        acc += expf(l - tot) * o[i * o_stride + c];
      }
      out[c] = acc;
    }
  }
}

// Local pages [begin, end) of chunk `chunk` of a pair: its k chunks split the
// pair's pages evenly (sizes differ by at most one), so no work item is more
// than one page longer than another of the same pair.
__device__ __forceinline__ void chunk_range(const PairPlan& pp, int chunk, int& begin, int& end) {
  const int k = pp.k > 0 ? pp.k : 1;
  const int base = pp.n_local / k, extra = pp.n_local - base * k;
  begin = chunk * base + min(chunk, extra);
  end = begin + base + (chunk < extra ? 1 : 0);
}

// Plan of chunk gc (pair < 0 when the planner made fewer chunks).
__device__ __forceinline__ ChunkPlan load_chunk(const AttnParams& p, int64_t gc) {
  if (gc >= p.max_chunks) return ChunkPlan{-1, 0, 0, -1};
  return p.chunks[gc];
}

// Value of an OCP e4m3fn code (bias 7) computed exactly: the code's exponent
// and mantissa bits placed in an IEEE half (bias 15) give the value / 2^8 for
// normal and subnormal codes alike.  The NaN codes 0x7F/0xFF decode to +-480.
__device__ __forceinline__ float e4m3fn_to_float(uint32_t b) {
  const uint16_t h = (uint16_t)(((b & 0x80u) << 8) | ((b & 0x7Fu) << 7));
  return (float)__builtin_bit_cast(_Float16, h) * 256.0f;
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

}  // namespace dcpkv
