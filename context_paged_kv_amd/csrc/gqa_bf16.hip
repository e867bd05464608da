// Partial decode attention for split-layout bf16 pages with head_dim 128 and
// 64-token pages (the GQA decode shape), on gfx950.
//
// [2DR] = "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding"
//         (section 5.2: each DCP rank attends over its own pages);
// [SGL] = "SGLang's path" (serving-k3, module 05): a shard's partial is its
//         weighted sum plus the log-sum-exp of its scores.
//
// One wavefront owns one work item: (shard d, request b, KV head, chunk of the
// pair's local pages).  The query rows sharing the KV head (group x q_len,
// at most 16) form the A operand of v_mfma_f32_16x16x32_bf16; K is fed from
// global memory straight into the B operand (lane l reads 64 contiguous bytes
// of token l % 16), so S = Q K^T needs no LDS.  The online softmax runs in
// base 2 inside 16-lane DPP rows (row group g = lane / 16 holds rows
// 4g..4g+3).  P goes through a 1 KB per-wave LDS slot to the PV stage, which
// runs on the VALU with fully coalesced V loads (lane l owns 8 dims of one
// token per 1 KB load); the four token groups are folded with two lane
// shuffles at the end of the chunk.  The decode path reads every K and V byte
// once and is HBM-bound: the MFMA and VALU work is a small fraction of the
// page streaming time.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "attn_common.h"
#include "attn_kernels.h"

namespace dcpkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGqaD = 128;
constexpr int kGqaPage = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 8, 16));
  v = fmaxf(v, __shfl_xor(v, 4, 16));
  v = fmaxf(v, __shfl_xor(v, 2, 16));
  v = fmaxf(v, __shfl_xor(v, 1, 16));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __shfl_xor(v, 8, 16);
  v += __shfl_xor(v, 4, 16);
  v += __shfl_xor(v, 2, 16);
  v += __shfl_xor(v, 1, 16);
  return v;
}

// NRG: row groups of 4 (rows = group * q_len <= 4 * NRG).
template <int NRG>
__global__ __launch_bounds__(256) void gqa_bf16_kernel(AttnParams p) {
  constexpr int ROWS = 4 * NRG;
  __shared__ float4 s_p[4][kGqaPage][NRG];  // per wave: P[token][row group] (4 rows each)
  __shared__ float s_alpha[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;   // 16-lane row group
  const int c = lane & 15;   // column within the row group
  const int total = p.hdr->total_chunks * p.hb_count;
  const int w = blockIdx.x * 4 + wave;
  if (w >= total) return;

  int pair, chunk, hb;
  decode_item(p, w, pair, chunk, hb);
  const PairPlan pp = p.pairs[pair];
  const int d = p.shard_begin + pair / p.batch, b = pair % p.batch;
  const int hk = hb;  // one head block per KV head (rows <= 16)
  const int rows = p.group * p.q_len;
  const int T = p.seq_lens[b];
  const float sl2 = p.scale * kLog2e;

  // Q as the A operand: lane l holds row l % 16, dims 32*g + 8*kk + [0, 8) for k-step kk.
  bf16x8 qa[4];
  {
    const int r = c;
    const uint16_t* q = static_cast<const uint16_t*>(p.q);
    if (r < rows) {
      const int t = r / p.group, h = hk * p.group + (r % p.group);
      const u32x4* qp = reinterpret_cast<const u32x4*>(q + (((int64_t)b * p.q_len + t) * p.hq + h) * kGqaD + 32 * g);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qa[kk] = __builtin_bit_cast(bf16x8, qp[kk]);
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qa[kk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }
  // query position limit of each row this lane's row group holds (rows 4g + i)
  int lim[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    lim[i] = r < rows ? T - p.q_len + r / p.group : -1;
  }

  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = kNegInf;
    l[i] = 0.f;
  }
  float o[ROWS][8];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.f;

  const int j_begin = chunk * p.chunk_pages;
  const int j_end = min(pp.n_local, j_begin + p.chunk_pages);
  const int32_t* bt = p.block_tables + ((int64_t)d * p.batch + b) * p.max_local;
  const int64_t head_bytes = (int64_t)kGqaPage * kGqaD * 2;  // one head's K (or V) of a page

  for (int jj = j_begin; jj < j_end; ++jj) {
    const int32_t slot = bt[jj];
    if (slot < 0 || slot >= p.pages_per_layer) continue;
    const uint8_t* page = p.pools[d] + ((int64_t)p.layer * p.pages_per_layer + slot) * p.page_bytes;
    const uint8_t* kb = page + (int64_t)hk * head_bytes;
    const uint8_t* vb = page + ((int64_t)p.hkv + hk) * head_bytes;
    const int64_t pos0 = ((int64_t)jj * p.n + d) * kGqaPage;
    const int64_t rem = (int64_t)T - pos0;
    const int valid = rem < kGqaPage ? (int)rem : kGqaPage;  // tokens of this page before T

    // K into B operands: tile tt, k-step kk -> token 16*tt + c, bytes 64*g + 16*kk
    u32x4 kr[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const u32x4* kp = reinterpret_cast<const u32x4*>(kb + (16 * tt + c) * (kGqaD * 2) + 64 * g);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kr[tt][kk] = __builtin_nontemporal_load(kp + kk);
    }
    // V rows: load i -> token 4*i + g, dims 8*c .. 8*c+7 (1 KB contiguous per load)
    u32x4 vr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (4 * i + g) * (kGqaD * 2) + 16 * c));

    f32x4 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(bf16x8, kr[tt][kk]), acc, 0, 0, 0);
      s[tt] = acc;
    }
    // scores (base 2), causal / length mask, page max per row
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int64_t pos = pos0 + 16 * tt + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = (pos <= lim[i]) ? s[tt][i] * sl2 : kNegInf;
        s[tt][i] = v;
        mx[i] = fmaxf(mx[i], v);
      }
    }
    float alpha[4], ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx[i] = row16_max(mx[i]);
      const float mn = fmaxf(m[i], mx[i]);
      alpha[i] = (m[i] == kNegInf) ? 0.f : exp2f(m[i] - mn);
      m[i] = mn;
      ps[i] = 0.f;
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float4 pv;
      float* pe = reinterpret_cast<float*>(&pv);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = (s[tt][i] == kNegInf) ? 0.f : exp2f(s[tt][i] - m[i]);
        pe[i] = x;
        ps[i] += x;
      }
      if (g < NRG) s_p[wave][16 * tt + c][g] = pv;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) l[i] = l[i] * alpha[i] + row16_sum(ps[i]);
    if (c == 0 && g < NRG) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_alpha[wave][4 * g + i] = alpha[i];
    }
    // the wave's own LDS writes must land before its reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float a = s_alpha[wave][r];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[r][e] *= a;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = 4 * i + g;
      u32x4 v = vr[i];
      if (tok >= valid) v = u32x4{0, 0, 0, 0};  // tail of the last page: never let garbage in
      float ve[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ve[2 * q] = bf16lo(v[q]);
        ve[2 * q + 1] = bf16hi(v[q]);
      }
#pragma unroll
      for (int rg = 0; rg < NRG; ++rg) {
        const float4 pr = s_p[wave][tok][rg];
        const float pe[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[4 * rg + i2][e] += pe[i2] * ve[e];
      }
    }
    __builtin_amdgcn_wave_barrier();  // reads of s_p / s_alpha done before the next page's writes
  }

  // fold the four token groups (lanes c, c+16, c+32, c+48 hold the same dims)
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[r][e];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      o[r][e] = x;
    }
  // per-row m, l live in row group r / 4 (lane 16 * (r / 4)); fetch them for all rows
  float mr[ROWS], lr[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    mr[r] = __shfl(m[r & 3], 16 * (r >> 2), 64);
    lr[r] = __shfl(l[r & 3], 16 * (r >> 2), 64);
  }
  const bool direct = pp.k == 1;
  const int64_t pair_row0 = ((int64_t)d * p.batch + b) * p.rows;
  const int64_t ws_row0 = direct ? 0 : ((int64_t)pp.ws_begin + chunk) * p.rows;
  if (g == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      if (r >= rows) continue;
      const int t = r / p.group, h = hk * p.group + (r % p.group);
      const int64_t row = t * p.hq + h;
      const float inv = lr[r] > 0.f ? 1.f / lr[r] : 0.f;
      float4 a = make_float4(o[r][0] * inv, o[r][1] * inv, o[r][2] * inv, o[r][3] * inv);
      float4 bq = make_float4(o[r][4] * inv, o[r][5] * inv, o[r][6] * inv, o[r][7] * inv);
      float* dst = direct ? p.partial_out + (pair_row0 + row) * kGqaD : p.ws_o + (ws_row0 + row) * kGqaD;
      reinterpret_cast<float4*>(dst + 8 * c)[0] = a;
      reinterpret_cast<float4*>(dst + 8 * c)[1] = bq;
      if (c == 0) {
        const float lse = lr[r] > 0.f ? (mr[r] + log2f(lr[r])) * kLn2 : kNegInf;
        if (direct)
          p.partial_lse[pair_row0 + row] = lse;
        else
          p.ws_lse[ws_row0 + row] = lse;
      }
    }
  }
}

bool gqa_bf16_supported(const dcp_attn_desc& D) {
  const int rows = (D.num_q_heads / D.num_kv_heads) * D.q_len;
  return D.kv_layout == DCPKV_LAYOUT_SPLIT && D.kv_dtype == DCPKV_KV_BF16 && D.q_dtype == DCPKV_Q_BF16 &&
         D.head_dim_qk == kGqaD && D.head_dim_v == kGqaD && D.page_size == kGqaPage && rows <= 16;
}

int launch_gqa_bf16(const AttnParams& p, const dcp_attn_desc& D, int64_t item_bound, hipStream_t st) {
  const int rows = (D.num_q_heads / D.num_kv_heads) * D.q_len;
  const int64_t blocks = std::max<int64_t>(1, (item_bound + 3) / 4);
  if (blocks > INT32_MAX / 256) return set_error(DCPKV_EINVAL, "attn: too many work items");
  if (rows <= 4)
    hipLaunchKernelGGL(gqa_bf16_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, p);
  else if (rows <= 8)
    hipLaunchKernelGGL(gqa_bf16_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(gqa_bf16_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "attn: gqa launch: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

}  // namespace dcpkv
