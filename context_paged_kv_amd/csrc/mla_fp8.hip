// Partial decode attention for fp8 MLA latent pages (576 = 512 latent + 64
// rope bytes per token, one bf16 scale per page, 64-token pages) on gfx950.
//
// [2DR] = "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding"
//         (section 5.3: the 576-byte fp8 latent; section 5.2: per-rank
//         partial attention; section 8: verify with several draft tokens);
// [SGL] = "SGLang's path" (serving-k3, module 05): partial = weighted sum +
//         log-sum-exp.
//
// Absorbed MLA: every query head has a 576-d query; K is the whole latent and
// V its first 512 entries, shared by all heads.  With 128 heads the work is
// about 480 flop per KV byte, so this kernel is bound by the matrix cores,
// not by HBM.
//
// Work item: (shard d, request b, chunk of local pages, block of 64 query
// rows); a workgroup of four wavefronts owns one item, each wavefront 16 rows
// (the N = 16 columns of its MFMAs).  Per page:
//   * the 36 KB of codes are fetched one page ahead with coalesced
//     non-temporal 16-byte loads (36 VGPRs per thread);
//   * the workgroup converts them once, exactly, to an fp16 tile
//     [64 tokens][576] in LDS (v_cvt_scalef32_pk_f16_fp8, two codes per
//     instruction; tokens past the sequence end are written as zeros);
//   * S^T = K Q^T on v_mfma_f32_16x16x32_f16: A = 16 token rows of the tile,
//     B = the wavefront's queries (fp16) held in registers;
//   * online softmax in base 2, scores scaled by softmax_scale x page scale;
//   * O^T += V^T P^T on the same MFMA: the V^T operand is read straight from
//     the row-major tile with ds_read_b64_tr_b16 (each lane receives four
//     tokens of one latent dim); the token order of the k slots is chosen so
//     that P^T is lane-local after the S^T MFMA.  The page scale of V is
//     folded into the running rescale of the accumulator.
// The tile row stride (1168 bytes) keeps both the 16-row K reads and the
// transposing V reads free of LDS bank conflicts.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "attn_common.h"
#include "attn_kernels.h"

namespace dcpkv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMlaPage = 64;
constexpr int kMlaDim = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaRowsPerBlock = 64;
constexpr int kTileStride = 2 * kMlaDim + 16;  // bytes per fp16 tile row
constexpr int kPageChunks = kMlaPage * kMlaDim / 16;  // 2304 16-byte chunks per page
constexpr int kChunksPerThread = kPageChunks / 256;   // 9
constexpr float kLog2eM = 1.4426950408889634f;
constexpr float kLn2M = 0.6931471805599453f;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ float mgrp4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float mgrp4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

__global__ __launch_bounds__(256) void mla_fp8_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[kMlaPage * kTileStride];  // 74752 B
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  // items sharing a chunk run on the same XCD (dispatch is round robin over 8)
  const int hbc = p.hb_count;
  const int blk = blockIdx.x;
  const int gc = (blk / (8 * hbc)) * 8 + (blk & 7);
  const int hb = (blk >> 3) % hbc;
  if (gc >= p.hdr->total_chunks) return;
  int pair = 0;
  {
    int lo = 0, hi = p.shard_count * p.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.pairs[mid].chunk_begin <= gc)
        lo = mid;
      else
        hi = mid - 1;
    }
    pair = lo;
  }
  const PairPlan pp = p.pairs[pair];
  const int chunk = gc - pp.chunk_begin;
  const int d = p.shard_begin + pair / p.batch, b = pair % p.batch;
  const int T = p.seq_lens[b];
  const int row = hb * kMlaRowsPerBlock + wave * 16 + c;  // this lane's query row within the pair
  const bool row_ok = row < p.rows;
  const int t_q = row_ok ? row / p.hq : 0, h_q = row_ok ? row % p.hq : 0;
  const int64_t lim = row_ok ? (int64_t)T - p.q_len + t_q : -1;  // last visible position
  const float sl2 = p.scale * kLog2eM;

  // Q^T as B operand: lane (g, c) holds row c of the wave, dims 32*kk + 8*g + [0, 8), fp16
  f16x8 qb[18];
  {
    const uint16_t* qbf = static_cast<const uint16_t*>(p.q);
    const uint16_t* qr = qbf + (((int64_t)b * p.q_len + t_q) * p.hq + h_q) * kMlaDim;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      u32x4 w = row_ok ? *reinterpret_cast<const u32x4*>(qr + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        qb[kk][2 * e2] = (_Float16)__builtin_bit_cast(float, w[e2] << 16);
        qb[kk][2 * e2 + 1] = (_Float16)__builtin_bit_cast(float, w[e2] & 0xFFFF0000u);
      }
    }
  }

  float m = kNegInf, l = 0.f, ps_prev = 1.f;
  f32x4 o[32];  // O^T tiles (in units of the current page scale): dims 16*mt + 4*g + i of row c
#pragma unroll
  for (int mt = 0; mt < 32; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int j_begin = chunk * p.chunk_pages;
  const int j_end = min(pp.n_local, j_begin + p.chunk_pages);
  const int32_t* bt = p.block_tables + ((int64_t)d * p.batch + b) * p.max_local;
  const uint8_t* pool = p.pools[d] + (int64_t)p.layer * p.pages_per_layer * p.page_bytes;
  const uint16_t* scl = p.scales[d] + (int64_t)p.layer * p.pages_per_layer;

  u32x4 raw[kChunksPerThread];
  int jj = j_begin;
  int32_t slot = -1;
  for (; jj < j_end; ++jj) {
    slot = bt[jj];
    if (slot >= 0 && slot < p.pages_per_layer) break;
  }
  float pscale = 1.f;
  if (jj < j_end) {
    const u32x4* src = reinterpret_cast<const u32x4*>(pool + (int64_t)slot * p.page_bytes);
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) raw[i] = __builtin_nontemporal_load(src + tid + 256 * i);
    pscale = bf16_to_float(scl[slot]);
  }

  while (jj < j_end) {
    const int64_t pos0 = ((int64_t)jj * p.n + d) * kMlaPage;
    const int64_t rem = (int64_t)T - pos0;
    const int valid = rem < kMlaPage ? (int)rem : kMlaPage;
    const float ps = fmaxf(pscale, 1e-30f);
    __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int q = tid + 256 * i;
      const int r = q / 36, cc = q - r * 36;
      u32x4 h0, h1;
      if (r < valid) {
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          h0[2 * e2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i][e2], 1.0f, false));
          h0[2 * e2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i][e2], 1.0f, true));
          h1[2 * e2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i][2 + e2], 1.0f, false));
          h1[2 * e2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i][2 + e2], 1.0f, true));
        }
      } else {
        h0 = u32x4{0, 0, 0, 0};
        h1 = u32x4{0, 0, 0, 0};
      }
      u32x4* dst = reinterpret_cast<u32x4*>(&s_tile[r * kTileStride + 32 * cc]);
      dst[0] = h0;
      dst[1] = h1;
    }
    __syncthreads();
    // next page in flight while this one is computed
    int jn = jj + 1;
    for (; jn < j_end; ++jn) {
      slot = bt[jn];
      if (slot >= 0 && slot < p.pages_per_layer) break;
    }
    if (jn < j_end) {
      const u32x4* src = reinterpret_cast<const u32x4*>(pool + (int64_t)slot * p.page_bytes);
#pragma unroll
      for (int i = 0; i < kChunksPerThread; ++i) raw[i] = __builtin_nontemporal_load(src + tid + 256 * i);
      pscale = bf16_to_float(scl[slot]);
    }

    // ---- S^T = K Q^T: tile tt covers tokens 16*tt + m; lane gets tokens 16*tt + 4*g + i of row c
    f32x4 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = &s_tile[(16 * tt + c) * kTileStride + 16 * g];
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        const f16x8 a = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(krow + 64 * kk));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[kk], acc, 0, 0, 0);
      }
      s[tt] = acc;
    }
    // ---- online softmax
    const float f = sl2 * ps;
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t pos = pos0 + 16 * tt + 4 * g + i;
        const float v = pos <= lim ? s[tt][i] * f : kNegInf;
        s[tt][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = mgrp4_max(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = (m == kNegInf) ? 0.f : exp2f(m - mn);
    m = mn;
    float psum = 0.f;
    f16x8 pb[2];  // P^T operands: k-step ks holds tokens 32ks + 4g + [0,4) and 32ks + 16 + 4g + [0,4)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = (s[tt][i] == kNegInf) ? 0.f : exp2f(s[tt][i] - mn);
        psum += x;
        pb[tt >> 1][4 * (tt & 1) + i] = (_Float16)x;
      }
    l = l * alpha + mgrp4_sum(psum);
    // ---- O^T = (alpha * ps_prev / ps) O^T + V^T P^T   (accumulator in units of this page's scale)
    const float resc = alpha * (ps_prev / ps);
    ps_prev = ps;
    // V^T via transposing reads: source lane 4k + q of group g points at token
    // (32ks + 16*half + 4g + k), dims 16*mt + 4q .. +3
    const int kq = c >> 2, qq = c & 3;
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      f32x4 acc = o[mt] * resc;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int tok0 = 32 * ks + 4 * g + kq;
        const uint8_t* a0 = &s_tile[tok0 * kTileStride + 2 * (16 * mt + 4 * qq)];
        const uint8_t* a1 = a0 + 16 * kTileStride;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a1));
        // whole-vector casts: an element-by-element rebuild of these results was
        // miscompiled (every element became element 0)
        const f16x8 av = __builtin_shufflevector(__builtin_bit_cast(f16x4, v0), __builtin_bit_cast(f16x4, v1),
                                                 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pb[ks], acc, 0, 0, 0);
      }
      o[mt] = acc;
    }
    jj = jn;
  }

  // ---- write the (chunk) partial of row c: O = ps_last * O^T / l
  if (row_ok) {
    const bool direct = pp.k == 1;
    const int64_t orow = (int64_t)t_q * p.hq + h_q;
    const int64_t pair_row0 = ((int64_t)d * p.batch + b) * p.rows;
    const int64_t ws_row0 = direct ? 0 : ((int64_t)pp.ws_begin + chunk) * p.rows;
    float* dst = direct ? p.partial_out + (pair_row0 + orow) * kMlaDv : p.ws_o + (ws_row0 + orow) * kMlaDv;
    const float inv = l > 0.f ? ps_prev / l : 0.f;
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const f32x4 v = o[mt] * inv;
      *reinterpret_cast<float4*>(dst + 16 * mt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (g == 0) {
      const float lse = l > 0.f ? (m + log2f(l)) * kLn2M : kNegInf;
      if (direct)
        p.partial_lse[pair_row0 + orow] = lse;
      else
        p.ws_lse[ws_row0 + orow] = lse;
    }
  }
}

bool mla_fp8_supported(const dcp_attn_desc& D) {
  return D.kv_layout == DCPKV_LAYOUT_MLA && D.kv_dtype == DCPKV_KV_FP8E4M3 && D.q_dtype == DCPKV_Q_BF16 &&
         D.head_dim_qk == kMlaDim && D.head_dim_v == kMlaDv && D.num_kv_heads == 1 && D.page_size == kMlaPage;
}

int launch_mla_fp8(const AttnParams& p, const dcp_attn_desc& D, int64_t item_bound, hipStream_t st) {
  (void)D;
  const int64_t chunks_bound = (item_bound + p.hb_count - 1) / p.hb_count;
  const int64_t blocks = ((chunks_bound + 7) / 8) * 8 * p.hb_count;
  if (blocks > INT32_MAX / 256) return set_error(DCPKV_EINVAL, "attn: too many work items");
  hipLaunchKernelGGL(mla_fp8_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "attn: mla launch: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

}  // namespace dcpkv
