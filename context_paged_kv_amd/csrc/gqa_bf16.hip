// Partial decode attention for split-layout bf16 pages with head_dim 128 and
// 64-token pages (the GQA decode shape), on gfx950.
//
// [2DR] = "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding"
//         (section 5.2: each DCP rank attends over its own pages);
// [SGL] = "SGLang's path" (serving-k3, module 05): a shard's partial is its
//         weighted sum plus the log-sum-exp of its scores.
//
// One wavefront owns one work item: (shard d, request b, KV head, chunk of the
// pair's local pages); the query rows sharing that KV head (group x q_len,
// at most 16) are the N = 16 columns of every MFMA.
//
// Per page (one head: 16 KB of K, 16 KB of V):
//   * K and V are fetched with fully coalesced non-temporal 16-byte loads, one
//     page ahead of the compute (the next page is in flight while the current
//     one is processed).
//   * K lands in a per-wave LDS tile with an XOR swizzle on its 16-byte
//     chunks; V lands transposed (V^T[dim][token]) after a v_perm packing of
//     token pairs.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = Q).
//     The token order of the A rows is chosen so that, after the MFMA, each
//     lane holds exactly the eight scores its P^T operand needs for PV.
//   * Online softmax in base 2 (each lane owns one query row; the four lane
//     groups that share a row combine with two shuffles).
//   * O^T += V^T P^T on the same MFMA, P split as bf16 hi + lo so the only
//     rounding left is fp32 accumulation.
// Every K and V byte is read from HBM once; the MFMA, VALU and LDS work is a
// fraction of the streaming time.

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
constexpr int kGqaRow = kGqaD * 2;            // bytes per token row of K or V
constexpr int kVtStride = 2 * kGqaPage + 16;  // bytes per V^T row (padded against bank conflicts)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct GqaWaveLds {
  uint8_t k[kGqaPage * kGqaRow];  // K tile, 16-byte chunks XOR-swizzled per row
  uint8_t vt[kGqaD * kVtStride];  // V^T tile
};

// Chunk swizzle of K row r: the 16 rows one MFMA reads land on 16 distinct chunks.
__device__ __forceinline__ int kswz(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }

// Token held by MFMA row m of S^T tile tt (see the header comment).
__device__ __forceinline__ int tok_of(int tt, int m) {
  return 32 * (tt >> 1) + 8 * (m >> 2) + 4 * (tt & 1) + (m & 3);
}

__device__ __forceinline__ float grp4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float grp4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

__device__ __forceinline__ void load_page(const uint8_t* kb, const uint8_t* vb, int c, int g,
                                          u32x4 (&kr)[16], u32x4 (&vr)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i)  // K: load i covers tokens 4i .. 4i+3 (1 KB contiguous)
    kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (4 * i + g) * kGqaRow + 16 * c));
#pragma unroll
  for (int i = 0; i < 16; ++i)  // V: load i covers tokens i, 16+i, 32+i, 48+i (4 x 256 B)
    vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (16 * g + i) * kGqaRow + 16 * c));
}

// One wavefront per workgroup: four fit a CU (34 KB of LDS each), and each one's LDS is
// released as soon as it finishes, whatever the length of its neighbours' chunks.
__global__ __launch_bounds__(64) void gqa_bf16_kernel(AttnParams p) {
  __shared__ GqaWaveLds s_lds;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;  // lane group
  const int c = lane & 15;  // MFMA row/column index within the group
  const int w = blockIdx.x;
  const int hb = w % p.hb_count;
  const ChunkPlan cp = load_chunk(p, w / p.hb_count);
  if (cp.pair < 0) return;
  GqaWaveLds& L = s_lds;
  const int pair = cp.pair;
  const int d = p.shard_begin + pair / p.batch, b = pair % p.batch;
  const int hk = hb;  // one head block per KV head (rows <= 16)
  const int rows = p.group * p.q_len;
  const int T = p.seq_lens[b];
  const float sl2 = p.scale * kLog2e;

  // Q^T as the B operand of S^T: lane (g, c) holds query row c, dims 32*kk + 8*g + [0, 8).
  bf16x8 qb[4];
  {
    const uint16_t* q = static_cast<const uint16_t*>(p.q);
    if (c < rows) {
      const int t = c / p.group, h = hk * p.group + (c % p.group);
      const uint16_t* qr = q + (((int64_t)b * p.q_len + t) * p.hq + h) * kGqaD;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qb[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + 32 * kk + 8 * g));
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[kk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
  }
  const int64_t lim = c < rows ? (int64_t)T - p.q_len + c / p.group : -1;  // last visible position

  float m = kNegInf, l = 0.f;
  f32x4 o[8];  // O^T tiles: lane holds dims 16*mt + 4*g + i of row c
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int j_begin = cp.j_begin, j_end = cp.j_end;
  const int32_t* bt = p.block_tables + ((int64_t)d * p.batch + b) * p.max_local;
  const int64_t head_bytes = (int64_t)kGqaPage * kGqaRow;
  const uint8_t* pool = p.pools[d] + (int64_t)p.layer * p.pages_per_layer * p.page_bytes;

  u32x4 kr[16], vr[16];
  // first page of the chunk with a valid slot
  int jj = j_begin;
  int32_t slot = -1;
  for (; jj < j_end; ++jj) {
    slot = bt[jj];
    if (slot >= 0 && slot < p.pages_per_layer) break;
  }
  if (jj < j_end) {
    const uint8_t* page = pool + (int64_t)slot * p.page_bytes;
    load_page(page + (int64_t)hk * head_bytes, page + ((int64_t)p.hkv + hk) * head_bytes, c, g, kr, vr);
  }

  while (jj < j_end) {
    // tokens of this page before T, and the last one this lane's row sees
    const int64_t vlast = local_limit((int64_t)T - 1, jj, kGqaPage, p.n, d, p.tok_il);
    const int valid = vlast + 1 < kGqaPage ? (int)(vlast + 1) : kGqaPage;
    const int64_t thr = local_limit(lim, jj, kGqaPage, p.n, d, p.tok_il);
    // ---- stage the current page into LDS
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 4 * i + g;
      *reinterpret_cast<u32x4*>(&L.k[r * kGqaRow + 16 * (c ^ kswz(r))]) = kr[i];
    }
    if (valid < kGqaPage) {  // tail of the last page: never let bytes past T into the sums
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * g + i >= valid) vr[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x4 lo, hi;
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        lo[k2] = __builtin_amdgcn_perm(vr[2 * k2 + 1][e >> 1], vr[2 * k2][e >> 1], sel);
        hi[k2] = __builtin_amdgcn_perm(vr[2 * k2 + 9][e >> 1], vr[2 * k2 + 8][e >> 1], sel);
      }
      uint8_t* row = &L.vt[(8 * c + e) * kVtStride + 32 * g];
      reinterpret_cast<u32x4*>(row)[0] = lo;
      reinterpret_cast<u32x4*>(row)[1] = hi;
    }
    // ---- next page in flight while this one is computed
    int jn = jj + 1;
    for (; jn < j_end; ++jn) {
      slot = bt[jn];
      if (slot >= 0 && slot < p.pages_per_layer) break;
    }
    if (jn < j_end) {
      const uint8_t* page = pool + (int64_t)slot * p.page_bytes;
      load_page(page + (int64_t)hk * head_bytes, page + ((int64_t)p.hkv + hk) * head_bytes, c, g, kr, vr);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- S^T = K Q^T
    f32x4 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int r = tok_of(tt, c);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&L.k[r * kGqaRow + 16 * ((4 * kk + g) ^ kswz(r))]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qb[kk], acc, 0, 0, 0);
      }
      s[tt] = acc;
    }
    // ---- online softmax (lane: row c, tokens tok_of(tt, 4g + i))
    float mx = kNegInf;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = tok_of(tt, 4 * g + i) <= thr ? s[tt][i] * sl2 : kNegInf;
        s[tt][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = grp4_max(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = (m == kNegInf) ? 0.f : exp2f(m - mn);
    m = mn;
    float ps = 0.f;
    bf16x8 phi[2], plo[2];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = (s[tt][i] == kNegInf) ? 0.f : exp2f(s[tt][i] - mn);
        ps += x;
        const __bf16 h = (__bf16)x;
        phi[tt >> 1][4 * (tt & 1) + i] = h;
        plo[tt >> 1][4 * (tt & 1) + i] = (__bf16)(x - (float)h);
      }
    l = l * alpha + grp4_sum(ps);
    // ---- O^T = alpha O^T + V^T P^T
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      f32x4 acc = o[mt] * alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&L.vt[(16 * mt + c) * kVtStride + 2 * (32 * ks + 8 * g)]);
        const bf16x8 av = __builtin_bit_cast(bf16x8, a);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, phi[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, plo[ks], acc, 0, 0, 0);
      }
      o[mt] = acc;
    }
    // this page's LDS reads precede the next page's writes (the fences keep the compiler from
    // moving one lane's accesses across the point where another lane's begin)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    jj = jn;
  }

  // ---- write the (chunk) partial of row c
  if (c < rows) {
    const bool direct = cp.out < 0;
    const int t = c / p.group, h = hk * p.group + (c % p.group);
    const int64_t row = (int64_t)t * p.hq + h;
    const int64_t pair_row0 = ((int64_t)d * p.batch + b) * p.rows;
    const int64_t ws_row0 = direct ? 0 : (int64_t)cp.out * p.rows;
    float* dst = direct ? p.partial_out + (pair_row0 + row) * kGqaD : p.ws_o + (ws_row0 + row) * kGqaD;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const f32x4 v = o[mt] * inv;
      *reinterpret_cast<float4*>(dst + 16 * mt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (g == 0) {
      const float lse = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
      if (direct)
        p.partial_lse[pair_row0 + row] = lse;
      else
        p.ws_lse[ws_row0 + row] = lse;
    }
  }
}

bool gqa_bf16_supported(const dcp_attn_desc& D) {
  const int rows = (D.num_q_heads / D.num_kv_heads) * D.q_len;
  return D.kv_layout == DCPKV_LAYOUT_SPLIT && D.kv_dtype == DCPKV_KV_BF16 && D.q_dtype == DCPKV_Q_BF16 &&
         D.head_dim_qk == kGqaD && D.head_dim_v == kGqaD && D.page_size == kGqaPage && rows <= 16;
}

int launch_gqa_bf16(const AttnParams& p, const dcp_attn_desc& D, int64_t item_bound, hipStream_t st) {
  (void)D;
  const int64_t blocks = std::max<int64_t>(1, item_bound);
  if (blocks > INT32_MAX) return set_error(DCPKV_EINVAL, "attn: too many work items");
  hipLaunchKernelGGL(gqa_bf16_kernel, dim3((unsigned)blocks), dim3(64), 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "attn: gqa launch: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

}  // namespace dcpkv
