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
//
// Two ways to hand out the work:
//   * even split (gqa_bf16_even_kernel, up to kEvenMaxPairs pairs): one
//     resident wave per slot, each streaming the same number of pages through
//     the sequence of (pair, KV head) segments.  The page pipeline runs across
//     segment boundaries (the next segment's slots, query and length are
//     fetched while the current one streams), so the memory system sees no
//     gaps between work items and all waves finish together;
//   * chunks (gqa_bf16_kernel): one workgroup per (chunk, KV head) item of the
//     chunk plan, for larger batches.

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

// Stage one page from registers into the wave's LDS tiles: K rows swizzled, V transposed.
// V rows at or past `valid` are zeroed first (the tail of the last page must never
// bring bytes past T into the sums, whatever they hold).
__device__ __forceinline__ void stage_page(GqaWaveLds& L, const u32x4 (&kr)[16], u32x4 (&vr)[16], int valid, int c,
                                           int g) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 4 * i + g;
    *reinterpret_cast<u32x4*>(&L.k[r * kGqaRow + 16 * (c ^ kswz(r))]) = kr[i];
  }
  if (valid < kGqaPage) {
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
}

// LDS hand-over point between the lanes of the wave (the fences keep the compiler from
// moving one lane's LDS accesses across the point where another lane's begin).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Scores, online softmax and O update for the staged page.  Tokens past `thr` (this
// lane's row's last visible token within the page) take no part.
__device__ __forceinline__ void compute_page(const GqaWaveLds& L, const bf16x8 (&qb)[4], int64_t thr, float sl2,
                                             float& m, float& l, f32x4 (&o)[8], int c, int g) {
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
}

// Q^T as the B operand of S^T: lane (g, c) holds query row c, dims 32*kk + 8*g + [0, 8).
__device__ __forceinline__ void load_q(const AttnParams& p, int b, int hk, int rows, int c, int g, bf16x8 (&qb)[4]) {
  // Columns c >= rows repeat the last row: their scores are masked out (no visible token)
  // and an MFMA column only ever feeds its own row, so the copy touches no result, and the
  // load needs no branch (it may be issued while pages are in flight).
  const uint16_t* q = static_cast<const uint16_t*>(p.q);
  const int cc = min(c, rows - 1);
  const int t = cc / p.group, h = hk * p.group + (cc % p.group);
  const uint16_t* qr = q + (((int64_t)b * p.q_len + t) * p.hq + h) * kGqaD;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qb[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + 32 * kk + 8 * g));
}

// Row c's normalised output (O / l) and LSE (natural log) to dst / *dst_lse.
__device__ __forceinline__ void write_row(float* dst, float* dst_lse, float m, float l, const f32x4 (&o)[8], int g) {
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const f32x4 v = o[mt] * inv;
    *reinterpret_cast<float4*>(dst + 16 * mt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
  }
  if (g == 0) *dst_lse = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
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

  bf16x8 qb[4];
  load_q(p, b, hk, rows, c, g, qb);
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
    stage_page(L, kr, vr, valid, c, g);
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
    wave_sync();
    compute_page(L, qb, thr, sl2, m, l, o, c, g);
    wave_sync();  // this page's LDS reads precede the next page's writes
    jj = jn;
  }

  // ---- write the (chunk) partial of row c
  if (c < rows) {
    const bool direct = cp.out < 0;
    const int t = c / p.group, h = hk * p.group + (c % p.group);
    const int64_t row = (int64_t)t * p.hq + h;
    const int64_t pair_row0 = ((int64_t)d * p.batch + b) * p.rows;
    const int64_t ws_row0 = direct ? 0 : (int64_t)cp.out * p.rows;
    if (direct)
      write_row(p.partial_out + (pair_row0 + row) * kGqaD, p.partial_lse + pair_row0 + row, m, l, o, g);
    else
      write_row(p.ws_o + (ws_row0 + row) * kGqaD, p.ws_lse + ws_row0 + row, m, l, o, g);
  }
}

// Pairs a wave plans by itself (SELF): four per lane.
constexpr int kSelfPlanBlocks = 4;

__device__ __forceinline__ int pick(const int (&v)[kSelfPlanBlocks], int k) {
  return k == 0 ? v[0] : (k == 1 ? v[1] : (k == 2 ? v[2] : v[3]));
}
__device__ __forceinline__ int64_t pick64(const int64_t (&v)[kSelfPlanBlocks], int k) {
  return k == 0 ? v[0] : (k == 1 ? v[1] : (k == 2 ? v[2] : v[3]));
}
__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Even split: wave w streams its page-items (see WaveStart), one page in flight ahead of the
// one being computed, across segment boundaries.  Each pass of the loop stages the page in
// flight, issues the next page's loads (one load site, so the page registers never move),
// computes the staged page and, at a segment's end, writes its part and moves on.
// SELF (at most 64 x kSelfPlanBlocks pairs): every wave computes the plan itself from the
// request lengths (pair k * 64 + lane in lane `lane`, block k): local pages, their prefix
// sums, its range and the pair that holds its first item; wave 0 also writes the prefix sums,
// pair entries and header the reduction reads.  Otherwise the starts come from the planner.
template <bool SELF>
__global__ __launch_bounds__(64) void gqa_bf16_even_kernel(AttnParams p) {
  __shared__ GqaWaveLds s_lds;
  GqaWaveLds& L = s_lds;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int w = blockIdx.x;
  const int rows = p.group * p.q_len;
  const int num_pairs = p.shard_count * p.batch;
  const float sl2 = p.scale * kLog2e;
  const int64_t head_bytes = (int64_t)kGqaPage * kGqaRow;
  const int64_t layer_off = (int64_t)p.layer * p.pages_per_layer * p.page_bytes;

  int sT[kSelfPlanBlocks], snl[kSelfPlanBlocks];
  int64_t spf[kSelfPlanBlocks];
  uint64_t nz[kSelfPlanBlocks];
  int after[kSelfPlanBlocks];  // first pair with pages in the blocks after block k
  // the next pair with pages after pair a (num_pairs if none)
  auto next_after = [&](int a) -> int {
    const int k0 = (a + 1) >> 6, sh = (a + 1) & 63;
    int r = num_pairs;
#pragma unroll
    for (int k = kSelfPlanBlocks - 1; k >= 0; --k) {
      if (k < k0) break;
      const uint64_t m = k == k0 ? (nz[k] & (~0ull << sh)) : nz[k];
      if (m) r = 64 * k + (int)__builtin_ctzll(m);
    }
    return r;
  };

  int pair, hb, j0, count, nl, next_pair, T;
  if constexpr (SELF) {
#pragma unroll
    for (int k = 0; k < kSelfPlanBlocks; ++k) {
      const int pr = min(64 * k + lane, num_pairs - 1);
      sT[k] = p.seq_lens[pr % p.batch];
    }
    int64_t carry = 0;
#pragma unroll
    for (int k = 0; k < kSelfPlanBlocks; ++k) {
      const int pr = 64 * k + lane;
      const int d = p.shard_begin + min(pr, num_pairs - 1) / p.batch;
      snl[k] = pr < num_pairs ? local_pages_of(sT[k], p.page_size, p.n, d, p.max_local, p.tok_il) : 0;
      int64_t incl = snl[k];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t u = __shfl_up(incl, off, 64);
        if (lane >= off) incl += u;
      }
      spf[k] = carry + incl - snl[k];
      carry += readlane64(incl, 63);
      nz[k] = __ballot(snl[k] > 0);
    }
    after[kSelfPlanBlocks - 1] = num_pairs;
#pragma unroll
    for (int k = kSelfPlanBlocks - 2; k >= 0; --k)
      after[k] = nz[k + 1] ? 64 * (k + 1) + (int)__builtin_ctzll(nz[k + 1]) : after[k + 1];
    const int64_t P = carry * p.hkv;
    const int G = (int)min<int64_t>(p.slots, P);
    if (w == 0) {  // what the reduction reads
#pragma unroll
      for (int k = 0; k < kSelfPlanBlocks; ++k) {
        const int pr = 64 * k + lane;
        if (pr < num_pairs) {
          const uint64_t m = lane == 63 ? 0ull : (nz[k] & (~0ull << (lane + 1)));
          const int nx = m ? 64 * k + (int)__builtin_ctzll(m) : after[k];
          p.pairs[pr] = PairPlan{0, -1, nx, snl[k]};
          p.pair_pfx[pr] = spf[k];
        }
      }
      if (lane == 0) {
        p.pair_pfx[num_pairs] = carry;
        p.hdr->total_chunks = 0;
        p.hdr->ws_chunks = 0;
        p.hdr->fallback = 0;
        p.hdr->waves = G;
        p.hdr->total_work = P;
      }
    }
    if (w >= G) return;
    const int64_t x0 = (int64_t)w * P / G, x1 = (int64_t)(w + 1) * P / G;
    // the pair of item x0: the last one whose first item is <= x0 (it has pages)
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kSelfPlanBlocks; ++k)
      cnt += __popcll(__ballot(64 * k + lane < num_pairs && spf[k] * p.hkv <= x0));
    pair = cnt - 1;
    const int blk = pair >> 6, ln = pair & 63;
    nl = __builtin_amdgcn_readlane(pick(snl, blk), ln);
    T = __builtin_amdgcn_readlane(pick(sT, blk), ln);
    const int64_t off = x0 - readlane64(pick64(spf, blk), ln) * p.hkv;
    hb = (int)(off / nl);
    j0 = (int)(off % nl);
    count = (int)(x1 - x0);
    next_pair = next_after(pair);
  } else {
    const WaveStart ws = p.wstarts[w];
    if (ws.count <= 0) return;
    pair = ws.pair;
    hb = ws.hb;
    j0 = ws.j0;
    count = ws.count;
    nl = ws.n_local;
    next_pair = ws.next_pair;
    T = ws.seq_len;
  }

  // current segment (pair, KV head hb): this wave's pages [jb, je) of the pair's nl
  int jb = j0, je = min(nl, jb + count);
  int left = count - (je - jb);  // page-items after the current segment
  int d = p.shard_begin + pair / p.batch, b = pair % p.batch;
  const int32_t* bt = p.block_tables + ((int64_t)d * p.batch + b) * p.max_local;
  const uint8_t* pool = p.pools[d] + layer_off;
  bool first_seg = true;
  bf16x8 qb[4];
  load_q(p, b, hb, rows, c, g, qb);

  // Slots of the current pair's pages win .. win + 63 (lane i: page win + i).  Entries past
  // the pair's pages are read from inside the table row (index clamped) and never selected:
  // every use checks the page against the segment's end first.
  int win = jb;
  int32_t wslot = bt[min(jb + lane, p.max_local - 1)];
  auto next_in_cur = [&](int j, int32_t& slot) -> int {
    while (j < je) {
      if (j < win || j >= win + 64) {
        win = j;
        wslot = bt[min(j + lane, p.max_local - 1)];
      }
      const uint64_t ok = __ballot(win + lane < je && wslot >= 0 && wslot < p.pages_per_layer);
      const uint64_t rest = ok >> (j - win);
      if (rest) {
        const int k = j + (int)__builtin_ctzll(rest);
        slot = __builtin_amdgcn_readlane(wslot, k - win);
        return k;
      }
      j = win + 64;
    }
    return je;
  };

  // The next segment, fetched while the current one streams: its pair's plan entry and
  // length and the slots of its pages 0 .. 63, by per-lane vector loads (lane 0's value is
  // the one used) that wait behind the page loads in flight and hold up nothing.
  int n_pair = -1, n_hb = 0;
  bool has_next = false;
  int32_t nwslot = -1, nv_nl = 0, nv_next = 0, nv_T = 0;
  auto prefetch = [&]() {
    has_next = false;
    if (left <= 0) return;
    n_pair = pair;
    n_hb = hb + 1;
    if (n_hb == p.hkv) {
      n_pair = next_pair;
      n_hb = 0;
    }
    if (n_pair >= num_pairs) return;  // no pair with pages left (the plan never leaves such a wave with work)
    has_next = true;
    if (n_pair != pair) {
      if constexpr (SELF) {
        const int blk = n_pair >> 6, ln = n_pair & 63;
        nv_nl = __builtin_amdgcn_readlane(pick(snl, blk), ln);
        nv_next = next_after(n_pair);
        nv_T = __builtin_amdgcn_readlane(pick(sT, blk), ln);
      } else {
        const PairPlan npp = p.pairs[min(n_pair + lane, num_pairs - 1)];
        nv_nl = npp.n_local;
        nv_next = npp.k;
        nv_T = p.seq_lens[min(n_pair % p.batch + lane, p.batch - 1)];
      }
      const int nb = n_pair % p.batch, nd = p.shard_begin + n_pair / p.batch;
      nwslot = p.block_tables[((int64_t)nd * p.batch + nb) * p.max_local + min(lane, p.max_local - 1)];
    } else {
      nv_nl = nl;
      nv_next = next_pair;
      nv_T = T;
      nwslot = win == 0 ? wslot : bt[min(lane, p.max_local - 1)];
    }
  };
  int n_je = 0;  // the next segment's page end, once known

  float m = kNegInf, l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 kr[16], vr[16];
  bool have = false;  // page jj of the current segment is in flight in kr / vr
  int jj = jb;        // without one: where to look for the next page
  prefetch();
  while (true) {
    int64_t thr = 0;
    if (have) {
      const int64_t lim = c < rows ? (int64_t)T - p.q_len + c / p.group : -1;
      const int64_t vlast = local_limit((int64_t)T - 1, jj, kGqaPage, p.n, d, p.tok_il);
      const int valid = vlast + 1 < kGqaPage ? (int)(vlast + 1) : kGqaPage;
      thr = local_limit(lim, jj, kGqaPage, p.n, d, p.tok_il);
      stage_page(L, kr, vr, valid, c, g);
    }
    // the page to fetch next: in this segment, else the next segment's first valid page
    int32_t slot = -1;
    const int jn = next_in_cur(have ? jj + 1 : jj, slot);
    int jx = -1;
    const uint8_t* page = nullptr;
    int page_hb = hb;
    if (jn < je) {
      page = pool + (int64_t)slot * p.page_bytes;
    } else if (have && has_next) {
      n_je = min(__builtin_amdgcn_readfirstlane(nv_nl), left);
      const uint64_t ok = __ballot(lane < n_je && nwslot >= 0 && nwslot < p.pages_per_layer);
      if (ok) {
        jx = (int)__builtin_ctzll(ok);
        const int nd = p.shard_begin + n_pair / p.batch;
        page = p.pools[nd] + layer_off + (int64_t)__builtin_amdgcn_readlane(nwslot, jx) * p.page_bytes;
        page_hb = n_hb;
      }
    }
    if (page) load_page(page + (int64_t)page_hb * head_bytes, page + ((int64_t)p.hkv + page_hb) * head_bytes, c, g, kr, vr);
    if (have) {
      wave_sync();
      compute_page(L, qb, thr, sl2, m, l, o, c, g);
      wave_sync();
    }
    if (jn < je) {
      jj = jn;
      have = true;
      continue;
    }
    // ---- the segment is done: row c's part straight to partial_out when this wave held the
    // whole segment, else to the wave's workspace slot for it
    if (c < rows) {
      const int t = c / p.group, h = hb * p.group + (c % p.group);
      if (jb == 0 && je == nl) {
        const int64_t row = ((int64_t)d * p.batch + b) * p.rows + (int64_t)t * p.hq + h;
        write_row(p.partial_out + row * kGqaD, p.partial_lse + row, m, l, o, g);
      } else {
        const int64_t row = (2 * (int64_t)w + (first_seg ? 0 : 1)) * kEvenRows + c;
        write_row(p.ws_o + row * kGqaD, p.ws_lse + row, m, l, o, g);
      }
    }
    if (!has_next) break;
    m = kNegInf;
    l = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // ---- switch to the next segment
    const bool same_pair = n_pair == pair;
    pair = n_pair;
    hb = n_hb;
    nl = __builtin_amdgcn_readfirstlane(nv_nl);
    next_pair = __builtin_amdgcn_readfirstlane(nv_next);
    T = __builtin_amdgcn_readfirstlane(nv_T);
    jb = 0;
    je = min(nl, left);
    left -= je;
    first_seg = false;
    if (!same_pair) {
      d = p.shard_begin + pair / p.batch;
      b = pair % p.batch;
      bt = p.block_tables + ((int64_t)d * p.batch + b) * p.max_local;
      pool = p.pools[d] + layer_off;
    }
    win = 0;
    wslot = nwslot;
    load_q(p, b, hb, rows, c, g, qb);
    prefetch();
    have = jx >= 0;
    jj = have ? jx : 0;
  }
}

bool gqa_bf16_supported(const dcp_attn_desc& D) {
  const int rows = (D.num_q_heads / D.num_kv_heads) * D.q_len;
  return D.kv_layout == DCPKV_LAYOUT_SPLIT && D.kv_dtype == DCPKV_KV_BF16 && D.q_dtype == DCPKV_Q_BF16 &&
         D.head_dim_qk == kGqaD && D.head_dim_v == kGqaD && D.page_size == kGqaPage && rows <= 16;
}

int launch_gqa_bf16(const AttnParams& p, const dcp_attn_desc& D, int64_t item_bound, hipStream_t st) {
  (void)D;
  if (p.even == 2) {
    hipLaunchKernelGGL(gqa_bf16_even_kernel<true>, dim3((unsigned)std::max(1, p.slots)), dim3(64), 0, st, p);
  } else if (p.even) {
    hipLaunchKernelGGL(gqa_bf16_even_kernel<false>, dim3((unsigned)std::max(1, p.slots)), dim3(64), 0, st, p);
  } else {
    const int64_t blocks = std::max<int64_t>(1, item_bound);
    if (blocks > INT32_MAX) return set_error(DCPKV_EINVAL, "attn: too many work items");
    hipLaunchKernelGGL(gqa_bf16_kernel, dim3((unsigned)blocks), dim3(64), 0, st, p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "attn: gqa launch: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

}  // namespace dcpkv
