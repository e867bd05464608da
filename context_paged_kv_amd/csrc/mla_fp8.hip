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
// about 480 flop per KV byte, so the matrix cores bind, not HBM.
//
// Work item: (shard d, request b, chunk of local pages, block of 64 query
// rows).  A workgroup owns one item.  Its wavefronts come in pairs (w and
// w ^ kPairStride) that own kNT column tiles of 16 rows each; half
// hh = w / kPairStride of the pair
//   * computes the scores over latent dims [256 hh, 256 hh + 256) and rope
//     dims [512 + 32 hh, 512 + 32 hh + 32), and swaps that partial S^T with
//     its partner through LDS, so both hold the full scores (the same sum,
//     bit for bit, hence the same softmax decisions);
//   * accumulates O over the value dims [256 hh, 256 hh + 256).
// With kNT = 2 every converted V operand feeds two MFMAs and one wavefront
// runs per SIMD (128 accumulator registers plus the query operands); kNT = 1
// runs two wavefronts per SIMD but converts twice as much and was slower.
// Per page:
//   * the 36 KB of fp8 codes are double buffered in LDS: the loads of page
//     j+1 go out between the score MFMAs of page j and land in registers,
//     and are written to the other buffer between its PV MFMAs (copies into
//     LDS by DMA were slower to issue and held up the wave's LDS reads).
//     LDS rows are 592 bytes (576 + 16 pad);
//   * latent scores on v_mfma_scale_f32_16x16x128_f8f6f4 straight from the
//     fp8 codes (unit scales): each query row is held as two e4m3 terms,
//     hi = e4m3(q) and lo = e4m3(q - hi), whose sum is the bf16 query
//     exactly (8 significant bits = 4 + 4), so no K conversion is needed;
//     the rope dims use v_mfma_f32_16x16x32_f16 with K converted by
//     v_cvt_scalef32_pk_f16_fp8 (exact).  The query is scaled by 2^qe per row
//     so its largest entry lies in [128, 256); the factor leaves with the
//     softmax scale.  The token order of the A rows puts, after the MFMA, the
//     eight scores a lane needs for its P^T operand in that lane;
//   * online softmax in base 2 with a lazy reference: a row's exponent offset
//     moves (and the accumulator is rescaled) only when the page maximum
//     exceeds it by more than 2^8, or when the page scale leaves
//     [1/4, 4] x the reference scale; in between P carries the page-scale
//     ratio and the accumulator is touched by MFMAs only;
//   * O^T += V^T P^T on the f16 MFMA: ds_read_b64_tr_b8 hands each lane eight
//     tokens of one latent dim straight from the row-major codes, converted
//     to fp16 as above.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "attn_common.h"
#include "attn_kernels.h"

namespace dcpkv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kMlaPage = 64;
constexpr int kMlaDim = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaRowsPerBlock = 64;
#ifndef MLA_NT
#define MLA_NT 2
#endif
constexpr int kNT = MLA_NT;                          // 16-row column tiles per wavefront
constexpr int kWaves = 8 / kNT;                      // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kPairStride = kWaves / 2;              // partner of wave w is w ^ kPairStride
constexpr int kLatHalf = 256;                       // latent score dims per wavefront (fp8 MFMA)
constexpr int kRopeHalf = 32;                       // rope score dims per wavefront (f16 MFMA)
constexpr int kRope0 = kMlaDv;                      // first rope dim
constexpr int kHalfV = kMlaDv / 2;                  // 256 value dims per wavefront
constexpr int kLatSteps = kLatHalf / 128;           // 2 k-steps of 128 dims
constexpr int kVTiles = kHalfV / 16;                // 16 M tiles of 16 dims
constexpr int kRawStride = 592;                     // LDS bytes per token row of codes
constexpr int kRawBuf = kMlaPage * kRawStride;      // 37888 bytes per page buffer
constexpr int kSlotsPerRow = kRawStride / 16;       // 37 16-byte slots (36 data + 1 pad)
constexpr int kSlots = kMlaPage * kSlotsPerRow;     // 2368
constexpr int kLoadIters = (kSlots + kThreads - 1) / kThreads;  // copy instructions per wave and page
constexpr int kWaitLgkm0 = 0xC07F;                 // s_waitcnt lgkmcnt(0), other counters untouched
constexpr float kTau = 8.f;                         // lazy-rescale threshold (log2 units)
constexpr float kLog2eM = 1.4426950408889634f;
constexpr float kLn2M = 0.6931471805599453f;

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one MFMA column).
// v_permlane16_swap a, b (v_permlane32_swap a, b) with a = b = v leaves, in
// every lane, v[l] and v[l ^ 16] (v[l ^ 32]) in the two registers.  Written as
// asm with both registers as operands: the compiler's builtin for these
// instructions loses track of the second result.  The s_nop gives the two wait
// states a swap needs after a VALU write of its operands.
__device__ __forceinline__ void xpair16(float v, float& a, float& b) {
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void xpair32(float v, float& a, float& b) {
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float mgrp4_max(float v) {
  float a, b;
  xpair16(v, a, b);
  xpair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float mgrp4_sum(float v) {
  float a, b;
  xpair16(v, a, b);
  xpair32(a + b, a, b);
  return a + b;
}

// Eight fp8 e4m3fn codes (two dwords) to eight fp16 values, exactly.
__device__ __forceinline__ f16x8 cvt8(u32x2 x) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.0f, true);
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3), __builtin_shufflevector(c, d, 0, 1, 2, 3),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// Four values (already scaled so |v| < 256) as two e4m3fn words: hi = e4m3(v),
// lo = e4m3(v - hi).  A bf16 value has 8 significant bits, each e4m3 term 4, so
// hi + lo is v itself for every value whose terms stay in the normal e4m3
// range (the rest lose less than 2^-9 of the row's largest entry).
__device__ __forceinline__ void split_e4m3(const float v[4], uint32_t& hi, uint32_t& lo) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], h, true);
  float r[4];
  r[0] = v[0] - __builtin_amdgcn_cvt_f32_fp8(h, 0);
  r[1] = v[1] - __builtin_amdgcn_cvt_f32_fp8(h, 1);
  r[2] = v[2] - __builtin_amdgcn_cvt_f32_fp8(h, 2);
  r[3] = v[3] - __builtin_amdgcn_cvt_f32_fp8(h, 3);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], w, true);
  hi = (uint32_t)h;
  lo = (uint32_t)w;
}

// Token held by MFMA row m of S^T tile tt: tiles 2ks and 2ks+1 give the lane of
// group g the tokens 32ks + 8g + [0, 8), the k slots of its P^T operand.
__device__ __forceinline__ int mla_tok(int tt, int m) {
  return 32 * (tt >> 1) + 8 * (m >> 2) + 4 * (tt & 1) + (m & 3);
}

// Start the global -> LDS copy of one page of codes into a 592-byte-row buffer.
// LDS slot q (16 bytes) of row q / 37, column q % 37 holds page bytes
// 16 * (q - q / 37) onwards; the pad column refetches a valid chunk.
// Per-lane source offsets of the page copy: load i of wave w moves the 64
// consecutive 16-byte LDS slots from kThreads * i + 64 * w (none past the page;
// the pad column of a row refetches a valid chunk).
struct CopyPlan {
  uint32_t off[kLoadIters];
};
__device__ __forceinline__ CopyPlan copy_plan(int wave, int lane) {
  CopyPlan cp;
#pragma unroll
  for (int i = 0; i < kLoadIters; ++i) {
    const int slot = kThreads * i + 64 * wave + lane;
    const int row = slot / kSlotsPerRow;
    cp.off[i] = (uint32_t)min(16 * (slot - row), kMlaPage * kMlaDim - 16);
  }
  return cp;
}

__global__ __launch_bounds__(kThreads) void mla_fp8_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[2][kRawBuf];  // 75776 B
  __shared__ u32x4 s_x[kWaves][4 * kNT][64];                          // score-partial swap, 32768 B
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < kWaves);
  const int rq = wave % kPairStride, hh = wave / kPairStride;
  const int partner = wave ^ kPairStride;
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

  // The lane's query rows (one per column tile) and their operands.  Latent dims
  // 256 hh + 128 ks + 32 g + [0, 32) go to the fp8 MFMA as two exact e4m3 terms
  // (hi, lo); rope dims 512 + 32 hh + 8 g + [0, 8) go to the f16 MFMA.  Both are
  // scaled by 2^qe per row (largest |q| in [128, 256)); the factor is taken out
  // of the scores with the softmax scale.
  int rowq[kNT];
  int lim[kNT];  // last visible position of the row (positions are below T <= INT32_MAX)
  float amax[kNT];
  u32x4 qraw[kNT][kLatSteps * 4 + 1];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int r = hb * kMlaRowsPerBlock + 16 * (kNT * rq + nt) + c;
    const bool ok = r < p.rows;
    rowq[nt] = ok ? r : -1;
    const int t = ok ? r / p.hq : 0, h = ok ? r % p.hq : 0;
    lim[nt] = ok ? T - p.q_len + t : -1;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (((int64_t)b * p.q_len + t) * p.hq + h) * kMlaDim;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < kLatSteps * 4 + 1; ++i) {
      const uint16_t* src = i < kLatSteps * 4 ? qr + kLatHalf * hh + 128 * (i >> 2) + 32 * g + 8 * (i & 3)
                                              : qr + kRope0 + kRopeHalf * hh + 8 * g;
      const u32x4 w = ok ? *reinterpret_cast<const u32x4*>(src) : u32x4{0, 0, 0, 0};
      qraw[nt][i] = w;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        mx = fmaxf(mx, fmaxf(fabsf(__builtin_bit_cast(float, w[e2] << 16)),
                             fabsf(__builtin_bit_cast(float, w[e2] & 0xFFFF0000u))));
    }
    amax[nt] = mgrp4_max(mx);
  }
  // both halves of a row use one scale: swap the half maxima once
  if (g == 0) {
    float* xm = reinterpret_cast<float*>(&s_x[wave][0][0]);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) xm[16 * nt + c] = amax[nt];
  }
  __syncthreads();
  float qscale[kNT];
  i32x8 qhi[kNT][kLatSteps], qlo[kNT][kLatSteps];
  f16x8 qrope[kNT];
  {
    const float* xo = reinterpret_cast<const float*>(&s_x[partner][0][0]);
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const float am = fmaxf(amax[nt], xo[16 * nt + c]);
      const int qe = am > 0.f ? 7 - ilogbf(am) : 0;
      qscale[nt] = ldexpf(1.f, qe);
#pragma unroll
      for (int ks = 0; ks < kLatSteps; ++ks) {
        i32x8 hv, lv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // 8 dims per u32x4 -> two words of four e4m3 codes
          const u32x4 w = qraw[nt][4 * ks + j];
#pragma unroll
          for (int hw = 0; hw < 2; ++hw) {
            const float v[4] = {ldexpf(__builtin_bit_cast(float, w[2 * hw] << 16), qe),
                                ldexpf(__builtin_bit_cast(float, w[2 * hw] & 0xFFFF0000u), qe),
                                ldexpf(__builtin_bit_cast(float, w[2 * hw + 1] << 16), qe),
                                ldexpf(__builtin_bit_cast(float, w[2 * hw + 1] & 0xFFFF0000u), qe)};
            uint32_t hw32, lw32;
            split_e4m3(v, hw32, lw32);
            hv[2 * j + hw] = (int)hw32;
            lv[2 * j + hw] = (int)lw32;
          }
        }
        qhi[nt][ks] = hv;
        qlo[nt][ks] = lv;
      }
      const u32x4 w = qraw[nt][kLatSteps * 4];
      f16x2 h2[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        h2[e2] = f16x2{(_Float16)ldexpf(__builtin_bit_cast(float, w[e2] << 16), qe),
                       (_Float16)ldexpf(__builtin_bit_cast(float, w[e2] & 0xFFFF0000u), qe)};
      qrope[nt] = __builtin_shufflevector(__builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3),
                                          __builtin_shufflevector(h2[2], h2[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5,
                                          6, 7);
    }
  }
  float sl2[kNT], mref[kNT], l[kNT];  // l: this lane's share of the row's denominator
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    sl2[nt] = p.scale * kLog2eM / qscale[nt];
    mref[nt] = kNegInf;
    l[nt] = 0.f;
  }
  float ps_ref = 1.f;  // the accumulator is in units of ps_ref
  f32x4 o[kNT][kVTiles];  // O^T tiles: dims 256 hh + 16 mt + 4 g + i of row (nt, c)
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int mt = 0; mt < kVTiles; ++mt) o[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int j_begin, j_end;
  chunk_range(pp, chunk, j_begin, j_end);
  const int32_t* bt = p.block_tables + ((int64_t)d * p.batch + b) * p.max_local;
  const uint8_t* pool = p.pools[d] + (int64_t)p.layer * p.pages_per_layer * p.page_bytes;
  const uint16_t* scl = p.scales[d] + (int64_t)p.layer * p.pages_per_layer;
  // Block-table entries come in windows of 64 (one per lane, the next window loaded a whole
  // window ahead) and page scales one page ahead, so no dependent load sits between a barrier
  // and the next page's copies.  Entries outside [0, pages_per_layer) are skipped.
  const uint32_t slots = (uint32_t)min<int64_t>(p.pages_per_layer, INT32_MAX);
  auto ok = [&](int32_t sl) { return (uint32_t)sl < slots; };
  int wbase = j_begin;
  int32_t win0 = j_begin + lane < j_end ? bt[j_begin + lane] : -1;
  int32_t win1 = j_begin + 64 + lane < j_end ? bt[j_begin + 64 + lane] : -1;
  int32_t slot_cur = __builtin_amdgcn_readlane(win0, 0);
  uint16_t sc_cur = 0, sc_nxt = 0;
  // The page copy goes through registers: load i of page j + 1 is issued next to k-step i of
  // page j's scores and written to the other LDS buffer next to the last M tiles of page j's
  // PV, so both hide behind MFMAs.
  const CopyPlan cp = copy_plan(wave, lane);
  if (j_begin < j_end && ok(slot_cur)) {
    const uint8_t* page = pool + (int64_t)slot_cur * p.page_bytes;
    u32x4 stg[kLoadIters];
#pragma unroll
    for (int i = 0; i < kLoadIters; ++i)
      if (kThreads * i + 64 * wave < kSlots)
        stg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(page + cp.off[i]));
#pragma unroll
    for (int i = 0; i < kLoadIters; ++i) {
      const int base = kThreads * i + 64 * wave;
      if (base < kSlots) *reinterpret_cast<u32x4*>(s_raw[0] + 16 * (base + lane)) = stg[i];
    }
    sc_cur = scl[slot_cur];
  }
  int buf = 0;
  for (int jj = j_begin; jj < j_end; ++jj) {
    __builtin_amdgcn_s_waitcnt(0);  // this thread's copies of page jj (and the prefetched words) have landed
    __syncthreads();                // ... and everyone's; the other buffer and the swap area are free
    if (jj + 1 - wbase == 64) {
      wbase += 64;
      win0 = win1;
      win1 = wbase + 64 + lane < j_end ? bt[wbase + 64 + lane] : -1;
    }
    const int32_t slot_nxt = jj + 1 < j_end ? __builtin_amdgcn_readlane(win0, jj + 1 - wbase) : -1;
    const bool have_nxt = ok(slot_nxt);
    const uint8_t* npage = pool + (int64_t)(have_nxt ? slot_nxt : 0) * p.page_bytes;
    uint8_t* nbuf = s_raw[buf ^ 1];
    u32x4 stg[kLoadIters];  // page j + 1 on its way to the other buffer
    // No test of have_nxt here: without a next page the loads read slot 0 (in bounds) and the
    // writes land in the buffer nothing reads before it is filled again; branch-free this way.
    auto ld = [&](int i) {
      if (kThreads * i + 64 * wave < kSlots)
        stg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(npage + cp.off[i]));
    };
    auto st = [&](int i) {
      const int base = kThreads * i + 64 * wave;
      if (base < kSlots) *reinterpret_cast<u32x4*>(nbuf + 16 * (base + lane)) = stg[i];
    };
    if (have_nxt) sc_nxt = scl[slot_nxt];
    if (!ok(slot_cur)) {
#pragma unroll
      for (int i = 0; i < kLoadIters; ++i) ld(i);
#pragma unroll
      for (int i = 0; i < kLoadIters; ++i) st(i);
    }
    if (ok(slot_cur)) {
      const int pos0 = (jj * p.n + d) * kMlaPage;  // local page jj holds positions below T
      const int valid = min(T - pos0, kMlaPage);
      const bool full = pos0 <= T - p.q_len - (kMlaPage - 1);  // no row masks a token of this page
      const float ps = fmaxf(bf16_to_float(sc_cur), 1e-30f);
      uint8_t* cur = s_raw[buf];
      if (valid < kMlaPage) {  // tail of the last page: no code past T reaches a product
        for (int i = tid; i < (kMlaPage - valid) * 36; i += kThreads) {
          const int r = valid + i / 36, cc = i - (i / 36) * 36;
          *reinterpret_cast<u32x4*>(cur + r * kRawStride + 16 * cc) = u32x4{0, 0, 0, 0};
        }
        __syncthreads();
      }

      // ---- partial S^T = K Q^T over this half's dims
      f32x4 s[kNT][4];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) s[nt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // latent: A = 32 fp8 codes of token mla_tok(tt, c) (two 16-byte LDS reads), B = the
      // row's hi and lo terms; rope: one f16 k-step as in the PV loop's operands
      const uint8_t* klat = cur + kLatHalf * hh + 32 * g;
      const uint8_t* krope = cur + kRope0 + kRopeHalf * hh + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kLatSteps; ++ks) {
        i32x8 a[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const uint8_t* kp = klat + mla_tok(tt, c) * kRawStride + 128 * ks;
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(kp);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(kp + 16);
          a[tt] = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < kLoadIters / kLatSteps; ++i) ld(ks * (kLoadIters / kLatSteps) + i);
        // each accumulator is touched every 8th MFMA: hi terms of all tiles, then lo terms
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            s[nt][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[tt], qhi[nt][ks], s[nt][tt], 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            s[nt][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[tt], qlo[nt][ks], s[nt][tt], 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int i = kLatSteps * (kLoadIters / kLatSteps); i < kLoadIters; ++i) ld(i);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const f16x8 a = cvt8(*reinterpret_cast<const u32x2*>(krope + mla_tok(tt, c) * kRawStride));
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          s[nt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qrope[nt], s[nt][tt], 0, 0, 0);
      }
      // ---- swap partials with the partner wavefront; both then hold the same full scores
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) s_x[wave][4 * nt + tt][lane] = __builtin_bit_cast(u32x4, s[nt][tt]);
      // LDS writes done, then a bare barrier: a full __syncthreads would also wait for the
      // next page's copy, which is still in flight
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) s[nt][tt] += __builtin_bit_cast(f32x4, s_x[partner][4 * nt + tt][lane]);

      // ---- row maxima in log2 units (lane: row (nt, c), tokens mla_tok(tt, 4g + i))
      float f[kNT], mx[kNT];
      bool move = false;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        f[nt] = sl2[nt] * ps;
        if (!full) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (mla_tok(tt, 4 * g + i) > lim[nt] - pos0) s[nt][tt][i] = kNegInf;
        }
        float v_max = kNegInf;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) v_max = fmaxf(v_max, s[nt][tt][i]);
        mx[nt] = v_max * f[nt];  // this lane's 16 scores; the row maximum is formed only on a move
        move = move || mx[nt] > mref[nt] + kTau;
      }
      // ---- move the references when a row's maximum outgrows its offset or the scale drifts
      const float ratio = ps * __builtin_amdgcn_rcpf(ps_ref);  // page scales are normal bf16 values
      if (__any(move) || ratio > 4.f || ratio < 0.25f) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const float mn = fmaxf(mref[nt], mgrp4_max(mx[nt]));
          const float a = mref[nt] == kNegInf ? 0.f : exp2f(mref[nt] - mn);
          mref[nt] = mn;
          l[nt] *= a;
          const float fo = a * ps_ref * __builtin_amdgcn_rcpf(ps);
          // the product goes back through an MFMA (adding 0 x 0) so the accumulator keeps one
          // register class across the loop and the common path carries no copies
          const f16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int mt = 0; mt < kVTiles; ++mt) {
            asm volatile("" : "+a"(o[nt][mt]));  // read the accumulator here, not ahead of the branch
            o[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(z, z, o[nt][mt] * fo, 0, 0, 0);
          }
        }
        ps_ref = ps;
      }
      // ---- P' = 2^(x - mref) * ps / ps_ref (fp16), l += sum 2^(x - mref)
      const float lr = __builtin_amdgcn_logf(ps * __builtin_amdgcn_rcpf(ps_ref));
      const float inv_ratio = ps_ref * __builtin_amdgcn_rcpf(ps);
      f16x8 pb[kNT][2];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const float off = mref[nt] == kNegInf ? 0.f : mref[nt] - lr;  // -inf only if every score so far is masked
        float psum = 0.f;
        f16x4 ph[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          float x4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = __builtin_amdgcn_exp2f(fmaf(s[nt][tt][i], f[nt], -off));
            psum += x;
            x4[i] = x;
          }
          ph[tt] = f16x4{(_Float16)x4[0], (_Float16)x4[1], (_Float16)x4[2], (_Float16)x4[3]};
        }
        // k step ks: tokens 32ks + 8g + [0, 4) from tile 2ks, + [4, 8) from tile 2ks + 1
        pb[nt][0] = __builtin_shufflevector(ph[0], ph[1], 0, 1, 2, 3, 4, 5, 6, 7);
        pb[nt][1] = __builtin_shufflevector(ph[2], ph[3], 0, 1, 2, 3, 4, 5, 6, 7);
        l[nt] += psum * inv_ratio;  // this lane's part of the row's denominator
      }
      // ---- O^T += V^T P^T over this half's value dims
      // source lane (g, c) of the transposing read points at token 32ks + 8g + (c >> 1),
      // dims 16*mt + 8*(c & 1) .. +7; lane (g, j) then holds dim 16*mt + j of those 8 tokens
      const uint8_t* vrow = cur + (8 * g + (c >> 1)) * kRawStride + 8 * (c & 1) + kHalfV * hh;
      i32x2 vx[2][2];  // codes of M tiles mt (in use) and mt + 1 (in flight)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        vx[0][ks] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vrow + 32 * ks * kRawStride));
#pragma unroll
      for (int mt = 0; mt < kVTiles; ++mt) {
        if (mt >= kVTiles - kLoadIters) st(mt - (kVTiles - kLoadIters));
        if (mt + 1 < kVTiles) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            vx[(mt + 1) & 1][ks] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2*)(vrow + 32 * ks * kRawStride + 16 * (mt + 1)));
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f16x8 a = cvt8(__builtin_bit_cast(u32x2, vx[mt & 1][ks]));
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            o[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[nt][ks], o[nt][mt], 0, 0, 0);
        }
      }
    }
    slot_cur = slot_nxt;
    sc_cur = sc_nxt;
    buf ^= 1;
  }

  // ---- write the (chunk) partial of the lane's two rows, this half's dims: O = ps_ref * O^T / l
  const bool direct = pp.k == 1;
  const int64_t pair_row0 = ((int64_t)d * p.batch + b) * p.rows;
  const int64_t ws_row0 = direct ? 0 : ((int64_t)pp.ws_begin + chunk) * p.rows;
  float lrow[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) lrow[nt] = mgrp4_sum(l[nt]);
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    if (rowq[nt] < 0) continue;
    const int r = rowq[nt];
    float* dst = (direct ? p.partial_out + (pair_row0 + r) * kMlaDv : p.ws_o + (ws_row0 + r) * kMlaDv) +
                 kHalfV * hh;
    const float inv = lrow[nt] > 0.f ? ps_ref / lrow[nt] : 0.f;
#pragma unroll
    for (int mt = 0; mt < kVTiles; ++mt) {
      const f32x4 v = o[nt][mt] * inv;
      *reinterpret_cast<float4*>(dst + 16 * mt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (g == 0 && hh == 0) {
      const float lse = lrow[nt] > 0.f ? (mref[nt] + log2f(lrow[nt])) * kLn2M : kNegInf;
      if (direct)
        p.partial_lse[pair_row0 + r] = lse;
      else
        p.ws_lse[ws_row0 + r] = lse;
    }
  }
}

bool mla_fp8_supported(const dcp_attn_desc& D) {
  return D.kv_layout == DCPKV_LAYOUT_MLA && D.kv_dtype == DCPKV_KV_FP8E4M3 && D.q_dtype == DCPKV_Q_BF16 &&
         D.head_dim_qk == kMlaDim && D.head_dim_v == kMlaDv && D.num_kv_heads == 1 && D.page_size == kMlaPage;
}

int mla_fp8_rows_per_block() { return kMlaRowsPerBlock; }

int launch_mla_fp8(const AttnParams& p, const dcp_attn_desc& D, int64_t item_bound, hipStream_t st) {
  (void)D;
  const int64_t chunks_bound = (item_bound + p.hb_count - 1) / p.hb_count;
  const int64_t blocks = ((chunks_bound + 7) / 8) * 8 * p.hb_count;
  if (blocks > INT32_MAX / 256) return set_error(DCPKV_EINVAL, "attn: too many work items");
  hipLaunchKernelGGL(mla_fp8_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(kThreads), 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "attn: mla launch: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

}  // namespace dcpkv
