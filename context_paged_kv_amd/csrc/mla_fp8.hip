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
// rows).  A workgroup of eight wavefronts owns one item, two wavefronts per
// SIMD of two kinds, one page apart, so one's vector work runs under the
// other's MFMAs:
//   * score wavefront w (w < 4): S^T for row tile w (16 rows) and all 64
//     tokens of page t over all 576 dims, the row offsets and the softmax
//     numerators P, handed to the value wavefronts through LDS (fp16, already
//     in the P^T operand layout, double buffered by page parity);
//   * value wavefront 4 + v: O^T for value dims [128 v, 128 v + 128) of all
//     64 rows from page t - 1's P, each converted V operand feeding four
//     MFMAs (one per row tile).
// Per page (one barrier each):
//   * the 36 KB of fp8 codes come by LDS DMA into three buffers, page t + 1
//     during step t.  LDS rows are 592 bytes (576 + 16 pad);
//   * latent scores on v_mfma_scale_f32_16x16x128_f8f6f4 straight from the
//     fp8 codes: each query row is held as two e4m3 terms per 32-dim block
//     of the instruction's block scaling, hi = e4m3(2^k q) and
//     lo = e4m3(16 (2^k q - hi)), with k chosen per block so that its largest
//     entry lies in [128, 256) and the block's scale operands 2^-k and 2^-k-4
//     taking the factors out inside the instruction.  A bf16 value has 8
//     significant bits, each term 4, so hi + lo is the query itself for every
//     entry within 2^13 of its block's largest; no K conversion is needed.  The
//     rope dims use v_mfma_f32_16x16x32_f16 with K converted by
//     v_cvt_scalef32_pk_f16_fp8 (exact).  The whole row is scaled by 2^qe
//     (largest entry in [128, 256)) for the fp16 rope operand and the latent
//     blocks' scales are relative to it; 2^qe leaves with the softmax scale;
//   * online softmax in base 2 with a lazy offset per row: the score wavefront
//     raises it only when the page's maximum exceeds it by more than 2^8, and
//     the value wavefronts rescale accumulator rows only then.  The page scale
//     rides in P as the ratio to a reference scale that moves (with a rescale)
//     only when the ratio leaves [1/4, 4];
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kMlaPage = 64;
constexpr int kMlaDim = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaRowsPerBlock = 64;
constexpr int kWaves = 8;                              // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kRowTiles = kMlaRowsPerBlock / 16;       // 4 column tiles of 16 query rows
constexpr int kLatSteps = kMlaDv / 128;                // 4 fp8 k-steps of 128 latent dims
constexpr int kRope0 = kMlaDv;                         // first rope dim
constexpr int kRopeSteps = (kMlaDim - kMlaDv) / 32;    // 2 f16 k-steps of 32 rope dims
constexpr int kQWords = kLatSteps * 4 + kRopeSteps;    // 16-byte query loads per lane
constexpr int kWaveDv = kMlaDv / kRowTiles;            // 128 value dims per accumulating wavefront
constexpr int kVTiles = kWaveDv / 16;                  // 8 M tiles of 16 dims
constexpr int kRawStride = 592;                        // LDS bytes per token row of codes
constexpr int kRawBuf = kMlaPage * kRawStride;         // 37888 bytes per page buffer
constexpr int kSlotsPerRow = kRawStride / 16;          // 37 16-byte slots (36 data + 1 pad)
constexpr int kSlots = kMlaPage * kSlotsPerRow;        // 2368
constexpr int kLoadIters = (kSlots + kThreads - 1) / kThreads;  // copy instructions per wave and page
constexpr int kPageBufs = 3;                           // page buffers in LDS
constexpr float kTau = 8.f;                            // lazy-rescale threshold (log2 units)
constexpr int kF16Steps = kMlaDim / 32;                // 18 f16 k-steps over all 576 dims (exact scores)
// A row whose largest |q| exceeds kOutlier times its root mean square takes the exact score path
// (fp16 operands): the fp8 instruction keeps about 2^-12 of the largest product of a block, so
// a row with outliers would lose more than the scores may.
constexpr float kOutlier = 16.f;
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
// lo = e4m3(16 (v - hi)).  A bf16 value has 8 significant bits, each e4m3 term
// 4 (the residual's 4 bits are scaled by 16 to keep them out of e4m3's
// subnormal range), so hi + lo / 16 is v itself for every |v| >= 2^-6; smaller
// values lose the bits below 2^-13, less than 2^-20 of a block whose largest
// entry lies in [128, 256).
__device__ __forceinline__ void split_e4m3(const float v[4], uint32_t& hi, uint32_t& lo) {
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], h, true);
  float r[4];
  r[0] = 16.f * (v[0] - __builtin_amdgcn_cvt_f32_fp8(h, 0));
  r[1] = 16.f * (v[1] - __builtin_amdgcn_cvt_f32_fp8(h, 1));
  r[2] = 16.f * (v[2] - __builtin_amdgcn_cvt_f32_fp8(h, 2));
  r[3] = 16.f * (v[3] - __builtin_amdgcn_cvt_f32_fp8(h, 3));
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], w, true);
  hi = (uint32_t)h;
  lo = (uint32_t)w;
}

// Token order of a 32-token half page.  The PV contraction takes, in k-step
// slot (g, k) of a lane (g = lane / 16), token mla_vtok(g, k); the score MFMA
// row m of S^T tile tt reads token mla_tok(tt, m) = mla_vtok(m / 4, 4 tt + m % 4),
// so the output lane of group g holds the eight scores of its P^T slots.  The
// order makes both LDS access patterns bank-conflict free with 592-byte rows:
// the 16 rows of a score tile and the 16 rows a transposing read touches in a
// half wave are distinct modulo 16.
__device__ __forceinline__ int mla_vtok(int g, int k) {
  return 4 * g + k + (k < 4 ? (g < 2 ? 0 : 16) : 4);
}
__device__ __forceinline__ int mla_tok(int tt, int m) { return mla_vtok(m >> 2, 4 * tt + (m & 3)); }

// Eight bf16 values (one 16-byte load) times 2^e as eight fp16 values (exact for the range a
// query row scaled to a largest entry in [128, 256) occupies).
__device__ __forceinline__ f16x8 bf16x8_to_f16(u32x4 w, int e) {
  f16x2 h2[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2)
    h2[e2] = f16x2{(_Float16)ldexpf(__builtin_bit_cast(float, w[e2] << 16), e),
                   (_Float16)ldexpf(__builtin_bit_cast(float, w[e2] & 0xFFFF0000u), e)};
  return __builtin_shufflevector(__builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3),
                                 __builtin_shufflevector(h2[2], h2[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// The two halves of an eight-dword register group as fp16 operands, and back.
__device__ __forceinline__ f16x8 f16_half(i32x8 v, int h) {
  const i32x4 q = h ? __builtin_shufflevector(v, v, 4, 5, 6, 7) : __builtin_shufflevector(v, v, 0, 1, 2, 3);
  return __builtin_bit_cast(f16x8, q);
}
__device__ __forceinline__ i32x8 f16_pair(f16x8 a, f16x8 b) {
  return __builtin_shufflevector(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), 0, 1, 2, 3, 4, 5, 6,
                                 7);
}

// Block scaling of v_mfma_scale_f32_16x16x128_f8f6f4 (lane layout checked with an in-bounds
// probe): lane (g, c) holds 32 bytes of row (or column) c; its bytes [0, 16) belong to the
// instruction's 32-element block g / 2 and bytes [16, 32) to block 2 + g / 2, so each block is
// shared by lanes g and g ^ 1, and the scale of block b of row c is the operand of lane
// (b, c).  Exponent k of a block with largest magnitude m (2^k m in [128, 256)), relative to
// the row's 2^qe and kept within 2^120 of it (a block that far below its row adds nothing).
__device__ __forceinline__ int mla_block_exp(float m, int qe) {
  return m > 0.f ? min(7 - ilogbf(m), qe + 120) : qe;
}

// One LDS DMA piece: 16 bytes per lane from gptr to LDS address m0 + 16 lane (4 bytes per
// lane for dma4).  Written as asm, so the compiler neither orders LDS reads behind it nor
// counts it: every wait for these pieces is explicit.  The LDS address is an operand bound
// to m0, so the compiler sets m0 itself and knows it is in use; the s_nop is the one wait
// state an SALU write of m0 needs before an LDS DMA reads it.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"{m0}"(lds_addr), "v"(gptr) : "memory");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %1, off" ::"{m0}"(lds_addr), "v"(gptr) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS slot q (16 bytes) of a page buffer, row q / 37 and column q % 37, holds
// page bytes 16 * (q - q / 37) onwards.  Per-lane source offsets of the page copy: load i of wave w moves the 64
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

// Largest token x of local page j of shard d at a position <= pos (the 32-bit form of
// local_limit: positions are below T <= INT32_MAX).
__device__ __forceinline__ int mla_llim(int pos, int j, int tok_il, int n, int d) {
  return tok_il ? (pos >= d ? (pos - d) / n : -1) - j * kMlaPage : pos - (j * n + d) * kMlaPage;
}

// Page copies: global -> LDS by DMA, no registers.  Every wavefront issues kLoadIters
// requests per page (those with one piece less fetch the page-scale dword instead), so
// counting requests tells when a page has landed.
struct MlaCopy {
  const int32_t* bt;    // the pair's block table, from its first local page of the chunk
  const uint8_t* pool;  // layer base of the shard's pool
  const uint16_t* scl;  // layer base of the shard's page scales
  int64_t page_bytes;
  uint32_t slots;       // M: entries outside [0, M) are missing pages
  int np, wave, lane, tid;
  int wbase;            // block-table entries come in windows of 64 (one per lane), the next
  int32_t win0, win1;   // window loaded a whole window ahead
};

__device__ __forceinline__ bool mla_ok(const MlaCopy& m, int32_t sl) { return (uint32_t)sl < m.slots; }

// Page q (local to the chunk, ascending) into buffer q % 3; its entry goes to s_slot.
__device__ __forceinline__ void mla_fetch(MlaCopy& m, const CopyPlan& cp, int q, uint8_t (*s_raw)[kRawBuf],
                                          uint32_t (*s_scw)[4], int32_t* s_slot) {
  if (q - m.wbase == 64) {
    m.wbase += 64;
    m.win0 = m.win1;
    m.win1 = m.wbase + 64 + m.lane < m.np ? m.bt[m.wbase + 64 + m.lane] : -1;
  }
  const int32_t sl = __builtin_amdgcn_readlane(m.win0, q - m.wbase);
  const int bi = q % kPageBufs;
  const int32_t sl0 = mla_ok(m, sl) ? sl : 0;  // a missing page reads slot 0 (in bounds)
  const uint8_t* page = m.pool + (int64_t)sl0 * m.page_bytes;
#pragma unroll
  for (int i = 0; i < kLoadIters; ++i) {
    const int base = kThreads * i + 64 * m.wave;
    if (base < kSlots) {
      dma16(page + cp.off[i], lds_addr_of(s_raw[bi] + 16 * base));
    } else if (m.lane == 0) {  // one lane: a dword request writes 4 bytes per active lane
      const uintptr_t sa = (uintptr_t)(m.scl + sl0);
      dma4((const void*)(sa & ~(uintptr_t)3), lds_addr_of(&s_scw[bi][m.wave & 3]));
    }
  }
  if (m.tid == 0) s_slot[bi] = sl;
}

// The bf16 scale of the page in buffer bi (entry sl), out of its dword.
__device__ __forceinline__ float mla_scale(const MlaCopy& m, int32_t sl, int bi, uint32_t (*s_scw)[4]) {
  const uint32_t w = s_scw[bi][((kSlots - kThreads * (kLoadIters - 1)) / 64) & 3];
  const uintptr_t sa = (uintptr_t)(m.scl + (mla_ok(m, sl) ? sl : 0));
  return fmaxf(bf16_to_float((uint16_t)((sa & 2) ? (w >> 16) : (w & 0xFFFFu))), 1e-30f);
}

// The reference page scale an accumulator is in units of moves (with a rescale) when a page's
// ratio to it leaves [1/4, 4].
__device__ __forceinline__ float mla_next_ref(float ps, float ref) {
  const float rat = ps * __builtin_amdgcn_rcpf(ref);
  return (rat > 4.f || rat < 0.25f) ? ps : ref;
}

// Scale the accumulator tile by f.  The product goes back through an MFMA
// (adding 0 x 0) so the accumulator keeps one register class across the loop
// and the common path carries no copies; the empty asm makes the read happen
// here, not ahead of the (rare) branch that calls this.
__device__ __forceinline__ void scale_acc(f32x4& o, float f) {
  const f16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  asm volatile("" : "+v"(o));
  o = __builtin_amdgcn_mfma_f32_16x16x32_f16(z, z, o * f, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads) void mla_fp8_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_raw[kPageBufs][kRawBuf];  // 113664 B
  __shared__ f16x8 s_p[2][kRowTiles][2][64];  // P^T operands by (step parity, row tile, token half, lane), 16 KB
  __shared__ float s_off[2][kMlaRowsPerBlock];  // each row's exponent offset for the page, by step parity
  __shared__ uint32_t s_scw[kPageBufs][4];      // the dword holding each buffer's page scale
  __shared__ float s_l[kMlaRowsPerBlock];       // final denominators
  __shared__ int32_t s_slot[kPageBufs];         // block-table entry of the page in each buffer
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < kWaves);
  const bool scorer = wave < kRowTiles;  // waves 0-3 score row tile `wave`; waves 4-7 accumulate values
  const int g = lane >> 4, c = lane & 15;

  // items sharing a chunk run on the same XCD (dispatch is round robin over 8)
  const int hbc = p.hb_count;
  const int blk = blockIdx.x;
  const int gc = (blk / (8 * hbc)) * 8 + (blk & 7);
  const int hb = (blk >> 3) % hbc;
  const ChunkPlan chk = load_chunk(p, gc);
  if (chk.pair < 0) return;
  const int pair = chk.pair;
  const int d = p.shard_begin + pair / p.batch, b = pair % p.batch;
  const int T = p.seq_lens[b];

  const int j_begin = chk.j_begin, np = chk.j_end - chk.j_begin;
  const int32_t* bt = p.block_tables + ((int64_t)d * p.batch + b) * p.max_local;
  const uint8_t* pool = p.pools[d] + (int64_t)p.layer * p.pages_per_layer * p.page_bytes;
  const uint16_t* scl = p.scales[d] + (int64_t)p.layer * p.pages_per_layer;
  const int tok_il = p.tok_il, nsh = p.n;
  MlaCopy mc;
  mc.bt = bt + j_begin;
  mc.pool = pool;
  mc.scl = scl;
  mc.page_bytes = p.page_bytes;
  mc.slots = (uint32_t)min<int64_t>(p.pages_per_layer, INT32_MAX);
  mc.np = np;
  mc.wave = wave;
  mc.lane = lane;
  mc.tid = tid;
  mc.wbase = 0;
  mc.win0 = lane < np ? mc.bt[lane] : -1;
  mc.win1 = 64 + lane < np ? mc.bt[64 + lane] : -1;
  const CopyPlan cp = copy_plan(wave, lane);
  // Page q + 1 is fetched during step q (three buffers: step q reads pages q - 1 and q).  A
  // missing page's tokens are all masked; its rows, and those of a page at or past T, are
  // zeroed before anyone reads them.
#define MLA_ZERO_TAIL(q)                                                                          \
  do {                                                                                            \
    const int32_t zsl = s_slot[(q) % kPageBufs];                                                  \
    const int valid = mla_ok(mc, zsl) ? min(mla_llim(T - 1, j_begin + (q), tok_il, nsh, d) + 1, kMlaPage) : 0; \
    if (valid < kMlaPage) {                                                                       \
      uint8_t* zcur = s_raw[(q) % kPageBufs];                                                     \
      for (int i = tid; i < (kMlaPage - valid) * 36; i += kThreads) {                             \
        const int r = valid + i / 36, cc = i - (i / 36) * 36;                                     \
        *reinterpret_cast<u32x4*>(zcur + r * kRawStride + 16 * cc) = u32x4{0, 0, 0, 0};           \
      }                                                                                           \
      __syncthreads();                                                                            \
    }                                                                                             \
  } while (0)
  if (np > 0) {
    mla_fetch(mc, cp, 0, s_raw, s_scw, s_slot);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    MLA_ZERO_TAIL(0);
  }
  // The reference page scale the accumulator is in units of moves (with a rescale) when a
  // page's ratio to it leaves [1/4, 4]; scorers and accumulators follow the same sequence.

  if (scorer) {
    // ======== scores and numerators of row tile rt = wave, all 64 tokens of page t in step t
    const int rt = wave;
    // The lane's query row 16 rt + c of the block.  Latent dims 128 ks + 32 g + [0, 32) go to
    // the fp8 MFMA as two e4m3 terms (hi, lo) scaled per block of the instruction; rope dims
    // 512 + 32 ks + 8 g + [0, 8) go to the f16 MFMA scaled by 2^qe (largest |q| of the row in
    // [128, 256)).  The latent blocks' scale operands are relative to 2^qe, which is taken out
    // of the scores with the softmax scale.
    const int r_s = hb * kMlaRowsPerBlock + 16 * rt + c;
    const bool row_ok = r_s < p.rows;
    const int lim = row_ok ? T - p.q_len + r_s / p.hq : -1;  // last visible position (below T <= INT32_MAX)
    // fp8 path: latent terms and scales in qhi, qlo, qsc, rope in qrope.  Exact path: the fp16
    // query of step kk in half kk & 1 of qhi[kk / 2] (kk < 8) or qlo[(kk - 8) / 2] (kk < 16), or
    // in qrope[kk - 16].
    i32x8 qhi[kLatSteps], qlo[kLatSteps];
    int qsc[kLatSteps];  // scale operand (E8M0) of the hi term's block this lane supplies; lo: qsc - 4
    f16x8 qrope[kRopeSteps];
    float sl2;
    bool exact;  // this wavefront's rows take the exact (fp16) score path
    {
      const int t = row_ok ? r_s / p.hq : 0, h = row_ok ? r_s % p.hq : 0;
      const uint16_t* qr = static_cast<const uint16_t*>(p.q) + (((int64_t)b * p.q_len + t) * p.hq + h) * kMlaDim;
      u32x4 qraw[kQWords];
      float mx = 0.f, ss = 0.f;
      float mh[kLatSteps][2];  // largest |q| of the lane's first and second 16 latent dims per k-step
#pragma unroll
      for (int i = 0; i < kQWords; ++i) {
        const uint16_t* src = i < kLatSteps * 4 ? qr + 128 * (i >> 2) + 32 * g + 8 * (i & 3)
                                                : qr + kRope0 + 32 * (i - kLatSteps * 4) + 8 * g;
        const u32x4 w = row_ok ? *reinterpret_cast<const u32x4*>(src) : u32x4{0, 0, 0, 0};
        qraw[i] = w;
        float m8 = 0.f;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float lo = __builtin_bit_cast(float, w[e2] << 16), hi = __builtin_bit_cast(float, w[e2] & 0xFFFF0000u);
          m8 = fmaxf(m8, fmaxf(fabsf(lo), fabsf(hi)));
          ss = fmaf(lo, lo, fmaf(hi, hi, ss));
        }
        mx = fmaxf(mx, m8);
        if (i < kLatSteps * 4) {
          float& slot = mh[i >> 2][(i & 3) >> 1];
          slot = (i & 1) ? fmaxf(slot, m8) : m8;
        }
      }
      const float am = mgrp4_max(mx);
      const int qe = am > 0.f ? 7 - ilogbf(am) : 0;
      const bool outlier_row = am * am * (float)kMlaDim > kOutlier * kOutlier * mgrp4_sum(ss);
      exact = p.mla_scores == 2 || (p.mla_scores == 0 && __any(outlier_row));
      if (exact) {  // fp16 query over all 576 dims, lane (g, c): dims 32 kk + 8 g + [0, 8) of step kk
#pragma unroll
        for (int kk = 0; kk < kF16Steps; ++kk) {
          const u32x4 w = row_ok ? *reinterpret_cast<const u32x4*>(qr + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
          const f16x8 h = bf16x8_to_f16(w, qe);
          if (kk < 2 * kLatSteps) {
            qhi[kk >> 1] = (kk & 1) ? f16_pair(f16_half(qhi[kk >> 1], 0), h) : f16_pair(h, h);
          } else if (kk < 4 * kLatSteps) {
            const int j = (kk - 2 * kLatSteps) >> 1;
            qlo[j] = (kk & 1) ? f16_pair(f16_half(qlo[j], 0), h) : f16_pair(h, h);
          } else {
            qrope[kk - 4 * kLatSteps] = h;
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < (exact ? 0 : kLatSteps); ++ks) {
        // mf, ms: largest |q| of the blocks this lane's first and second halves belong to (each
        // shared with lane g ^ 1); mine: that of block g, whose scale operand this lane supplies
        // (lane 1 takes block 1, the first halves of lanes 2 and 3, from lane 2; lane 2 takes
        // block 2, the second halves of lanes 0 and 1, from lane 1)
        const float mf = fmaxf(mh[ks][0], __shfl_xor(mh[ks][0], 16, 64));
        const float ms = fmaxf(mh[ks][1], __shfl_xor(mh[ks][1], 16, 64));
        const float other = __shfl_xor(g == 2 ? mf : ms, 48, 64);  // lane 1 gets block 1, lane 2 block 2
        const float mine = g == 0 ? mf : (g == 3 ? ms : other);
        const int kf = mla_block_exp(mf, qe), ksec = mla_block_exp(ms, qe);
        qsc[ks] = 127 + qe - mla_block_exp(mine, qe);
        i32x8 hv, lv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // 8 dims per u32x4 -> two words of four e4m3 codes
          const u32x4 w = qraw[4 * ks + j];
          const int kx = j < 2 ? kf : ksec;
#pragma unroll
          for (int hw = 0; hw < 2; ++hw) {
            const float v[4] = {ldexpf(__builtin_bit_cast(float, w[2 * hw] << 16), kx),
                                ldexpf(__builtin_bit_cast(float, w[2 * hw] & 0xFFFF0000u), kx),
                                ldexpf(__builtin_bit_cast(float, w[2 * hw + 1] << 16), kx),
                                ldexpf(__builtin_bit_cast(float, w[2 * hw + 1] & 0xFFFF0000u), kx)};
            uint32_t hw32, lw32;
            split_e4m3(v, hw32, lw32);
            hv[2 * j + hw] = (int)hw32;
            lv[2 * j + hw] = (int)lw32;
          }
        }
        qhi[ks] = hv;
        qlo[ks] = lv;
      }
#pragma unroll
      for (int ks = 0; ks < (exact ? 0 : kRopeSteps); ++ks) qrope[ks] = bf16x8_to_f16(qraw[kLatSteps * 4 + ks], qe);
      sl2 = p.scale * kLog2eM / ldexpf(1.f, qe);
    }
    float ref_s = kNegInf;  // the row's exponent offset (log2 units), the same in its four lanes
    float l_s = 0.f;        // this lane's share of the row's denominator, in units of 2^ref_s
    float ps_ref = 1.f;
    for (int t = 0; t <= np; ++t) {
      if (t + 1 < np) mla_fetch(mc, cp, t + 1, s_raw, s_scw, s_slot);
      if (t < np) {
        const int bt_ = t % kPageBufs, jj = j_begin + t;
        const uint8_t* cur = s_raw[bt_];
        const int32_t sl = s_slot[bt_];
        const float ps = mla_scale(mc, sl, bt_, s_scw);
        const bool exists = mla_ok(mc, sl);
        ps_ref = mla_next_ref(ps, ps_ref);
        const float lrat = __builtin_amdgcn_logf(ps * __builtin_amdgcn_rcpf(ps_ref));  // log2 of the ratio
        // ---- S^T = K Q^T: tile 2 th + tt holds tokens 32 th + mla_tok(tt, m).  Per k-step the four
        // tiles' hi products go first, then their lo products, so no MFMA waits on the one
        // just before it.
        f32x4 sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (exact) {
#pragma unroll
          for (int kk = 0; kk < kF16Steps; ++kk) {
            const f16x8 bq = kk < 2 * kLatSteps ? f16_half(qhi[kk >> 1], kk & 1)
                             : kk < 4 * kLatSteps ? f16_half(qlo[(kk - 2 * kLatSteps) >> 1], kk & 1)
                                                  : qrope[kk - 4 * kLatSteps];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const f16x8 a = cvt8(*reinterpret_cast<const u32x2*>(
                  cur + (32 * (u >> 1) + mla_tok(u & 1, c)) * kRawStride + 32 * kk + 8 * g));
              sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq, sc[u], 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int ks = 0; ks < kLatSteps; ++ks) {
            i32x8 a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint8_t* kp = cur + (32 * (u >> 1) + mla_tok(u & 1, c)) * kRawStride + 128 * ks + 32 * g;
              const u32x4 a0 = *reinterpret_cast<const u32x4*>(kp);
              const u32x4 a1 = *reinterpret_cast<const u32x4*>(kp + 16);
              a[u] = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
              sc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[u], qhi[ks], sc[u], 0, 0, 0, 127, 0, qsc[ks]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
              sc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[u], qlo[ks], sc[u], 0, 0, 0, 127, 0,
                                                                       qsc[ks] - 4);
          }
#pragma unroll
          for (int ks = 0; ks < kRopeSteps; ++ks)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const f16x8 a = cvt8(*reinterpret_cast<const u32x2*>(
                  cur + (32 * (u >> 1) + mla_tok(u & 1, c)) * kRawStride + kRope0 + 32 * ks + 8 * g));
              sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qrope[ks], sc[u], 0, 0, 0);
            }
        }
        // ---- numerators (lane: row 16 rt + c, tokens 32 th + mla_vtok(g, [0, 8)) of each half)
        const float f = sl2 * ps;
        const bool full = exists && mla_llim(T - p.q_len, jj, tok_il, nsh, d) >= kMlaPage - 1;
        if (!full) {
          const int thr = exists ? mla_llim(lim, jj, tok_il, nsh, d) : -1;  // this row's last visible token
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (32 * (u >> 1) + mla_tok(u & 1, 4 * g + i) > thr) sc[u][i] = kNegInf;
        }
        float v_max = kNegInf;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) v_max = fmaxf(v_max, sc[u][i]);
        const float lane_max = v_max * f;
        if (__any(lane_max > ref_s + kTau)) {  // the offset moves only past the threshold
          const float m_row = mgrp4_max(lane_max);
          if (m_row > ref_s + kTau) {
            l_s *= ref_s == kNegInf ? 0.f : exp2f(ref_s - m_row);
            ref_s = m_row;
          }
        }
        const float off = ref_s == kNegInf ? 0.f : ref_s - lrat;  // -inf only while every score is masked
        float psum = 0.f;
#pragma unroll
        for (int th = 0; th < 2; ++th) {
          float x[8];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[4 * tt + i] = __builtin_amdgcn_exp2f(fmaf(sc[2 * th + tt][i], f, -off));
              psum += x[4 * tt + i];
            }
          s_p[t & 1][rt][th][lane] = f16x8{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3],
                                           (_Float16)x[4], (_Float16)x[5], (_Float16)x[6], (_Float16)x[7]};
        }
        l_s += psum * ps_ref * __builtin_amdgcn_rcpf(ps);  // P carries ps / ps_ref; the denominator not
        if (g == 0) s_off[t & 1][16 * rt + c] = ref_s;
      }
      // this step's LDS writes are done and page t + 1 has landed; then its tail, if any, is cleared.
      // The workgroup fences keep the compiler from moving LDS accesses across the barrier (the
      // explicit wait already covers what they would make the hardware wait for).
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (t + 1 < np) MLA_ZERO_TAIL(t + 1);
    }
    const float lh = mgrp4_sum(l_s);
    if (g == 0) s_l[16 * rt + c] = lh;
    __syncthreads();
  } else {
    // ======== O^T += V^T P^T for value dims [128 vw, 128 vw + 128) of all 64 rows, page t - 1 in step t
    const int vw = wave - kRowTiles;
    float ref[kRowTiles];  // offsets of rows 16 nt + c the accumulator is in units of
#pragma unroll
    for (int nt = 0; nt < kRowTiles; ++nt) ref[nt] = kNegInf;
    float ps_ref = 1.f;
    f32x4 o[kRowTiles][kVTiles];  // O^T tiles: dims 128 vw + 16 mt + 4 g + i of row 16 nt + c
#pragma unroll
    for (int nt = 0; nt < kRowTiles; ++nt)
#pragma unroll
      for (int mt = 0; mt < kVTiles; ++mt) o[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t <= np; ++t) {
      if (t + 1 < np) mla_fetch(mc, cp, t + 1, s_raw, s_scw, s_slot);
      if (t >= 1) {
        const int bv = (t - 1) % kPageBufs, pb = (t - 1) & 1;
        const uint8_t* cur = s_raw[bv];
        const float ps = mla_scale(mc, s_slot[bv], bv, s_scw);
        const float nps = mla_next_ref(ps, ps_ref);
        if (nps != ps_ref) {
          const float fo = ps_ref * __builtin_amdgcn_rcpf(nps);
#pragma unroll
          for (int nt = 0; nt < kRowTiles; ++nt)
#pragma unroll
            for (int mt = 0; mt < kVTiles; ++mt) scale_acc(o[nt][mt], fo);
          ps_ref = nps;
        }
        float nref[kRowTiles];
        bool mv = false;
#pragma unroll
        for (int nt = 0; nt < kRowTiles; ++nt) {
          nref[nt] = s_off[pb][16 * nt + c];
          mv = mv || nref[nt] != ref[nt];
        }
        if (__any(mv)) {
#pragma unroll
          for (int nt = 0; nt < kRowTiles; ++nt) {
            const float a = nref[nt] == ref[nt] ? 1.f : (ref[nt] == kNegInf ? 0.f : exp2f(ref[nt] - nref[nt]));
#pragma unroll
            for (int mt = 0; mt < kVTiles; ++mt) scale_acc(o[nt][mt], a);
            ref[nt] = nref[nt];
          }
        }
        // source lane (g, c) of the transposing read points at token 32 ks + mla_vtok(g, c >> 1),
        // dims 16 mt + 8 (c & 1) .. +7; lane (g, j) then holds dim 16 mt + j of those 8 tokens
        const uint8_t* vrow = cur + mla_vtok(g, c >> 1) * kRawStride + 8 * (c & 1) + kWaveDv * vw;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f16x8 pk[kRowTiles];
#pragma unroll
          for (int nt = 0; nt < kRowTiles; ++nt) pk[nt] = s_p[pb][nt][ks][lane];
#pragma unroll
          for (int mh = 0; mh < kVTiles; mh += 4) {
            i32x2 vx4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
              vx4[u] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (lds_i32x2*)(vrow + 32 * ks * kRawStride + 16 * (mh + u)));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const f16x8 a = cvt8(__builtin_bit_cast(u32x2, vx4[u]));
#pragma unroll
              for (int nt = 0; nt < kRowTiles; ++nt)
                o[nt][mh + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pk[nt], o[nt][mh + u], 0, 0, 0);
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (t + 1 < np) MLA_ZERO_TAIL(t + 1);
    }
    __syncthreads();  // the scorers' final denominators
    // ---- write the (chunk) partial of rows 16 nt + c, this wave's dims: O = ps_ref * O^T / l
    const bool direct = chk.out < 0;
    const int64_t pair_row0 = ((int64_t)d * p.batch + b) * p.rows;
    const int64_t ws_row0 = direct ? 0 : (int64_t)chk.out * p.rows;
#pragma unroll
    for (int nt = 0; nt < kRowTiles; ++nt) {
      const int r = hb * kMlaRowsPerBlock + 16 * nt + c;
      if (r >= p.rows) continue;
      const float lrow = s_l[16 * nt + c];
      float* dst = (direct ? p.partial_out + (pair_row0 + r) * kMlaDv : p.ws_o + (ws_row0 + r) * kMlaDv) +
                   kWaveDv * vw;
      const float inv = lrow > 0.f ? ps_ref / lrow : 0.f;
#pragma unroll
      for (int mt = 0; mt < kVTiles; ++mt) {
        const f32x4 v = o[nt][mt] * inv;
        *reinterpret_cast<float4*>(dst + 16 * mt + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g == 0 && vw == 0) {
        const float lse = lrow > 0.f ? (ref[nt] + log2f(lrow)) * kLn2M : kNegInf;
        if (direct)
          p.partial_lse[pair_row0 + r] = lse;
        else
          p.ws_lse[ws_row0 + r] = lse;
      }
    }
  }
#undef MLA_ZERO_TAIL
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
