// Page-level 2D reshard ([2DR] = "Serving Macaron-V1 at Scale: Page-Level
// 2D KV Resharding", sections 2, 4.1, 6.2-6.6).
//
// One launch moves one request's uncached pages over every (layer-split
// source r, DCP destination d) path.  The source-side filter of section 6.2
// is fused: the destination global page VALUE g picks the shard (g mod N) and
// the local slot (g div N), pairing with the source page id at the same list
// position (section 6.3).
//
// Work is split into items (layer, entry, segment): each page is cut into
// segments of 12-24 KB (a 256 KB bf16 GQA page into 16 of 16 KB, a 576-byte x
// 64-token fp8 page into 3 of 12 KB).  A persistent grid of two workgroups per
// CU strides over the items; every thread issues all of its 16-byte
// non-temporal loads for the segment (three to six) before its stores, in
// straight-line code, and the page ids of the workgroup's next item are read
// while the current one is in flight.  The side work per (layer, entry) --
// page scales, counts of bad entries and of pages per destination -- runs
// before the copy loop, spread over all threads.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <vector>

#include "common.h"

namespace dcpkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Division of a 32-bit n < 2^31 by a launch constant d >= 1 without a divide: with
// s = ceil(log2 d) and m = ceil(2^(32+s) / d), floor(n / d) = (n * m) >> (32 + s) exactly (the
// rounding error of m times n stays below 2^(31+s)).
struct FastDiv {
  uint64_t m;
  uint32_t s, d;
};
static FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const unsigned __int128 num = (unsigned __int128)1 << (32 + s);
  return FastDiv{(uint64_t)((num + d - 1) / d), s, d};
}
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((unsigned __int128)n * f.m) >> (32 + f.s));
}

struct ReshardArgs {
  const uint8_t* src[kMaxSources];
  uint8_t* dst[kMaxShards];
  const uint16_t* src_scale[kMaxSources];
  uint16_t* dst_scale[kMaxShards];
  const int32_t* src_ids;
  const int64_t* dst_ids;
  int32_t* bad;
  int64_t* per_dst;    // entries written per destination (nullable)
  int64_t page_bytes;
  int64_t seg_bytes;   // bytes per segment (a multiple of 16)
  int64_t src_pages;   // S
  int64_t dst_pages;   // M
  int64_t first;       // first uncached entry
  int64_t work;        // entries to move (num_pages - first)
  int64_t items;       // num_layers * work * segs
  int32_t segs;        // segments per page
  int32_t num_layers;
  int32_t num_sources;
  int32_t n;           // DCP size
  int32_t dst_filter;
  int32_t has_scales;
  FastDiv div_layer;   // by work * segs: item -> layer
  FastDiv div_seg;     // by segs: item within a layer -> entry
  FastDiv div_n;       // by n: global page -> slot
};

// Copy geometry, measured on MI355X over page-permuted copies and both page sizes of the
// workloads: two 256-thread workgroups per CU with three to five 16-byte loads per thread in
// flight (segments of 12-20 KB) stream better than deeper queues (nine loads, three or four
// workgroups: 2-5% slower) or one workgroup per CU (25% slower).
constexpr int kReshardThreads = 256;
constexpr int kReshardBlocksPerCU = 2;
constexpr int kReshardMaxUnroll = 6;

// Loads per thread for pages of page_bytes: four when 16 KB segments cut the page exactly (the
// fastest in the sweep; 256 KB pages), else the first of 6, 5 and 3 that does (36 KB pages: three
// segments of 12 KB, 5% faster than two of 18 KB with a partial round), else of 4, 5 and 6 the one
// whose near-equal segments leave the fewest lanes idle (ties to the smaller).
static int reshard_unroll(int64_t page_bytes) {
  for (int u : {4, 6, 5, 3})
    if (page_bytes % (16LL * kReshardThreads * u) == 0) return u;
  int best = 4;
  double best_fill = 0.0;
  for (int u = 4; u <= kReshardMaxUnroll; ++u) {
    const int64_t cap = 16LL * kReshardThreads * u;
    const int64_t nseg = (page_bytes + cap - 1) / cap;
    const double fill = (double)page_bytes / (double)(nseg * cap);
    if (fill > best_fill + 1e-9) {
      best_fill = fill;
      best = u;
    }
  }
  return best;
}

// One segment of `chunks` 16-byte chunks, every load issued before the first store.  A segment
// of the launch's full size (UF rounds of all threads, plus one round of the first `chunks mod
// 256` threads when PART) runs as straight-line code, so the compiler counts the loads in flight
// exactly instead of waiting for every earlier access before each store; the partial round's
// load is clamped into the segment and only its store is predicated.  A shorter segment (the
// last of a page) copies one chunk per thread at a time.  store(c, v) writes chunk c.
template <int UF, bool PART, typename Store, typename Between>
__device__ __forceinline__ void copy_segment(const u32x4* __restrict__ src, int chunks, int full_chunks,
                                             Store store, Between between) {
  const int t = threadIdx.x;
  if (chunks == full_chunks) {
    u32x4 v[UF > 0 ? UF : 1], x;
#pragma unroll
    for (int u = 0; u < UF; ++u) v[u] = __builtin_nontemporal_load(src + u * kReshardThreads + t);
    const int cx = UF * kReshardThreads + t;
    if (PART) x = __builtin_nontemporal_load(src + (cx < chunks ? cx : chunks - 1));
    between();  // while the loads are in flight
#pragma unroll
    for (int u = 0; u < UF; ++u) store(u * kReshardThreads + t, v[u]);
    if (PART && cx < chunks) store(cx, x);
  } else {
    between();
    for (int c = t; c < chunks; c += kReshardThreads) store(c, __builtin_nontemporal_load(src + c));
  }
}

// Owner of `layer` under the section 4.1 split, and the first layer it owns.
__device__ __forceinline__ void layer_owner(int layer, int num_layers, int num_sources, int& r,
                                            int& begin) {
  const int base = num_layers / num_sources, extra = num_layers % num_sources;
  const int big = extra * (base + 1);  // layers held by the sources with one extra layer
  if (layer < big) {
    r = layer / (base + 1);
    begin = r * (base + 1);
  } else {
    r = extra + (layer - big) / base;
    begin = r * base + extra;
  }
}

// Entry e of the list: source page id and destination global page.
struct ReshardEntry {
  int64_t g;
  int32_t sp;
};

// The entry of item `it`, clamped into range instead of branched on, and with divisions by
// launch constants, so the loop around it has no data-dependent branch.  (Reading the entries
// with scalar loads instead, so that the next segment's loads need not wait for the previous
// segment's stores, measured 1-3% slower: the wait keeps fewer bytes in flight per CU, which
// this memory system prefers.)
__device__ __forceinline__ ReshardEntry reshard_entry(const ReshardArgs& a, uint32_t it) {
  const uint32_t itc = it < (uint32_t)a.items ? it : (uint32_t)a.items - 1;
  const uint32_t layer = fdiv(itc, a.div_layer);
  const uint32_t e = fdiv(itc - layer * a.div_layer.d, a.div_seg);
  const int64_t* gp = a.dst_ids + a.first + e;
  const int32_t* sp = a.src_ids + a.first + e;
  return ReshardEntry{*gp, *sp};
}

// Destination shard and slot of global page g, and whether the entry is copied at all (page ids
// are below 2^31: the host limits M * N).
__device__ __forceinline__ bool reshard_target(const ReshardArgs& a, int64_t g, int32_t sp, int& d, int64_t& s) {
  const bool in = g >= 0 && g < (int64_t)a.dst_pages * a.n && sp >= 0 && sp < a.src_pages;
  const uint32_t g32 = in ? (uint32_t)g : 0u;
  const uint32_t q = a.n > 1 ? fdiv(g32, a.div_n) : g32;
  d = (int)(g32 - q * (uint32_t)a.n);
  s = q;
  return in;
}

template <int UF, bool PART>
__global__ __launch_bounds__(kReshardThreads) void reshard_kernel(ReshardArgs a) {
  // The per-(layer, entry) side work first, spread over all threads: the page scales, the count
  // of entries out of range and the per-destination page counts.  The copy loop below then
  // holds no per-lane memory access, so the compiler keeps its loads and stores overlapped.
  if (a.has_scales || a.bad || a.per_dst) {
    const int64_t pairs = (int64_t)a.num_layers * a.work;
    for (int64_t q = (int64_t)blockIdx.x * kReshardThreads + threadIdx.x; q < pairs;
         q += (int64_t)gridDim.x * kReshardThreads) {
      const int layer = (int)(q / a.work);
      const int64_t e = q - (int64_t)layer * a.work;
      const int64_t g = a.dst_ids[a.first + e];
      const int32_t sp = a.src_ids[a.first + e];
      int d;
      int64_t s;
      if (!reshard_target(a, g, sp, d, s)) {
        if (a.bad) atomicAdd(a.bad, 1);
        continue;
      }
      if (a.dst_filter >= 0 && d != a.dst_filter) continue;
      if (a.per_dst && layer == 0) atomicAdd((unsigned long long*)&a.per_dst[d], 1ull);
      if (a.has_scales) {
        int r, begin;
        layer_owner(layer, a.num_layers, a.num_sources, r, begin);
        a.dst_scale[d][(int64_t)layer * a.dst_pages + s] = a.src_scale[r][(int64_t)(layer - begin) * a.src_pages + sp];
      }
    }
  }
  ReshardEntry en = reshard_entry(a, blockIdx.x);
  for (uint32_t it = blockIdx.x; it < (uint32_t)a.items; it += gridDim.x) {
    const uint32_t layer = fdiv(it, a.div_layer);
    const uint32_t rest = it - layer * a.div_layer.d;
    const uint32_t e = fdiv(rest, a.div_seg);
    const int sg = (int)(rest - e * (uint32_t)a.segs);
    const ReshardEntry cur = en;
    int d;
    int64_t s;
    const uint32_t nxt = it + gridDim.x;
    if (!reshard_target(a, cur.g, cur.sp, d, s) || (a.dst_filter >= 0 && d != a.dst_filter)) {
      en = reshard_entry(a, nxt);
      continue;
    }
    int r, begin;
    layer_owner((int)layer, a.num_layers, a.num_sources, r, begin);
    const int64_t off = (int64_t)sg * a.seg_bytes;
    const int64_t src_off = ((int64_t)((int)layer - begin) * a.src_pages + cur.sp) * a.page_bytes + off;
    const int64_t dst_off = ((int64_t)layer * a.dst_pages + s) * a.page_bytes + off;
    const u32x4* __restrict__ src = reinterpret_cast<const u32x4*>(a.src[r] + src_off);
    u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(a.dst[d] + dst_off);
    const int64_t len = (a.page_bytes - off) < a.seg_bytes ? (a.page_bytes - off) : a.seg_bytes;
    copy_segment<UF, PART>(src, (int)(len >> 4), (int)(a.seg_bytes >> 4),
                           [dst](int c, const u32x4& v) { __builtin_nontemporal_store(v, dst + c); },
                           [&]() { en = reshard_entry(a, nxt); });
  }
}

// ---------------------------------------------------------------------------
// Token scatter under token ownership ([SGL]: token t on shard t mod N)
// ---------------------------------------------------------------------------

struct TokenReshardArgs {
  const uint8_t* src[kMaxSources];
  uint8_t* dst[kMaxShards];
  const int32_t* src_ids;
  const int64_t* dst_ids;
  const int64_t* req_off;  // request b owns list entries [req_off[b], req_off[b+1]); NULL: one request
  int32_t* bad;
  int64_t page_bytes, seg_bytes, src_pages, dst_pages, first, work, items, num_pages;
  int32_t segs, num_layers, num_sources, n, page_size, row_bytes, num_req;
  int32_t row16, block16;  // 16-byte chunks per token row and per block (page_size rows)
  float r_row16, r_block16, r_n;  // their reciprocals and 1 / n, for the quotients below
};

// floor(a / b) for 0 <= a < 2^22 and b >= 1 from a float reciprocal: the product is within
// 1/2 of a / b, so one correction step makes it exact.
__device__ __forceinline__ int small_div(int a, int b, float rb) {
  int q = (int)((float)a * rb);
  const int r = a - q * b;
  q += (r >= b ? 1 : 0) - (r < 0 ? 1 : 0);
  return q;
}

// First list entry of the request that holds entry i (i < num_pages), or -1 when the offsets
// name no request that contains i (offsets out of order or out of range).
__device__ __forceinline__ int64_t token_request_base(const TokenReshardArgs& a, int64_t i) {
  if (!a.req_off) return 0;
  int lo = 0, hi = a.num_req - 1;
  while (lo < hi) {  // last request whose first entry is <= i
    const int mid = (lo + hi + 1) >> 1;
    if (a.req_off[mid] <= i)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int64_t b0 = a.req_off[lo], b1 = a.req_off[lo + 1];
  return (b0 >= 0 && b0 <= i && i < b1 && b1 <= a.num_pages) ? b0 : -1;
}

// Item (layer, list entry i, segment): entry i is sequence page k = i - o of the request whose
// entries start at o.  The page's tokens x land on shard (k*P + x) mod N as local token
// u = (k*P + x) div N, row u mod P of the request's virtual page k div N, whose slot is
// g_{o + (k div N) N} div N on every shard.  A page is token_rows blocks of P rows of row_bytes;
// token x is row x of each block, and so is its destination row.
template <int UF, bool PART>
__global__ __launch_bounds__(kReshardThreads) void reshard_tokens_kernel(TokenReshardArgs a) {
  // the destination pools' base addresses, indexed per lane below, from LDS
  __shared__ uint8_t* s_dst[kMaxShards];
  if ((int)threadIdx.x < a.n) s_dst[threadIdx.x] = a.dst[threadIdx.x];
  __syncthreads();
  const int64_t per_layer = a.work * a.segs;
  for (int64_t it = blockIdx.x; it < a.items; it += gridDim.x) {
    const int layer = (int)(it / per_layer);
    const int64_t rest = it - (int64_t)layer * per_layer;
    const int64_t i = a.first + rest / a.segs;
    const int sg = (int)(rest % a.segs);
    const int32_t sp = a.src_ids[i];
    const int64_t o = token_request_base(a, i);
    const int64_t k = i - o;  // sequence page within the request (o >= 0 keeps o + (k/N)*N in [o, i])
    const int64_t g = o >= 0 ? a.dst_ids[o + (k / a.n) * a.n] : -1;
    const int64_t slot = a.n > 1 ? g / a.n : g;
    if (o < 0 || sp < 0 || sp >= a.src_pages || g < 0 || slot >= a.dst_pages) {
      if (sg == 0 && threadIdx.x == 0 && a.bad) atomicAdd(a.bad, 1);
      continue;
    }
    int r, begin;
    layer_owner(layer, a.num_layers, a.num_sources, r, begin);
    const int64_t off0 = (int64_t)sg * a.seg_bytes;
    const uint8_t* src = a.src[r] + ((int64_t)(layer - begin) * a.src_pages + sp) * a.page_bytes;
    const int64_t dst_page = ((int64_t)layer * a.dst_pages + slot) * a.page_bytes;
    const int64_t len = (a.page_bytes - off0) < a.seg_bytes ? (a.page_bytes - off0) : a.seg_bytes;
    const int chunks = (int)(len >> 4);
    // token t = k * page_size + x of the page goes to shard t mod n, row (t div n) mod page_size;
    // with t0 = k * page_size = u0 * n + d0 that is shard (d0 + x) mod n, row
    // (u0 + (d0 + x) div n) mod page_size
    const int64_t t0 = k * a.page_size;
    const int d0 = (int)(t0 % a.n);
    const int y0 = (int)((t0 / a.n) % a.page_size);
    const int c0 = (int)(off0 >> 4);  // first 16-byte chunk of the segment in the page
    uint8_t* const* dsts = s_dst;
    copy_segment<UF, PART>(reinterpret_cast<const u32x4*>(src + off0), chunks, (int)(a.seg_bytes >> 4),
                           [&a, dsts, dst_page, c0, d0, y0](int c, const u32x4& v) {
      const int ci = c0 + c;  // chunk in the page: block, token row, chunk within the row
      const int blk = small_div(ci, a.block16, a.r_block16), rem = ci - blk * a.block16;
      const int x = small_div(rem, a.row16, a.r_row16), cr = rem - x * a.row16;
      const int sx = d0 + x, dq = small_div(sx, a.n, a.r_n);
      const int d = sx - dq * a.n;
      const int y = y0 + dq >= a.page_size ? y0 + dq - a.page_size : y0 + dq;
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4*>(dsts[d] + dst_page) + ((int64_t)blk * a.page_size + y) * a.row16 + cr);
    }, []() {});
  }
}

// DCPKV_CHECK_PRECONDITIONS=1: the reshard calls copy the destination page list to the host
// (synchronising the caller's stream) and refuse a list that names a page twice.
static bool check_preconditions() {
  const char* e = std::getenv("DCPKV_CHECK_PRECONDITIONS");
  return e && e[0] == '1';
}

static int check_unique_on_device(const int64_t* dst_ids, int64_t num_pages, int64_t first, void* stream,
                                  const char* who) {
  std::vector<int64_t> h((size_t)num_pages);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(h.data(), dst_ids, (size_t)num_pages * sizeof(int64_t), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return set_error(DCPKV_EDEVICE, "%s: copying the page list for the precondition check failed", who);
  int64_t dup = -1;
  if (kv_check_unique_pages(h.data(), num_pages, first, &dup) != DCPKV_OK)
    return set_error(DCPKV_EINVAL, "%s: destination page %lld appears twice (again at entry %lld)", who,
                     (long long)h[(size_t)dup], (long long)dup);
  return DCPKV_OK;
}

// Launch KERNEL<UF, PART> for full segments of SEG_CHUNKS chunks: UF = SEG_CHUNKS / 256 whole
// rounds (at most kReshardMaxUnroll) and PART when a partial round is left.
#define DCPKV_SEGMENT_DISPATCH(KERNEL, SEG_CHUNKS, GRID, ST, ARGS)                                     \
  do {                                                                                              \
    const int uf_ = (int)((SEG_CHUNKS) / kReshardThreads);                                          \
    const bool part_ = ((SEG_CHUNKS) % kReshardThreads) != 0;                                       \
    const dim3 g_((unsigned)(GRID)), b_(kReshardThreads);                                           \
    switch (uf_ * 2 + (part_ ? 1 : 0)) {                                                            \
      case 1: hipLaunchKernelGGL((KERNEL<0, true>), g_, b_, 0, ST, ARGS); break;                    \
      case 2: hipLaunchKernelGGL((KERNEL<1, false>), g_, b_, 0, ST, ARGS); break;                   \
      case 3: hipLaunchKernelGGL((KERNEL<1, true>), g_, b_, 0, ST, ARGS); break;                    \
      case 4: hipLaunchKernelGGL((KERNEL<2, false>), g_, b_, 0, ST, ARGS); break;                   \
      case 5: hipLaunchKernelGGL((KERNEL<2, true>), g_, b_, 0, ST, ARGS); break;                    \
      case 6: hipLaunchKernelGGL((KERNEL<3, false>), g_, b_, 0, ST, ARGS); break;                   \
      case 7: hipLaunchKernelGGL((KERNEL<3, true>), g_, b_, 0, ST, ARGS); break;                    \
      case 8: hipLaunchKernelGGL((KERNEL<4, false>), g_, b_, 0, ST, ARGS); break;                   \
      case 9: hipLaunchKernelGGL((KERNEL<4, true>), g_, b_, 0, ST, ARGS); break;                    \
      case 10: hipLaunchKernelGGL((KERNEL<5, false>), g_, b_, 0, ST, ARGS); break;                  \
      case 11: hipLaunchKernelGGL((KERNEL<5, true>), g_, b_, 0, ST, ARGS); break;                   \
      default: hipLaunchKernelGGL((KERNEL<6, false>), g_, b_, 0, ST, ARGS); break;                  \
    }                                                                                               \
  } while (0)

static int device_cus_reshard() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

}  // namespace dcpkv

using namespace dcpkv;

extern "C" int kv_reshard_pages(const kv_reshard_desc* desc, const void* const* src_pools,
                                void* const* dst_pools, const void* const* src_scales,
                                void* const* dst_scales, const int32_t* src_page_ids,
                                const int64_t* dst_global_pages, int64_t num_pages,
                                int64_t first_uncached, int32_t* bad_entries, int64_t* pages_per_dst,
                                void* stream) {
  if (!desc || !src_pools || !dst_pools) return set_error(DCPKV_EINVAL, "reshard: NULL argument");
  const kv_reshard_desc& D = *desc;
  if (D.num_sources < 1 || D.num_sources > kMaxSources || D.num_layers < D.num_sources ||
      D.num_layers > kMaxLayers || D.dcp_size < 1 || D.dcp_size > kMaxShards ||
      D.dst_filter < -1 || D.dst_filter >= D.dcp_size || D.page_bytes <= 0 ||
      D.page_bytes % 16 != 0 || D.src_pages < 1 || D.dst_pages < 1)
    return set_error(DCPKV_EINVAL,
                     "reshard: bad descriptor (N_cp=%d L=%d N=%d filter=%d page_bytes=%lld S=%lld "
                     "M=%lld)",
                     D.num_sources, D.num_layers, D.dcp_size, D.dst_filter,
                     (long long)D.page_bytes, (long long)D.src_pages, (long long)D.dst_pages);
  if (num_pages < 0 || first_uncached < 0 || first_uncached > num_pages)
    return set_error(DCPKV_EINVAL, "reshard: first_uncached %lld outside [0, %lld]",
                     (long long)first_uncached, (long long)num_pages);
  if ((src_scales == nullptr) != (dst_scales == nullptr))
    return set_error(DCPKV_EINVAL, "reshard: src_scales and dst_scales must both be set or NULL");
  const int64_t work = num_pages - first_uncached;
  if (work == 0) return DCPKV_OK;
  if (!src_page_ids || !dst_global_pages)
    return set_error(DCPKV_EINVAL, "reshard: NULL page id arrays");
  if (pages_per_dst && (reinterpret_cast<uintptr_t>(pages_per_dst) & 7u))
    return set_error(DCPKV_EINVAL, "reshard: pages_per_dst must be 8-byte aligned");
  if (check_preconditions()) {
    const int rc = check_unique_on_device(dst_global_pages, num_pages, first_uncached, stream, "reshard");
    if (rc) return rc;
  }
  ReshardArgs a = {};
  for (int r = 0; r < D.num_sources; ++r) {
    if (!src_pools[r] || !aligned16(src_pools[r]))
      return set_error(DCPKV_EINVAL, "reshard: source pool %d is NULL or not 16-byte aligned", r);
    a.src[r] = static_cast<const uint8_t*>(src_pools[r]);
    if (src_scales) {
      if (!src_scales[r]) return set_error(DCPKV_EINVAL, "reshard: source scale %d is NULL", r);
      a.src_scale[r] = static_cast<const uint16_t*>(src_scales[r]);
    }
  }
  for (int d = 0; d < D.dcp_size; ++d) {
    if (!dst_pools[d] || !aligned16(dst_pools[d]))
      return set_error(DCPKV_EINVAL, "reshard: destination pool %d is NULL or not 16-byte aligned",
                       d);
    a.dst[d] = static_cast<uint8_t*>(dst_pools[d]);
    if (dst_scales) {
      if (!dst_scales[d]) return set_error(DCPKV_EINVAL, "reshard: destination scale %d is NULL", d);
      a.dst_scale[d] = static_cast<uint16_t*>(dst_scales[d]);
    }
  }
  a.src_ids = src_page_ids;
  a.dst_ids = dst_global_pages;
  a.bad = bad_entries;
  a.per_dst = pages_per_dst;
  a.page_bytes = D.page_bytes;
  const int unroll = reshard_unroll(D.page_bytes);
  {  // near-equal segments of at most 16 * 256 * unroll bytes, 16-byte multiples, covering the page
    const int64_t seg_max = 16LL * kReshardThreads * unroll;
    const int64_t nseg = (D.page_bytes + seg_max - 1) / seg_max;
    a.seg_bytes = (((D.page_bytes + nseg - 1) / nseg + 15) / 16) * 16;
    a.segs = (int32_t)((D.page_bytes + a.seg_bytes - 1) / a.seg_bytes);
  }
  a.src_pages = D.src_pages;
  a.dst_pages = D.dst_pages;
  a.first = first_uncached;
  a.work = work;
  a.items = (int64_t)D.num_layers * work * a.segs;
  if (a.items + (int64_t)device_cus_reshard() * kReshardBlocksPerCU >= (1LL << 31) ||
      D.dst_pages * D.dcp_size >= (1LL << 31) || D.src_pages >= (1LL << 31))
    return set_error(DCPKV_EINVAL, "reshard: %lld (layer, page, segment) items or %lld destination pages per layer "
                     "(limit 2^31)", (long long)a.items, (long long)(D.dst_pages * D.dcp_size));
  a.div_layer = make_fastdiv((uint32_t)(work * a.segs));
  a.div_seg = make_fastdiv((uint32_t)a.segs);
  a.div_n = make_fastdiv((uint32_t)D.dcp_size);
  a.num_layers = D.num_layers;
  a.num_sources = D.num_sources;
  a.n = D.dcp_size;
  a.dst_filter = D.dst_filter;
  a.has_scales = src_scales != nullptr;
  const int64_t grid = std::min<int64_t>(a.items, (int64_t)device_cus_reshard() * kReshardBlocksPerCU);
  hipStream_t st = static_cast<hipStream_t>(stream);
  DCPKV_SEGMENT_DISPATCH(reshard_kernel, a.seg_bytes >> 4, grid, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "reshard: launch failed: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

extern "C" int kv_reshard_tokens(const kv_token_reshard_desc* desc, const void* const* src_pools,
                                 void* const* dst_pools, const int32_t* src_page_ids,
                                 const int64_t* dst_global_pages, int64_t num_pages,
                                 const int64_t* request_offsets, int32_t num_requests, int64_t first_uncached,
                                 int32_t* bad_entries, void* stream) {
  if (!desc || !src_pools || !dst_pools) return set_error(DCPKV_EINVAL, "token reshard: NULL argument");
  const kv_token_reshard_desc& D = *desc;
  const int64_t page_bytes = (int64_t)D.token_rows * D.page_size * D.row_bytes;
  if (D.num_sources < 1 || D.num_sources > kMaxSources || D.num_layers < D.num_sources ||
      D.num_layers > kMaxLayers || D.dcp_size < 1 || D.dcp_size > kMaxShards || D.page_size < 1 ||
      D.token_rows < 1 || D.row_bytes < 16 || D.row_bytes % 16 != 0 || page_bytes >= (1LL << 26) ||
      D.src_pages < 1 || D.dst_pages < 1)
    return set_error(DCPKV_EINVAL,
                     "token reshard: bad descriptor (N_cp=%d L=%d N=%d page=%d rows=%d row_bytes=%d S=%lld M=%lld)",
                     D.num_sources, D.num_layers, D.dcp_size, D.page_size, D.token_rows, D.row_bytes,
                     (long long)D.src_pages, (long long)D.dst_pages);
  if (num_pages < 0 || first_uncached < 0 || first_uncached > num_pages)
    return set_error(DCPKV_EINVAL, "token reshard: first_uncached %lld outside [0, %lld]",
                     (long long)first_uncached, (long long)num_pages);
  if (num_requests < 0 || (num_requests > 1 && !request_offsets) || (request_offsets && num_requests < 1))
    return set_error(DCPKV_EINVAL, "token reshard: %d requests with%s request_offsets", num_requests,
                     request_offsets ? "" : "out");
  const int64_t work = num_pages - first_uncached;
  if (work == 0) return DCPKV_OK;
  if (!src_page_ids || !dst_global_pages) return set_error(DCPKV_EINVAL, "token reshard: NULL page id arrays");
  if (check_preconditions()) {
    const int rc = check_unique_on_device(dst_global_pages, num_pages, first_uncached, stream, "token reshard");
    if (rc) return rc;
  }
  TokenReshardArgs a = {};
  a.req_off = request_offsets;
  a.num_req = request_offsets ? num_requests : 1;
  a.num_pages = num_pages;
  for (int r = 0; r < D.num_sources; ++r) {
    if (!src_pools[r] || !aligned16(src_pools[r]))
      return set_error(DCPKV_EINVAL, "token reshard: source pool %d is NULL or not 16-byte aligned", r);
    a.src[r] = static_cast<const uint8_t*>(src_pools[r]);
  }
  for (int d = 0; d < D.dcp_size; ++d) {
    if (!dst_pools[d] || !aligned16(dst_pools[d]))
      return set_error(DCPKV_EINVAL, "token reshard: destination pool %d is NULL or not 16-byte aligned", d);
    a.dst[d] = static_cast<uint8_t*>(dst_pools[d]);
  }
  a.src_ids = src_page_ids;
  a.dst_ids = dst_global_pages;
  a.bad = bad_entries;
  a.page_bytes = page_bytes;
  const int unroll = reshard_unroll(page_bytes);
  {
    const int64_t seg_max = 16LL * kReshardThreads * unroll;
    const int64_t nseg = (page_bytes + seg_max - 1) / seg_max;
    a.seg_bytes = (((page_bytes + nseg - 1) / nseg + 15) / 16) * 16;
    a.segs = (int32_t)((page_bytes + a.seg_bytes - 1) / a.seg_bytes);
  }
  a.src_pages = D.src_pages;
  a.dst_pages = D.dst_pages;
  a.first = first_uncached;
  a.work = work;
  a.items = (int64_t)D.num_layers * work * a.segs;
  a.num_layers = D.num_layers;
  a.num_sources = D.num_sources;
  a.n = D.dcp_size;
  a.page_size = D.page_size;
  a.row_bytes = D.row_bytes;
  a.row16 = D.row_bytes / 16;
  a.block16 = D.page_size * a.row16;
  a.r_row16 = 1.0f / (float)a.row16;
  a.r_block16 = 1.0f / (float)a.block16;
  a.r_n = 1.0f / (float)D.dcp_size;
  const int64_t grid = std::min<int64_t>(a.items, (int64_t)device_cus_reshard() * kReshardBlocksPerCU);
  hipStream_t st = static_cast<hipStream_t>(stream);
  DCPKV_SEGMENT_DISPATCH(reshard_tokens_kernel, a.seg_bytes >> 4, grid, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "token reshard: launch failed: %s", hipGetErrorString(e));
  return DCPKV_OK;
}
