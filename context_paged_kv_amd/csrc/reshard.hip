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
// near-equal segments of at most 36 KB (a whole 576-byte x 64-token fp8 page
// is one segment).  A persistent grid strides over the items; every thread
// issues all of its 16-byte non-temporal loads for the segment (up to nine)
// before its stores, and the page ids of the workgroup's next item are read
// while the current one is in flight, so neither the id lookup nor the data
// latency is exposed per item.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <vector>

#include "common.h"

namespace dcpkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
};

constexpr int kReshardThreads = 256;
constexpr int kReshardUnroll = 9;                                          // 16-byte loads per thread
constexpr int64_t kReshardSegMax = 16 * kReshardThreads * kReshardUnroll;  // 36864 bytes
#ifndef RESHARD_BLOCKS_PER_CU
#define RESHARD_BLOCKS_PER_CU 4
#endif
constexpr int kReshardBlocksPerCU = RESHARD_BLOCKS_PER_CU;

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

// Entry e of the list: source page id and destination global page (plain loads; the
// compiler turns them into scalar loads since every lane reads the same word).
struct ReshardEntry {
  int64_t g;
  int32_t sp;
};
__device__ __forceinline__ ReshardEntry reshard_entry(const ReshardArgs& a, int64_t it) {
  ReshardEntry en{-1, -1};
  if (it < a.items) {
    const int64_t e = (it % (a.work * a.segs)) / a.segs;
    en.g = a.dst_ids[a.first + e];
    en.sp = a.src_ids[a.first + e];
  }
  return en;
}

__global__ __launch_bounds__(kReshardThreads) void reshard_kernel(ReshardArgs a) {
  const int64_t per_layer = a.work * a.segs;
  ReshardEntry en = reshard_entry(a, blockIdx.x);
  for (int64_t it = blockIdx.x; it < a.items; it += gridDim.x) {
    const ReshardEntry nx = reshard_entry(a, it + gridDim.x);  // in flight during this copy
    const int layer = (int)(it / per_layer);
    const int64_t rest = it - (int64_t)layer * per_layer;
    const int sg = (int)(rest % a.segs);
    const int64_t g = en.g;
    const int32_t sp = en.sp;
    en = nx;
    int d;
    int64_t s;
    if (a.n > 1) {
      d = (int)(g % a.n);
      s = g / a.n;
    } else {
      d = 0;
      s = g;
    }
    const bool ok = g >= 0 && s < a.dst_pages && sp >= 0 && sp < a.src_pages;
    if (!ok) {
      if (sg == 0 && threadIdx.x == 0 && a.bad) atomicAdd(a.bad, 1);
      continue;
    }
    if (a.dst_filter >= 0 && d != a.dst_filter) continue;
    if (a.per_dst && layer == 0 && sg == 0 && threadIdx.x == 0) atomicAdd((unsigned long long*)&a.per_dst[d], 1ull);
    int r, begin;
    layer_owner(layer, a.num_layers, a.num_sources, r, begin);
    const int64_t off = (int64_t)sg * a.seg_bytes;
    const int64_t src_off = ((int64_t)(layer - begin) * a.src_pages + sp) * a.page_bytes + off;
    const int64_t dst_off = ((int64_t)layer * a.dst_pages + s) * a.page_bytes + off;
    const u32x4* __restrict__ src = reinterpret_cast<const u32x4*>(a.src[r] + src_off);
    u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(a.dst[d] + dst_off);
    const int64_t len = (a.page_bytes - off) < a.seg_bytes ? (a.page_bytes - off) : a.seg_bytes;
    const int chunks = (int)(len >> 4);  // <= kReshardThreads * kReshardUnroll
    u32x4 v[kReshardUnroll];
#pragma unroll
    for (int u = 0; u < kReshardUnroll; ++u) {
      const int c = u * kReshardThreads + threadIdx.x;
      if (c < chunks) v[u] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int u = 0; u < kReshardUnroll; ++u) {
      const int c = u * kReshardThreads + threadIdx.x;
      if (c < chunks) __builtin_nontemporal_store(v[u], dst + c);
    }
    if (a.has_scales && sg == 0 && threadIdx.x == 0) {
      a.dst_scale[d][(int64_t)layer * a.dst_pages + s] =
          a.src_scale[r][(int64_t)(layer - begin) * a.src_pages + sp];
    }
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
    u32x4 v[kReshardUnroll];
#pragma unroll
    for (int q = 0; q < kReshardUnroll; ++q) {
      const int c = q * kReshardThreads + threadIdx.x;
      if (c < chunks) v[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off0) + c);
    }
#pragma unroll
    for (int q = 0; q < kReshardUnroll; ++q) {
      const int c = q * kReshardThreads + threadIdx.x;
      if (c < chunks) {
        const int ci = c0 + c;  // chunk in the page: block, token row, chunk within the row
        const int blk = small_div(ci, a.block16, a.r_block16), rem = ci - blk * a.block16;
        const int x = small_div(rem, a.row16, a.r_row16), cr = rem - x * a.row16;
        const int sx = d0 + x, dq = small_div(sx, a.n, a.r_n);
        const int d = sx - dq * a.n;
        const int y = y0 + dq >= a.page_size ? y0 + dq - a.page_size : y0 + dq;
        __builtin_nontemporal_store(
            v[q], reinterpret_cast<u32x4*>(s_dst[d] + dst_page) + ((int64_t)blk * a.page_size + y) * a.row16 + cr);
      }
    }
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
  {  // near-equal segments of at most 36 KB, 16-byte multiples, covering the page exactly
    const int64_t nseg = (D.page_bytes + kReshardSegMax - 1) / kReshardSegMax;
    a.seg_bytes = (((D.page_bytes + nseg - 1) / nseg + 15) / 16) * 16;
    a.segs = (int32_t)((D.page_bytes + a.seg_bytes - 1) / a.seg_bytes);
  }
  a.src_pages = D.src_pages;
  a.dst_pages = D.dst_pages;
  a.first = first_uncached;
  a.work = work;
  a.items = (int64_t)D.num_layers * work * a.segs;
  a.num_layers = D.num_layers;
  a.num_sources = D.num_sources;
  a.n = D.dcp_size;
  a.dst_filter = D.dst_filter;
  a.has_scales = src_scales != nullptr;
  const int64_t grid = std::min<int64_t>(a.items, (int64_t)device_cus_reshard() * kReshardBlocksPerCU);
  hipLaunchKernelGGL(reshard_kernel, dim3((unsigned)grid), dim3(kReshardThreads), 0,
                     static_cast<hipStream_t>(stream), a);
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
  {
    const int64_t nseg = (page_bytes + kReshardSegMax - 1) / kReshardSegMax;
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
  hipLaunchKernelGGL(reshard_tokens_kernel, dim3((unsigned)grid), dim3(kReshardThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "token reshard: launch failed: %s", hipGetErrorString(e));
  return DCPKV_OK;
}
