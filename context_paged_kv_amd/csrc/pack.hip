// Bounded pack / unpack of one (layer-split source r, DCP destination d)
// path of the page-level reshard.
//
// [2DR] = "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding"
//         (section 2: each path carries L_r x P_d pages; sections 6.2-6.3:
//         the destination page VALUE picks the rank, lists pair by position).
// [PR28] = the fivechenxi/sglang pull request #28 thread, the review of the
//         bounded-pack commit: a fixed-size, pre-registered pack buffer that is
//         reused in chunks when a transfer does not fit, instead of falling back
//         to many small non-contiguous transfers; it moves the same bytes.
//
// A path's units are (entry, layer) pairs, entry-major: unit u is layer
// begin_r + (u mod |L_r|) of the (u div |L_r|)-th entry of the path.  The
// entries are the list positions kv_path_entries selects (uncached, ids in
// range, owned by d), in list order.  kv_pack_pages gathers a window of units
// into a contiguous staging buffer, kv_unpack_pages scatters it into the
// destination pool; run over every window of every path they reproduce
// kv_reshard_pages byte for byte.
//
// The copies use the reshard's segment loop: near-equal segments of at most
// 36 KB per (unit, segment) item, every 16-byte non-temporal load of a thread
// in flight before its stores, a persistent grid striding over the items.  The
// entry count stays on the device (no host synchronisation); items past the
// window the count allows exit.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace dcpkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPathThreads = 1024;
constexpr int kPackThreads = 256;
constexpr int kPackUnroll = 9;
constexpr int64_t kPackSegMax = 16 * kPackThreads * kPackUnroll;  // 36864 bytes
constexpr int kPackBlocksPerCU = 4;

// ---------------------------------------------------------------------------
// Entries of a path: order-preserving compaction in one workgroup
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kPathThreads) void path_entries_kernel(const int32_t* __restrict__ src_ids,
                                                                    const int64_t* __restrict__ dst_ids,
                                                                    int64_t num_pages, int64_t first,
                                                                    int32_t n, int32_t dest, int64_t src_pages,
                                                                    int64_t dst_pages, int32_t* __restrict__ pos,
                                                                    int64_t* __restrict__ count) {
  __shared__ int s_wave[kPathThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t carry = 0;
  for (int64_t base = first; base < num_pages; base += kPathThreads) {
    const int64_t i = base + tid;
    bool take = false;
    if (i < num_pages) {
      const int64_t g = dst_ids[i];
      const int32_t sp = src_ids[i];
      const int64_t s = n > 1 ? g / n : g;
      const int d = n > 1 ? (int)(g % n) : 0;
      take = g >= 0 && s < dst_pages && sp >= 0 && sp < src_pages && d == dest;
    }
    const unsigned long long m = __ballot(take);
    const int below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kPathThreads / 64; ++w) {
      const int c = s_wave[w];
      before += w < wave ? c : 0;
      total += c;
    }
    if (take) pos[carry + before + below] = (int32_t)i;
    carry += total;
    __syncthreads();  // s_wave is rewritten by the next round
  }
  if (tid == 0) *count = carry;
}

// ---------------------------------------------------------------------------
// Pack (PACK = true) and unpack of a window of units
// ---------------------------------------------------------------------------

struct PackArgs {
  const uint8_t* src;      // pack: source pool r [|L_r|+1][S][page_bytes]; unpack: staging
  uint8_t* dst;            // pack: staging [cap][page_bytes]; unpack: destination pool d [L][M][page_bytes]
  const uint16_t* src_sc;  // scales, same roles (nullable together with dst_sc)
  uint16_t* dst_sc;
  const int32_t* src_ids;  // pack
  const int64_t* dst_ids;  // unpack
  const int32_t* pos;
  const int64_t* count;
  int64_t* out_units;      // pack, nullable
  int64_t page_bytes, seg_bytes, src_pages, dst_pages;
  int64_t unit_begin, cap;
  int32_t segs, nl, begin, n, dest;
};

template <bool PACK>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(PackArgs a) {
  // units of the window: n = min(cap, count * |L_r| - unit_begin), at least 0
  const int64_t total = *a.count * a.nl;
  const int64_t nw = std::max<int64_t>(0, std::min<int64_t>(a.cap, total - a.unit_begin));
  if (PACK && a.out_units && blockIdx.x == 0 && threadIdx.x == 0) *a.out_units = nw;
  const int64_t items = nw * a.segs;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t k = it / a.segs;
    const int sg = (int)(it - k * a.segs);
    const int64_t u = a.unit_begin + k;
    const int64_t j = u / a.nl;
    const int lr = (int)(u - j * a.nl);  // layer slot within source r
    const int32_t i = a.pos[j];
    int64_t src_page, dst_page;  // page indices of the two sides (in page_bytes units)
    if (PACK) {
      const int32_t sp = a.src_ids[i];
      if (sp < 0 || sp >= a.src_pages) continue;  // the entry list never holds these
      src_page = (int64_t)lr * a.src_pages + sp;
      dst_page = k;
    } else {
      const int64_t g = a.dst_ids[i];
      const int64_t s = a.n > 1 ? g / a.n : g;
      if (g < 0 || s >= a.dst_pages || (a.n > 1 && g % a.n != a.dest)) continue;
      src_page = k;
      dst_page = (int64_t)(a.begin + lr) * a.dst_pages + s;
    }
    const int64_t off = (int64_t)sg * a.seg_bytes;
    const u32x4* __restrict__ src = reinterpret_cast<const u32x4*>(a.src + src_page * a.page_bytes + off);
    u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(a.dst + dst_page * a.page_bytes + off);
    const int64_t len = std::min<int64_t>(a.page_bytes - off, a.seg_bytes);
    const int chunks = (int)(len >> 4);  // <= kPackThreads * kPackUnroll
    u32x4 v[kPackUnroll];
#pragma unroll
    for (int q = 0; q < kPackUnroll; ++q) {
      const int c = q * kPackThreads + threadIdx.x;
      if (c < chunks) v[q] = __builtin_nontemporal_load(src + c);
    }
#pragma unroll
    for (int q = 0; q < kPackUnroll; ++q) {
      const int c = q * kPackThreads + threadIdx.x;
      if (c < chunks) __builtin_nontemporal_store(v[q], dst + c);
    }
    if (a.src_sc && sg == 0 && threadIdx.x == 0) a.dst_sc[dst_page] = a.src_sc[src_page];
  }
}

static int device_cus_pack() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// Shared checks of the path calls; fills the geometry of source r.
static int check_path_desc(const kv_reshard_desc* desc, int32_t source, const char* who, int& begin, int& nl) {
  if (!desc) return set_error(DCPKV_EINVAL, "%s: NULL descriptor", who);
  const kv_reshard_desc& D = *desc;
  if (D.num_sources < 1 || D.num_sources > kMaxSources || D.num_layers < D.num_sources ||
      D.num_layers > kMaxLayers || D.dcp_size < 1 || D.dcp_size > kMaxShards || D.page_bytes <= 0 ||
      D.page_bytes % 16 != 0 || D.src_pages < 1 || D.dst_pages < 1)
    return set_error(DCPKV_EINVAL, "%s: bad descriptor (N_cp=%d L=%d N=%d page_bytes=%lld S=%lld M=%lld)", who,
                     D.num_sources, D.num_layers, D.dcp_size, (long long)D.page_bytes,
                     (long long)D.src_pages, (long long)D.dst_pages);
  if (source < 0 || source >= D.num_sources)
    return set_error(DCPKV_EINVAL, "%s: source %d outside [0, %d)", who, source, D.num_sources);
  const int base = D.num_layers / D.num_sources, extra = D.num_layers % D.num_sources;
  begin = source * base + std::min(source, extra);
  nl = base + (source < extra ? 1 : 0);
  return DCPKV_OK;
}

static void fill_segments(PackArgs& a, int64_t page_bytes) {
  const int64_t nseg = (page_bytes + kPackSegMax - 1) / kPackSegMax;
  a.seg_bytes = (((page_bytes + nseg - 1) / nseg + 15) / 16) * 16;
  a.segs = (int32_t)((page_bytes + a.seg_bytes - 1) / a.seg_bytes);
  a.page_bytes = page_bytes;
}

static int launch_pack(bool pack, const PackArgs& a, void* stream, const char* who) {
  const int64_t grid =
      std::max<int64_t>(1, std::min<int64_t>(a.cap * a.segs, (int64_t)device_cus_pack() * kPackBlocksPerCU));
  if (pack)
    hipLaunchKernelGGL(pack_kernel<true>, dim3((unsigned)grid), dim3(kPackThreads), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(pack_kernel<false>, dim3((unsigned)grid), dim3(kPackThreads), 0,
                       static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "%s: launch failed: %s", who, hipGetErrorString(e));
  return DCPKV_OK;
}

}  // namespace dcpkv

using namespace dcpkv;

extern "C" int kv_path_entries(const kv_reshard_desc* desc, int32_t dest, const int32_t* src_page_ids,
                               const int64_t* dst_global_pages, int64_t num_pages, int64_t first_uncached,
                               int32_t* out_positions, int64_t* out_count, void* stream) {
  int begin = 0, nl = 0;
  if (int rc = check_path_desc(desc, 0, "path entries", begin, nl)) return rc;
  const kv_reshard_desc& D = *desc;
  if (dest < 0 || dest >= D.dcp_size)
    return set_error(DCPKV_EINVAL, "path entries: destination %d outside [0, %d)", dest, D.dcp_size);
  if (num_pages < 0 || num_pages > INT32_MAX || first_uncached < 0 || first_uncached > num_pages)
    return set_error(DCPKV_EINVAL, "path entries: num_pages %lld / first_uncached %lld out of range",
                     (long long)num_pages, (long long)first_uncached);
  if (!out_count || (num_pages > first_uncached && (!src_page_ids || !dst_global_pages || !out_positions)))
    return set_error(DCPKV_EINVAL, "path entries: NULL array");
  hipLaunchKernelGGL(path_entries_kernel, dim3(1), dim3(kPathThreads), 0, static_cast<hipStream_t>(stream),
                     src_page_ids, dst_global_pages, num_pages, first_uncached, D.dcp_size, dest, D.src_pages,
                     D.dst_pages, out_positions, out_count);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "path entries: launch failed: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

extern "C" int kv_pack_pages(const kv_reshard_desc* desc, int32_t source, const void* src_pool,
                             const void* src_scales, const int32_t* src_page_ids, const int32_t* positions,
                             const int64_t* count, int64_t unit_begin, int64_t cap_units, void* staging,
                             void* staging_scales, int64_t* out_units, void* stream) {
  int begin = 0, nl = 0;
  if (int rc = check_path_desc(desc, source, "pack", begin, nl)) return rc;
  if (unit_begin < 0 || cap_units < 1)
    return set_error(DCPKV_EINVAL, "pack: unit_begin %lld < 0 or cap_units %lld < 1", (long long)unit_begin,
                     (long long)cap_units);
  if (!src_pool || !staging || !src_page_ids || !positions || !count)
    return set_error(DCPKV_EINVAL, "pack: NULL pointer");
  if (!aligned16(src_pool) || !aligned16(staging))
    return set_error(DCPKV_EINVAL, "pack: source pool and staging must be 16-byte aligned");
  if ((src_scales == nullptr) != (staging_scales == nullptr))
    return set_error(DCPKV_EINVAL, "pack: src_scales and staging_scales must both be set or NULL");
  PackArgs a = {};
  fill_segments(a, desc->page_bytes);
  a.src = static_cast<const uint8_t*>(src_pool);
  a.dst = static_cast<uint8_t*>(staging);
  a.src_sc = static_cast<const uint16_t*>(src_scales);
  a.dst_sc = static_cast<uint16_t*>(staging_scales);
  a.src_ids = src_page_ids;
  a.pos = positions;
  a.count = count;
  a.out_units = out_units;
  a.src_pages = desc->src_pages;
  a.dst_pages = desc->dst_pages;
  a.unit_begin = unit_begin;
  a.cap = cap_units;
  a.nl = nl;
  a.begin = begin;
  a.n = desc->dcp_size;
  return launch_pack(true, a, stream, "pack");
}

extern "C" int kv_unpack_pages(const kv_reshard_desc* desc, int32_t source, int32_t dest, void* dst_pool,
                               void* dst_scales, const int64_t* dst_global_pages, const int32_t* positions,
                               const int64_t* count, int64_t unit_begin, int64_t cap_units, const void* staging,
                               const void* staging_scales, void* stream) {
  int begin = 0, nl = 0;
  if (int rc = check_path_desc(desc, source, "unpack", begin, nl)) return rc;
  if (dest < 0 || dest >= desc->dcp_size)
    return set_error(DCPKV_EINVAL, "unpack: destination %d outside [0, %d)", dest, desc->dcp_size);
  if (unit_begin < 0 || cap_units < 1)
    return set_error(DCPKV_EINVAL, "unpack: unit_begin %lld < 0 or cap_units %lld < 1", (long long)unit_begin,
                     (long long)cap_units);
  if (!dst_pool || !staging || !dst_global_pages || !positions || !count)
    return set_error(DCPKV_EINVAL, "unpack: NULL pointer");
  if (!aligned16(dst_pool) || !aligned16(staging))
    return set_error(DCPKV_EINVAL, "unpack: destination pool and staging must be 16-byte aligned");
  if ((dst_scales == nullptr) != (staging_scales == nullptr))
    return set_error(DCPKV_EINVAL, "unpack: dst_scales and staging_scales must both be set or NULL");
  PackArgs a = {};
  fill_segments(a, desc->page_bytes);
  a.src = static_cast<const uint8_t*>(staging);
  a.dst = static_cast<uint8_t*>(dst_pool);
  a.src_sc = static_cast<const uint16_t*>(staging_scales);
  a.dst_sc = static_cast<uint16_t*>(dst_scales);
  a.dst_ids = dst_global_pages;
  a.pos = positions;
  a.count = count;
  a.src_pages = desc->src_pages;
  a.dst_pages = desc->dst_pages;
  a.unit_begin = unit_begin;
  a.cap = cap_units;
  a.nl = nl;
  a.begin = begin;
  a.n = desc->dcp_size;
  a.dest = dest;
  return launch_pack(false, a, stream, "unpack");
}
