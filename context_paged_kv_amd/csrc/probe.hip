// Measurement aid, not on the decode path: the matrix-core rate a kernel of
// back-to-back independent MFMAs reaches on this device, for the two
// instruction kinds the fp8 MLA kernel issues.  One workgroup of eight
// wavefronts per CU (two per SIMD, as in the MLA kernel); its shared-memory
// request keeps a second workgroup off the CU.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace dcpkv {

typedef _Float16 f16x8p __attribute__((ext_vector_type(8)));
typedef float f32x4p __attribute__((ext_vector_type(4)));
typedef int i32x8p __attribute__((ext_vector_type(8)));

constexpr int kProbeThreads = 512;
constexpr int kProbeChains = 8;  // independent accumulators per wavefront
constexpr int kProbeMaxGrid = 1024;
constexpr size_t kProbeLds = 96 * 1024;

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void mfma_rate_kernel(int iters, float* sink) {
  extern __shared__ float probe_lds[];
  const int lane = threadIdx.x & 63;
  f32x4p acc[kProbeChains];
#pragma unroll
  for (int u = 0; u < kProbeChains; ++u) acc[u] = f32x4p{0.f, 0.f, 0.f, 0.f};
  if (KIND == 0) {
    f16x8p a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (_Float16)(0.001f * (lane + i));
      b[i] = (_Float16)(0.002f * (lane - i));
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int u = 0; u < kProbeChains; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[u], 0, 0, 0);
  } else {
    i32x8p a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x30303030 + lane + i;  // small e4m3 codes
      b[i] = 0x28282828 + lane - i;
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int u = 0; u < kProbeChains; ++u)
        acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[u], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kProbeChains; ++u) s += acc[u][0] + acc[u][1] + acc[u][2] + acc[u][3];
  if (iters < 0) probe_lds[threadIdx.x] = s;  // never taken; keeps the request meaningful
  sink[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace dcpkv

using namespace dcpkv;

extern "C" int dcpkv_probe_mfma(int32_t kind, int32_t iters, float* sink, int64_t sink_floats, int64_t* out_flops,
                                void* stream) {
  if ((kind != 0 && kind != 1) || iters < 1 || !sink || !out_flops)
    return set_error(DCPKV_EINVAL, "probe_mfma: bad arguments (kind %d, iters %d)", kind, iters);
  if (sink_floats < (int64_t)kProbeMaxGrid * kProbeThreads)
    return set_error(DCPKV_EINVAL, "probe_mfma: sink holds %lld floats, needs %d", (long long)sink_floats,
                     kProbeMaxGrid * kProbeThreads);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return set_error(DCPKV_EDEVICE, "probe_mfma: no device");
  const int grid = std::min(cus, kProbeMaxGrid);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const void* fn = kind == 0 ? reinterpret_cast<const void*>(&mfma_rate_kernel<0>)
                             : reinterpret_cast<const void*>(&mfma_rate_kernel<1>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kProbeLds) != hipSuccess)
    return set_error(DCPKV_EDEVICE, "probe_mfma: cannot request %zu bytes of LDS", kProbeLds);
  if (kind == 0)
    hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(grid), dim3(kProbeThreads), kProbeLds, st, iters, sink);
  else
    hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(grid), dim3(kProbeThreads), kProbeLds, st, iters, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "probe_mfma: launch failed: %s", hipGetErrorString(e));
  const int64_t per_mfma = kind == 0 ? 2LL * 16 * 16 * 32 : 2LL * 16 * 16 * 128;
  *out_flops = (int64_t)grid * (kProbeThreads / 64) * (int64_t)iters * kProbeChains * per_mfma;
  return DCPKV_OK;
}

// ---------------------------------------------------------------------------
// Streaming copy: the copy ceiling the reshard is read against
// ---------------------------------------------------------------------------

namespace dcpkv {

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte loads in flight per thread
constexpr int kCopyBlocksPerCU = 2;

// A persistent grid over segments of kCopyThreads * kCopyUnroll chunks: every thread issues
// all of its non-temporal 16-byte loads before its stores (the reshard's segment loop over one
// contiguous range instead of a page list, in the geometry that streamed fastest in a sweep of
// loads per thread, threads per workgroup, workgroups per CU and cache hints).
__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4p* __restrict__ src,
                                                                   u32x4p* __restrict__ dst, int64_t chunks) {
  constexpr int64_t seg = (int64_t)kCopyThreads * kCopyUnroll;
  const int64_t items = (chunks + seg - 1) / seg;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t base = it * seg;
    const int64_t n = chunks - base < seg ? chunks - base : seg;
    if (n == seg) {  // straight-line: every load in flight before the first store
      u32x4p v[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u)
        v[u] = __builtin_nontemporal_load(src + base + u * kCopyThreads + threadIdx.x);
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u)
        __builtin_nontemporal_store(v[u], dst + base + u * kCopyThreads + threadIdx.x);
    } else {
      for (int64_t c = threadIdx.x; c < n; c += kCopyThreads)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + base + c), dst + base + c);
    }
  }
}

// The same segment loop over a page list: page src_pages[i] of src to page dst_pages[i] of dst,
// entries outside the buffers skipped.
__global__ __launch_bounds__(kCopyThreads) void page_copy_kernel(const u32x4p* __restrict__ src,
                                                                 u32x4p* __restrict__ dst,
                                                                 const int32_t* __restrict__ src_pages,
                                                                 const int32_t* __restrict__ dst_pages,
                                                                 int64_t num_pages, int64_t src_cap, int64_t dst_cap,
                                                                 int64_t page_chunks) {
  constexpr int64_t seg = (int64_t)kCopyThreads * kCopyUnroll;
  const int64_t per_page = (page_chunks + seg - 1) / seg;
  const int64_t items = num_pages * per_page;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t pg = it / per_page, off = (it - pg * per_page) * seg;
    const int64_t sp = src_pages[pg], dp = dst_pages[pg];
    if (sp < 0 || sp >= src_cap || dp < 0 || dp >= dst_cap) continue;
    const u32x4p* s = src + sp * page_chunks + off;
    u32x4p* d = dst + dp * page_chunks + off;
    const int64_t n = page_chunks - off < seg ? page_chunks - off : seg;
    if (n == seg) {
      u32x4p v[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(s + u * kCopyThreads + threadIdx.x);
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], d + u * kCopyThreads + threadIdx.x);
    } else {
      for (int64_t c = threadIdx.x; c < n; c += kCopyThreads)
        __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
    }
  }
}

static int probe_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *cus <= 0)
    return set_error(DCPKV_EDEVICE, "probe: no device");
  return DCPKV_OK;
}

}  // namespace dcpkv

extern "C" int dcpkv_probe_copy_pages(const void* src, void* dst, const int32_t* src_pages, const int32_t* dst_pages,
                                      int64_t num_pages, int64_t src_capacity, int64_t dst_capacity,
                                      int64_t page_bytes, void* stream) {
  if (num_pages < 0 || page_bytes < 16 || page_bytes % 16 || src_capacity < 1 || dst_capacity < 1)
    return set_error(DCPKV_EINVAL, "probe_copy_pages: bad sizes (%lld pages of %lld bytes)", (long long)num_pages,
                     (long long)page_bytes);
  if (num_pages == 0) return DCPKV_OK;
  if (!src || !dst || !src_pages || !dst_pages || !aligned16(src) || !aligned16(dst) ||
      (reinterpret_cast<uintptr_t>(src_pages) & 3u) || (reinterpret_cast<uintptr_t>(dst_pages) & 3u))
    return set_error(DCPKV_EINVAL, "probe_copy_pages: NULL or misaligned pointer");
  if (src_capacity > INT64_MAX / page_bytes || dst_capacity > INT64_MAX / page_bytes)
    return set_error(DCPKV_EINVAL, "probe_copy_pages: buffers too large");
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  if (s < d + dst_capacity * page_bytes && d < s + src_capacity * page_bytes)
    return set_error(DCPKV_EINVAL, "probe_copy_pages: source and destination overlap");
  int cus = 0;
  int rc = probe_cus(&cus);
  if (rc) return rc;
  const int64_t seg = (int64_t)kCopyThreads * kCopyUnroll, chunks = page_bytes / 16;
  const int64_t per_page = (chunks + seg - 1) / seg;
  if (num_pages > INT64_MAX / per_page) return set_error(DCPKV_EINVAL, "probe_copy_pages: too many pages");
  const int64_t grid = std::min<int64_t>(num_pages * per_page, (int64_t)cus * kCopyBlocksPerCU);
  hipLaunchKernelGGL(page_copy_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4p*>(src), static_cast<u32x4p*>(dst), src_pages, dst_pages, num_pages,
                     src_capacity, dst_capacity, chunks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "probe_copy_pages: launch failed: %s", hipGetErrorString(e));
  return DCPKV_OK;
}

extern "C" int dcpkv_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes < 16 || bytes % 16 || !aligned16(src) || !aligned16(dst))
    return set_error(DCPKV_EINVAL, "probe_copy: bad arguments (%lld bytes; 16-byte multiples and alignment)",
                     (long long)bytes);
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  if (s < d + bytes && d < s + bytes) return set_error(DCPKV_EINVAL, "probe_copy: source and destination overlap");
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return set_error(DCPKV_EDEVICE, "probe_copy: no device");
  const int64_t chunks = bytes / 16;
  const int64_t items = (chunks + (int64_t)kCopyThreads * kCopyUnroll - 1) / ((int64_t)kCopyThreads * kCopyUnroll);
  const int64_t grid = std::min<int64_t>(items, (int64_t)cus * kCopyBlocksPerCU);
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4p*>(src), static_cast<u32x4p*>(dst), chunks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(DCPKV_EDEVICE, "probe_copy: launch failed: %s", hipGetErrorString(e));
  return DCPKV_OK;
}
