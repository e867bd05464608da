// Host-side part of the library: error reporting, the layer split, the page
// index filter, the page map (free list + allocator) and block tables.
//
// [2DR] = "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding".

#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <utility>
#include <vector>

#include "common.h"

namespace dcpkv {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace dcpkv

using namespace dcpkv;

extern "C" const char* dcpkv_last_error(void) { return g_err; }

extern "C" int dcpkv_abi_version(void) { return 7; }

// [2DR] section 4.1: start_r = r*floor(L/N) + min(r, L mod N), end_r = start_{r+1}.
extern "C" int cp_layersplit_layer_range(int32_t num_layers, int32_t num_sources, int32_t r,
                                         int32_t* begin, int32_t* end) {
  if (!begin || !end) return set_error(DCPKV_EINVAL, "layer_range: NULL output");
  if (num_sources < 1 || num_layers < num_sources || r < 0 || r >= num_sources)
    return set_error(DCPKV_EINVAL, "layer_range: bad split L=%d N_cp=%d r=%d", num_layers,
                     num_sources, r);
  const int32_t base = num_layers / num_sources, extra = num_layers % num_sources;
  *begin = r * base + std::min(r, extra);
  *end = (r + 1) * base + std::min(r + 1, extra);
  return DCPKV_OK;
}

// [2DR] section 6.2: keep p with p mod N == d, compressed to floor(p / N).
extern "C" int dcp_filter_kv_indices(const int64_t* kv_indices, int64_t n, int32_t dcp_size,
                                     int32_t dcp_rank, int64_t* out_local, int64_t* out_count) {
  if (n < 0 || (n > 0 && (!kv_indices || !out_local)) || !out_count)
    return set_error(DCPKV_EINVAL, "filter: bad arguments");
  if (dcp_size > 1 && (dcp_rank < 0 || dcp_rank >= dcp_size))
    return set_error(DCPKV_EINVAL, "filter: rank %d outside [0, %d)", dcp_rank, dcp_size);
  int64_t k = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t p = kv_indices[i];
    if (p < 0) return set_error(DCPKV_EINVAL, "filter: negative page index at %lld", (long long)i);
    if (dcp_size <= 1) {
      out_local[k++] = p;
    } else if (p % dcp_size == dcp_rank) {
      out_local[k++] = p / dcp_size;
    }
  }
  *out_count = k;
  return DCPKV_OK;
}

// ---------------------------------------------------------------------------
// Page map ([2DR] sections 5.1 and 6.4)
// ---------------------------------------------------------------------------

struct dcp_pagemap {
  int32_t n;
  int32_t page_size;
  int64_t m;
  std::deque<int64_t> free_list;
  std::vector<uint8_t> used;  // per virtual page
};

extern "C" int dcp_pagemap_create(int32_t dcp_size, int32_t page_size, int64_t num_virtual_pages,
                                  const int64_t* free_order, dcp_pagemap** out) {
  if (!out) return set_error(DCPKV_EINVAL, "pagemap_create: NULL out");
  *out = nullptr;
  if (dcp_size < 1 || dcp_size > kMaxShards || page_size < 1 || num_virtual_pages < 1)
    return set_error(DCPKV_EINVAL, "pagemap_create: bad geometry N=%d page=%d M=%lld", dcp_size,
                     page_size, (long long)num_virtual_pages);
  dcp_pagemap* pm = new (std::nothrow) dcp_pagemap();
  if (!pm) return set_error(DCPKV_ENOMEM, "pagemap_create: out of host memory");
  try {
    pm->n = dcp_size;
    pm->page_size = page_size;
    pm->m = num_virtual_pages;
    pm->used.assign((size_t)num_virtual_pages, 0);
    std::vector<uint8_t> seen((size_t)num_virtual_pages, 0);
    for (int64_t i = 0; i < num_virtual_pages; ++i) {
      const int64_t v = free_order ? free_order[i] : i;
      if (v < 0 || v >= num_virtual_pages || seen[(size_t)v]) {
        delete pm;
        return set_error(DCPKV_EINVAL, "pagemap_create: free_order is not a permutation of [0, %lld)",
                         (long long)num_virtual_pages);
      }
      seen[(size_t)v] = 1;
      pm->free_list.push_back(v);
    }
  } catch (const std::bad_alloc&) {
    delete pm;
    return set_error(DCPKV_ENOMEM, "pagemap_create: out of host memory");
  }
  *out = pm;
  return DCPKV_OK;
}

extern "C" void dcp_pagemap_destroy(dcp_pagemap* pm) { delete pm; }

extern "C" int64_t dcp_pagemap_num_free(const dcp_pagemap* pm) {
  return pm ? (int64_t)pm->free_list.size() : -1;
}

extern "C" int dcp_pagemap_alloc(dcp_pagemap* pm, int64_t num_tokens, int64_t* out_global_pages,
                                 int64_t capacity) {
  if (!pm || !out_global_pages) return set_error(DCPKV_EINVAL, "pagemap_alloc: NULL argument");
  if (num_tokens < 1) return set_error(DCPKV_EINVAL, "pagemap_alloc: empty request");
  const int64_t pages = (num_tokens + pm->page_size - 1) / pm->page_size;
  const int64_t virt = (pages + pm->n - 1) / pm->n;
  if (capacity < pages)
    return set_error(DCPKV_EINVAL, "pagemap_alloc: capacity %lld < %lld pages", (long long)capacity,
                     (long long)pages);
  if (virt > (int64_t)pm->free_list.size())
    return set_error(DCPKV_ENOSPC, "pagemap_alloc: need %lld virtual pages, %zu free",
                     (long long)virt, pm->free_list.size());
  // virtual page k of the request covers sequence pages k*N .. k*N+N-1
  int64_t v = -1;
  for (int64_t i = 0; i < pages; ++i) {
    if (i % pm->n == 0) {
      v = pm->free_list.front();
      pm->free_list.pop_front();
      pm->used[(size_t)v] = 1;
    }
    out_global_pages[i] = v * pm->n + (i % pm->n);
  }
  return DCPKV_OK;
}

extern "C" int dcp_pagemap_release(dcp_pagemap* pm, const int64_t* global_pages, int64_t n) {
  if (!pm || (n > 0 && !global_pages) || n < 0)
    return set_error(DCPKV_EINVAL, "pagemap_release: bad arguments");
  std::vector<int64_t> vs;  // the distinct virtual pages, in first-seen order (that order is appended)
  try {
    vs.reserve((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
      const int64_t g = global_pages[i];
      if (g < 0 || g >= pm->m * pm->n)
        return set_error(DCPKV_EINVAL, "pagemap_release: page %lld out of range", (long long)g);
      vs.push_back(g / pm->n);
    }
    std::vector<int64_t> sorted = vs;
    std::sort(sorted.begin(), sorted.end());
    sorted.erase(std::unique(sorted.begin(), sorted.end()), sorted.end());
    std::vector<uint8_t> taken(sorted.size(), 0);
    size_t k = 0;
    for (size_t i = 0; i < vs.size(); ++i) {  // keep the first occurrence of each, in list order
      const size_t at = (size_t)(std::lower_bound(sorted.begin(), sorted.end(), vs[i]) - sorted.begin());
      if (!taken[at]) {
        taken[at] = 1;
        vs[k++] = vs[i];
      }
    }
    vs.resize(k);
  } catch (const std::bad_alloc&) {
    return set_error(DCPKV_ENOMEM, "pagemap_release: out of host memory");
  }
  for (int64_t v : vs)
    if (!pm->used[(size_t)v])
      return set_error(DCPKV_EINVAL, "pagemap_release: virtual page %lld is not allocated",
                       (long long)v);
  for (int64_t v : vs) {
    pm->used[(size_t)v] = 0;
    pm->free_list.push_back(v);
  }
  return DCPKV_OK;
}

extern "C" int dcp_build_block_tables(int32_t dcp_size, int32_t batch, const int64_t* global_pages,
                                      const int64_t* page_offsets, int32_t max_local_pages,
                                      int32_t token_interleave, int32_t* out_tables, int32_t* out_counts) {
  if (dcp_size < 1 || dcp_size > kMaxShards || batch < 0 || max_local_pages < 0 || !page_offsets ||
      !out_tables || (!global_pages && batch > 0 && page_offsets[batch] > 0) ||
      (token_interleave != DCPKV_OWN_PAGE && token_interleave != DCPKV_OWN_TOKEN))
    return set_error(DCPKV_EINVAL, "block_tables: bad arguments");
  const size_t total = (size_t)dcp_size * batch * max_local_pages;
  for (size_t i = 0; i < total; ++i) out_tables[i] = -1;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t a = page_offsets[b], e = page_offsets[b + 1];
    if (a < 0 || e < a) return set_error(DCPKV_EINVAL, "block_tables: bad offsets at %d", b);
    std::vector<int32_t> cnt(dcp_size, 0);
    for (int64_t i = a; i < e; ++i) {
      const int64_t g = global_pages[i];
      const int64_t seq_page = i - a;
      if (g < 0) return set_error(DCPKV_EINVAL, "block_tables: negative page id");
      const int32_t d = (int32_t)(g % dcp_size);
      if (d != (int32_t)(seq_page % dcp_size))
        return set_error(DCPKV_EINVAL,
                         "block_tables: request %d page %lld (id %lld) is not on rank %lld mod %d",
                         b, (long long)seq_page, (long long)g, (long long)seq_page, dcp_size);
      const int64_t slot = g / dcp_size;
      if (slot > INT32_MAX) return set_error(DCPKV_EINVAL, "block_tables: slot overflows int32");
      if (cnt[d] >= max_local_pages)
        return set_error(DCPKV_EINVAL, "block_tables: request %d needs more than %d local pages",
                         b, max_local_pages);
      if (!token_interleave) out_tables[((size_t)d * batch + b) * max_local_pages + cnt[d]] = (int32_t)slot;
      ++cnt[d];
    }
    if (token_interleave) {  // local page j of every shard sits at virtual page j's slot
      const int64_t nv = (e - a + dcp_size - 1) / dcp_size;
      if (nv > max_local_pages)
        return set_error(DCPKV_EINVAL, "block_tables: request %d needs more than %d local pages", b,
                         max_local_pages);
      // the N pages of virtual page j must share one slot: every shard reads its tokens of that
      // virtual page from the same slot
      for (int64_t i = a; i < e; ++i) {
        const int64_t head = a + ((i - a) / dcp_size) * dcp_size;
        if (global_pages[i] / dcp_size != global_pages[head] / dcp_size)
          return set_error(DCPKV_EINVAL,
                           "block_tables: request %d page %lld (id %lld) is not in the slot of virtual page %lld "
                           "(id %lld)", b, (long long)(i - a), (long long)global_pages[i],
                           (long long)((i - a) / dcp_size), (long long)global_pages[head]);
      }
      for (int32_t d = 0; d < dcp_size; ++d) {
        for (int64_t j = 0; j < nv; ++j)
          out_tables[((size_t)d * batch + b) * max_local_pages + j] = (int32_t)(global_pages[a + j * dcp_size] / dcp_size);
        cnt[d] = (int32_t)nv;
      }
    }
    if (out_counts)
      for (int32_t d = 0; d < dcp_size; ++d) out_counts[(size_t)d * batch + b] = cnt[d];
  }
  return DCPKV_OK;
}

// The reshard's precondition that no destination page is written twice in one call: the
// destination global pages of the uncached entries are pairwise distinct.
extern "C" int kv_check_unique_pages(const int64_t* dst_global_pages, int64_t num_pages, int64_t first_uncached,
                                     int64_t* out_first_duplicate) {
  if (num_pages < 0 || first_uncached < 0 || first_uncached > num_pages ||
      (num_pages > first_uncached && !dst_global_pages))
    return set_error(DCPKV_EINVAL, "check_unique: bad arguments");
  if (out_first_duplicate) *out_first_duplicate = -1;
  std::vector<std::pair<int64_t, int64_t>> v;  // (page, list position)
  try {
    v.reserve((size_t)(num_pages - first_uncached));
    for (int64_t i = first_uncached; i < num_pages; ++i) v.emplace_back(dst_global_pages[i], i);
  } catch (const std::bad_alloc&) {
    return set_error(DCPKV_ENOMEM, "check_unique: out of host memory");
  }
  std::sort(v.begin(), v.end());
  int64_t first = -1;  // the smallest list position whose page appeared earlier in the list
  for (size_t k = 1; k < v.size(); ++k)
    if (v[k].first == v[k - 1].first && (first < 0 || v[k].second < first)) first = v[k].second;
  if (first >= 0) {
    if (out_first_duplicate) *out_first_duplicate = first;
    return set_error(DCPKV_EINVAL, "check_unique: destination page %lld appears twice (again at entry %lld)",
                     (long long)dst_global_pages[first], (long long)first);
  }
  return DCPKV_OK;
}
