/*
 * dcpkv.h -- C ABI of the Decode Context Parallelism (DCP) paged-KV library
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (cited by short name):
 *   [2DR]  "Serving Macaron-V1 at Scale: Page-Level 2D KV Resharding"
 *   [SGL]  "SGLang's path" (serving-k3, module 05, the DCP paragraph)
 *   [PR28] the fivechenxi/sglang pull request #28 thread (the bounded-pack
 *          review and the address-translation comment)
 *
 * Conventions shared by every entry point
 *   - Status: 0 (DCPKV_OK) on success, a negative errno-style code on error.
 *     Argument errors are detected on the host before anything is enqueued;
 *     dcpkv_last_error() then returns a thread-local description.
 *   - Device calls enqueue work on the caller's stream (a hipStream_t passed as
 *     void*, NULL = the default stream) and return without waiting.  A failed
 *     launch returns DCPKV_EDEVICE.  Faults surface at the caller's next
 *     synchronisation.
 *   - Memory: the caller owns every buffer (device pointers unless marked
 *     "host").  Device calls never allocate; scratch space is the caller's
 *     workspace.  The library owns only dcp_pagemap objects.
 *   - Page contents are opaque bytes to the reshard.  Attention reads pages in
 *     one of two layouts, both contiguous per (layer, page):
 *       SPLIT: [2 (K, V)][num_kv_heads][page_size][head_dim], f32 or bf16
 *       MLA:   [page_size][576] fp8 e4m3fn (512 latent + 64 rope), with one
 *              bf16 scale per (layer, page) in a separate array.
 *   - A DCP pool is [num_layers][pages_per_layer][page_bytes]; local slot s of
 *     layer l lives at byte offset (l * pages_per_layer + s) * page_bytes.
 *   - Not thread-safe per object; distinct objects/streams may be used from
 *     distinct threads.
 */
#ifndef DCPKV_H
#define DCPKV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DCPKV_API __attribute__((visibility("default")))
#else
#define DCPKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DCPKV_OK = 0,
  DCPKV_EDEVICE = -5,   /* a HIP call or kernel launch failed */
  DCPKV_ENOMEM = -12,   /* host allocation failed */
  DCPKV_EINVAL = -22,   /* bad argument */
  DCPKV_ENOSPC = -28,   /* page map exhausted */
  DCPKV_ENOTSUP = -95   /* valid request this build does not implement */
};

enum { DCPKV_KV_F32 = 0, DCPKV_KV_BF16 = 1, DCPKV_KV_FP8E4M3 = 2 };
enum { DCPKV_LAYOUT_SPLIT = 0, DCPKV_LAYOUT_MLA = 1 };
enum { DCPKV_Q_F32 = 0, DCPKV_Q_BF16 = 1 };
/* Which shard holds a token: its page's owner (page p on rank p mod N, [2DR]
 * section 5.1) or the token's own residue (token t on rank t mod N, [SGL]). */
enum { DCPKV_OWN_PAGE = 0, DCPKV_OWN_TOKEN = 1 };

/* Thread-local text describing the last non-OK status returned on this thread. */
DCPKV_API const char* dcpkv_last_error(void);

/* ABI version of this header (bumped on any signature change). */
DCPKV_API int dcpkv_abi_version(void);

/* ------------------------------------------------------------------------ *
 * Host-side geometry helpers                                                *
 * ------------------------------------------------------------------------ */

/* [2DR] section 4.1, layer-assignment equation.  Half-open range
 * [*begin, *end) of layers owned by layer-split source r out of num_sources:
 * floor(L / N_cp) layers each, the first (L mod N_cp) sources one more.
 * EINVAL if num_layers < num_sources, num_sources < 1 or r out of range. */
DCPKV_API int cp_layersplit_layer_range(int32_t num_layers, int32_t num_sources, int32_t r,
                              int32_t* begin, int32_t* end);

/* [2DR] section 6.2, page index filter.  Writes to out_local (host, capacity
 * n) the local slots floor(p / N) of the pages p in kv_indices (host, n) with
 * p mod N == dcp_rank, in input order, and their count to *out_count.  With
 * dcp_size <= 1 the list is copied unchanged.  EINVAL on a negative index, a
 * rank outside [0, N) or NULL pointers. */
DCPKV_API int dcp_filter_kv_indices(const int64_t* kv_indices, int64_t n, int32_t dcp_size,
                          int32_t dcp_rank, int64_t* out_local, int64_t* out_count);

/* ------------------------------------------------------------------------ *
 * Page map: free list and allocator ([2DR] sections 5.1 and 6.4)           *
 * ------------------------------------------------------------------------ */

typedef struct dcp_pagemap dcp_pagemap;

/* An allocator of num_virtual_pages virtual pages (M), each covering
 * page_size * dcp_size tokens: virtual page v is global pages v*N .. v*N+N-1,
 * i.e. local slot v on every DCP rank (owner(p) = p mod N, slot = p div N).
 * free_order (host, nullable): a permutation of [0, M) giving the initial
 * free-list order (NULL = ascending).  The free list is FIFO: allocation
 * takes from the front, release appends to the back.
 * EINVAL on bad geometry or a free_order that is not a permutation;
 * ENOMEM if the host object cannot be allocated. */
DCPKV_API int dcp_pagemap_create(int32_t dcp_size, int32_t page_size, int64_t num_virtual_pages,
                       const int64_t* free_order, dcp_pagemap** out);
DCPKV_API void dcp_pagemap_destroy(dcp_pagemap* pm);

/* Virtual pages currently on the free list (-1 if pm is NULL). */
DCPKV_API int64_t dcp_pagemap_num_free(const dcp_pagemap* pm);

/* Allocate a request of num_tokens (>= 1) tokens: P = ceil(T / page_size)
 * pages from ceil(P / N) virtual pages v_0, v_1, ...; sequence page i gets
 * global page v_{i div N} * N + (i mod N), so it lands on rank i mod N.
 * Writes P ids to out_global_pages (host, capacity >= P).
 * ENOSPC (and nothing allocated) if the free list is too short. */
DCPKV_API int dcp_pagemap_alloc(dcp_pagemap* pm, int64_t num_tokens, int64_t* out_global_pages,
                      int64_t capacity);

/* Return the virtual pages behind a request's global pages (host, n) to the
 * back of the free list.  EINVAL (nothing released) on an id out of range or
 * a virtual page that is not allocated (double free). */
DCPKV_API int dcp_pagemap_release(dcp_pagemap* pm, const int64_t* global_pages, int64_t n);

/* Per-shard block tables for a batch ([2DR] section 5.1).  Request b's
 * global pages are global_pages[page_offsets[b] .. page_offsets[b+1]) (host).
 * out_tables (host, int32 [N][batch][max_local_pages]) receives, for shard d
 * and request b, the local slots of its local pages in order; unused entries
 * are -1.  out_counts (host, int32 [N][batch], nullable) receives the number
 * of entries per (d, b).  Requires the allocator's canonical placement:
 * sequence page i must be owned by rank i mod N (EINVAL otherwise), so that
 * virtual page j of the request is slot v_j = g_{jN} div N on every rank.
 *   token_interleave = DCPKV_OWN_PAGE: shard d's local page j is sequence page
 *     j*N + d (the pages d owns, in sequence order);
 *   token_interleave = DCPKV_OWN_TOKEN ([SGL]: token t on rank t mod N): local
 *     page j of every shard holds that shard's tokens of virtual page j, so every
 *     shard lists v_0 .. v_{ceil(P/N)-1}; the N pages of virtual page j must
 *     share its slot (g_{jN+d} div N == g_{jN} div N), EINVAL otherwise.
 * EINVAL if a count exceeds max_local_pages or token_interleave is neither. */
DCPKV_API int dcp_build_block_tables(int32_t dcp_size, int32_t batch, const int64_t* global_pages,
                           const int64_t* page_offsets, int32_t max_local_pages, int32_t token_interleave,
                           int32_t* out_tables, int32_t* out_counts);

/* ------------------------------------------------------------------------ *
 * (1) Page-level 2D reshard ([2DR] sections 2, 4.1, 6.2-6.6)               *
 * ------------------------------------------------------------------------ */

typedef struct {
  int32_t num_sources;  /* N_cp layer-split sources, >= 1 */
  int32_t num_layers;   /* L, >= num_sources */
  int32_t dcp_size;     /* N destination pools, >= 1 */
  int32_t dst_filter;   /* -1: every destination; d: only pages owned by d */
  int64_t page_bytes;   /* bytes per (layer, page); a multiple of 16 */
  int64_t src_pages;    /* S: page slots per layer slot in each source pool */
  int64_t dst_pages;    /* M: local page slots per layer in each destination */
} kv_reshard_desc;

/* One transfer of one request's pages over every (source r, destination d)
 * path at once.  Source r holds the contiguous layer range of
 * cp_layersplit_layer_range (section 4.1) in a pool of (|L_r| + 1) layer slots
 * x S pages x page_bytes; the extra slot is the transient broadcast slot and is
 * never read.  Destination d is a DCP pool [L][M][page_bytes].
 *
 * The i-th entry pairs source page src_page_ids[i] with destination global page
 * dst_global_pages[i] (pairing by position).  Ownership is decided by the
 * destination VALUE: d = g mod N, slot s = g div N (section 6.3); with N == 1
 * the slot is g.  For every layer l (from its owner r) and every
 * i in [first_uncached, num_pages):
 *     dst[d][l][s] = src[r][l - begin_r][src_page_ids[i]]     (page_bytes bytes)
 * Entries before first_uncached are prefix-cached: neither read nor written.
 * No CP-side filtering happens under layer split (section 6.6).
 *
 * src_pools (host array [N_cp] of device pointers), dst_pools (host array [N]).
 * src_scales / dst_scales (both NULL or both set): host arrays of device
 * pointers to bf16 per-page scales, [|L_r|+1][S] and [L][M]; each scale moves
 * with its page.  src_page_ids: device int32 [num_pages]; dst_global_pages:
 * device int64 [num_pages].  Destination global pages must be unique within a
 * call (each (layer, page) then has one writer).
 * bad_entries (device int32 [1], nullable): incremented by one for each
 * (layer, entry) whose ids fall outside [0, S) or [0, M*N); such entries are
 * skipped, never written.
 * pages_per_dst (device int64 [N], nullable, 8-byte aligned): pages_per_dst[d]
 * is incremented by the number of entries written to destination d (each on
 * every layer), the per-destination page count of the transfer worker's
 * "pages: 256 -> 64" log line (section 6.3); the caller zeroes it first.
 * Pointers must be 16-byte aligned.
 * With the environment variable DCPKV_CHECK_PRECONDITIONS=1 the call first
 * copies dst_global_pages to the host (synchronising `stream`) and returns
 * EINVAL, writing nothing, if a page repeats among the uncached entries.
 * EINVAL on a bad descriptor, NULL pool pointers, page_bytes % 16 != 0,
 * first_uncached outside [0, num_pages] or misaligned pointers. */
DCPKV_API int kv_reshard_pages(const kv_reshard_desc* desc, const void* const* src_pools,
                     void* const* dst_pools, const void* const* src_scales,
                     void* const* dst_scales, const int32_t* src_page_ids,
                     const int64_t* dst_global_pages, int64_t num_pages,
                     int64_t first_uncached, int32_t* bad_entries, int64_t* pages_per_dst,
                     void* stream);

/* The reshard's one-writer precondition, on the host: the destination global
 * pages dst_global_pages[first_uncached .. num_pages) (host) are pairwise
 * distinct, so every (layer, destination page) of a call has one writer
 * ([2DR] section 6.2, the guarantee that each rank's pages are written once).
 * Returns OK, or EINVAL with *out_first_duplicate (host, nullable) set to the
 * first list position whose page appeared earlier (-1 when none).  EINVAL also
 * on bad sizes or a NULL list. */
DCPKV_API int kv_check_unique_pages(const int64_t* dst_global_pages, int64_t num_pages,
                                    int64_t first_uncached, int64_t* out_first_duplicate);

/* ------------------------------------------------------------------------ *
 * (1c) Token scatter reshard for pools under token ownership                *
 *      ([2DR] section 2 per path; [SGL]: token t on rank t mod N)           *
 * ------------------------------------------------------------------------ */

typedef struct {
  int32_t num_sources;  /* N_cp layer-split sources, >= 1 */
  int32_t num_layers;   /* L, >= num_sources */
  int32_t dcp_size;     /* N destination pools, >= 1 */
  int32_t page_size;    /* tokens per page */
  int32_t token_rows;   /* R: a page is R blocks of page_size rows (SPLIT: 2 * Hkv; MLA: 1) */
  int32_t row_bytes;    /* bytes per row, a multiple of 16 (SPLIT: head_dim * elem; MLA: 576);
                           a page (token_rows * page_size * row_bytes) is below 64 MiB */
  int64_t src_pages;    /* S: page slots per layer slot in each source pool */
  int64_t dst_pages;    /* M: local page slots per layer in each destination */
} kv_token_reshard_desc;

/* A batch of requests' transfers into pools that hold tokens under token
 * ownership (DCPKV_OWN_TOKEN), in one launch.  The lists concatenate the
 * requests: request b owns entries [request_offsets[b], request_offsets[b+1])
 * (device int64 [num_requests + 1], non-decreasing, from 0 to num_pages), and
 * its entry i is its sequence page k = i - request_offsets[b]: source page
 * src_page_ids[i] (device int32) and global page dst_global_pages[i] (device
 * int64, the allocator's canonical placement).  request_offsets == NULL with
 * num_requests <= 1 is one request over the whole list.  For every layer l
 * (from its owner r, as in kv_reshard_pages), every entry i in
 * [first_uncached, num_pages) and every token x < page_size of its page, with
 * t = k*page_size + x the token's position in its request:
 *     d = t mod N,  u = t div N,
 *     slot = g_{o_b + (k div N) N} div N        (N == 1: g_i)
 *     dst[d][l][slot] row (u mod page_size) of block b'  =  src[r][l - begin_r]
 *         [src_page_ids[i]] row x of block b',   for every block b' < token_rows
 * i.e. a source page's tokens land on every shard, in its request's virtual
 * page k div N.  Whole uncached pages move, tail rows included.  first_uncached
 * counts list entries, as in kv_reshard_pages.  Page scales cannot follow
 * tokens that leave their page, so this call takes no scales (pools with
 * per-page fp8 scales under token ownership are out of its scope).
 * bad_entries (device int32 [1], nullable): incremented once per (layer, entry)
 * whose source id is outside [0, S), whose virtual page slot is outside
 * [0, M), or that no request of request_offsets contains consistently; such
 * entries are skipped.  Every access stays in bounds whatever the id arrays
 * and offsets hold.  DCPKV_CHECK_PRECONDITIONS=1 checks the destination pages
 * for repeats first, as in kv_reshard_pages.  EINVAL on a bad descriptor, NULL or misaligned pools,
 * first_uncached outside [0, num_pages], num_requests < 0, num_requests > 1
 * without offsets, or offsets with num_requests < 1. */
DCPKV_API int kv_reshard_tokens(const kv_token_reshard_desc* desc, const void* const* src_pools,
                      void* const* dst_pools, const int32_t* src_page_ids, const int64_t* dst_global_pages,
                      int64_t num_pages, const int64_t* request_offsets, int32_t num_requests,
                      int64_t first_uncached, int32_t* bad_entries, void* stream);

/* ------------------------------------------------------------------------ *
 * (1b) Bounded pack / unpack of one (source, destination) path              *
 *      ([2DR] section 2: a path carries L_r x P_d pages; sections 6.2-6.3:   *
 *      ownership by destination page value; [PR28]: a fixed-size pack       *
 *      buffer reused in chunks when a transfer does not fit)                 *
 * ------------------------------------------------------------------------ */

/* Entries of the path to destination `dest`: the list positions
 * i in [first_uncached, num_pages) whose ids are in range (src_page_ids[i] in
 * [0, S), g = dst_global_pages[i] in [0, M*N)) and whose owner is dest
 * (g mod N == dest; with N == 1 every entry), in list order.  Writes them to
 * out_positions (device int32, capacity num_pages - first_uncached) and their
 * number to out_count (device int64 [1]).  desc gives N, S and M (its
 * dst_filter is ignored).  One workgroup reads each list once.
 * EINVAL on a bad descriptor, dest outside [0, N), num_pages > INT32_MAX,
 * first_uncached outside [0, num_pages] or NULL arrays. */
DCPKV_API int kv_path_entries(const kv_reshard_desc* desc, int32_t dest, const int32_t* src_page_ids,
                    const int64_t* dst_global_pages, int64_t num_pages, int64_t first_uncached,
                    int32_t* out_positions, int64_t* out_count, void* stream);

/* The path (source r, destination d) carries count * |L_r| units, count being
 * the out_count of kv_path_entries (read on the device; no host wait).  Unit u
 * is layer l_u = begin_r + (u mod |L_r|) of entry i_u = positions[u div |L_r|]
 * (entry-major: one page's layers are consecutive).  kv_pack_pages copies the
 * window of n = min(cap_units, count * |L_r| - unit_begin) units (none if that
 * is negative) starting at unit_begin into a contiguous staging buffer:
 *     staging[k] = src_pool[l_u - begin_r][src_page_ids[i_u]]   (page_bytes bytes)
 *     staging_scales[k] = src_scales[l_u - begin_r][src_page_ids[i_u]]
 * for k = u - unit_begin, and writes n to out_units (device int64 [1],
 * nullable).  src_pool is source r's pool [|L_r|+1][S][page_bytes] (device),
 * src_scales its bf16 scales [|L_r|+1][S] or NULL (then staging_scales must
 * be NULL too).  staging holds cap_units pages (16-byte aligned),
 * staging_scales cap_units bf16 values.  A caller packs windows
 * unit_begin = 0, cap, 2 cap, ... until the unit count (read back once, or
 * known on the host) is covered; the staging buffer is reused per window.
 * EINVAL on a bad descriptor, source outside [0, N_cp), unit_begin < 0,
 * cap_units < 1, NULL or misaligned pointers, scales given on one side only. */
DCPKV_API int kv_pack_pages(const kv_reshard_desc* desc, int32_t source, const void* src_pool,
                  const void* src_scales, const int32_t* src_page_ids, const int32_t* positions,
                  const int64_t* count, int64_t unit_begin, int64_t cap_units, void* staging,
                  void* staging_scales, int64_t* out_units, void* stream);

/* The destination side of the same window:
 *     dst_pool[l_u][g div N] = staging[k],   g = dst_global_pages[i_u]  (N == 1: slot g)
 *     dst_scales[l_u][g div N] = staging_scales[k]
 * dst_pool is destination `dest`'s pool [L][M][page_bytes], dst_scales its
 * [L][M] bf16 scales or NULL (with staging_scales NULL).  Run over every window
 * of every path (r, d), pack + unpack write exactly what kv_reshard_pages
 * writes, byte for byte.  Errors as kv_pack_pages, plus dest outside [0, N). */
DCPKV_API int kv_unpack_pages(const kv_reshard_desc* desc, int32_t source, int32_t dest, void* dst_pool,
                    void* dst_scales, const int64_t* dst_global_pages, const int32_t* positions,
                    const int64_t* count, int64_t unit_begin, int64_t cap_units, const void* staging,
                    const void* staging_scales, void* stream);

/* ------------------------------------------------------------------------ *
 * (2) Per-shard partial decode attention ([2DR] sections 5.2, 8; [SGL])    *
 * ------------------------------------------------------------------------ */

typedef struct {
  int32_t kv_dtype;        /* DCPKV_KV_* */
  int32_t kv_layout;       /* DCPKV_LAYOUT_* (MLA requires FP8E4M3) */
  int32_t q_dtype;         /* DCPKV_Q_* */
  int32_t num_q_heads;     /* Hq */
  int32_t num_kv_heads;    /* Hkv (MLA: 1); Hq % Hkv == 0 */
  int32_t head_dim_qk;     /* SPLIT: D (== head_dim_v, <= 256); MLA: 576 */
  int32_t head_dim_v;      /* SPLIT: D; MLA: 512 */
  int32_t page_size;       /* tokens per page */
  int32_t dcp_size;        /* N shards */
  int32_t batch;           /* B requests */
  int32_t q_len;           /* queries per request (1 = decode, >1 = draft verify) */
  int32_t max_local_pages; /* row length of each block table */
  int32_t layer;           /* layer to read from the pools, < num_layers */
  int32_t num_layers;      /* L: layers in each pool */
  int64_t pages_per_layer; /* M: local slots per layer in each pool */
  float softmax_scale;     /* scores are softmax_scale * q . k; positive and finite */
  int32_t token_interleave; /* DCPKV_OWN_PAGE (0): page p of a sequence lives on shard
                               p mod N ([2DR] section 5.1).  DCPKV_OWN_TOKEN (1): token t
                               lives on shard t mod N, local token t div N ([SGL], the
                               DCP paragraph).  The block tables are the same for both:
                               entry j of (d, b) is the slot of local page j. */
} dcp_attn_desc;

/* Workspace bytes dcp_decode_partial needs for this batch.  total_tokens is
 * the sum of the batch's sequence lengths (a host-side figure that sizes the
 * split of long sequences into chunks; pass the same figure to
 * dcp_decode_partial).  A figure below the true sum only makes the split
 * coarser, down to one chunk per (shard, request); results do not depend on it.
 * Returns 0 on a bad descriptor. */
DCPKV_API size_t dcp_decode_partial_workspace(const dcp_attn_desc* desc, int64_t total_tokens);

/* For shards d in [shard_begin, shard_begin + shard_count), every request b,
 * query t < q_len and head h:
 *     pos_t = T_b - q_len + t  (T_b counts the q_len draft tokens, whose KV
 *                               is already in the pools)
 *     J     = { j <= pos_t : token j is owned by shard d }  (through its page, or
 *                               itself under DCPKV_OWN_TOKEN)
 *     s_j   = softmax_scale * q[b][t][h] . k_j   (k, v of KV head h / (Hq/Hkv))
 *     LSE_d = log sum_{j in J} exp(s_j)
 *     O_d   = sum_{j in J} exp(s_j - LSE_d) v_j
 * i.e. the shard's output normalised by its own denominator plus the
 * log-sum-exp of its scores; exp(LSE_d) * O_d is the weighted sum [SGL]
 * describes before normalisation.  An empty J gives O_d = 0, LSE_d = -inf.  MLA: k_j is the
 * whole dequantised 576-d latent (code x page scale), v_j its first 512.
 *
 * q: [B][q_len][Hq][head_dim_qk] (f32 or bf16).  kv_pools: host array [N] of
 * device pointers to DCP pools; kv_scales: host array [N] of device pointers
 * to bf16 [L][M] page scales (MLA), else NULL; page scales must be positive
 * and finite (a zero or negative scale gives undefined results).  block_tables: device int32
 * [N][B][max_local_pages] as built by dcp_build_block_tables: entry j of
 * (d, b) is the slot of shard d's local page j, which holds sequence page
 * j*N + d (DCPKV_OWN_PAGE) or the tokens (j*page_size + x)*N + d, x < page_size
 * (DCPKV_OWN_TOKEN).  seq_lens: device int32
 * [B], each T_b >= q_len.  Out: partial_out fp32 [N][B][q_len][Hq][head_dim_v],
 * partial_lse fp32 [N][B][q_len][Hq] (natural log); only the requested shards'
 * slices are written.  workspace: device, >= dcp_decode_partial_workspace()
 * bytes, 256-byte aligned; its contents need not be initialised.  q, the pools
 * and partial_out must be 16-byte aligned, partial_lse and the scale arrays
 * 4-byte aligned.
 * A table entry outside [0, M) is treated as a page of no tokens.
 * Limits: q_len * Hq <= 262,140 query rows per request, B * N <= 2^24.
 * EINVAL on a bad descriptor/pointer (a softmax_scale that is not positive and
 * finite included), a misaligned pointer, a limit exceeded or too small a
 * workspace (every descriptor that passes these checks has a kernel). */
DCPKV_API int dcp_decode_partial(const dcp_attn_desc* desc, const void* q, const void* const* kv_pools,
                       const void* const* kv_scales, const int32_t* block_tables,
                       const int32_t* seq_lens, int64_t total_tokens, int32_t shard_begin,
                       int32_t shard_count, float* partial_out, float* partial_lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * operation, arguments, layouts and errors as dcp_decode_partial, without a
 * workspace.  The library's own scratch array of DCPKV_NOALLOC_SCRATCH_BYTES
 * per device (held from the library's load until the process ends) takes its
 * place; the call allocates nothing.  When the split the planner wants needs
 * more chunk partials than the scratch holds, the split is coarser (down to
 * one chunk per (shard, request)), which changes results only by rounding.
 * EINVAL, before anything is enqueued, when even the plan without chunk
 * partials does not fit (about 32 bytes per (shard, request) pair plus 16 per
 * chunk).  Every call on a device shares that device's scratch: calls that can
 * overlap on one device (other streams, other threads) race and must be
 * serialised by the caller.  The scratch needs no clearing between calls. */
#define DCPKV_NOALLOC_SCRATCH_BYTES (64u << 20)
DCPKV_API int dcp_decode_partial_noalloc(const dcp_attn_desc* desc, const void* q, const void* const* kv_pools,
                       const void* const* kv_scales, const int32_t* block_tables,
                       const int32_t* seq_lens, int64_t total_tokens, int32_t shard_begin,
                       int32_t shard_count, float* partial_out, float* partial_lse, void* stream);

/* ------------------------------------------------------------------------ *
 * (3) Exact LSE merge over N partials ([2DR] section 5.2; [SGL])           *
 * ------------------------------------------------------------------------ */

/* For each of rows rows (rows = B * q_len * Hq when fed by
 * dcp_decode_partial):
 *     m   = max_d LSE_d
 *     LSE = m + log sum_d exp(LSE_d - m)
 *     out = sum_d exp(LSE_d - LSE) * O_d
 * partial_out fp32 [N][rows][head_dim_v], partial_lse fp32 [N][rows];
 * out fp32 [rows][head_dim_v]; out_lse fp32 [rows], nullable.  Rows whose
 * every LSE_d is -inf give out = 0, LSE = -inf.  The result does not depend on
 * the order of the shards beyond rounding.  out may not alias the inputs.
 * partial_out and out must be 16-byte aligned, the LSE arrays 4-byte aligned.
 * EINVAL on bad sizes, NULL or misaligned pointers. */
DCPKV_API int dcp_lse_merge(int32_t dcp_size, int64_t rows, int32_t head_dim_v, const float* partial_out,
                  const float* partial_lse, float* out, float* out_lse, void* stream);

/* ------------------------------------------------------------------------ *
 * (4) Measurement aid (not on the path)                                     *
 * ------------------------------------------------------------------------ */

/* The matrix-core rate this device reaches on back-to-back independent MFMAs
 * of one kind, to set the fp8 MLA kernel's time against what the hardware
 * delivers as well as against its published peak.  kind 0:
 * v_mfma_f32_16x16x32_f16 (the PV and rope products); kind 1:
 * v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 (the latent scores).  One
 * workgroup of eight wavefronts (two per SIMD) per CU runs `iters` rounds of
 * eight independent MFMAs each.  sink: device float array of at least
 * 1024 * 512 entries (caller-owned), written so the work is kept; *out_flops
 * (host) receives the flops of the launch.  Time it with events on `stream`.
 * EINVAL on bad arguments or too small a sink; EDEVICE if the launch fails. */
DCPKV_API int dcpkv_probe_mfma(int32_t kind, int32_t iters, float* sink, int64_t sink_floats, int64_t* out_flops,
                     void* stream);

/* The copy ceiling the reshard is read against: `bytes` (a multiple of 16)
 * from src to dst (device, 16-byte aligned, not overlapping) with the
 * reshard's own copy loop (a persistent grid of 256-thread workgroups, two per
 * CU, each thread issuing four non-temporal 16-byte loads before its stores)
 * over one contiguous range instead of a page list.  Time it with events on
 * `stream`.  EINVAL on bad arguments, EDEVICE if the launch fails. */
DCPKV_API int dcpkv_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* The same copy loop over a page list, the ceiling of a scattered page copy:
 * page src_pages[i] of src (src_capacity pages of page_bytes) to page
 * dst_pages[i] of dst (dst_capacity pages), i < num_pages, 16 KB segments per
 * workgroup step.  Entries outside [0, capacity) are skipped.  src, dst:
 * device, 16-byte aligned, not overlapping; the page lists: device int32,
 * caller-owned.  page_bytes a positive multiple of 16.  Time it with events on
 * `stream`.  EINVAL on bad arguments, EDEVICE if the launch fails. */
DCPKV_API int dcpkv_probe_copy_pages(const void* src, void* dst, const int32_t* src_pages, const int32_t* dst_pages,
                                     int64_t num_pages, int64_t src_capacity, int64_t dst_capacity,
                                     int64_t page_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCPKV_H */
