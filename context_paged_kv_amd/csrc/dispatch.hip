// Kernel choice for dcp_decode_partial.
#include <cstdlib>

#include "attn_kernels.h"

namespace dcpkv {

// DCPKV_FORCE_GENERIC=1 routes every call to the generic kernel (used to
// compare the two kernels of this library against each other).
static bool force_generic() {
  const char* e = std::getenv("DCPKV_FORCE_GENERIC");
  return e && e[0] == '1';
}

int choose_kernel(const dcp_attn_desc& D) {
  if (force_generic()) return KK_GENERIC;
  if (gqa_bf16_supported(D)) return KK_GQA_BF16;
  if (mla_fp8_supported(D)) return KK_MLA_FP8;
  return KK_GENERIC;
}

int kernel_rows_per_block(int kind, const dcp_attn_desc& D) {
  switch (kind) {
    case KK_GQA_BF16:
      return (D.num_q_heads / D.num_kv_heads) * D.q_len;  // the whole group in one MFMA row block
    case KK_MLA_FP8:
      return mla_fp8_rows_per_block();  // 64 query rows: four 16-row tiles
    default:
      return D.kv_layout == DCPKV_LAYOUT_MLA ? 8 : 16;
  }
}

int kernel_items_per_cu(int kind) {
  switch (kind) {
    case KK_GQA_BF16:
      return 16;  // one wavefront per item
    case KK_MLA_FP8:
      return 8;  // one workgroup per compute unit at a time: eight rounds of chunks balance mixed lengths
    default:
      return 4;
  }
}

// Workgroups of the kind one compute unit runs at once: the GQA kernel's one-wave
// workgroups are bounded by their 34 KB of LDS, the MLA kernel's by its 128 KB, and the
// generic kernel launches a grid of two per compute unit.
int kernel_resident_per_cu(int kind) {
  switch (kind) {
    case KK_GQA_BF16:
      return 4;
    case KK_MLA_FP8:
      return 1;
    default:
      return 2;
  }
}

int kernel_min_chunk_pages(int kind, const dcp_attn_desc& D) {
  (void)D;
  switch (kind) {
    default:
      return 4;
  }
}

int launch_partial(int kind, const AttnParams& p, const dcp_attn_desc& D, int cus,
                   int64_t item_bound, hipStream_t st) {
  switch (kind) {
    case KK_GQA_BF16:
      return launch_gqa_bf16(p, D, item_bound, st);
    case KK_MLA_FP8:
      return launch_mla_fp8(p, D, item_bound, st);
    default:
      return launch_generic(p, D, cus, item_bound, st);
  }
}

}  // namespace dcpkv
