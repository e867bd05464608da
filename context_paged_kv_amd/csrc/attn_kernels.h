// Kernel selection for dcp_decode_partial.  Each kernel kind states how many
// query rows one work item covers, how many items per compute unit the
// planner should aim for, how many of its workgroups one compute unit holds at
// once, the smallest chunk it wants, and how it launches.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_common.h"

namespace dcpkv {

enum KernelKind : int {
  KK_GENERIC = 0,  // VALU, any supported dtype / layout / shape
  KK_GQA_BF16 = 1, // split layout, bf16 KV, MFMA scores
  KK_MLA_FP8 = 2,  // MLA fp8 latent, MFMA QK^T and PV
};

int choose_kernel(const dcp_attn_desc& D);
int kernel_rows_per_block(int kind, const dcp_attn_desc& D);
int kernel_items_per_cu(int kind);
int kernel_resident_per_cu(int kind);
int kernel_min_chunk_pages(int kind, const dcp_attn_desc& D);
int launch_partial(int kind, const AttnParams& p, const dcp_attn_desc& D, int cus,
                   int64_t item_bound, hipStream_t st);
int launch_generic(const AttnParams& p, const dcp_attn_desc& D, int cus, int64_t item_bound,
                   hipStream_t st);
bool gqa_bf16_supported(const dcp_attn_desc& D);
int launch_gqa_bf16(const AttnParams& p, const dcp_attn_desc& D, int64_t item_bound, hipStream_t st);
bool mla_fp8_supported(const dcp_attn_desc& D);
int mla_fp8_rows_per_block();
int launch_mla_fp8(const AttnParams& p, const dcp_attn_desc& D, int64_t item_bound, hipStream_t st);

}  // namespace dcpkv
