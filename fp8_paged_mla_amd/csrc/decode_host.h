// Host-side pieces shared by the decode and extend translation units (internal).
#pragma once

#include "decode_common.h"
#include "launch.h"

namespace fp8mla {

decode::SplitParams make_split_params(const uint16_t* q, const void* kv_rows, int64_t num_slots,
                                      const int32_t* kv_indptr, const int32_t* kv_indices,
                                      int64_t total_tokens, int32_t batch, int32_t num_heads,
                                      float scale, float sm_scale, uint16_t* out,
                                      void* workspace, const DecodePlan& pl);

// Merge of the partials of requests spanning several segments (one wave per
// request and head).
hipError_t launch_mla_combine(const decode::SplitParams& sp, hipStream_t stream);

// The 64-row split kernel in its extend form (virtual requests, causal limits).
hipError_t launch_mla_split_h64_extend(const decode::SplitParams& sp, int grid, hipStream_t stream);

}  // namespace fp8mla
