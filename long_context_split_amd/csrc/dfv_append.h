// Internal interface of the paged E4M3 KV-append kernel (gfx950).  See
// kv_append_kernel.hip.
#pragma once

#include "dfv_common.h"

namespace dfv {

struct AppendArgs {
  const _Float16* k_new;        // [N][256] FP16 key rows of the new tokens
  const _Float16* v_new;        // [N][256]
  const int64_t* slot_mapping;  // [N]: page * 16 + row, or outside [0, num_slots) to skip
  const float* k_scale;         // device scalars
  const float* v_scale;
  uint8_t* k_cache;             // [num_blocks][16][1][256] E4M3
  uint8_t* v_cache;
  long long num_slots;          // num_blocks * 16
  int num_tokens;
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);

}  // namespace dfv
