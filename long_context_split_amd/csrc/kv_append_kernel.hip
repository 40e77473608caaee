// Paged E4M3 KV append of new tokens (the q verification tokens), on gfx950.
//
// Pages cited by PR number and section:
//   [#556] "[Perf] Add opt-in DFlash2 schedules and numerical audits"
//   [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK reuse"
//
// What one launch computes.  The pages hold the target model's KV cache in
// E4M3 with per-tensor FP32 scales ([#589] Test Plan; [#556] Test Plan) and
// leave the write path unstated; the reading taken here: each new token's FP16
// key and value rows are divided by the layer's scale in FP32 (correctly
// rounded), saturated at +-448 (the largest finite E4M3 magnitude; NaN stays
// NaN), rounded to the nearest E4M3 code with ties to even, and written to row
// slot % 16 of page slot / 16.  A slot outside [0, num_blocks * 16) is padding
// and writes nothing.
//
// Decomposition: one wave per (token, K or V) row; lane l converts dimensions
// 4l..4l+3 with two v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950, round to nearest
// even) and writes one dword, so a row is one coalesced 256-byte store.  The
// work is a few kilobytes per call: the launch is latency-bound.
#include "dfv_append.h"

namespace dfv {
namespace {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

constexpr int kAppendWaves = 4;
constexpr float kE4M3Max = 448.0f;

// x / scale, saturated to the finite E4M3 range; NaN passes through.
__device__ __forceinline__ float scaled_sat(float x, float scale) {
  const float y = __fdiv_rn(x, scale);
  return fabsf(y) > kE4M3Max ? copysignf(kE4M3Max, y) : y;
}

__global__ __launch_bounds__(kAppendWaves * 64) void kv_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  const int tok = gw >> 1;
  if (tok >= a.num_tokens) return;
  const bool is_v = gw & 1;
  const long long slot = a.slot_mapping[tok];
  if (slot < 0 || slot >= a.num_slots) return;
  const _Float16* src = (is_v ? a.v_new : a.k_new) + (size_t)tok * kHeadDim + 4 * lane;
  const float scale = is_v ? a.v_scale[0] : a.k_scale[0];
  const half4 h = *(const half4*)src;
  int packed = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_sat((float)h[0], scale), scaled_sat((float)h[1], scale),
                                               0, false);
  packed = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_sat((float)h[2], scale), scaled_sat((float)h[3], scale),
                                           packed, true);
  uint8_t* dst = (is_v ? a.v_cache : a.k_cache) + (size_t)slot * kHeadDim + 4 * lane;
  *(int*)dst = packed;
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int waves = 2 * a.num_tokens;
  const dim3 grid((waves + kAppendWaves - 1) / kAppendWaves);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(kAppendWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dfv
