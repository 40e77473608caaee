// Internal definitions shared by the gfx950 kernels and the C-ABI host code.
//
// Pages cited by PR number and section:
//   [#587] "[Perf] Reduce DFlash2 long-context verification decay"
//   [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK reuse"
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfv {

constexpr int kHeadDim = 256;
constexpr int kQHeads = 6;
constexpr int kPage = 16;                       // tokens per KV page
constexpr int kTile = 32;                       // keys per online-softmax update ([#587] Implementation: N32)
constexpr int kMaxQ = 8;
constexpr int kMaxRows = kMaxQ * kQHeads;       // 48 query rows = three 16-row MFMA blocks
constexpr int kMaxSplits = 256;
constexpr int kWaves = 4;                       // one wave per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kPageBytes = kPage * kHeadDim;    // 4096 B of E4M3 per page per cache
constexpr int kStageBytes = 4 * kPageBytes;     // K pages 0,1 then V pages 0,1 of one tile
constexpr int kStageArray = kWaves * kStageBytes;   // one LDS array per pipeline stage
constexpr int kPartStride = kHeadDim + 4;       // LDS row stride (floats) of a folded partial
constexpr int kPartFloats = kMaxRows * kPartStride + 3 * kMaxRows;
constexpr int kSlotFloats = kMaxRows * kHeadDim + 2 * kMaxRows;   // scratch partial: o, m, l
constexpr float kRestartLog2 = 64.0f;           // P may reach 2^64 before a wave restarts its tiles
constexpr float kLog2e = 1.4426950408889634f;

struct SplitArgs {
  const _Float16* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  float* ws_max;
  float* ws_sum;
  float* ws_num;
  int* counters;      // [batch * num_splits], zero between calls
  float* partials;    // [num_workgroups + batch * num_splits][kSlotFloats]
  int batch;
  int num_q;
  int max_blocks;
  int num_splits;
  int split_tokens;   // 0 = per-sequence rule
  int max_context_len;
  float softmax_scale;
};

struct CombineArgs {
  const float* ws_max;
  const float* ws_sum;
  const float* ws_num;
  _Float16* out;
  int rows;           // batch * num_q * 6
  int num_splits;
};

// Scratch layout: counters first (rounded to 256 B), then partial slots.
inline size_t counter_bytes(int batch, int num_splits) {
  size_t b = (size_t)batch * (size_t)num_splits * sizeof(int);
  return (b + 255) & ~(size_t)255;
}
inline size_t scratch_bytes(int batch, int num_splits, int workgroups) {
  return counter_bytes(batch, num_splits) +
         ((size_t)workgroups + (size_t)batch * (size_t)num_splits) * kSlotFloats * sizeof(float);
}

hipError_t launch_split(const SplitArgs& a, int workgroups, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

}  // namespace dfv
