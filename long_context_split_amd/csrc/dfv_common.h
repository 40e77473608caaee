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
constexpr int kTile = 32;                       // split boundaries fall on 32-key tiles ([#587] Implementation: N32)
constexpr int kMaxQ = 8;
constexpr int kMaxRows = kMaxQ * kQHeads;       // 48 query rows = three 16-row MFMA blocks
constexpr int kMaxSplits = 256;
constexpr int kMaxContext = 1 << 22;            // admitted bound on max_context_len (keeps key arithmetic in int)
constexpr int kTargetCUs = 256;                 // MI355X compute units (sizes the key chunking)
constexpr int kMaxChunks = 4;                   // key chunks per logical split, at most
constexpr int kWaves = 4;                       // one wave per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kPageBytes = kPage * kHeadDim;    // 4096 B of E4M3 per page per cache
constexpr float kLog2e = 1.4426950408889634f;

struct SplitArgs {
  const _Float16* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  // Where the states go: the workspace itself (chunks = 1) or scratch laid out
  // as the workspace with the chunk index innermost (chunks > 1).
  float* st_max;      // [rows][NS][chunks]
  float* st_sum;      // [rows][NS][chunks]
  float* st_num;      // [rows][NS][chunks][256]
  int chunks;         // key chunks per logical split
  int batch;
  int num_q;
  int max_blocks;
  int num_splits;
  int split_tokens;   // 0 = per-sequence rule
  int max_context_len;
  float softmax_scale;
};

struct CombineArgs {
  // Source states: the workspace (chunks = 1) or the split kernel's chunk
  // states in scratch (chunks > 1).
  const float* src_max;
  const float* src_sum;
  const float* src_num;
  int chunks;
  // Merged workspace, written when write_ws is set (always when chunks > 1).
  float* ws_max;
  float* ws_sum;
  float* ws_num;
  int write_ws;
  _Float16* out;      // NULL: merge only (no output)
  int rows;           // batch * num_q * 6
  int num_splits;
};

int split_chunks(int batch, int num_splits);

// Scratch (chunks > 1): chunk numerators, then maxima, then sums.
inline size_t scratch_floats(int rows, int num_splits, int chunks) {
  return (size_t)rows * num_splits * chunks;
}
inline size_t scratch_bytes(int batch, int num_q, int num_splits) {
  const int chunks = split_chunks(batch, num_splits);
  if (chunks == 1) return 0;
  const size_t n = scratch_floats(batch * num_q * kQHeads, num_splits, chunks);
  return (n * (kHeadDim + 2) * sizeof(float) + 255) & ~(size_t)255;
}
int split_grid(int batch, int num_q, int num_splits);
hipError_t launch_split(const SplitArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

}  // namespace dfv
