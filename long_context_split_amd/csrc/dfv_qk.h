// Internal interface of the QK-stage kernel (gfx950): the launch arguments and
// the grid it uses.  See qk_kernel.hip.
#pragma once

#include "dfv_common.h"

namespace dfv {

struct QkArgs {
  const _Float16* q;           // [B][q][6][256]
  const uint8_t* k_cache;      // [num_blocks][16][1][256] E4M3
  const int32_t* block_table;  // [B][max_blocks]
  const int32_t* context_lens; // [B]
  const float* k_scale;        // device scalar
  float* scores;               // [B][tiles_per_seq][6q][32]
  long long tiles_per_seq;     // tile capacity per sequence, >= ceil(max_context_len / 32)
  int batch;
  int num_q;
  int max_blocks;
  int max_context_len;
  float softmax_scale;
};

constexpr int kQkWaves = 8;     // waves per workgroup
constexpr int kQkWindow = 32;   // tiles per wave at most (one page-id window)

// Workgroups per sequence: enough to fill the GPU, and enough that no wave
// gets more than kQkWindow tiles of 32 keys.
inline int qk_groups_per_seq(int batch, int max_context_len) {
  const int tiles = (max_context_len + kTile - 1) / kTile;
  const int fill = (kTargetCUs + batch - 1) / batch;
  const int need = (tiles + kQkWaves * kQkWindow - 1) / (kQkWaves * kQkWindow);
  return fill > need ? fill : need;
}

hipError_t launch_qk(const QkArgs& a, hipStream_t stream);

}  // namespace dfv
