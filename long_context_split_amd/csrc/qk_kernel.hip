// QK stage of DFlash2 verification attention on its own, on gfx950 (MI355X).
//
// Pages cited by PR number and section:
//   [#587] "[Perf] Reduce DFlash2 long-context verification decay"
//   [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK reuse"
//
// What one launch computes: every FP32 score
//   s[b][r][t] = c * <Q[b, i, h, :], K_t>,   r = 6i + h,   c = softmax_scale * k_scale,
// with K_t the E4M3-decoded key row of token t read through the block table,
// in whole 32-key tiles (the update tile of [#587] Implementation), stored
// tile-major: tile u of sequence b is one contiguous [6q][32] block.  A tile
// is written when it starts inside the context; inside it, keys that row r
// must not see (t > p_i = L_b - q + i, which covers t >= L_b) hold -inf.
// Tiles from ceil(L_b / 32) on are guard tiles: never written, they keep
// whatever the caller put there.  This is the QK producer that the pages time and check by
// itself, score by score and guard tile by guard tile ([#589] Purpose, Test
// Plan); as there, one decoded K fragment feeds the products of all three
// 16-row blocks.
//
// Work decomposition (MI355X: 256 CUs, 64-wide waves, 160 KB LDS per CU):
//   * Workgroups of eight waves, each workgroup on one sequence; a wave takes
//     the sequence's tiles t = t0 + k * W (t0 its index among the sequence's
//     waves, W their count, at most 32 tiles per wave).  The page ids of all
//     its tiles arrive in one vector load (lane j: page j / 32 of tile j % 32)
//     and are then read with v_readlane, so no memory latency sits between
//     one tile and the next tile's DMA.
//   * Each tile's two 4 KiB K pages land in one of the wave's two LDS slots by
//     16-byte direct-to-LDS loads (global_load_lds_dwordx4); a slot is read
//     into registers as soon as its tile lands and refilled at once, so two
//     tiles are in flight per wave while the products run; inside a 256-byte
//     token row the 16-byte chunks are XOR-swizzled by row and page parity so
//     that the operand reads fall on distinct banks.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_f16 with Q (staged once per workgroup
//     through LDS) in registers; E4M3 is decoded with v_cvt_scalef32_pk_f16_fp8
//     (exact in FP16), the per-tensor scale folded into c.
//   * Each lane ends with 4 consecutive keys of one row per page; eight lanes
//     cover a row's 32 keys, and a tile's rows are adjacent, so a tile leaves
//     as one contiguous 6q x 128-byte block, with non-temporal stores (nothing
//     in the launch reads it back), one tile after it was computed.
#include "dfv_qk.h"
#include "dfv_device.h"

namespace dfv {
namespace {

#define LDS_AS DFV_LDS

constexpr int kQkThreads = kQkWaves * 64;
constexpr int kQkTileBytes = 2 * kPageBytes;   // the K pages of one 32-key tile
constexpr int kQkRB = kMaxRows / 16;           // three 16-row blocks at most
constexpr float kNegInfQk = -__builtin_inff();

__shared__ __attribute__((aligned(16))) uint8_t g_qk_k[kQkWaves][2][kQkTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_qk_q[kQkRB * 8][64 * 16];

template <int RB>
__global__ __launch_bounds__(kQkThreads) void qk_kernel(QkArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int NQ = a.num_q;
  const int ROWS = NQ * kQHeads;
  const int gps = gridDim.x / a.batch;               // workgroups per sequence
  const int b = blockIdx.x / gps;
  const int W = gps * kQkWaves;                      // waves per sequence
  const int t0 = (blockIdx.x % gps) * kQkWaves + wave;
  // The page ids are gathered for the tiles a context of max_context_len would
  // have (entries below 16 * max_blocks, so in bounds), at the same time as the
  // context length and Q arrive: no dependent load precedes the first DMA.
  const int Tcap = (a.max_context_len + kTile - 1) / kTile;
  const int ncap = min(t0 < Tcap ? (Tcap - t0 + W - 1) / W : 0, kQkWindow);
  // Q in MFMA B-operand order, staged once per workgroup: fragment f = rb*8 + m,
  // lane (n, g) holds Q[row 16rb + n][64g + 8m + 0..7]; rows past 6q repeat the
  // last real row (their scores are never stored).
  {
    const _Float16* qb = a.q + (size_t)b * ROWS * kHeadDim;
    for (int f = wave; f < RB * 8; f += kQkWaves) {
      const int row = min(16 * (f >> 3) + n, ROWS - 1);
      lds_dma16(qb, (unsigned)(row * kHeadDim * 2 + 128 * g + 16 * (f & 7)),
                   (LDS_AS uint8_t*)&g_qk_q[f][0]);
    }
  }
  // Page ids of this wave's tiles: lane j holds page j / 32 of tile j % 32
  // (0 past the capacity; a page past the context is never loaded).
  int page_v = 0;
  {
    const int k = lane & 31;
    const int pg = 2 * (t0 + k * W) + (lane >> 5);
    if (k < ncap && kPage * pg < a.max_context_len) page_v = a.block_table[(size_t)b * a.max_blocks + pg];
  }
  const int L = min(max(a.context_lens[b], NQ), a.max_context_len);
  const int Tb = (L + kTile - 1) / kTile;            // tiles written for this sequence
  // At most kQkWindow by the launch geometry; the bound keeps every page-id
  // read inside the window whatever the lengths.
  const int ntiles = min(t0 < Tb ? (Tb - t0 + W - 1) / W : 0, kQkWindow);

  // DMA lane offsets: load qq of page p fills LDS row r = 4qq + lane/16, chunk
  // position lane%16, with global chunk (lane%16) ^ r ^ 4p of that row.
  unsigned lane_off[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const unsigned r = 4 * qq + (lane >> 4);
      lane_off[p][qq] = r * 256u + 16u * ((unsigned)(lane & 15) ^ r ^ (4u * p));
    }
  // Number of 16-byte loads issue(k) puts out: 4 per page, the second page
  // only when it starts inside the context; 0 past the wave's tiles.
  auto nops = [&](int k) -> int {
    if (k >= ntiles) return 0;
    return (kTile * (t0 + k * W) + kPage < L) ? 8 : 4;
  };
  auto issue = [&](int k) {
    if (k >= ntiles) return;
    const int t = t0 + k * W;
    LDS_AS uint8_t* slot = (LDS_AS uint8_t*)&g_qk_k[wave][k & 1][0];
    const int id0 = __builtin_amdgcn_readlane(page_v, k);
    const uint8_t* p0 = a.k_cache + (size_t)id0 * kPageBytes;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) lds_dma16_nt(p0, lane_off[0][qq], slot + qq * 1024);
    if (kTile * t + kPage < L) {
      const int id1 = __builtin_amdgcn_readlane(page_v, 32 + k);
      const uint8_t* p1 = a.k_cache + (size_t)id1 * kPageBytes;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) lds_dma16_nt(p1, lane_off[1][qq], slot + kPageBytes + qq * 1024);
    }
  };
  // Page ids, the length, the scale and this wave's Q fragments have landed;
  // c passes through the wait so that no later wait is placed for its load.
  float c = a.softmax_scale * a.k_scale[0];
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(c) :: "memory");
  issue(0);                                           // two tiles go out before the barrier
  issue(1);
  __syncthreads();                                    // every wave's Q fragments staged
  half8 qf[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int m = 0; m < 8; ++m) qf[rb][m] = *(const LDS_AS half8*)(&g_qk_q[rb * 8 + m][lane * 16]);

  // Causal bound of each of this lane's rows.
  int limit[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) limit[rb] = L - NQ + min(16 * rb + n, ROWS - 1) / kQHeads;
  float* const out_b = a.scores + (size_t)b * a.tiles_per_seq * ROWS * kTile;

  // Two tiles in flight per wave: tile k's slot is read into registers as
  // soon as it lands and refilled with tile k + 2 before the products.  The
  // wait for tile k lets the loads of tile k + 1 stay outstanding: loads
  // complete in issue order, so at most nops(k + 1) operations outstanding
  // means tile k has landed, whatever the stores issued in between (they may
  // complete in any order, and are counted as still to wait for).  A tile's
  // scores are stored one iteration later, after the refill.
  float4v res[2][RB];
  int res_t = -1;
  auto store_res = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = 16 * rb + n;
      if (row >= ROWS) continue;
      float* const dst = out_b + ((size_t)res_t * ROWS + row) * kTile + 4 * g;
#pragma unroll
      for (int p = 0; p < 2; ++p) __builtin_nontemporal_store(res[p][rb], (float4v*)(dst + 16 * p));
    }
  };
  for (int k = 0; k < ntiles; ++k) {
    const int after = nops(k + 1);
    if (after == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (after == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int t = t0 + k * W;
    const LDS_AS uint8_t* ks = (const LDS_AS uint8_t*)&g_qk_k[wave][k & 1][0] + n * 256;
    uint4v kr[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const LDS_AS uint8_t* krow = ks + p * kPageBytes;
      const unsigned swz = 16u * ((unsigned)n ^ (4u * p));
#pragma unroll
      for (int j = 0; j < 4; ++j) kr[p][j] = *(const volatile LDS_AS uint4v*)(krow + ((16u * (4 * g + j)) ^ swz));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the slot is read before its refill
    issue(k + 2);
    if (res_t >= 0) store_res();
    float4v sacc[2][RB];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[p][rb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8 k0 = decode8(kr[p][j][0], kr[p][j][1]);
        const half8 k1 = decode8(kr[p][j][2], kr[p][j][3]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[p][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[rb][2 * j], sacc[p][rb], 0, 0, 0);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[p][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qf[rb][2 * j + 1], sacc[p][rb], 0, 0, 0);
      }
    }
    // Scale and mask (a page past the context was not loaded: its keys are all
    // masked, whatever the slot held).
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int key = kTile * t + 16 * p + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) res[p][rb][r] = (key + r <= limit[rb]) ? sacc[p][rb][r] * c : kNegInfQk;
      }
    res_t = t;
  }
  if (res_t >= 0) store_res();
}

}  // namespace

hipError_t launch_qk(const QkArgs& a, hipStream_t stream) {
  const int rb = (a.num_q * kQHeads + 15) / 16;
  const dim3 grid(a.batch * qk_groups_per_seq(a.batch, a.max_context_len));
  const dim3 block(kQkThreads);
  switch (rb) {
    case 1: hipLaunchKernelGGL(qk_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(qk_kernel<2>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(qk_kernel<3>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace dfv
