// Combine stage of DFlash2 verification attention on gfx950 (MI355X), and the
// merge of key-chunk states into the per-split workspace.
//
// Page cited: [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK
// reuse", Test Result (each q8 attention kernel is followed by a combine kernel
// that merges the logical splits).
//
// For one query row the NS split states (m_j, l_j, o_j) merge by log-sum-exp:
//   M = max_j m_j,  out = sum_j e^(m_j - M) o_j / sum_j e^(m_j - M) l_j,
// empty splits (m_j = -inf) carrying no weight; the result is rounded to FP16
// with round-to-nearest-even.  When the split kernel cut every split into C key
// chunks, the chunk states of split j merge the same way first,
//   m_j = max_c m_jc,  l_j = sum_c e^(m_jc - m_j) l_jc,  o_j = sum_c e^(m_jc - m_j) o_jc,
// in chunk order, and (m_j, l_j, o_j) is written to the workspace.  The output
// is then formed from exactly the values written, so merge-and-combine gives
// the same bytes as a merge followed by a combine of the workspace.
//
// The work is small (NS * C KB per row) and latency-bound, so it is spread
// wide: one workgroup per (row, quarter of the 256 dimensions), ten waves.
// Every wave reduces M over all states itself (no barrier), then wave v takes
// the groups of four splits g = v, v+10, ... (two per load batch, so the 20
// groups of an 80-split row are one batch) with each lane owning four
// dimensions of one split and all loads of a batch issued before use; the ten
// partial sums are added in wave order through LDS.  Every sum has a fixed order, so results are byte-deterministic.
// Workspace stores are non-temporal: nothing in the launch reads them back;
// the state loads are non-temporal too (each state is read once).
#include "dfv_common.h"

namespace dfv {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kCombineWaves = 10;
constexpr int kGroupsPerBatch = 2;   // 4-split groups per wave per load batch

typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// C = chunks per split in the source (1: the source is the workspace itself).
// OUT = form the FP16 output (else only merge chunk states into the workspace).
// Lane (k, d) = (lane / 16, lane % 16) covers split 4*gi + k of each of its
// wave's split groups gi and dimensions 64*quarter + 4d .. +3.
template <int C, bool OUT>
__global__ __launch_bounds__(kCombineWaves * 64) void combine_kernel(CombineArgs a) {
  __shared__ float4v s_num[kCombineWaves][16];
  __shared__ float s_den[kCombineWaves];
  const int row = blockIdx.x >> 2;
  const int quarter = blockIdx.x & 3;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int k = lane >> 4;
  const int d = lane & 15;
  const int NS = a.num_splits;
  const int NG = (NS + 3) >> 2;
  const float* mrow = a.src_max + (size_t)row * NS * C;
  const float* lrow = a.src_sum + (size_t)row * NS * C;
  const float* orow = a.src_num + (size_t)row * NS * C * kHeadDim + 64 * quarter + 4 * d;

  float M = kNegInf;
  float4v num = float4v{0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int g0 = wave; g0 < NG; g0 += kCombineWaves * kGroupsPerBatch) {
    float4v ov[kGroupsPerBatch][C];
    float mv[kGroupsPerBatch][C], lv[kGroupsPerBatch][C];
#pragma unroll
    for (int b = 0; b < kGroupsPerBatch; ++b) {
      const int j = 4 * (g0 + kCombineWaves * b) + k;
      const bool in = j < NS;
      const size_t s0 = (size_t)(in ? j : 0) * C;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        ov[b][c] = __builtin_nontemporal_load((const float4v*)(orow + (s0 + c) * kHeadDim));
        mv[b][c] = mrow[s0 + c];
        lv[b][c] = lrow[s0 + c];
        if (!in) mv[b][c] = kNegInf;
      }
    }
    if (OUT && g0 == wave) {   // row max over every state, while the batch is in flight
      for (int s = lane; s < NS * C; s += 64) M = fmaxf(M, mrow[s]);
      M = wave_max(M);
    }
#pragma unroll
    for (int b = 0; b < kGroupsPerBatch; ++b) {
      const int j = 4 * (g0 + kCombineWaves * b) + k;
      float mj = mv[b][0], lj = lv[b][0];
      float4v oj = ov[b][0];
      if (C > 1) {
#pragma unroll
        for (int c = 1; c < C; ++c) mj = fmaxf(mj, mv[b][c]);
        lj = 0.f;
        oj = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float e = (mv[b][c] == kNegInf) ? 0.f : __expf(mv[b][c] - mj);
          lj = __builtin_fmaf(lv[b][c], e, lj);
#pragma unroll
          for (int i = 0; i < 4; ++i) oj[i] = __builtin_fmaf(ov[b][c][i], e, oj[i]);
        }
      }
      if ((C > 1 || a.write_ws) && j < NS) {
        const size_t w = (size_t)row * NS + j;
        __builtin_nontemporal_store(oj, (float4v*)(a.ws_num + w * kHeadDim + 64 * quarter + 4 * d));
        if (quarter == 0 && d == 0) {
          __builtin_nontemporal_store(mj, a.ws_max + w);
          __builtin_nontemporal_store(lj, a.ws_sum + w);
        }
      }
      if (OUT) {
        const float e = (mj == kNegInf) ? 0.f : __expf(mj - M);
#pragma unroll
        for (int i = 0; i < 4; ++i) num[i] = __builtin_fmaf(oj[i], e, num[i]);
        den = __builtin_fmaf(lj, e, den);
      }
    }
  }
  if (!OUT) return;
  // Splits 4g + k, then the four k (pairwise), then the waves, all in fixed order.
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) num[i] += __shfl_xor(num[i], off, 64);
    den += __shfl_xor(den, off, 64);
  }
  if (lane < 16) s_num[wave][lane] = num;
  if (lane == 0) s_den[wave] = den;
  __syncthreads();
  if (wave == 0 && lane < 16) {
    float4v n = float4v{0.f, 0.f, 0.f, 0.f};
    float dd = 0.f;
#pragma unroll
    for (int v = 0; v < kCombineWaves; ++v) {
      n += s_num[v][lane];
      dd += s_den[v];
    }
    _Float16* o = a.out + (size_t)row * kHeadDim + 64 * quarter + 4 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (_Float16)(n[i] / dd);
  }
}

template <int C>
void launch_c(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(4 * a.rows), block(kCombineWaves * 64);
  if (a.out)
    hipLaunchKernelGGL((combine_kernel<C, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((combine_kernel<C, false>), grid, block, 0, stream, a);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  switch (a.chunks) {
    case 1: launch_c<1>(a, stream); break;
    case 2: launch_c<2>(a, stream); break;
    case 3: launch_c<3>(a, stream); break;
    case 4: launch_c<4>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dfv
