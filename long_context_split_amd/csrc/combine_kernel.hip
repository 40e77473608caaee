// Combine stage of DFlash2 verification attention on gfx950 (MI355X).
//
// Page cited: [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK
// reuse", Test Result (each q8 attention kernel is followed by a combine kernel
// that merges the logical splits).
//
// For one query row the NS split states (m_j, l_j, o_j) merge by log-sum-exp:
//   M = max_j m_j,  out = sum_j e^(m_j - M) o_j / sum_j e^(m_j - M) l_j,
// empty splits (m_j = -inf) carrying no weight; the result is rounded to FP16
// with round-to-nearest-even.
//
// The workload is small (NS KB per row) and latency-bound, so it is spread
// wide: one workgroup per (row, quarter of the 256 dimensions), four waves per
// workgroup.  Every wave reduces M over all splits itself (no barrier), then
// wave v accumulates splits j = v, v+4, ... with each lane owning one dimension
// and all of its loads issued before use; the four partial sums are added in
// wave order through LDS.  Every sum has a fixed order, so results are
// byte-deterministic.
#include "dfv_common.h"

namespace dfv {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kChunk = 8;   // loads in flight per lane and batch

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  __shared__ float s_num[kWaves][64];
  __shared__ float s_den[kWaves];
  const int row = blockIdx.x >> 2;
  const int quarter = blockIdx.x & 3;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int NS = a.num_splits;
  const float* mrow = a.ws_max + (size_t)row * NS;
  const float* lrow = a.ws_sum + (size_t)row * NS;
  const float* orow = a.ws_num + (size_t)row * NS * kHeadDim + 64 * quarter + lane;

  float M = kNegInf;
  for (int j = lane; j < NS; j += 64) M = fmaxf(M, mrow[j]);
  M = wave_max(M);

  float num = 0.f, den = 0.f;
  if (M != kNegInf) {
    for (int j0 = wave; j0 < NS; j0 += kWaves * kChunk) {
      float ov[kChunk];
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int j = j0 + kWaves * k;
        ov[k] = j < NS ? orow[(size_t)j * kHeadDim] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int j = j0 + kWaves * k;
        if (j < NS) {
          const float mj = mrow[j];
          const float e = (mj == kNegInf) ? 0.f : __expf(mj - M);
          num += ov[k] * e;
          den += lrow[j] * e;
        }
      }
    }
  }
  s_num[wave][lane] = num;
  if (lane == 0) s_den[wave] = den;
  __syncthreads();
  if (wave == 0) {
    float n = 0.f, d = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      n += s_num[v][lane];
      d += s_den[v];
    }
    a.out[(size_t)row * kHeadDim + 64 * quarter + lane] = (_Float16)(n / d);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(4 * a.rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dfv
