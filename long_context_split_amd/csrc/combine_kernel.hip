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
// One workgroup per row, four waves; wave v merges splits j = v, v+4, ... with
// lane l owning dimensions 4l..4l+3 (16-byte loads of the numerator rows), then
// the four wave partials are merged in wave order through LDS.  The order of
// every sum is fixed, so results are byte-deterministic.  The workload is tiny
// (NS * 1 KB per row), so the kernel is latency-bound; four waves per row keep
// four independent load streams in flight.
#include "dfv_common.h"

namespace dfv {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));
constexpr float kNegInf = -__builtin_inff();

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  __shared__ float s_m[kWaves];
  __shared__ float s_l[kWaves];
  __shared__ __attribute__((aligned(16))) float s_o[kWaves][kHeadDim];
  const int row = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int NS = a.num_splits;
  const float* mrow = a.ws_max + (size_t)row * NS;
  const float* lrow = a.ws_sum + (size_t)row * NS;
  const float* orow = a.ws_num + (size_t)row * NS * kHeadDim;

  float M = kNegInf;
  for (int j = wave; j < NS; j += kWaves) M = fmaxf(M, mrow[j]);
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (M != kNegInf) {
    for (int j = wave; j < NS; j += kWaves) {
      const float mj = mrow[j];
      if (mj == kNegInf) continue;
      const float e = __expf(mj - M);
      acc += *(const float4v*)(orow + (size_t)j * kHeadDim + 4 * lane) * e;
      l += lrow[j] * e;
    }
  }
  if (lane == 0) {
    s_m[wave] = M;
    s_l[wave] = l;
  }
  *(float4v*)&s_o[wave][4 * lane] = acc;
  __syncthreads();
  if (wave == 0) {
    float Mt = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) Mt = fmaxf(Mt, s_m[v]);
    float4v num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      if (s_m[v] == kNegInf) continue;
      const float e = __expf(s_m[v] - Mt);
      num += *(const float4v*)&s_o[v][4 * lane] * e;
      den += s_l[v] * e;
    }
    _Float16* o = a.out + (size_t)row * kHeadDim + 4 * lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = (_Float16)(num[k] / den);
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.rows), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dfv
