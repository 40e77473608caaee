// Split stage of DFlash2 verification attention on gfx950 (MI355X).
//
// Pages cited by PR number and section:
//   [#587] "[Perf] Reduce DFlash2 long-context verification decay"
//   [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK reuse"
//
// What one launch computes: for every sequence b, query row r = 6*i + h and
// logical split j, the FP32 state (max, sum, numerator) of causal softmax
// attention restricted to the split's keys ([#587] Implementation: 80 logical
// splits, N32 online updates, compensated FP32 sums, probability residual
// products, FP32 state; [#589] Test Plan: the full FP32 workspace is output).
//
// Work decomposition (MI355X: 256 CUs, 64-wide waves, 160 KB LDS per CU):
//   * The 32-key tiles of all sequences form one list, cut evenly into one
//     contiguous range per workgroup (one workgroup per CU).  A range may start
//     or end inside a logical split; workgroups that share a split store their
//     partial state in scratch and the last one to arrive merges the partials in
//     workgroup order, so results are byte-deterministic.
//   * Inside a workgroup, four waves (one per SIMD) take the range's tiles in
//     turn.  Each wave owns all 6q query rows, so every K and V byte is decoded
//     once and each decoded K fragment feeds the three 16-row MFMA products
//     (the pages' three M16 products per K fragment, [#589] Purpose).
//   * Each wave streams its tiles through a private two-stage LDS ring with
//     16-byte direct-to-LDS loads (global_load_lds_dwordx4), one 4 KB page per
//     four wave instructions, fully coalesced.  Within a 256-byte token row the
//     16-byte chunks are XOR-swizzled by the row's slot so MFMA operand reads are
//     bank-conflict free.
//   * QK^T runs as S^T = K * Q^T with v_mfma_f32_16x16x32_f16: A = 16 keys x 32
//     dims of decoded K, B = 32 dims x 16 rows of Q (Q stays in registers).  The
//     C layout leaves each lane with 4 keys of one row, so the row max needs two
//     cross-lane steps (permlane16/32 swaps).
//   * Each wave fixes a per-row reference max at the first tile where the row
//     sees a key and never rescales its accumulators inside the tile loop:
//     P = exp(s - m_ref) is carried as three bf16 terms (the pages' probability
//     residual products; 24 significant bits, fp32 exponent range), so P may
//     grow far above 1.  Should a row's running max outgrow its reference by
//     more than 2^64, the wave raises the reference and redoes its tiles (only
//     adversarial score growth gets there).  The fold renormalises every state
//     to its true max.  This is an exact re-association of the pages' 32-key
//     online update, chosen because a data-dependent rescale of the AGPR
//     accumulators makes the compiler shadow them in VGPRs.
//   * PV runs as O^T += V^T * P^T with v_mfma_f32_16x16x32_bf16 (E4M3 is exact
//     in bf16); the V operand (8 keys of one dimension per lane) comes straight
//     out of LDS with the transposing read ds_read_b64_tr_b8.
//   * E4M3 is decoded in registers with v_cvt_pk_f32_fp8 (OCP on gfx950) and
//     packed to FP16 for K and bf16 for V (both exact).  The scales are
//     not applied during decode: k_scale is folded into the score scale and
//     v_scale into the stored numerator.
#include "dfv_common.h"

namespace dfv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ half8 decode8(unsigned lo, unsigned hi) {
  float2v a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  float2v b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  float2v c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  float2v d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  half8 r;
  r[0] = (_Float16)a[0]; r[1] = (_Float16)a[1];
  r[2] = (_Float16)b[0]; r[3] = (_Float16)b[1];
  r[4] = (_Float16)c[0]; r[5] = (_Float16)c[1];
  r[6] = (_Float16)d[0]; r[7] = (_Float16)d[1];
  return r;
}

__device__ __forceinline__ bf16x8 decode8_bf16(unsigned lo, unsigned hi) {
  float2v a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  float2v b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  float2v c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  float2v d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1];
  r[2] = (__bf16)b[0]; r[3] = (__bf16)b[1];
  r[4] = (__bf16)c[0]; r[5] = (__bf16)c[1];
  r[6] = (__bf16)d[0]; r[7] = (__bf16)d[1];
  return r;
}

// Pairwise exchange with lane ^ 16 and lane ^ 32: both lanes of a pair receive
// the same (low-lane, high-lane) values, so symmetric reductions agree bitwise.
__device__ __forceinline__ float max_x16(float x) {
  uint2v r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  uint2v r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  uint2v r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  uint2v r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Neumaier compensated add of x into (sum, comp).
__device__ __forceinline__ void comp_add(float& sum, float& comp, float x) {
  float t = sum + x;
  comp += (fabsf(sum) >= fabsf(x)) ? ((sum - t) + x) : ((x - t) + sum);
  sum = t;
}

// 16-byte direct-to-LDS load: lane l's 16 bytes (uniform base + per-lane offset)
// land at LDS address dst + 16*l.  Issued through inline asm so the compiler
// does not add its conservative "wait for every LDS DMA" before unrelated LDS
// reads; the tile loop waits on vmcnt itself (vector loads complete in order,
// so extra outstanding loads only ever make the compiler's own waits stricter).
// s_nop covers the M0 write -> LDS-DMA wait state.
__device__ __forceinline__ void lds_dma16(const uint8_t* base, unsigned off, LDS_AS uint8_t* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(m0) : "memory", "m0");
}

// a ^ k computed in the loop body.  The swizzled LDS addresses of a tile are
// loop-invariant; left to itself the compiler hoists all of them out of the tile
// loop and spills them, and every spill reload waits for the in-flight DMAs.
__device__ __forceinline__ unsigned xor_in_loop(unsigned a, unsigned k) {
  unsigned r;
  asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(k), "v"(a));
  return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
}

// Issue the 16 direct-to-LDS loads of one 32-key tile (K pages 0,1 then V pages
// 0,1).  Lane l of load qq fills LDS row r = 4*qq + l/16, chunk position l%16,
// with global chunk (l%16) ^ r of that row.
__device__ __forceinline__ void issue_tile(const uint8_t* kc, const uint8_t* vc, int page0, int page1,
                                           LDS_AS uint8_t* dst, const unsigned (&lane_off)[4]) {
  const uint8_t* k0 = kc + (size_t)page0 * kPageBytes;
  const uint8_t* k1 = kc + (size_t)page1 * kPageBytes;
  const uint8_t* v0 = vc + (size_t)page0 * kPageBytes;
  const uint8_t* v1 = vc + (size_t)page1 * kPageBytes;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    lds_dma16(k0, lane_off[qq], dst + 0 * kPageBytes + qq * 1024);
    lds_dma16(k1, lane_off[qq], dst + 1 * kPageBytes + qq * 1024);
    lds_dma16(v0, lane_off[qq], dst + 2 * kPageBytes + qq * 1024);
    lds_dma16(v1, lane_off[qq], dst + 3 * kPageBytes + qq * 1024);
  }
}

template <int RB>
struct WaveState {
  float4v o[16][RB];   // O^T accumulators relative to m_ref: lane (n,g) holds row 16rb+n, dims 16mb+4g+0..3
  float m_ref[RB];     // reference max (raw dot-product units); -inf until the row sees a key
  float m_max[RB];     // true running max (raw units)
  float l_sum[RB];     // this lane's compensated partial sum of P (relative to m_ref)
  float l_cmp[RB];
};

template <int RB>
__device__ __forceinline__ void state_reset(WaveState<RB>& st) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    st.m_ref[rb] = kNegInf;
    st.m_max[rb] = kNegInf;
    st.l_sum[rb] = 0.f;
    st.l_cmp[rb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) st.o[mb][rb] = float4v{0.f, 0.f, 0.f, 0.f};
  }
}

// Split p into three bf16 terms p = hi + mid + lo (24 significant bits; each
// residual is exact in fp32).  bf16 keeps fp32's exponent range, so p may run
// far above 1 without overflow.
__device__ __forceinline__ void split3(float p, __bf16& hi, __bf16& mid, __bf16& lo) {
  hi = (__bf16)p;
  const float r1 = p - (float)hi;
  mid = (__bf16)r1;
  lo = (__bf16)(r1 - (float)mid);
}

// One 32-key tile: QK^T, masked softmax against a fixed reference max, and
// PV with the three-term P.  Returns true (before touching O) when some row's
// running max has outgrown its reference by more than 2^kRestartLog2; the
// caller then restarts the wave's tiles from a raised reference.
// qlane points at this lane's Q fragments in LDS: fragment (rb, m) holds
// Q[row 16rb+n][64g + 8m + 0..7] at qlane + (rb*8 + m)*1024.
template <int RB>
__device__ __forceinline__ bool compute_tile(WaveState<RB>& st, const LDS_AS uint8_t* qlane,
                                             const LDS_AS uint8_t* kl, int t0, int L,
                                             const int (&limit)[RB], float c2, int n, int g) {
  const LDS_AS uint8_t* vl = kl + 2 * kPageBytes;
  // ---- S^T = K * Q^T over the tile's two 16-key blocks; each decoded K
  // fragment feeds RB row blocks, each Q fragment both key blocks.
  float4v sacc[2][RB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sacc[kb][rb] = float4v{0.f, 0.f, 0.f, 0.f};
  const LDS_AS uint8_t* krow0 = kl + n * 256;
  const LDS_AS uint8_t* krow1 = kl + kPageBytes + n * 256;
  uint4v kr0 = *(const LDS_AS uint4v*)(krow0 + 16 * ((4 * g) ^ n));
  uint4v kr1 = *(const LDS_AS uint4v*)(krow1 + 16 * ((4 * g) ^ n));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4v c0 = kr0, c1 = kr1;
    if (i < 3) {   // prefetch the next 16-byte chunk of both key rows
      const int chunk = 16 * ((4 * g + i + 1) ^ n);
      kr0 = *(const LDS_AS uint4v*)(krow0 + chunk);
      kr1 = *(const LDS_AS uint4v*)(krow1 + chunk);
    }
    const half8 k00 = decode8(c0[0], c0[1]);
    const half8 k01 = decode8(c0[2], c0[3]);
    const half8 k10 = decode8(c1[0], c1[1]);
    const half8 k11 = decode8(c1[2], c1[3]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const half8 qa = *(const LDS_AS half8*)(qlane + (rb * 8 + 2 * i) * 1024);
      const half8 qb = *(const LDS_AS half8*)(qlane + (rb * 8 + 2 * i + 1) * 1024);
      sacc[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k00, qa, sacc[0][rb], 0, 0, 0);
      sacc[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k01, qb, sacc[0][rb], 0, 0, 0);
      sacc[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k10, qa, sacc[1][rb], 0, 0, 0);
      sacc[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k11, qb, sacc[1][rb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- masked scores, row max, reference max (lane holds keys t0 + 16kb + 4g + r)
  float s[RB][8];
  bool restart = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float tmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = t0 + 16 * kb + 4 * g + r;
        const float v = (key <= limit[rb]) ? sacc[kb][rb][r] : kNegInf;
        s[rb][kb * 4 + r] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = max_x16(tmax);
    tmax = max_x32(tmax);
    st.m_max[rb] = fmaxf(st.m_max[rb], tmax);
    if (st.m_ref[rb] == kNegInf) st.m_ref[rb] = tmax;   // first visible keys of this row (or still -inf)
    restart |= (st.m_max[rb] - st.m_ref[rb]) * c2 > kRestartLog2;   // false while -inf
  }
  if (__builtin_amdgcn_ballot_w64(restart)) return true;
  __builtin_amdgcn_sched_barrier(0);
  // ---- P = exp(s - m_ref) as three bf16 terms (the pages' probability residual
  // products), compensated row sums
  bf16x8 phi[RB], pmid[RB], plo[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bool live = st.m_ref[rb] != kNegInf;
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // (s - m_ref) first: exact for keys near the max, so P keeps full
      // relative precision even when |m_ref * c2| is large.
      const float p = live ? fast_exp2((s[rb][k] - st.m_ref[rb]) * c2) : 0.f;
      psum += p;
      __bf16 h, m, l;
      split3(p, h, m, l);
      phi[rb][k] = h;
      pmid[rb][k] = m;
      plo[rb][k] = l;
    }
    comp_add(st.l_sum[rb], st.l_cmp[rb], psum);
  }
  // ---- O^T += V^T * P^T; lane (n,g) reads 8 keys of dimension 16mb + n.
  // Keys at or past L (last tile of a sequence) hold unrelated bytes; their
  // codes are cleared to +0 before decode so 0 * NaN never reaches the sum.
  const int j = n >> 1;
  const int vslot = 4 * g + (j & 3);
  const unsigned vrow = (unsigned)(uintptr_t)(vl + (j >> 2) * kPageBytes + vslot * 256 + 8 * (n & 1));
  const unsigned vsw = 16u * vslot;
  unsigned keep_lo = 0xffffffffu, keep_hi = 0xffffffffu;
  if (t0 + kTile > L) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (t0 + 4 * g + k >= L) keep_lo &= ~(0xffu << (8 * k));
      if (t0 + 16 + 4 * g + k >= L) keep_hi &= ~(0xffu << (8 * k));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  int2v vnext = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS int2v*)(uintptr_t)(vrow + vsw));
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) {
    const int2v vr = vnext;
    if (mb < 15)
      vnext = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (LDS_AS int2v*)(uintptr_t)(vrow + xor_in_loop(vsw, 16u * (mb + 1))));
    const bf16x8 va = decode8_bf16((unsigned)vr[0] & keep_lo, (unsigned)vr[1] & keep_hi);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      st.o[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi[rb], st.o[mb][rb], 0, 0, 0);
      st.o[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pmid[rb], st.o[mb][rb], 0, 0, 0);
      st.o[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo[rb], st.o[mb][rb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  return false;
}

// Reduce the per-lane sums over the four lanes of each row (l_sum then holds
// the row sum relative to m_ref).
template <int RB>
__device__ __forceinline__ void finalize_wave(WaveState<RB>& st) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    st.l_sum[rb] = sum_x32(sum_x16(st.l_sum[rb])) + sum_x32(sum_x16(st.l_cmp[rb]));
}

// LDS partial of one wave: o[48][kPartStride] (relative to m_ref), then m_ref,
// m_max and l per row.
template <int RB>
__device__ __forceinline__ void write_lds_partial(const WaveState<RB>& st, LDS_AS float* buf, int n, int g) {
  LDS_AS float* mref = buf + kMaxRows * kPartStride;
  LDS_AS float* mmax = mref + kMaxRows;
  LDS_AS float* lbuf = mmax + kMaxRows;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 16 * rb + n;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) {
      *(LDS_AS float4v*)(buf + row * kPartStride + 16 * mb + 4 * g) = st.o[mb][rb];
      __builtin_amdgcn_sched_barrier(0);
    }
    if (g == 0) {
      mref[row] = st.m_ref[rb];
      mmax[row] = st.m_max[rb];
      lbuf[row] = st.l_sum[rb];
    }
  }
}

// Merge another wave's LDS partial into this wave's state.  Both are rescaled
// to the common true max M, after which m_ref = m_max = M.
template <int RB>
__device__ __forceinline__ void merge_lds_partial(WaveState<RB>& st, const LDS_AS float* buf, float c2, int n, int g) {
  const LDS_AS float* mref = buf + kMaxRows * kPartStride;
  const LDS_AS float* mmax = mref + kMaxRows;
  const LDS_AS float* lbuf = mmax + kMaxRows;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 16 * rb + n;
    const float rb_ref = mref[row];
    const float M = fmaxf(st.m_max[rb], mmax[row]);
    const float ea = (st.m_ref[rb] != kNegInf) ? fast_exp2((st.m_ref[rb] - M) * c2) : 0.f;
    const float eb = (rb_ref != kNegInf) ? fast_exp2((rb_ref - M) * c2) : 0.f;
#pragma unroll
    for (int mb = 0; mb < 16; ++mb) {
      const float4v ob = *(const LDS_AS float4v*)(buf + row * kPartStride + 16 * mb + 4 * g);
      st.o[mb][rb] = st.o[mb][rb] * ea + ob * eb;
      __builtin_amdgcn_sched_barrier(0);
    }
    st.l_sum[rb] = st.l_sum[rb] * ea + lbuf[row] * eb;
    st.m_ref[rb] = M;
    st.m_max[rb] = M;
  }
}

__shared__ __attribute__((aligned(16))) uint8_t g_stage0[kStageArray];
__shared__ __attribute__((aligned(16))) uint8_t g_stage1[kStageArray];
__shared__ __attribute__((aligned(16))) uint8_t g_qfrag[(kMaxRows / 16) * 8 * 1024];
__shared__ int g_last_flag;

__device__ __forceinline__ int split_size_of(int L, int ns, int fixed) {
  if (fixed) return fixed;
  const int per = (L + ns - 1) / ns;
  return kTile * ((per + kTile - 1) / kTile);
}

__device__ __forceinline__ int clamp_len(int L, int nq, int maxL) { return min(max(L, nq), maxL); }

// Workgroup owning flattened tile f when T tiles are cut into G even ranges
// [floor(w*T/G), floor((w+1)*T/G)).
__device__ __forceinline__ int owner_of(long long f, long long T, int G) {
  return (int)(((f + 1) * (long long)G - 1) / T);
}

template <int RB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void split_kernel(const _Float16* __restrict__ q, const uint8_t* __restrict__ k_cache,
                  const uint8_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
                  const int32_t* __restrict__ context_lens, const float* __restrict__ k_scale,
                  const float* __restrict__ v_scale, SplitArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int G = gridDim.x;
  const int w = blockIdx.x;
  const int NQ = a.num_q;
  const int ROWS = NQ * kQHeads;
  const int NS = a.num_splits;

  const float c = a.softmax_scale * k_scale[0];
  const float c2 = c * kLog2e;
  const float ofac = v_scale[0];

  long long T = 0;
  for (int b = 0; b < a.batch; ++b) {
    const int L = clamp_len(context_lens[b], NQ, a.max_context_len);
    T += (L + kTile - 1) / kTile;
  }
  const long long f0 = (long long)w * T / G;
  const long long f1 = (long long)(w + 1) * T / G;

  unsigned lane_off[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const unsigned r = 4 * qq + (lane >> 4);
    lane_off[qq] = r * 256u + 16u * ((unsigned)(lane & 15) ^ r);
  }

  LDS_AS uint8_t* ring0 = (LDS_AS uint8_t*)g_stage0 + wave * kStageBytes;
  LDS_AS uint8_t* ring1 = (LDS_AS uint8_t*)g_stage1 + wave * kStageBytes;
  LDS_AS float* part0 = (LDS_AS float*)g_stage0;   // fold buffers reuse the rings once a segment is done
  LDS_AS float* part1 = (LDS_AS float*)g_stage1;

  WaveState<RB> st;
  const LDS_AS uint8_t* qlane = (const LDS_AS uint8_t*)g_qfrag + lane * 16;

  long long off = 0;
  for (int b = 0; b < a.batch && off < f1; ++b) {
    const int L = clamp_len(context_lens[b], NQ, a.max_context_len);
    const int Tb = (L + kTile - 1) / kTile;
    if (off + Tb <= f0) {
      off += Tb;
      continue;
    }
    const int S = split_size_of(L, NS, a.split_tokens);
    const int tps = S / kTile;
    const int npages = (L + kPage - 1) / kPage;
    const int t_lo = (int)max(f0 - off, 0LL);
    const int t_hi = (int)min(f1 - off, (long long)Tb);
    const int32_t* bt = block_table + (size_t)b * a.max_blocks;

    // Stage Q of sequence b in LDS in MFMA B-operand order: fragment (rb, m),
    // lane (n,g) = Q[row 16rb+n][64g + 8m + 0..7] (zero for padding rows).
    int limit[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = 16 * rb + n;
      limit[rb] = row < ROWS ? (L - NQ + row / kQHeads) : -1;
    }
    __syncthreads();
    for (int u = tid; u < RB * 8 * 64; u += kThreads) {
      const int ul = u & 63, um = (u >> 6) & 7, urb = u >> 9;
      const int row = 16 * urb + (ul & 15);
      half8 v = half8{};
      if (row < ROWS) v = *(const half8*)(q + ((size_t)b * ROWS + row) * kHeadDim + 64 * (ul >> 4) + 8 * um);
      *(LDS_AS half8*)((LDS_AS uint8_t*)g_qfrag + u * 16) = v;
    }
    __syncthreads();

    for (int jsp = t_lo / tps; jsp * tps < t_hi; ++jsp) {
      const int split_lo = jsp * tps;
      const int split_hi = min(split_lo + tps, Tb);
      const int s_lo = max(t_lo, split_lo);
      const int s_hi = min(t_hi, split_hi);

      __syncthreads();   // previous segment's fold buffers overlap the rings
      state_reset(st);
      const int t_first = s_lo + wave;
      int t = t_first;
      int stage = 0;
      if (t < s_hi) {
        const int p0 = bt[2 * t];
        const int p1 = (2 * t + 1 < npages) ? bt[2 * t + 1] : p0;
        issue_tile(k_cache, v_cache, p0, p1, ring0, lane_off);
      }
      while (t < s_hi) {
        const int tn = t + kWaves;
        if (tn < s_hi) {
          const int p0 = bt[2 * tn];
          const int p1 = (2 * tn + 1 < npages) ? bt[2 * tn + 1] : p0;
          issue_tile(k_cache, v_cache, p0, p1, stage ? ring0 : ring1, lane_off);
          wait_vmcnt<16>();
        } else {
          wait_vmcnt<0>();
        }
        if (compute_tile<RB>(st, qlane, stage ? ring1 : ring0, t * kTile, L, limit, c2, n, g)) {
          // A row outgrew its reference max: raise every reference to the running
          // max and redo this wave's tiles (only adversarial score growth gets here).
          wait_vmcnt<0>();
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            st.m_ref[rb] = st.m_max[rb];
            st.l_sum[rb] = 0.f;
            st.l_cmp[rb] = 0.f;
#pragma unroll
            for (int mb = 0; mb < 16; ++mb) st.o[mb][rb] = float4v{0.f, 0.f, 0.f, 0.f};
          }
          t = t_first;
          stage = 0;
          const int p0 = bt[2 * t];
          const int p1 = (2 * t + 1 < npages) ? bt[2 * t + 1] : p0;
          issue_tile(k_cache, v_cache, p0, p1, ring0, lane_off);
          continue;
        }
        stage ^= 1;
        t = tn;
      }
      finalize_wave<RB>(st);

      // ---- fold the four waves: (0<-1, 2<-3), then 0<-2
      __syncthreads();
      if (wave == 1) write_lds_partial<RB>(st, part0, n, g);
      if (wave == 3) write_lds_partial<RB>(st, part1, n, g);
      __syncthreads();
      if (wave == 0) merge_lds_partial<RB>(st, part0, c2, n, g);
      if (wave == 2) merge_lds_partial<RB>(st, part1, c2, n, g);
      __syncthreads();
      if (wave == 2) write_lds_partial<RB>(st, part0, n, g);
      __syncthreads();
      if (wave == 0) merge_lds_partial<RB>(st, part0, c2, n, g);

      const size_t gsi = (size_t)b * NS + jsp;
      const bool whole = (s_lo == split_lo) && (s_hi == split_hi);
      if (whole) {
        if (wave == 0) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int row = 16 * rb + n;
            if (row < ROWS) {
              const size_t ws = ((size_t)b * ROWS + row) * NS + jsp;
              const bool empty = st.m_max[rb] == kNegInf;
#pragma unroll
              for (int mb = 0; mb < 16; ++mb) {
                *(float4v*)(a.ws_num + ws * kHeadDim + 16 * mb + 4 * g) = st.o[mb][rb] * ofac;
                __builtin_amdgcn_sched_barrier(0);
              }
              if (g == 0) {
                a.ws_max[ws] = empty ? kNegInf : st.m_max[rb] * c;
                a.ws_sum[ws] = st.l_sum[rb];
              }
            }
          }
        }
      } else {
        // Partial of a shared split: publish it, then the last arriver merges.
        const long long fs = off + split_lo;
        const long long fe = off + split_hi - 1;
        const int w_first = owner_of(fs, T, G);
        const int w_last = owner_of(fe, T, G);
        float* slot = a.partials + ((size_t)w + gsi) * kSlotFloats;
        if (wave == 0) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int row = 16 * rb + n;
#pragma unroll
            for (int mb = 0; mb < 16; ++mb) {
              *(float4v*)(slot + row * kHeadDim + 16 * mb + 4 * g) = st.o[mb][rb];
              __builtin_amdgcn_sched_barrier(0);
            }
            if (g == 0) {
              slot[kMaxRows * kHeadDim + row] = st.m_max[rb];
              slot[kMaxRows * kHeadDim + kMaxRows + row] = st.l_sum[rb];
            }
          }
        }
        __threadfence();
        __syncthreads();
        if (tid == 0) {
          const int prev = atomicAdd(a.counters + gsi, 1);
          g_last_flag = (prev == w_last - w_first);
        }
        __syncthreads();
        if (g_last_flag) {
          __threadfence();
          if (tid == 0) a.counters[gsi] = 0;   // ready for the next call
          const int np = w_last - w_first + 1;
          for (int u = tid; u < ROWS * (kHeadDim / 4); u += kThreads) {
            const int row = u / (kHeadDim / 4);
            const int dq = u % (kHeadDim / 4);
            float M = kNegInf;
            for (int pi = 0; pi < np; ++pi) {
              const float* ps = a.partials + ((size_t)(w_first + pi) + gsi) * kSlotFloats;
              M = fmaxf(M, __builtin_nontemporal_load(ps + kMaxRows * kHeadDim + row));
            }
            float4v acc = {0.f, 0.f, 0.f, 0.f};
            float l = 0.f;
            if (M != kNegInf) {
              for (int pi = 0; pi < np; ++pi) {
                const float* ps = a.partials + ((size_t)(w_first + pi) + gsi) * kSlotFloats;
                const float mp = __builtin_nontemporal_load(ps + kMaxRows * kHeadDim + row);
                if (mp == kNegInf) continue;
                const float e = fast_exp2((mp - M) * c2);
                const float4v op = __builtin_nontemporal_load((const float4v*)(ps + row * kHeadDim + 4 * dq));
                acc += op * e;
                l += __builtin_nontemporal_load(ps + kMaxRows * kHeadDim + kMaxRows + row) * e;
              }
            }
            const size_t ws = ((size_t)b * ROWS + row) * NS + jsp;
            *(float4v*)(a.ws_num + ws * kHeadDim + 4 * dq) = acc * ofac;
            if (dq == 0) {
              a.ws_max[ws] = (M == kNegInf) ? kNegInf : M * c;
              a.ws_sum[ws] = l;
            }
          }
        }
      }
    }
    // The workgroup holding the sequence's last tile also writes the splits
    // that start at or beyond L (empty for every row).
    if (off + Tb - 1 >= f0 && off + Tb - 1 < f1) {
      const int first_empty = (Tb + tps - 1) / tps;
      const int n_empty = NS - first_empty;
      for (int u = tid; u < ROWS * n_empty * (kHeadDim / 4); u += kThreads) {
        const int dq = u % (kHeadDim / 4);
        const int rj = u / (kHeadDim / 4);
        const int row = rj / n_empty;
        const int jj = first_empty + rj % n_empty;
        const size_t ws = ((size_t)b * ROWS + row) * NS + jj;
        *(float4v*)(a.ws_num + ws * kHeadDim + 4 * dq) = float4v{0.f, 0.f, 0.f, 0.f};
        if (dq == 0) {
          a.ws_max[ws] = kNegInf;
          a.ws_sum[ws] = 0.f;
        }
      }
    }
    off += Tb;
  }
}

}  // namespace

hipError_t launch_split(const SplitArgs& a, int workgroups, hipStream_t stream) {
  const int rb = (a.num_q * kQHeads + 15) / 16;
  dim3 grid(workgroups), block(kThreads);
  switch (rb) {
    case 1: hipLaunchKernelGGL(split_kernel<1>, grid, block, 0, stream, a.q, a.k_cache, a.v_cache,
                                 a.block_table, a.context_lens, a.k_scale, a.v_scale, a); break;
    case 2: hipLaunchKernelGGL(split_kernel<2>, grid, block, 0, stream, a.q, a.k_cache, a.v_cache,
                                 a.block_table, a.context_lens, a.k_scale, a.v_scale, a); break;
    default: hipLaunchKernelGGL(split_kernel<3>, grid, block, 0, stream, a.q, a.k_cache, a.v_cache,
                                 a.block_table, a.context_lens, a.k_scale, a.v_scale, a); break;
  }
  return hipGetLastError();
}

}  // namespace dfv
