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
// Work decomposition (MI355X: 256 CUs in 8 XCDs, 64-wide waves, 160 KB LDS/CU):
//   * One workgroup per (sequence, logical split, 16-row block of the 6q query
//     rows): 80 * 3 = 240 workgroups at q8, each streaming its whole split, so
//     no state ever crosses workgroups and every split state is written once,
//     straight into the workspace.  Workgroups are dispatched to XCDs round
//     robin (workgroup w runs on XCD w % 8); the row blocks of one split get ids
//     congruent mod 8, so they share that XCD's L2 and the split's KV bytes come
//     from HBM once.
//   * Four waves (one per SIMD) take the split's 32-key tiles in turn, each with
//     its own state for the 16 rows; at the end the four states are folded in
//     LDS in wave order (byte-deterministic).
//   * Each wave streams its tiles through a private two-stage LDS ring with
//     16-byte direct-to-LDS loads (global_load_lds_dwordx4); one 4 KB page is four
//     fully coalesced wave instructions.  Inside a 256-byte token row the 16-byte
//     chunks are XOR-swizzled by the row's page slot so operand reads from LDS
//     are bank-conflict free.
//   * QK^T runs as S^T = K * Q^T on v_mfma_f32_16x16x32_f16 (A = 16 keys x 32
//     dims of K, B = 32 dims x 16 rows of Q held in registers).  The C layout
//     leaves each lane 4 keys of one row, so a row max is an in-lane max plus
//     two cross-lane steps (permlane16/32 swaps).
//   * Each wave fixes a per-row reference max at the first tile where the row
//     sees a key and never rescales its accumulators inside the tile loop.
//     P = exp(s - m_ref) * 2^3 is carried as FP16 hi + FP16 lo (the pages'
//     probability residual products, ~22 bits of P); should a row's running max
//     outgrow its reference by more than 2^12 (beyond FP16 range for P), the
//     wave raises the reference and redoes its tiles, which only strongly
//     growing scores trigger.  The fold renormalises every state to its true max.
//     This is an exact re-association of the pages' 32-key online update; it is
//     used because a data-dependent rescale of the AGPR accumulators makes the
//     compiler shadow them in VGPRs.
//   * PV runs as O^T += V^T * P^T on the same MFMA; the V operand (8 keys of one
//     dimension per lane) comes straight out of LDS with the transposing read
//     ds_read_b64_tr_b8.
//   * E4M3 is decoded in registers with v_cvt_scalef32_pk_f16_fp8 (OCP on gfx950,
//     two codes per instruction, exact in FP16).  The per-tensor scales are not
//     applied during decode: k_scale is folded into the score scale and v_scale
//     into the stored numerator.
#include "dfv_common.h"

namespace dfv {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
constexpr float kPScale = 8.0f;              // 2^3: P * 2^3 <= 2^15 keeps FP16 hi finite
constexpr float kRestartLog2 = 12.0f;        // P may reach 2^12 before a wave restarts

// Eight E4M3 codes (two dwords) to eight FP16 values, two codes per instruction.
__device__ __forceinline__ half8 decode8(unsigned lo, unsigned hi) {
  const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
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
  const float t = sum + x;
  comp += (fabsf(sum) >= fabsf(x)) ? ((sum - t) + x) : ((x - t) + sum);
  sum = t;
}

// 16-byte direct-to-LDS load: lane l's 16 bytes (uniform base + per-lane offset)
// land at LDS address dst + 16*l.  Issued through inline asm so the compiler does
// not add its conservative "wait for every LDS DMA" before unrelated LDS reads;
// the tile loop waits on vmcnt itself (vector loads complete in order, so extra
// outstanding loads only ever make the compiler's own waits stricter).  s_nop
// covers the M0 write -> LDS-DMA wait state.
__device__ __forceinline__ void lds_dma16(const uint8_t* base, unsigned off, LDS_AS uint8_t* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(m0) : "memory", "m0");
}

// a ^ k computed in the loop body.  The swizzled LDS addresses of a tile are
// loop-invariant; left to itself the compiler hoists all of them out of the
// tile loop and spills them, and every spill reload waits for in-flight DMAs.
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

// Per-wave softmax state for the 16 rows of the block; lane (n, g) owns row n.
struct WaveState {
  float4v o[16];   // O^T accumulators (x 2^3, relative to m_ref): dims 16mb + 4g + 0..3 of row n
  float m_ref;     // reference max (raw dot-product units); -inf until the row sees a key
  float m_max;     // true running max (raw units)
  float l_sum;     // this lane's compensated partial sum of P (relative to m_ref)
  float l_cmp;
};

__device__ __forceinline__ void state_reset(WaveState& st) {
  st.m_ref = kNegInf;
  st.m_max = kNegInf;
  st.l_sum = 0.f;
  st.l_cmp = 0.f;
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) st.o[mb] = float4v{0.f, 0.f, 0.f, 0.f};
}

// One 32-key tile: QK^T, softmax against the fixed reference max, PV with
// P = hi + lo.  Returns true (before touching O) when the row max has outgrown
// the reference by more than 2^kRestartLog2; the caller then restarts.
// `masked` tiles hold keys past some row's causal bound or past L.
__device__ __forceinline__ bool compute_tile(WaveState& st, const half8 (&qf)[8],
                                             const LDS_AS uint8_t* kl, int t0, int L, int limit,
                                             bool masked, float c2, int n, int g) {
  const LDS_AS uint8_t* vl = kl + 2 * kPageBytes;
  // ---- S^T = K * Q^T for the tile's two 16-key blocks
  float4v sacc0 = {0.f, 0.f, 0.f, 0.f}, sacc1 = {0.f, 0.f, 0.f, 0.f};
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
    sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(c0[0], c0[1]), qf[2 * i], sacc0, 0, 0, 0);
    sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(c1[0], c1[1]), qf[2 * i], sacc1, 0, 0, 0);
    sacc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(c0[2], c0[3]), qf[2 * i + 1], sacc0, 0, 0, 0);
    sacc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(c1[2], c1[3]), qf[2 * i + 1], sacc1, 0, 0, 0);
  }
  // ---- scores (lane holds keys t0 + 16kb + 4g + r of row n), row max, reference
  float s[8] = {sacc0[0], sacc0[1], sacc0[2], sacc0[3], sacc1[0], sacc1[1], sacc1[2], sacc1[3]};
  if (masked) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (t0 + 16 * (k >> 2) + 4 * g + (k & 3) > limit) s[k] = kNegInf;
  }
  float tmax = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
  tmax = max_x32(max_x16(tmax));
  st.m_max = fmaxf(st.m_max, tmax);
  if (st.m_ref == kNegInf) st.m_ref = tmax;            // first visible keys of the row (or still -inf)
  const bool restart = (st.m_max - st.m_ref) * c2 > kRestartLog2;   // false while -inf
  if (__builtin_amdgcn_ballot_w64(restart)) return true;
  // ---- P * 2^3 = exp2((s - m_ref) * c2) * 2^3 as FP16 hi + lo; compensated sums.
  // (s - m_ref) first: exact for keys near the max, so P keeps full relative
  // precision even when |m_ref * c2| is large.
  const bool live = st.m_ref != kNegInf;
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    p[k] = live ? fast_exp2((s[k] - st.m_ref) * c2) : 0.f;
    psum += p[k];
  }
  comp_add(st.l_sum, st.l_cmp, psum);
  half8 phi, plo;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float ph = p[k] * kPScale;
    phi[k] = (_Float16)ph;
    plo[k] = (_Float16)(ph - (float)phi[k]);
  }
  // ---- O^T += V^T * P^T; lane (n, g) reads 8 keys of dimension 16mb + n.
  // MFMA K-index 8g + k of this lane holds key 4g + k (k < 4) or 16 + 4g + k - 4,
  // matching the score layout above.  Keys at or past L hold unrelated bytes;
  // their codes are cleared to +0 before decode so 0 * NaN never reaches O.
  const int j = n >> 1;
  const int vslot = 4 * g + (j & 3);
  const unsigned vrow = (unsigned)(uintptr_t)(vl + (j >> 2) * kPageBytes + vslot * 256 + 8 * (n & 1));
  const unsigned vsw = 16u * vslot;
  unsigned keep_lo = 0xffffffffu, keep_hi = 0xffffffffu;
  if (masked) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (t0 + 4 * g + k >= L) keep_lo &= ~(0xffu << (8 * k));
      if (t0 + 16 + 4 * g + k >= L) keep_hi &= ~(0xffu << (8 * k));
    }
  }
  int2v vnext = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS int2v*)(uintptr_t)(vrow + vsw));
#pragma unroll
  for (int mb = 0; mb < 16; ++mb) {
    const int2v vr = vnext;
    if (mb < 15)
      vnext = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (LDS_AS int2v*)(uintptr_t)(vrow + xor_in_loop(vsw, 16u * (mb + 1))));
    const half8 va = decode8((unsigned)vr[0] & keep_lo, (unsigned)vr[1] & keep_hi);
    st.o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, phi, st.o[mb], 0, 0, 0);
    st.o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, plo, st.o[mb], 0, 0, 0);
  }
  return false;
}

__shared__ __attribute__((aligned(16))) uint8_t g_stage0[kStageArray];
__shared__ __attribute__((aligned(16))) uint8_t g_stage1[kStageArray];

__device__ __forceinline__ int split_size_of(int L, int ns, int fixed) {
  if (fixed) return fixed;
  const int per = (L + ns - 1) / ns;
  return kTile * ((per + kTile - 1) / kTile);
}

__device__ __forceinline__ int clamp_len(int L, int nq, int maxL) { return min(max(L, nq), maxL); }

// Workgroup w -> (split group, row block): groups (sequence, split) are dealt
// to XCDs round robin and the RB row blocks of a group get workgroup ids
// 8*(RB*(grp/8) + r) + grp%8, all on XCD grp % 8.
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
  const int NQ = a.num_q;
  const int ROWS = NQ * kQHeads;
  const int RB = (ROWS + 15) / 16;
  const int NS = a.num_splits;
  const int w = blockIdx.x;
  const int grp = 8 * ((w >> 3) / RB) + (w & 7);
  const int rb = (w >> 3) % RB;
  if (grp >= a.batch * NS) return;
  const int b = grp / NS;
  const int jsp = grp % NS;

  const float c = a.softmax_scale * k_scale[0];
  const float c2 = c * kLog2e;
  const float ofac = v_scale[0] * (1.0f / kPScale);
  const int L = clamp_len(context_lens[b], NQ, a.max_context_len);
  const int S = split_size_of(L, NS, a.split_tokens);
  const int t_lo = jsp * (S / kTile);
  const int t_hi = min((jsp + 1) * (S / kTile), (L + kTile - 1) / kTile);
  const int npages = (L + kPage - 1) / kPage;
  const int32_t* bt = block_table + (size_t)b * a.max_blocks;

  // Q of the block's 16 rows in the B-operand layout: lane (n,g), fragment m
  // holds Q[row 16rb+n][64g + 8m + 0..7] (zero for rows past 6q).
  const int row = 16 * rb + n;
  const bool row_ok = row < ROWS;
  const int limit = row_ok ? (L - NQ + row / kQHeads) : -1;
  half8 qf[8];
  {
    const _Float16* qrow = q + ((size_t)b * ROWS + (row_ok ? row : 0)) * kHeadDim + 64 * g;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const half8 v = *(const half8*)(qrow + 8 * m);
      qf[m] = row_ok ? v : half8{};
    }
  }
  const int first_masked = (L - NQ) / kTile;   // tiles from here on hold keys some row must not see

  unsigned lane_off[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const unsigned r = 4 * qq + (lane >> 4);
    lane_off[qq] = r * 256u + 16u * ((unsigned)(lane & 15) ^ r);
  }
  LDS_AS uint8_t* ring0 = (LDS_AS uint8_t*)g_stage0 + wave * kStageBytes;
  LDS_AS uint8_t* ring1 = (LDS_AS uint8_t*)g_stage1 + wave * kStageBytes;

  WaveState st;
  state_reset(st);
  const int t_first = t_lo + wave;
  int t = t_first;
  int stage = 0;
  if (t < t_hi) {
    const int p0 = bt[2 * t];
    const int p1 = (2 * t + 1 < npages) ? bt[2 * t + 1] : p0;
    issue_tile(k_cache, v_cache, p0, p1, ring0, lane_off);
  }
  while (t < t_hi) {
    const int tn = t + kWaves;
    if (tn < t_hi) {
      const int p0 = bt[2 * tn];
      const int p1 = (2 * tn + 1 < npages) ? bt[2 * tn + 1] : p0;
      issue_tile(k_cache, v_cache, p0, p1, stage ? ring0 : ring1, lane_off);
      wait_vmcnt<16>();
    } else {
      wait_vmcnt<0>();
    }
    if (compute_tile(st, qf, stage ? ring1 : ring0, t * kTile, L, limit, t >= first_masked, c2, n, g)) {
      // The row max outgrew its reference: raise the reference to the running
      // max and redo this wave's tiles.
      wait_vmcnt<0>();
      st.m_ref = st.m_max;
      st.l_sum = 0.f;
      st.l_cmp = 0.f;
#pragma unroll
      for (int mb = 0; mb < 16; ++mb) st.o[mb] = float4v{0.f, 0.f, 0.f, 0.f};
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
  // Row sum of this wave: the four lanes of a row hold disjoint key subsets.
  const float l_wave = sum_x32(sum_x16(st.l_sum)) + sum_x32(sum_x16(st.l_cmp));

  // ---- fold the four waves in LDS, in wave order.  Each wave parks its state
  // in its own ring areas (its DMAs are complete and it no longer reads them):
  // O rows of 1 KB in stage 0, 16-byte chunk c of row r at position c ^ r (bank
  // conflict free), and (m_ref, m_max, l) per row in stage 1.  Then every
  // thread merges 16 dimensions of one row.
  LDS_AS float* park_o = (LDS_AS float*)((LDS_AS uint8_t*)g_stage0 + wave * kStageBytes);
  LDS_AS float* park_m = (LDS_AS float*)((LDS_AS uint8_t*)g_stage1 + wave * kStageBytes);
#pragma unroll
  for (int mb = 0; mb < 16; ++mb)
    *(LDS_AS float4v*)(park_o + n * kHeadDim + 4 * ((4 * mb + g) ^ n)) = st.o[mb];
  if (g == 0) {
    park_m[n] = st.m_ref;
    park_m[16 + n] = st.m_max;
    park_m[32 + n] = l_wave;
  }
  __syncthreads();
  const int fr = tid >> 4;          // row within the block
  const int fq = (tid & 15) * 4;    // first of 4 float4 chunks (16 dimensions)
  float mref[kWaves];
  float M = kNegInf;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const LDS_AS float* pm = (const LDS_AS float*)((LDS_AS uint8_t*)g_stage1 + v * kStageBytes);
    mref[v] = pm[fr];
    M = fmaxf(M, pm[16 + fr]);
  }
  float4v acc[4] = {};
  float l = 0.f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const LDS_AS float* po = (const LDS_AS float*)((LDS_AS uint8_t*)g_stage0 + v * kStageBytes);
    const LDS_AS float* pm = (const LDS_AS float*)((LDS_AS uint8_t*)g_stage1 + v * kStageBytes);
    const float e = (mref[v] != kNegInf) ? fast_exp2((mref[v] - M) * c2) : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      acc[k] += *(const LDS_AS float4v*)(po + fr * kHeadDim + 4 * ((fq + k) ^ fr)) * e;
    l += pm[32 + fr] * e;
  }
  const int grow = 16 * rb + fr;
  if (grow < ROWS) {
    const size_t ws = ((size_t)b * ROWS + grow) * NS + jsp;
#pragma unroll
    for (int k = 0; k < 4; ++k) *(float4v*)(a.ws_num + ws * kHeadDim + 4 * (fq + k)) = acc[k] * ofac;
    if ((tid & 15) == 0) {
      a.ws_max[ws] = (M == kNegInf) ? kNegInf : M * c;
      a.ws_sum[ws] = l;
    }
  }
}

}  // namespace

int split_grid(int batch, int num_q, int num_splits) {
  const int rb = (num_q * kQHeads + 15) / 16;
  const int groups = batch * num_splits;
  return 8 * rb * ((groups + 7) / 8);
}

hipError_t launch_split(const SplitArgs& a, hipStream_t stream) {
  const int grid = split_grid(a.batch, a.num_q, a.num_splits);
  hipLaunchKernelGGL(split_kernel, dim3(grid), dim3(kThreads), 0, stream, a.q, a.k_cache, a.v_cache,
                     a.block_table, a.context_lens, a.k_scale, a.v_scale, a);
  return hipGetLastError();
}

}  // namespace dfv
