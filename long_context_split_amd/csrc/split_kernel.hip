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
//   * Each logical split is cut into C key chunks (C = 3 for one sequence and
//     80 splits: 240 workgroups, about one per CU).  Workgroups never talk to
//     each other: with C = 1 a workgroup writes its split's workspace entry,
//     with C > 1 it writes its chunk state to scratch and a separate merge
//     pass (fused into the combine kernel when the output is wanted) reduces
//     the C states of a split in chunk order, so results are deterministic.
//   * Four waves (one per SIMD) take the chunk's 32-key tiles in turn.  Each
//     wave owns all 6q query rows (up to three 16-row blocks), so every K and V
//     byte is decoded once and each decoded K fragment feeds every row block
//     (the pages' reuse of one K fragment across three M16 products, [#589]
//     Purpose).
//   * Each wave streams its tiles through a private two-stage LDS ring with
//     16-byte direct-to-LDS loads (global_load_lds_dwordx4); one 4 KB page is four
//     fully coalesced wave instructions.  Inside a 256-byte token row the 16-byte
//     chunks are XOR-swizzled by the row's page slot so operand reads from LDS
//     are bank-conflict free.
//   * QK^T runs as S^T = K * Q^T on v_mfma_f32_16x16x32_f16 (A = 16 keys x 32
//     dims of K, B = 32 dims x 16 rows of Q, staged once in LDS in operand
//     order).  The C layout leaves each lane 4 keys of one row, so a row max is
//     an in-lane max plus two cross-lane steps (permlane16/32 swaps).
//   * Each wave fixes a per-row reference max at the first tile where the row
//     sees a key and never rescales its accumulators inside the tile loop.
//     P = exp(s - m_ref) * 2^3 is carried as FP16 hi + FP16 lo (the pages'
//     probability residual products, ~22 bits of P); should a row's running max
//     outgrow its reference by more than 2^12 (beyond FP16 range for P), the
//     wave raises the reference and redoes its tiles, which only strongly
//     growing scores trigger.  The folds renormalise every state to its true
//     max.  This is an exact re-association of the pages' 32-key online update;
//     it is used because a data-dependent rescale of the AGPR accumulators makes
//     the compiler shadow them in VGPRs.
//   * PV runs as O^T += V^T * P^T on the same MFMA; the V operand (8 keys of one
//     dimension per lane) comes straight out of LDS with the transposing read
//     ds_read_b64_tr_b8.
//   * The four wave states are folded in LDS as a reduce-scatter: afterwards
//     wave v holds dimensions 64v..64v+63 of all rows, merged in wave order.
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

// Per-wave softmax state for RB 16-row blocks; lane (n, g) owns row 16rb + n.
template <int RB>
struct WaveState {
  float4v o[16][RB];   // O^T accumulators (x 2^3, relative to m_ref): dims 16mb + 4g + 0..3
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

// One 32-key tile: QK^T, softmax against the fixed reference max, PV with
// P = hi + lo.  Returns true (before touching O) when some row max has outgrown
// its reference by more than 2^kRestartLog2; the caller then restarts.
// `masked` tiles hold keys past some row's causal bound or past L.
// qlane points at this lane's Q fragments in LDS: fragment (rb, m) holds
// Q[row 16rb+n][64g + 8m + 0..7] at qlane + (rb*8 + m)*1024.
template <int RB>
__device__ __forceinline__ bool compute_tile(WaveState<RB>& st, const LDS_AS uint8_t* qlane,
                                             const LDS_AS uint8_t* kl, int t0, int L,
                                             const int (&limit)[RB], bool masked, float c2, int n, int g) {
  const LDS_AS uint8_t* vl = kl + 2 * kPageBytes;
  // ---- S^T = K * Q^T for the tile's two 16-key blocks and every row block
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
      sacc[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k10, qa, sacc[1][rb], 0, 0, 0);
      sacc[0][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k01, qb, sacc[0][rb], 0, 0, 0);
      sacc[1][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k11, qb, sacc[1][rb], 0, 0, 0);
    }
  }
  // ---- scores (lane holds keys t0 + 16kb + 4g + r of its row), row max, reference
  float s[RB][8];
  bool restart = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int k = 0; k < 8; ++k) s[rb][k] = sacc[k >> 2][rb][k & 3];
    if (masked) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + 16 * (k >> 2) + 4 * g + (k & 3) > limit[rb]) s[rb][k] = kNegInf;
    }
    float tmax = fmaxf(fmaxf(fmaxf(s[rb][0], s[rb][1]), fmaxf(s[rb][2], s[rb][3])),
                       fmaxf(fmaxf(s[rb][4], s[rb][5]), fmaxf(s[rb][6], s[rb][7])));
    tmax = max_x32(max_x16(tmax));
    st.m_max[rb] = fmaxf(st.m_max[rb], tmax);
    if (st.m_ref[rb] == kNegInf) st.m_ref[rb] = tmax;   // first visible keys of the row (or still -inf)
    restart |= (st.m_max[rb] - st.m_ref[rb]) * c2 > kRestartLog2;   // false while -inf
  }
  if (__builtin_amdgcn_ballot_w64(restart)) return true;
  // ---- P * 2^3 = exp2((s - m_ref) * c2) * 2^3 as FP16 hi + lo; compensated sums.
  // (s - m_ref) first: exact for keys near the max, so P keeps full relative
  // precision even when |m_ref * c2| is large.
  half8 phi[RB], plo[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bool live = st.m_ref[rb] != kNegInf;
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = live ? fast_exp2((s[rb][k] - st.m_ref[rb]) * c2) : 0.f;
      psum += p;
      const float ph = p * kPScale;
      phi[rb][k] = (_Float16)ph;
      plo[rb][k] = (_Float16)(ph - (float)phi[rb][k]);
    }
    comp_add(st.l_sum[rb], st.l_cmp[rb], psum);
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
    // hi products of every row block first, then lo: dependent MFMAs on one
    // accumulator are RB instructions apart instead of back to back.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      st.o[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, phi[rb], st.o[mb][rb], 0, 0, 0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      st.o[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, plo[rb], st.o[mb][rb], 0, 0, 0);
  }
  return false;
}

__shared__ __attribute__((aligned(16))) uint8_t g_stage0[kStageArray];
__shared__ __attribute__((aligned(16))) uint8_t g_stage1[kStageArray];
__shared__ __attribute__((aligned(16))) uint8_t g_qfrag[(kMaxRows / 16) * 8 * 1024];
__shared__ float g_meta[kWaves][3][kMaxRows];   // per wave: m_ref, m_max, l of every row

__device__ __forceinline__ int split_size_of(int L, int ns, int fixed) {
  if (fixed) return fixed;
  const int per = (L + ns - 1) / ns;
  return kTile * ((per + kTile - 1) / kTile);
}

__device__ __forceinline__ int clamp_len(int L, int nq, int maxL) { return min(max(L, nq), maxL); }

// LDS slot of wave s during the fold (4 slots of RB * 8 KB over the two rings).
template <int RB>
__device__ __forceinline__ LDS_AS uint8_t* fold_slot(int s) {
  return (LDS_AS uint8_t*)(s < 2 ? g_stage0 : g_stage1) + (s & 1) * (RB * 8 * 1024);
}

// Workgroup w -> (split group, chunk): groups (sequence, split) are dealt to
// XCDs round robin and the C chunks of a group get workgroup ids
// 8*(C*(grp/8) + c) + grp%8, all on XCD grp % 8.
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
  const int NQ = a.num_q;
  const int ROWS = NQ * kQHeads;
  const int NS = a.num_splits;
  const int C = a.chunks;
  const int w = blockIdx.x;
  const int grp = 8 * ((w >> 3) / C) + (w & 7);
  const int chunk = (w >> 3) % C;
  if (grp >= a.batch * NS) return;
  const int b = grp / NS;
  const int jsp = grp % NS;

  const float c = a.softmax_scale * k_scale[0];
  const float c2 = c * kLog2e;
  const float ofac = v_scale[0] * (1.0f / kPScale);
  const int L = clamp_len(context_lens[b], NQ, a.max_context_len);
  const int S = split_size_of(L, NS, a.split_tokens);
  const int Tb = (L + kTile - 1) / kTile;
  const int s_lo = min(jsp * (S / kTile), Tb);
  const int s_hi = min((jsp + 1) * (S / kTile), Tb);
  const int nt = s_hi - s_lo;
  const int t_lo = s_lo + (chunk * nt) / C;
  const int t_hi = s_lo + ((chunk + 1) * nt) / C;
  const int npages = (L + kPage - 1) / kPage;
  const int32_t* bt = block_table + (size_t)b * a.max_blocks;

  unsigned lane_off[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const unsigned r = 4 * qq + (lane >> 4);
    lane_off[qq] = r * 256u + 16u * ((unsigned)(lane & 15) ^ r);
  }
  LDS_AS uint8_t* ring0 = (LDS_AS uint8_t*)g_stage0 + wave * kStageBytes;
  LDS_AS uint8_t* ring1 = (LDS_AS uint8_t*)g_stage1 + wave * kStageBytes;
  const int t_first = t_lo + wave;
  // First tile in flight before anything else.
  if (t_first < t_hi) {
    const int p0 = bt[2 * t_first];
    const int p1 = (2 * t_first + 1 < npages) ? bt[2 * t_first + 1] : p0;
    issue_tile(k_cache, v_cache, p0, p1, ring0, lane_off);
  }

  // Q of sequence b in LDS in MFMA B-operand order: fragment (rb, m), lane
  // (n,g) = Q[row 16rb+n][64g + 8m + 0..7], zero for rows past 6q.
  for (int u = tid; u < RB * 8 * 64; u += kThreads) {
    const int ul = u & 63, um = (u >> 6) & 7, urb = u >> 9;
    const int row = 16 * urb + (ul & 15);
    half8 v = half8{};
    if (row < ROWS) v = *(const half8*)(q + ((size_t)b * ROWS + row) * kHeadDim + 64 * (ul >> 4) + 8 * um);
    *(LDS_AS half8*)((LDS_AS uint8_t*)g_qfrag + u * 16) = v;
  }
  __syncthreads();
  const LDS_AS uint8_t* qlane = (const LDS_AS uint8_t*)g_qfrag + lane * 16;
  int limit[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 16 * rb + n;
    limit[rb] = row < ROWS ? (L - NQ + row / kQHeads) : -1;
  }
  const int first_masked = (L - NQ) / kTile;   // tiles from here on hold keys some row must not see

  WaveState<RB> st;
  state_reset(st);
  int t = t_first;
  int stage = 0;
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
    if (compute_tile<RB>(st, qlane, stage ? ring1 : ring0, t * kTile, L, limit, t >= first_masked, c2, n,
                         g)) {
      // A row max outgrew its reference: raise every reference to the running
      // max and redo this wave's tiles.
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

  // ---- fold the four wave states (reduce-scatter through LDS).  Row sums: the
  // four lanes of a row hold disjoint key subsets.
  if (g == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      g_meta[wave][0][16 * rb + n] = st.m_ref[rb];
      g_meta[wave][1][16 * rb + n] = st.m_max[rb];
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l = sum_x32(sum_x16(st.l_sum[rb])) + sum_x32(sum_x16(st.l_cmp[rb]));
    if (g == 0) g_meta[wave][2][16 * rb + n] = l;
  }
  __syncthreads();   // every wave is done with its ring; meta is complete
  // Merge weights of this lane's rows: M = max over waves of m_max, wave s
  // contributes with e_s = 2^((m_ref_s - M) * c2).
  float M[RB], e[kWaves][RB], Lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 16 * rb + n;
    M[rb] = kNegInf;
#pragma unroll
    for (int s = 0; s < kWaves; ++s) M[rb] = fmaxf(M[rb], g_meta[s][1][row]);
    Lsum[rb] = 0.f;
#pragma unroll
    for (int s = 0; s < kWaves; ++s) {
      const float mr = g_meta[s][0][row];
      e[s][rb] = (mr != kNegInf) ? fast_exp2((mr - M[rb]) * c2) : 0.f;
      Lsum[rb] += g_meta[s][2][row] * e[s][rb];
    }
  }
  // Two halves of the dimensions; in half h, waves 2h and 2h+1 merge the
  // quarters 2h and 2h+1 (16-dim blocks mb = 4v .. 4v+3).
  float4v res[4][RB];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h) __syncthreads();   // readers of the first half are done
    LDS_AS uint8_t* mine = fold_slot<RB>(wave);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int mbl = 0; mbl < 8; ++mbl)
        *(LDS_AS float4v*)(mine + ((rb * 8 + mbl) * 64 + lane) * 16) = st.o[8 * h + mbl][rb];
    __syncthreads();
    if ((wave >> 1) == h) {
      const int base = 4 * (wave & 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int k = 0; k < 4; ++k) res[k][rb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kWaves; ++s) {
        const LDS_AS uint8_t* src = fold_slot<RB>(s);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            res[k][rb] += *(const LDS_AS float4v*)(src + ((rb * 8 + base + k) * 64 + lane) * 16) * e[s][rb];
      }
    }
  }
  // Wave v now holds dims 16mb + 4g + 0..3 for mb = 4v..4v+3 of rows 16rb + n.
  // One chunk per split: the state goes straight to the workspace.  Several:
  // chunk states go to scratch in the workspace layout with the chunk index
  // innermost, and the merge kernel reduces them in chunk order.
  const size_t row0 = (size_t)b * ROWS;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 16 * rb + n;
    if (row < ROWS) {
      const size_t idx = ((row0 + row) * NS + jsp) * C + chunk;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *(float4v*)(a.st_num + idx * kHeadDim + 16 * (4 * wave + k) + 4 * g) = res[k][rb] * ofac;
      if (wave == 0 && g == 0) {
        a.st_max[idx] = (M[rb] == kNegInf) ? kNegInf : M[rb] * c;
        a.st_sum[idx] = Lsum[rb];
      }
    }
  }
}

}  // namespace

int split_chunks(int batch, int num_splits) {
  const int groups = batch * num_splits;
  return max(1, min(kMaxChunks, kTargetCUs / groups));
}

int split_grid(int batch, int num_q, int num_splits) {
  const int groups = batch * num_splits;
  return 8 * split_chunks(batch, num_splits) * ((groups + 7) / 8);
}

hipError_t launch_split(const SplitArgs& a, hipStream_t stream) {
  const int rb = (a.num_q * kQHeads + 15) / 16;
  const dim3 grid(split_grid(a.batch, a.num_q, a.num_splits)), block(kThreads);
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
