// Split stage of DFlash2 verification attention on gfx950 (MI355X).
//
// Pages cited by PR number and section:
//   [#587] "[Perf] Reduce DFlash2 long-context verification decay"
//   [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK reuse"
//
// What one launch computes: for every sequence b, query row r = 6*i + h and
// logical split j (or key chunk of a split), the FP32 state (max, sum,
// numerator) of causal softmax attention restricted to those keys ([#587]
// Implementation: 80 logical splits, compensated FP32 sums, probability
// residual products, FP32 state; [#589] Test Plan: the FP32 workspace is an
// output).
//
// Work decomposition (MI355X: 256 CUs in 8 XCDs, 64-wide waves, 160 KB LDS/CU):
//   * Each logical split is cut into C key chunks (C = 3 for one sequence and
//     80 splits: 240 workgroups, about one per CU).  Workgroups never talk to
//     each other: with C = 1 a workgroup writes its split's workspace entry,
//     with C > 1 it writes its chunk state and a separate merge pass (fused
//     into the combine kernel when the output is wanted) reduces the C states
//     of a split in chunk order, so results are deterministic.
//   * A workgroup walks its chunk in 64-key tiles, four 16-token pages, through
//     a four-stage LDS ring fed by 16-byte direct-to-LDS loads
//     (global_load_lds_dwordx4); the first tile goes out alone as soon as the
//     block table has arrived, the next two once it has landed and the fourth
//     with the first loop iteration; afterwards two tiles are in flight while
//     one is scored and one is multiplied into V.  The page loads carry the
//     non-temporal hint (every page is read once; 6% on this pattern).  Inside
//     a 256-byte token row the 16-byte chunks are XOR-swizzled by the row's
//     slot, and the K, V and P operand orders are chosen so that the LDS
//     serves every operand read without a bank conflict.
//   * Eight waves, two per SIMD, split each tile by role.  For QK^T score wave
//     w takes page w: S^T = K_w * Q^T on v_mfma_f32_16x16x32_f16 for all 6q rows
//     (up to three 16-row blocks, Q held in registers), so every K byte is
//     decoded once and each decoded K fragment feeds every row block (the
//     pages' reuse of one K fragment across three M16 products, [#589]
//     Purpose).  Each wave turns its scores into P = exp(s - m_ref) * 2^3 as
//     FP16 hi + FP16 lo (the pages' probability residual products, ~22 bits)
//     and publishes them in LDS; after one barrier per tile, PV wave w forms
//     O^T += V^T * P^T for its own 64 of the 256 dimensions over all 64 keys,
//     with the V operand read straight out of LDS by the transposing
//     ds_read_b64_tr_b8.  No wave ever holds another wave's dimensions, so
//     there is nothing to fold at the end.  The chunk state leaves through LDS
//     as whole 1 KB numerator rows, with non-temporal stores.
//   * m_ref is a per-row reference max shared by the four waves: the max of
//     the chunk's first tile (every row that sees any key of the chunk sees
//     its first key).  Accumulators are never rescaled in the tile loop.
//     Should a row's scores outgrow the reference by more than 2^12 (beyond
//     FP16 range for P), the workgroup notices at the end of the chunk, takes
//     the chunk's true row max as the reference and redoes the chunk once;
//     only strongly growing scores trigger this.  The
//     end of the chunk renormalises to the true max.  This is an exact
//     re-association of the pages' 32-key online update.
//   * E4M3 is decoded in registers with v_cvt_scalef32_pk_f16_fp8 (OCP on gfx950,
//     two codes per instruction, exact in FP16).  The per-tensor scales are not
//     applied during decode: k_scale is folded into the score scale and v_scale
//     into the stored numerator.
#include "dfv_common.h"
#include "dfv_device.h"

namespace dfv {
namespace {

#define LDS_AS DFV_LDS

constexpr float kNegInf = -__builtin_inff();
constexpr float kPScale = 8.0f;              // 2^3: P * 2^3 <= 2^15 keeps FP16 hi finite
constexpr float kPScaleLog2 = 3.0f;
constexpr float kRestartLog2 = 12.0f;        // P may reach 2^12 before the workgroup restarts
constexpr int kMaxRB = kMaxRows / 16;        // three 16-row blocks
constexpr int kTileKeys = 64;                // one 16-token page per wave
constexpr int kStages = 4;                   // LDS ring depth
constexpr int kTileBytes = 8 * kPageBytes;   // K pages 0..3, then V pages 0..3 (32 KB)
constexpr int kVOffset = 4 * kPageBytes;
constexpr int kPSlot = 64 * 16;              // one (k-step, row block, hi|lo) P operand: 64 lanes x 16 B
constexpr int kSplitThreads = 2 * kThreads;  // four score waves + four PV waves, two per SIMD
constexpr int kORowBytes = 4 * kHeadDim + 16;  // numerator row staged in LDS; the pad spreads 16 rows over all banks
constexpr int kORowsPerStage = kTileBytes / kORowBytes;   // 31 rows of one ring stage
static_assert(2 * kORowsPerStage >= kMaxRows, "two ring stages hold the staged numerator rows");

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

// max(a, b, c); the compiler folds the pair into one v_max3_f32.  It must stay
// visible to the compiler: its operands come straight from MFMA accumulators,
// and only the compiler inserts the wait states that a VALU read of an MFMA
// result needs (the hardware does not check that dependency; an inline-asm
// read right after the MFMA sees the register's old contents).
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Kahan compensated add of x into (sum, comp), comp holding minus the low part
// lost so far: every term is a probability (x >= 0), so the sum only grows
// and Kahan's bound (about 2u of the sum) holds without Neumaier's branch.
__device__ __forceinline__ void comp_add(float& sum, float& comp, float x) {
  const float y = x - comp;
  const float t = sum + y;
  comp = (t - sum) - y;
  sum = t;
}

// FP16 of pa - hi.lo and pb - hi.hi, packed, where hi holds two FP16 values:
// v_fma_mixlo_f16 and v_fma_mixhi_f16 (each difference exact in FP32 and
// rounded once to FP16; the second instruction fills the high half and keeps
// the low one).  No operand is an MFMA result.
__device__ __forceinline__ unsigned residual_pair(unsigned hi, float pa, float pb) {
  unsigned out;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(out) : "v"(hi), "v"(pa));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(out) : "v"(hi), "v"(pb));
  return out;
}

// Wait until at most `pending` (0, 8, 16 or 24) of this wave's LDS loads are in flight.
__device__ __forceinline__ void wait_dma(int pending) {
  if (pending >= 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if (pending >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (pending >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__shared__ __attribute__((aligned(16))) uint8_t g_ring[kStages * kTileBytes];
// P operands, double-buffered by tile parity: [ks][rb][hi|lo][page parity][lane][4 halves],
// as the score waves hold them (each wave writes 512 contiguous bytes per operand).
__shared__ __attribute__((aligned(16))) uint8_t g_p[2][2 * kMaxRB * 2 * kPSlot];
__shared__ float g_meta[3][kWaves][kMaxRows];   // per score wave: row max, row sum, reference
__shared__ int g_flag[kWaves];                  // a wave's rows outgrew m_ref somewhere in the chunk
__shared__ int g_pages[2][kWaves][64];          // block-table windows: wave w's pages of 64 tiles

__device__ __forceinline__ int split_size_of(int L, int ns, int fixed) {
  if (fixed) return fixed;
  const int per = (L + ns - 1) / ns;
  return kTile * ((per + kTile - 1) / kTile);
}

__device__ __forceinline__ int clamp_len(int L, int nq, int maxL) { return min(max(L, nq), maxL); }

// Workgroup w -> (split group, chunk): groups (sequence, split) are dealt to
// XCDs round robin and the C chunks of a group get workgroup ids
// 8*(C*(grp/8) + c) + grp%8, all on XCD grp % 8 (a locality nicety only).
//
// Eight waves, two per SIMD, in two roles: waves 0-3 ("score waves") own page
// w of every tile for QK^T, softmax and the P operands; waves 4-7 ("PV
// waves") own dimensions 64w..64w+63 (V decode and the PV products) and the
// DMA stream of page w (block-table windows, the tile loads and the waits
// that precede each hand-over barrier).  On each SIMD one wave of each kind
// runs, so the MFMA pipe works on one wave's products while the other wave's
// VALU work (decode, exp, packing) proceeds.
template <int RB>
__global__ __launch_bounds__(kSplitThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void split_kernel(const _Float16* __restrict__ q, const uint8_t* __restrict__ k_cache,
                  const uint8_t* __restrict__ v_cache, const int32_t* __restrict__ block_table,
                  const int32_t* __restrict__ context_lens, const float* __restrict__ k_scale,
                  const float* __restrict__ v_scale, SplitArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool scorer = wid < kWaves;
  const int wave = wid & (kWaves - 1);   // page (score wave) or dimension slice (PV wave)
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

  // The chunk's 32-key tiles [t_lo, t_hi) for a context of L keys.
  auto chunk_tiles = [&](int L, int& t_lo, int& t_hi) {
    const int S = split_size_of(L, NS, a.split_tokens);
    const int Tb = (L + kTile - 1) / kTile;
    const int s_lo = min(jsp * (S / kTile), Tb);
    const int s_hi = min((jsp + 1) * (S / kTile), Tb);
    const int ns32 = s_hi - s_lo;
    t_lo = s_lo + (chunk * ns32) / C;
    t_hi = s_lo + ((chunk + 1) * ns32) / C;
  };
  // Block-table window k of page slot `wave` (one dword per lane: the page of
  // 64-key tile 64k + lane, or the chunk's first page past the chunk), landing
  // in g_pages[k & 1][wave] by direct-to-LDS load.
  const int32_t* bt = block_table + (size_t)b * a.max_blocks;
  auto window_dma = [&](int k, int plo, int pend, int nu_) {
    const int tu = 64 * k + lane;
    const int e = (tu < nu_ && plo + 4 * tu + wave < pend) ? plo + 4 * tu + wave : plo;
    lds_dma4(bt, (unsigned)e * 4u, (LDS_AS void*)&g_pages[k & 1][wave][0]);
  };
  // The PV waves fetch the first windows before the context length is known,
  // for the chunk that a context of max_context_len keys would give (entries
  // below 16 * max_blocks, so always in bounds).  Once the length arrives the
  // windows are kept if the chunk's pages are the same (a single sequence at
  // its bound, or a fixed split size whose chunk lies below the true length)
  // and fetched again otherwise.  This takes one memory latency off the start.
  int spec_lo = 0, spec_end = 0, spec_nu = 0;
  if (!scorer) {
    int tl, th;
    chunk_tiles(a.max_context_len, tl, th);
    spec_lo = 2 * tl;
    spec_end = min(2 * th, (a.max_context_len + kPage - 1) / kPage);
    spec_nu = (th - tl + 1) / 2;
    if (spec_nu > 0) window_dma(0, spec_lo, spec_end, spec_nu);
    if (spec_nu > 64) window_dma(1, spec_lo, spec_end, spec_nu);
  }

  const float c = a.softmax_scale * k_scale[0];
  const float c2 = c * kLog2e;
  const float ofac = v_scale[0] * (1.0f / kPScale);
  const int L = clamp_len(context_lens[b], NQ, a.max_context_len);
  int t_lo, t_hi;                                      // chunk = 32-key tiles [t_lo, t_hi)
  chunk_tiles(L, t_lo, t_hi);
  const int npages = (L + kPage - 1) / kPage;
  const int page_lo = 2 * t_lo;
  const int page_end = min(2 * t_hi, npages);          // pages of the chunk that exist
  const int key_lo = kTile * t_lo;
  const int key_end = min(kTile * t_hi, L);            // keys of the chunk
  const int nu = (t_hi - t_lo + 1) / 2;                // 64-key tiles

  auto stage_of = [&](int t) { return (LDS_AS uint8_t*)g_ring + (t % kStages) * kTileBytes; };

  // ------------------------------------------------------------------ score waves
  // DMA lane offsets: load qq of a page fills LDS row r = 4qq + lane/16, chunk
  // position lane%16, with global chunk (lane%16) ^ r of that row.
  unsigned lane_off[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const unsigned r = 4 * qq + (lane >> 4);
    lane_off[qq] = r * 256u + 16u * ((unsigned)(lane & 15) ^ r);
  }
  // Wave w's page of tile u is page_lo + 4u + w; pages past the chunk are skipped.
  auto tile_valid = [&](int u) { return u < nu && page_lo + 4 * u + wave < page_end; };
  auto issue_page = [&](int u, int page) {
    if (!tile_valid(u)) return;
    LDS_AS uint8_t* st = stage_of(u) + wave * kPageBytes;
    const uint8_t* kp = k_cache + (size_t)page * kPageBytes;
    const uint8_t* vp = v_cache + (size_t)page * kPageBytes;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) lds_dma16_nt(kp, lane_off[qq], st + qq * 1024);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) lds_dma16_nt(vp, lane_off[qq], st + kVOffset + qq * 1024);
  };
  // Block-table entries come through LDS windows (one dword per lane, window
  // k = tiles 64k..64k+63, double-buffered) and then one VGPR, so no scalar
  // load sits between a tile's turn and its DMA; the block table is never read
  // any other way.  Lanes past the chunk read a valid entry whose value is
  // never used.
  auto load_window = [&](int k) { window_dma(k, page_lo, page_end, nu); };
  auto issue_tile = [&](int u, int pg) { issue_page(u, __builtin_amdgcn_readlane(pg, u & 63)); };
  // This wave's LDS loads still allowed in flight once tile u has landed, when
  // tiles u+1..u+ahead have been issued after it.
  auto pending_after = [&](int u, int ahead) {
    int p = 0;
#pragma unroll
    for (int d = 1; d <= kStages - 1; ++d) p += (d <= ahead && tile_valid(u + d)) ? 8 : 0;
    return p;
  };

  // Causal bound of each of this lane's rows (rows past 6q act as the last
  // real row), also cut at the chunk end; mask_from is the first key that some
  // row must not see, so tiles below it need no mask.
  const int mask_from = min(L - NQ + 1, key_end);
  int limit[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = min(16 * rb + n, ROWS - 1);
    limit[rb] = min(L - NQ + row / kQHeads, key_end - 1);
  }

  // Rows of this wave's K and V pages at or past the chunk end hold unrelated
  // bytes (or nothing, for a page that was not loaded): clear their codes to +0
  // so that neither a masked score (-inf plus the products) nor P = 0 times V
  // turns into NaN.  Only the chunk's last tile.
  auto clear_tail = [&](int t) {
    const int r0 = max(0, key_end - kPage * (page_lo + 4 * t + wave));
    if (r0 >= kPage) return;
    LDS_AS uint8_t* kp = stage_of(t) + wave * kPageBytes;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = e * 64 + lane;   // 16-byte chunk idx of the page, row idx / 16
      if ((idx >> 4) >= r0) {
        *(LDS_AS uint4v*)(kp + idx * 16) = uint4v{0u, 0u, 0u, 0u};
        *(LDS_AS uint4v*)(kp + kVOffset + idx * 16) = uint4v{0u, 0u, 0u, 0u};
      }
    }
  };

  half8 qf[RB][8];       // Q in MFMA B-operand order (score waves; AGPRs)
  // m_ref: the row's reference max (-inf until known, and for a row that sees no
  // key of the chunk); mr: m_ref, or 0 for such a row; m_lane: this lane's
  // largest s - mr.
  float m_ref[RB], mr[RB], m_lane[RB], l_sum[RB], l_cmp[RB];
  int pg = 0;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_ref[rb] = kNegInf;
    mr[rb] = 0.f;
    m_lane[rb] = kNegInf;
    l_sum[rb] = 0.f;
    l_cmp[rb] = 0.f;
  }
  const unsigned kswz = 16u * (unsigned)n;   // K row n, chunk c at n*256 + 16*(c ^ n)

  // S^T - mr = K_w * Q^T - mr for this wave's page of tile t (the products
  // accumulate onto -mr); lane holds keys key_lo + 64t + 16w + 4g + r of row
  // 16rb + n.  Masked keys start at -inf instead, which the (finite) products
  // leave at -inf; only tiles that reach mask_from choose per key.  The
  // choice is made before the MFMAs, so no branch separates an MFMA from the
  // first reader of its result (the hardware does not check that dependency,
  // and at such a join the compiler has been seen to leave out the wait states).
  auto qk = [&](int t, float (&s)[RB][4]) {
    float4v sacc[RB];
    if (key_lo + kTileKeys * (t + 1) > mask_from) {
      const int kb = key_lo + kTileKeys * t + 16 * wave + 4 * g;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[rb][r] = (kb + r > limit[rb]) ? kNegInf : -mr[rb];
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb] = float4v{-mr[rb], -mr[rb], -mr[rb], -mr[rb]};
    }
    const LDS_AS uint8_t* krow = stage_of(t) + wave * kPageBytes + n * 256;
    // Read i of lane (n, g) is 16-byte chunk g + 4i of its row: the four lane
    // groups of one read take four neighbouring chunks, which the LDS serves
    // without bank conflicts (chunks 4g + i, the other natural order, cost a
    // second pass on gfx950).
    uint4v kr[4];   // all four reads in flight at once: one LDS latency per tile
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = *(const LDS_AS uint4v*)(krow + ((16u * (g + 4 * i)) ^ kswz));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half8 k0 = decode8(kr[i][0], kr[i][1]);
      const half8 k1 = decode8(kr[i][2], kr[i][3]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[rb][2 * i], sacc[rb], 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qf[rb][2 * i + 1], sacc[rb], 0, 0, 0);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[rb][r] = sacc[rb][r];
  };
  // Running max of this lane's s - mr (cross-lane reduction only at the chunk end).
  auto lane_max = [&](const float (&s)[RB][4]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) m_lane[rb] = max3(max3(m_lane[rb], s[rb][0], s[rb][1]), s[rb][2], s[rb][3]);
  };
  // P * 2^3 = exp2((s - mr) * c2 + 3) as FP16 hi (truncated) + FP16 lo (the
  // exact remainder, rounded); compensated row sums.  s - mr comes straight
  // from the accumulation, so keys near the max keep full relative precision
  // even when |m_ref * c2| is large.  Published for every PV wave: operand
  // (ks, rb, hi|lo) with ks = w/2, this lane's 8 bytes at 512 (w%2) + 8 lane.
  auto publish_p = [&](int t, const float (&s)[RB][4]) {
    LDS_AS uint8_t* pw = (LDS_AS uint8_t*)g_p[t & 1] + 512 * (wave & 1) + 8 * lane;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float p8[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p8[r] = fast_exp2(__builtin_fmaf(s[rb][r], c2, kPScaleLog2));
      const unsigned h01 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(p8[0], p8[1]));
      const unsigned h23 = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(p8[2], p8[3]));
      const uint2v hi = uint2v{h01, h23};
      const uint2v lo = uint2v{residual_pair(h01, p8[0], p8[1]), residual_pair(h23, p8[2], p8[3])};
      comp_add(l_sum[rb], l_cmp[rb], (p8[0] + p8[1]) + (p8[2] + p8[3]));
      const int slot = ((wave >> 1) * RB + rb) * 2;
      // volatile: two separate ds_write_b64 (the compiler would pair them into
      // one ds_write2st64_b64, which the LDS serves at half the rate)
      *(volatile LDS_AS uint2v*)(pw + slot * kPSlot) = hi;
      *(volatile LDS_AS uint2v*)(pw + (slot + 1) * kPSlot) = lo;
    }
  };
  // Scores of tile t up to (not including) publishing: tail, QK.  The PV waves
  // have waited for the tile's DMAs before the barrier that precedes.
  auto front = [&](int t, float (&s)[RB][4]) {
    if (key_lo + kTileKeys * (t + 1) > key_end) clear_tail(t);
    qk(t, s);
  };

  // ------------------------------------------------------------------ PV waves
  float4v o[4][RB];      // O^T (x 2^3, relative to m_ref): dims 16(4w+mb) + 4g + 0..3 of row 16rb + n
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) o[mb][rb] = float4v{0.f, 0.f, 0.f, 0.f};
  // V operand addresses (ds_read_b64_tr_b8): lane (n, g) reads row (page g/2,
  // slot 8(g%2) + (j ^ 4(g%2))), j = n/2, bytes 8(n%2)..+7 of 16-byte chunk
  // mb; after the transpose it holds 8 keys of dimension 16mb + n, MFMA
  // K-index 8g + k being key 8(g%2) + (k ^ 4(g%2)) of page g/2.  Each half
  // wave reads all 16 rows of one page, which spreads its 32 reads over every
  // bank.  The P operand follows the same key order: for even g, halves 0-3
  // and 4-7 are the 8 bytes that score lanes (n, 0) and (n, 1) of page g/2
  // wrote; for odd g, those of lanes (n, 3) and (n, 2).  Read in that order
  // (as two 8-byte reads), every half wave again covers all banks.
  unsigned voff[4];
  {
    const int vslot = 8 * (g & 1) + ((n >> 1) ^ (4 * (g & 1)));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      voff[mb] = kVOffset + (g >> 1) * kPageBytes + vslot * 256 + 8 * (n & 1) +
                 ((16u * (4 * wave + mb)) ^ (16u * (unsigned)vslot));
  }
  // PV of tile t: 64 keys as two 32-key MFMA steps (pages 2ks, 2ks+1), for
  // this wave's four 16-dimension blocks; hi products of every row block first,
  // then lo, so dependent MFMAs on one accumulator are RB instructions apart.
  //
  // When tn >= 0 this wave's page of tile tn goes out in two halves: its
  // four K loads before the operand reads (the score waves need tile tn one
  // iteration before the PV waves do), its four V loads after the products.
  // A wave is held at each load issue until the memory system takes it; with
  // the V half after the products that hold overlaps the wave's MFMAs still
  // in the pipe (all eight first: the step about 1% slower).
  auto pv = [&](int t, int tn) {
    const unsigned sbase = (unsigned)(uintptr_t)stage_of(t);
    const LDS_AS uint8_t* pr1 = (const LDS_AS uint8_t*)g_p[t & 1] + 512 * (g >> 1) + 384 * (g & 1) + 8 * n;
    const LDS_AS uint8_t* pr2 = (const LDS_AS uint8_t*)g_p[t & 1] + 512 * (g >> 1) + 128 * ((g & 1) + 1) + 8 * n;
    const bool dma = tn >= 0 && tile_valid(tn);
    const int page = dma ? __builtin_amdgcn_readlane(pg, tn & 63) : 0;
    const uint8_t* kvp[2] = {k_cache + (size_t)page * kPageBytes, v_cache + (size_t)page * kPageBytes};
    LDS_AS uint8_t* dst = stage_of(dma ? tn : 0) + wave * kPageBytes;
    if (dma) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) lds_dma16_nt(kvp[0], lane_off[mb], dst + mb * 1024);
    }
    // A tile whose pages 2 and 3 lie past the chunk (the last tile of a chunk
    // of an odd number of 32-key tiles) needs only the first 32-key step.
    const int nks = (page_lo + 4 * t + 2 >= page_end) ? 1 : 2;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks >= nks) break;
      half8 phi[RB], plo[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        // volatile: four separate ds_read_b64, not ds_read2st64_b64 pairs
        // (those take twice the LDS cycles)
        const int shi = ((ks * RB + rb) * 2) * kPSlot, slo = shi + kPSlot;
        const half4 h0 = *(volatile const LDS_AS half4*)(pr1 + shi), h1 = *(volatile const LDS_AS half4*)(pr2 + shi);
        const half4 l0 = *(volatile const LDS_AS half4*)(pr1 + slo), l1 = *(volatile const LDS_AS half4*)(pr2 + slo);
        phi[rb] = half8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        plo[rb] = half8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
      }
      int2v vr[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        vr[mb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (LDS_AS int2v*)(uintptr_t)(sbase + ks * 2 * kPageBytes + voff[mb]));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const half8 va = decode8((unsigned)vr[mb][0], (unsigned)vr[mb][1]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, phi[rb], o[mb][rb], 0, 0, 0);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[mb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, plo[rb], o[mb][rb], 0, 0, 0);
      }
    }
    if (dma) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) lds_dma16_nt(kvp[1], lane_off[mb], dst + kVOffset + mb * 1024);
    }
  };

  // The numerator rows of the finished chunk, unscaled, in the two ring stages
  // that the last tile does not occupy (rows 0..30 in one, 31..47 in the
  // other); no load targets them any more once the last tile is in flight.
  auto ostage = [&](int row) {
    return row < kORowsPerStage ? stage_of(nu) + row * kORowBytes
                                : stage_of(nu + 1) + (row - kORowsPerStage) * kORowBytes;
  };
  auto stage_o = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        *(LDS_AS float4v*)(ostage(16 * rb + n) + 4 * (16 * (4 * wave + mb) + 4 * g)) = o[mb][rb];
  };

  // ------------------------------------------------------------------ prologue
  // The PV waves own the DMA stream: PV wave w fetches the block-table windows
  // of page w (0 and 1) and, as soon as those land, puts page w of tile 0 in
  // flight alone, so that it lands as early as the start allows (every
  // workgroup issues at once, and a wave is held at each load until the memory
  // system takes it); tiles 1 and 2 follow once tile 0 is in, while the score
  // waves compute its scores, and tile 3 goes out in the first loop iteration
  // like every later tile (the less the start issues, the sooner the loop
  // begins: 0.3-0.8 us against issuing tiles 1-3 here).  A wave waits for each tile before the
  // barrier that hands the tile to the score waves.  Meanwhile the score waves
  // stage Q, in MFMA B-operand order, in the P buffers, which nothing else
  // uses before P(0) is published.
  // Fragment f = rb*8 + m, lane (n, g) holds Q[row 16rb+n][64(m/2) + 16g +
  // 8(m%2) + 0..7] (the dimensions of K read m/2); rows past 6q repeat the
  // last real row.
  LDS_AS uint8_t* const qstage = (LDS_AS uint8_t*)&g_p[0][0];
  static_assert(sizeof(g_p) >= kMaxRB * 8 * 1024, "Q staging fits in the P buffers");
  // PV waves: windows 0 and 1 (unless the speculative ones hold the same
  // pages), then tiles 0..last (the first start: tile 0 alone; a restart:
  // tiles 0-2).
  auto start_stream = [&](bool spec_ok, int last) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!spec_ok) {
      if (nu > 0) load_window(0);
      if (nu > 64) load_window(1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    pg = g_pages[0][wave][lane];
#pragma unroll
    for (int u = 0; u < kStages; ++u)
      if (u <= last) issue_tile(u, pg);
  };
  if (!scorer) {
    start_stream(spec_lo == page_lo && spec_end == page_end && spec_nu == nu, 0);
    // Tile 0's K is all the first scores need: when the tile has no keys past
    // the chunk end (nothing for the score waves to clear in its V), the V
    // half may still be in flight at the barrier; the wait for tile 1 before
    // the loop covers it.
    if (key_lo + kTileKeys <= key_end) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    const _Float16* qb = q + (size_t)b * ROWS * kHeadDim;
    for (int f = wave; f < RB * 8; f += kWaves) {
      const int row = min(16 * (f >> 3) + n, ROWS - 1);
      const int m = f & 7;
      lds_dma16(qb, (unsigned)(row * kHeadDim * 2 + 128 * (m >> 1) + 32 * g + 16 * (m & 1)), qstage + f * 1024);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();   // Q staged; tile 0 landed
  if (scorer) {
    const LDS_AS uint8_t* qs = qstage + lane * 16;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        qf[rb][m] = *(const LDS_AS half8*)(qs + (rb * 8 + m) * 1024);
        asm volatile("" : "+a"(qf[rb][m]));   // Q lives in AGPRs: MFMA reads B from there directly
      }
  }
  const size_t row0 = (size_t)b * ROWS;
  float M[RB], lsum[RB], mref_all[RB];
  // Row max, sum and reference of the chunk, shared by the score waves through
  // LDS at the end of a pass (after the barrier that follows the writes).
  auto read_meta = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = 16 * rb + n;
      M[rb] = fmaxf(fmaxf(g_meta[0][0][row], g_meta[0][1][row]), fmaxf(g_meta[0][2][row], g_meta[0][3][row]));
      lsum[rb] = ((g_meta[1][0][row] + g_meta[1][1][row]) + g_meta[1][2][row]) + g_meta[1][3][row];
      mref_all[rb] = g_meta[2][0][row];
    }
    return (g_flag[0] | g_flag[1] | g_flag[2] | g_flag[3]) != 0;
  };

  // The two roles run separate loops with the same barrier sequence:
  //   nu > 0: first-tile max exchange, P(0) published;
  //   per tile u: one barrier (P(u+1) published, PV(u) done);
  //   end of pass: one barrier (meta written); on a restart one more (P(0)).
  if (scorer) {
    // First tile: the shared reference m_ref is its row max over all four pages
    // (every row that sees any key of the chunk sees its first key).
    if (nu > 0) {
      float s[RB][4];
      front(0, s);   // mr = 0 still: plain scores
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float t = max3(max3(kNegInf, s[rb][0], s[rb][1]), s[rb][2], s[rb][3]);
        const float tm = max_x32(max_x16(t));
        if (g == 0) g_meta[0][wave][16 * rb + n] = tm;
      }
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = 16 * rb + n;
        m_ref[rb] = fmaxf(fmaxf(g_meta[0][0][row], g_meta[0][1][row]),
                          fmaxf(g_meta[0][2][row], g_meta[0][3][row]));
        mr[rb] = (m_ref[rb] == kNegInf) ? 0.f : m_ref[rb];   // a row without keys has s = -inf
#pragma unroll
        for (int r = 0; r < 4; ++r) s[rb][r] -= mr[rb];
      }
      lane_max(s);
      publish_p(0, s);
      __syncthreads();   // P(0) published; tile 1 landed
    }
    // End of pass: true row max and sum over the four pages (in wave order),
    // the reference, and whether a row outgrew it.  Written while the PV
    // waves work on the last tile, published by the barrier that ends it.
    auto end_meta = [&]() {
      bool ovf = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        ovf |= m_lane[rb] * c2 > kRestartLog2;   // false while -inf
        const float mx = mr[rb] + max_x32(max_x16(m_lane[rb]));   // -inf stays -inf
        const float l = sum_x32(sum_x16(l_sum[rb])) - sum_x32(sum_x16(l_cmp[rb]));
        if (g == 0) {
          g_meta[0][wave][16 * rb + n] = mx;
          g_meta[1][wave][16 * rb + n] = l;
          g_meta[2][wave][16 * rb + n] = m_ref[rb];
        }
      }
      g_flag[wave] = __builtin_amdgcn_ballot_w64(ovf) != 0;
    };
    for (;;) {
      for (int u = 0; u < nu; ++u) {
        if (u + 1 < nu) {
          float s[RB][4];
          front(u + 1, s);
          lane_max(s);
          publish_p(u + 1, s);
        } else {
          end_meta();
        }
        __syncthreads();   // P(u+1) published (meta, after the last tile); PV(u) done; tile u+2 landed
      }
      if (nu == 0) {
        end_meta();
        __syncthreads();
      }
      if (!read_meta()) break;
      // Some row max outgrew its reference (P beyond FP16 range somewhere):
      // take the chunk's true row max as the reference and redo the chunk.
      // The reference now bounds every score, so this happens at most once.
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        m_ref[rb] = M[rb];
        mr[rb] = (M[rb] == kNegInf) ? 0.f : M[rb];
        m_lane[rb] = kNegInf;
        l_sum[rb] = 0.f;
        l_cmp[rb] = 0.f;
      }
      __syncthreads();   // restart: tile 0 landed; every read of g_meta / g_flag above is done
      float s[RB][4];
      front(0, s);
      lane_max(s);
      publish_p(0, s);
      __syncthreads();   // P(0) published; tile 1 landed
    }
    if (wave == 0 && g == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = 16 * rb + n;
        if (row < ROWS) {
          const float e = (mref_all[rb] == kNegInf) ? 0.f : fast_exp2((mref_all[rb] - M[rb]) * c2);
          const size_t idx = ((row0 + row) * NS + jsp) * C + chunk;
          __builtin_nontemporal_store((M[rb] == kNegInf) ? kNegInf : M[rb] * c, a.st_max + idx);
          __builtin_nontemporal_store(lsum[rb] * e * (1.0f / kPScale), a.st_sum + idx);
        }
      }
    }
  } else {
    // The PV waves carry the tile loop's critical path (the score waves wait at
    // its barrier): they win issue ties on their SIMD (about 3% per launch).
    __builtin_amdgcn_s_setprio(1);
    if (nu > 0) {
#pragma unroll
      for (int u = 1; u < kStages - 1; ++u) issue_tile(u, pg);   // while the score waves work on tile 0
      __syncthreads();   // first-tile max exchange
      wait_dma(pending_after(1, kStages - 3));
      __syncthreads();   // P(0) published; tile 1 landed
    }
    for (;;) {
      for (int u = 0; u < nu; ++u) {
        // Every wave is past the barrier that ended tile u-1: its stage is free
        // (tiles 0..kStages-2 went out before the loop; tile kStages-1 goes
        // out now, in iteration 0).
        const int tn = u + kStages - 1;
        int tdma = -1;
        if (tn < nu) {
          if ((tn & 63) == 0) {
            pg = g_pages[(tn >> 6) & 1][wave][lane];
            if (tn + 64 < nu) load_window((tn >> 6) + 1);
          }
          tdma = tn;
        }
        pv(u, tdma);
        if (u + 1 < nu)
          wait_dma(pending_after(u + 2, 1));   // tile u+2, which the score waves read next
        else
          stage_o();
        __syncthreads();   // P(u+1) published (meta, after the last tile); PV(u) done; tile u+2 landed
      }
      if (nu == 0) {
        stage_o();
        __syncthreads();
      }
      if (!read_meta()) break;
      // Restart (see the score waves): refill the ring from the first tile.
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb][rb] = float4v{0.f, 0.f, 0.f, 0.f};
      start_stream(false, kStages - 2);
      wait_dma(pending_after(0, kStages - 2));
      __syncthreads();   // restart: tile 0 landed
      wait_dma(pending_after(1, kStages - 3));
      __syncthreads();   // P(0) published; tile 1 landed
    }
  }
  // Numerator rows leave as whole 1 KB rows, one row per wave instruction,
  // renormalised to the true row max on the way.  The stores are
  // non-temporal: nothing in this launch reads them back, and streamed out
  // they no longer pile up as dirty cache lines that the end of the launch
  // would have to write back all at once.
  for (int row = wid; row < ROWS; row += 2 * kWaves) {
    const float mx = fmaxf(fmaxf(g_meta[0][0][row], g_meta[0][1][row]), fmaxf(g_meta[0][2][row], g_meta[0][3][row]));
    const float rf = g_meta[2][0][row];
    const float of = (rf == kNegInf) ? 0.f : fast_exp2((rf - mx) * c2) * ofac;
    const size_t idx = ((row0 + row) * NS + jsp) * C + chunk;
    __builtin_nontemporal_store(*(const LDS_AS float4v*)(ostage(row) + 16 * lane) * of,
                                (float4v*)(a.st_num + idx * kHeadDim + 4 * lane));
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
  const dim3 grid(split_grid(a.batch, a.num_q, a.num_splits)), block(kSplitThreads);
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
