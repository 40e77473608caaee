// Page-read ceiling probe for gfx950 (MI355X): measurement infrastructure, not
// part of the attention path.
//
// It streams exactly the bytes the split kernel must read for one layer -- the
// K page and the V page named by every block-table entry of a sequence, in the
// table's (shuffled) order -- through LDS with direct-to-LDS 16-byte loads and
// does nothing else.  Its time is what random 4 KiB pages cost on this machine, the
// practical ceiling against which the split kernel's rate is read.
//
// The loads carry the non-temporal hint, as the split kernel's page loads do
// (each page is read once; the hint is worth about 6% on this pattern).
//
// Decomposition: 240 workgroups x 8 waves; wave i takes a contiguous run of the
// block table and keeps one page pair (K + V, 8 KB) in flight through a private
// two-slot LDS ring (16 KB per wave, 128 KB per workgroup).  A wave that issues
// direct-to-LDS loads is held at each issue until the memory system takes it,
// so eight issuing waves per workgroup read faster than four with more pages
// in flight each (21.5 against 24.8 us per layer in one sweep); the depth in
// flight per wave makes no difference.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dfv_device.h"
#include "dfv_probe.h"

namespace {

#define LDS_AS DFV_LDS

constexpr int kWavesPerWG = 8;
constexpr int kPageBytes = 4096;
constexpr int kSlots = 2;
constexpr int kDepth = 1;   // page pairs in flight per wave besides the one waited for

__shared__ __attribute__((aligned(16))) uint8_t g_slots[kWavesPerWG][kSlots][2 * kPageBytes];

__global__ __launch_bounds__(kWavesPerWG * 64) void page_read_probe(const uint8_t* __restrict__ k,
                                                                   const uint8_t* __restrict__ v,
                                                                   const int32_t* __restrict__ pages,
                                                                   int npages, unsigned* sink) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * kWavesPerWG;
  const int gw = blockIdx.x * kWavesPerWG + wave;
  const int p0 = (int)((long long)gw * npages / nw);
  const int p1 = (int)((long long)(gw + 1) * npages / nw);
  const int cnt = p1 - p0;
  unsigned acc = 0;
  for (int i = 0; i < cnt + kDepth; ++i) {
    if (i < cnt) {
      const size_t pg = (size_t)pages[p0 + i] * kPageBytes;
      LDS_AS uint8_t* dst = (LDS_AS uint8_t*)&g_slots[wave][i % kSlots][0];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) dfv::lds_dma16_nt(k + pg, qq * 1024 + lane * 16, dst + qq * 1024);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) dfv::lds_dma16_nt(v + pg, qq * 1024 + lane * 16, dst + kPageBytes + qq * 1024);
    }
    if (i >= kDepth) {
      // page i - kDepth has landed once at most the pages issued after it remain
      static_assert(kDepth == 1, "the waits below assume one page pair issued after the one waited for");
      if (i < cnt) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      acc ^= *(volatile LDS_AS unsigned*)&g_slots[wave][(i - kDepth) % kSlots][lane * 4];
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;   // keeps the reads; practically never stores
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int dfv_probe_page_read(const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* pages,
                                   int32_t npages, uint32_t* sink, hipStream_t stream) {
  if (!k_cache || !v_cache || !pages || !sink || npages < 1) return -1;
  hipLaunchKernelGGL(page_read_probe, dim3(kProbeWorkgroups), dim3(kWavesPerWG * 64), 0, stream,
                     k_cache, v_cache, pages, (int)npages, (unsigned*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
