// dfv_attn_noalloc: dfv_attn with the split kernel's scratch in a static device
// array, for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Nothing here allocates.
//
// The array `scratch` lives in this library's code object; each GPU the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol: the device address is
// taken once per device with hipGetSymbolAddress (with that device current)
// and kept, and only that address is ever handed to a kernel.
#include <mutex>

#include "dfv.h"
#include "dfv_common.h"

namespace {

// The largest scratch any admitted descriptor needs: at most 256 key-chunk
// states (batch * splits * chunks <= 256 whenever chunks > 1) of 48 rows x
// (256 + 2) floats = 12,681,216 bytes; 16 MiB leaves room.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of this GPU's copy of `scratch` (the current device's).
dfv_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFV_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFV_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DFV_OK;
}

}  // namespace

extern "C" {

dfv_status dfv_attn_noalloc(const dfv_attn_desc* desc, const void* q, const uint8_t* k_cache,
                            const uint8_t* v_cache, const int32_t* block_table,
                            const int32_t* context_lens, const float* k_scale, const float* v_scale,
                            float* ws_max, float* ws_sum, float* ws_num, void* out, void* stream) {
  size_t need = 0;
  const dfv_status s = dfv_attn_scratch_bytes(desc, &need);   // validates the descriptor, host only
  if (s != DFV_OK) return s;
  if (need > kStaticScratchBytes) return DFV_ERR_SCRATCH;
  void* p = nullptr;
  const dfv_status sp = device_scratch(&p);
  if (sp != DFV_OK) return sp;
  // The chunk states need no initialisation: the split kernel writes every
  // state the merge reads.
  return dfv_attn(desc, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, ws_max, ws_sum,
                  ws_num, p, kStaticScratchBytes, out, stream);
}

}  // extern "C"
