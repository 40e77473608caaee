// Page-read ceiling probe (measurement infrastructure, not part of the attention
// boundary in include/dfv.h).  Built into its own library, libdfv_probe.so,
// which only the benchmark loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Workgroups of the probe launch: the split kernel's count at one sequence and
// 80 splits, so both put the same number of CUs to work.
constexpr int kProbeWorkgroups = 240;

// Streams the K page and the V page of every entry of pages[0..npages) (4 KiB
// each, E4M3 cache layout [block][16][256]) through LDS and discards them.
// k_cache, v_cache, pages: device pointers; sink: one device uint32 that is
// practically never written.  Returns 0, -1 on a NULL pointer or npages < 1
// (nothing launched), -5 if the launch failed.  Asynchronous on `stream`.
extern "C" __attribute__((visibility("default"))) int dfv_probe_page_read(const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* pages,
                                   int32_t npages, uint32_t* sink, hipStream_t stream);
