// host_common.h -- host-side checks shared by the entry points of this
// library: the current device must be a gfx950 (its compute-unit count is
// cached per device), and byte ranges that must not overlap.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "attn.h"

namespace {

// Per-device cache: 0 unknown, -1 not gfx950, else the compute-unit count.
std::atomic<int> g_dev_cu[64];

int check_device(int* n_cu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_E_DEVICE;
  if (dev < 64) {
    const int s = g_dev_cu[dev].load(std::memory_order_relaxed);
    if (s > 0) {
      *n_cu = s;
      return ATTN_OK;
    }
    if (s < 0) return ATTN_E_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_E_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && prop.multiProcessorCount > 0;
  if (dev < 64) g_dev_cu[dev].store(ok ? prop.multiProcessorCount : -1, std::memory_order_relaxed);
  *n_cu = prop.multiProcessorCount;
  return ok ? ATTN_OK : ATTN_E_DEVICE;
}

bool ranges_overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uint64_t pa = (uint64_t)(uintptr_t)a, pb = (uint64_t)(uintptr_t)b;
  return pa < pb + nb && pb < pa + na;
}

}  // namespace
