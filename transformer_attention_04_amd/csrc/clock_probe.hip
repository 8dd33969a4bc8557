// Probes for the benchmark (declared in attn_clock.h), not part of the
// attention path.  The shader-clock probe: each wave brackets a dependent
// multiply-add chain with reads of the shader cycle counter and the 100 MHz
// reference counter; the ratio of the two deltas is the shader clock while the
// chain ran.  The MFMA probe: each wave streams 32x32 MFMAs in four
// independent accumulator chains, nothing else, so its rate is the matrix
// throughput the chip sustains at the clock it holds under that load.  The
// copy probe: a plain 16-byte-per-lane streaming copy, the HBM counterpart.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "attn_clock.h"

namespace {

__global__ void __launch_bounds__(64) clock_probe_kernel(uint64_t* out, int iters) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  float x = (float)threadIdx.x * 1e-3f, y = 1.0f - x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      x = __builtin_fmaf(x, 0.999f, y);
      y = __builtin_fmaf(y, 0.999f, x);
    }
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    // Keeps the chain live: x + y is never exactly -1 for these inputs.
    const uint64_t keep = (x + y == -1.0f) ? 1u : 0u;
    out[2 * blockIdx.x] = c1 - c0 + keep;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// 16 MFMAs per iteration in four chains; the operands depend on the lane so
// nothing folds, and one sum per wave keeps the chains live.
template <int DT>
__global__ void __launch_bounds__(256) mfma_probe_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if constexpr (DT == 0) {
    const float a = 1e-3f * lane, b = 1e-3f * (63 - lane);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(b, b, c3, 0, 0, 0);
      }
    }
  } else {
    typedef typename std::conditional<DT == 1, f16x8, bf16x8>::type V;
    typedef typename std::conditional<DT == 1, _Float16, __bf16>::type E;
    V a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (E)(1e-3f * (lane + e));
      b[e] = (E)(1e-3f * (63 - lane + e));
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (DT == 1) {
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
          c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
          c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
        } else {
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
          c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
          c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
        }
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Streaming copy, 16 bytes per lane per access and four accesses in flight
// per lane: the HBM rate a plain read-and-write stream reaches.  A workgroup
// moves one contiguous 16 KB chunk per round (four 4 KB rows of 256 lanes),
// and the chunks are dealt to the workgroups round-robin.
__global__ void __launch_bounds__(256) copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n) {
  constexpr int CHUNK = 4 * 256;  // 16-byte units per chunk
  const int64_t full = n / CHUNK;
  for (int64_t ch = blockIdx.x; ch < full; ch += gridDim.x) {
    const int64_t i = ch * CHUNK + threadIdx.x;
    const u32x4 a = src[i], b = src[i + 256], c = src[i + 512], d = src[i + 768];
    dst[i] = a;
    dst[i + 256] = b;
    dst[i + 512] = c;
    dst[i + 768] = d;
  }
  // the tail (fewer than CHUNK units), by workgroup 0
  if (blockIdx.x == 0)
    for (int64_t i = full * CHUNK + threadIdx.x; i < n; i += 256) dst[i] = src[i];
}

}  // namespace

extern "C" int attn_copy_probe(const void* src, void* dst, int64_t bytes, int n_wg, void* stream) {
  if (!src || !dst || (((uintptr_t)src | (uintptr_t)dst) & 15u)) return 1;
  if (bytes < 16 || (bytes & 15) || n_wg < 1 || n_wg > 65536) return 2;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + (uint64_t)bytes && d0 < s0 + (uint64_t)bytes) return 2;  // overlapping ranges
  hipLaunchKernelGGL(copy_probe_kernel, dim3(n_wg), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 10;
}

extern "C" int attn_mfma_probe(float* out, int n_wg, int iters, int dtype, void* stream) {
  if (!out || ((uintptr_t)out & 3u)) return 1;
  if (n_wg < 1 || n_wg > 65536 || iters < 1 || iters > (1 << 24) || dtype < 0 || dtype > 2) return 2;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(n_wg), dim3(256), 0, st, out, iters);
  else if (dtype == 1)
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(n_wg), dim3(256), 0, st, out, iters);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<2>, dim3(n_wg), dim3(256), 0, st, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 10;
}

extern "C" int attn_clock_probe(uint64_t* out, int n_wg, int iters, void* stream) {
  if (!out || ((uintptr_t)out & 7u)) return 1;
  if (n_wg < 1 || n_wg > 4096 || iters < 1 || iters > (1 << 24)) return 2;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(n_wg), dim3(64), 0, static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 10;
}
