// gfx950.h -- CDNA4 (gfx950) building blocks shared by the kernels of this
// library: vector types, direct global-to-LDS copies and their waits, the
// 32x32x16 16-bit MFMA, and the swizzled LDS layout of 64-element 16-bit rows.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4)
// from this lane's 64-bit address gsrc (a VGPR pair); lane l's bytes land at
// LDS address m0 + 16*l, m0 wave-uniform.  Issued as inline assembly so the
// compiler does not add its own conservative waits for it before unrelated
// LDS reads; completion is tracked explicitly with wait_vmem (vmcnt counts
// these copies, in issue order).  The compiler's hazard recognizer cannot see
// inside the assembly, so the operands are chosen to need no help from it:
// the address comes from VGPRs (a VMEM read of an SGPR written by a VALU
// instruction would need wait states the compiler cannot insert here), and
// the one wait state an SALU write of M0 needs before an LDS-DMA instruction
// reads it is the s_nop inside the assembly.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t m0) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
}

// Two copies whose sources and destinations both lie 2 * HALF bytes apart,
// from one address and one M0 at their midpoint: the instruction offset
// (13-bit signed) applies to the global and the LDS address alike, so the
// copies take offsets -HALF and +HALF.  Same operand rules as dma16.
template <int HALF = 2048>
__device__ __forceinline__ void dma16_pair(const void* gmid, uint32_t m0mid) {
  static_assert(HALF == 1024 || HALF == 2048, "offsets within the 13-bit signed field");
  if constexpr (HALF == 2048)
    asm volatile(
        "s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:-2048\n\tglobal_load_lds_dwordx4 %0, off offset:2048" ::"v"(
            gmid),
        "{m0}"(m0mid)
        : "memory");
  else
    asm volatile(
        "s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:-1024\n\tglobal_load_lds_dwordx4 %0, off offset:1024" ::"v"(
            gmid),
        "{m0}"(m0mid)
        : "memory");
}

// LDS byte address of a __shared__ location (what M0 takes).
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (the direct-to-LDS copies of later tiles may stay in flight).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(N | (0x7 << 4) | (0xF << 8));  // vmcnt=N, expcnt/lgkmcnt: no wait
}

// Workgroup barrier that does not drain in-flight direct-to-LDS copies (the
// fence in __syncthreads would wait for all of them).  LDS reads of this wave
// are complete before it arrives; the clobbers stop the compiler from moving
// memory operations across it.
__device__ __forceinline__ void barrier_keep_dma() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14) | (0x0 << 8));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename T>
struct Half16;

template <>
struct Half16<__bf16> {
  typedef bf16x8 vec8;
  static constexpr unsigned ONE2 = 0x3f803f80u;  // two 1.0 values
  __device__ static __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ unsigned pack2(float x, float y) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x, y}, bf16x2));
  }
};

template <>
struct Half16<_Float16> {
  typedef f16x8 vec8;
  static constexpr unsigned ONE2 = 0x3c003c00u;  // two 1.0 values
  __device__ static __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ unsigned pack2(float x, float y) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){x, y}, f16x2));
  }
};

// LDS tile of 64 rows x 128 bytes (64 16-bit values) = 8 KB.  16-byte chunks
// are XOR-swizzled per row to keep the MFMA operand reads conflict-free.
// K is read as one 16-byte chunk per lane, 16 consecutive rows per access.
__device__ __forceinline__ int k16_off(int row, int c16) {
  return row * 128 + ((c16 ^ ((row & 7) ^ ((row >> 3) & 1))) << 4);
}
}  // namespace
