// Device helpers for the gfx950 layer kernels: vector types, MFMA wrappers, bf16
// rounding, wave reductions, LDS-only workgroup barrier, grid barrier.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moel_params.h"

namespace moel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;  // 8 wavefronts of 64
constexpr int kWaves = 8;
constexpr int kMaxT = 16;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ uint16_t f2bf(float f) {
  // round to nearest even (inputs are finite in this path; NaN stays NaN)
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
// two fp32 values -> {packed bf16 (nearest), packed bf16 of the remainders}
__device__ __forceinline__ u32x2 split_bf16(float a, float b) {
  const uint16_t ha = f2bf(a), hb = f2bf(b);
  return u32x2{(uint32_t)ha | ((uint32_t)hb << 16), pack2bf(a - bf2f(ha), b - bf2f(hb))};
}

// ---------------------------------------------------------------- global memory access
// Pointers reach the phases through a reference to the launch parameters, which hides their
// address space; without this cast the compiler emits flat accesses, and flat loads also
// count against lgkmcnt, so every LDS wait would drain the whole in-flight weight stream.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gl(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}
__device__ __forceinline__ u32x4 ldg_stream(const void* p) {
  return __builtin_nontemporal_load(gl(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ uint32_t ldg_stream32(const void* p) {
  return __builtin_nontemporal_load(gl(reinterpret_cast<const uint32_t*>(p)));
}
__device__ __forceinline__ u32x4 ldg16(const void* p) { return *gl(reinterpret_cast<const u32x4*>(p)); }
__device__ __forceinline__ u32x2 ldg8(const void* p) { return *gl(reinterpret_cast<const u32x2*>(p)); }
__device__ __forceinline__ float4 ldgf4(const float* p) {
  const f32x4 v = *gl(reinterpret_cast<const f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 16 independent 4x4x4 products; A of block ABID broadcast to all 16 blocks.
template <int ABID>
__device__ __forceinline__ f32x4 mfma4x4x4_bcast(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(short4v, a),
                                                __builtin_bit_cast(short4v, b), c, 4, ABID, 0);
}

// E2M1 pair (one byte of a dword, low nibble first) -> two bf16, unscaled (exact)
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t codes) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, r);
}
// E4M3 (OCP) byte of a dword -> fp32 (exact)
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t bytes) {
  return __builtin_amdgcn_cvt_f32_fp8((int)bytes, SEL);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Workgroup barrier for LDS traffic only: does not wait for outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------- control block
enum CtrlWord { kBar = 0, kExit = 1, kStatus = 2, kAbort = 3 };

__device__ __forceinline__ bool aborted(KP& p) {
  return __hip_atomic_load(gl(p.ctrl) + kAbort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Grid-wide barrier of the persistent launch.  `target` grows by nwg per barrier within one
// launch; the counter is reset by the last workgroup to leave the kernel.  Every wait is
// bounded: after ~0.5 s the status word records a timeout and the wait ends.
//
// Visibility: every wave first waits for its own stores to reach the L2 of its XCD; one wave
// per workgroup then writes the XCD's L2 back (release), arrives, spins, and invalidates the
// CU's L1 and the XCD's L2 (acquire).  Those cache operations act on the whole CU / XCD, so a
// single wave's fences cover the stores and later loads of all eight waves.
__device__ __forceinline__ void grid_barrier(KP& p, unsigned target) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(gl(p.ctrl) + kBar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(gl(p.ctrl) + kBar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (__builtin_amdgcn_s_memrealtime() - t0 > 50000000ull) {
        __hip_atomic_store(gl(p.ctrl) + kStatus, (unsigned)MOEL_DEV_TIMEOUT, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

__device__ __forceinline__ void stamp(KP& p, int slot) {
  if (p.dbg_ts != nullptr && threadIdx.x == 0)
    gl(p.dbg_ts)[blockIdx.x * MOEL_N_STAMPS_DEV + slot] = __builtin_amdgcn_s_memrealtime();
}

}  // namespace moel
