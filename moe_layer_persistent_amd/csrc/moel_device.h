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
constexpr int kMaxT = MOEL_MAX_TOKENS;  // tokens of one step at most
constexpr int kTile = 16;               // tokens per MFMA token tile
constexpr int kMaxTiles = kMaxT / kTile;
static_assert(kMaxTiles * kTile == kMaxT && kMaxTiles <= 2, "one or two token tiles");

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
// A value known to be equal on every lane, moved to a scalar register so that branches and
// address arithmetic on it stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// No 64-bit integer overload: the int one would take such a value by narrowing it (a parameter
// handle would lose its upper half).  Handles go through params_from, pointers through the
// overload below.
__device__ int uniform(long) = delete;
__device__ int uniform(unsigned long) = delete;
__device__ int uniform(long long) = delete;
__device__ int uniform(unsigned long long) = delete;
template <class T>
__device__ __forceinline__ T* uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// The launch parameters live in the kernel-argument segment.  The segment pointer exists only
// in the kernel itself (non-kernel functions do not receive it), so the kernel takes its
// address and passes it down as a plain 64-bit value; callees move it back to scalar
// registers, so every parameter read there is a scalar load.
__device__ __forceinline__ KP& kernel_params() {
  return *(KP*)__builtin_amdgcn_kernarg_segment_ptr();
}
__device__ __forceinline__ uint64_t params_handle(KP& p) { return (uint64_t)(&p); }
__device__ __forceinline__ KP& params_from(uint64_t h) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)h);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(h >> 32));
  return *(KP*)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- bf16
// Round to nearest even through the hardware conversion (v_cvt_pk_bf16_f32, two values per
// instruction, no branches).
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint16_t f2bf(float f) { return (uint16_t)(pack2bf(f, 0.f) & 0xffffu); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
// element c of a row in the split-operand layout: quad c/4 holds 4 bf16 of the nearest
// values, then 4 bf16 of the remainders
template <class Ptr>
__device__ __forceinline__ void store_split(Ptr row, int c, float v) {
  const uint16_t h = f2bf(v);
  row[(c >> 2) * 8 + (c & 3)] = h;
  row[(c >> 2) * 8 + 4 + (c & 3)] = f2bf(v - bf2f(h));
}
// two fp32 values -> {packed bf16 (nearest), packed bf16 of the remainders}
__device__ __forceinline__ u32x2 split_bf16(float a, float b) {
  const uint32_t h = pack2bf(a, b);
  return u32x2{h, pack2bf(a - bf_lo(h), b - bf_hi(h))};
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

// Keeps the instruction scheduler from moving anything across this point.  Placed after the
// loads of each ring step so that they stay spread over the loop body: left alone, the
// scheduler sinks them all to the end of the iteration, where they are consumed right after
// issue and the stream runs with one batch in flight at a time.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

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
// Words of the plan's control block (unsigned, 4 KiB).  The barrier words sit on separate
// 128-byte lines so that arrivals of different groups do not contend.
enum CtrlWord {
  kExit = 1,      // workgroups that have left the launch
  kStatus = 2,    // MOEL_DEV_* (0 = ok)
  kAbort = 3,     // set by the host: skip all work
  kFlag = 32,     // number of the last grid barrier released in this launch
  kTop = 64,      // group leaders arrived (monotonic within a launch)
  kGroup = 96,    // + 32 * g: workgroups of group g arrived (monotonic within a launch)
  kWork = 352,    // + 32 * i: tiles handed out so far by expert phase i (0 gate/up, 1 down)
  kXccMask = 416, // + 32 * g: bit x set when a workgroup of barrier group g runs on XCC x
  kEntered = 672, // workgroups that have recorded their XCC in kXccMask
  kAttnDone = 704,// + 32 * q: attention items of group q written (merged per barrier group)
  kFix = 1024,    // + kFixPerPhase * i + b: split-K units of block b of dense phase i arrived
  kCtrlWords = 2048
};
constexpr int kFixPerPhase = 256;
constexpr int kBarGroups = 8;

__device__ __forceinline__ bool aborted(KP& p) {
  return __hip_atomic_load(gl(p.ctrl) + kAbort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Acquire side of the grid barrier.  Other workgroups' data reaches this CU through its L1,
// which is not coherent and is always invalidated, and the XCD's L2.  The device may keep a
// clean copy that an XCD's L2 took of a line coherent with a later write from another XCD
// (probed when the plan is created); it does not for a line that the XCD itself wrote earlier
// in the launch (observed: such a copy outlives the other XCD's write and its write-back).
// Within one layer every line that crosses XCDs is written once (split-K partials either stay
// on one XCD or their reader takes the full acquire), so on a device that passes the probe the
// L1-only acquire suffices and the L2 is left alone: the agent-scope acquire of the memory
// model would also drop the L2's clean lines, read-only weights included.  Where one launch
// runs several layers, every XCD drops its L2's clean lines at the layer boundary.
__device__ __forceinline__ void acquire_fence(int l2_coherent) {
  if (l2_coherent) asm volatile("buffer_inv sc0" ::: "memory");  // L1 only
  else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ void acq_rel_fence(int l2_coherent) {
  if (l2_coherent) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // no reads follow before the flag
  else __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");
}

// XCC (accelerator complex die, one L2) of the calling wave.
__device__ __forceinline__ unsigned xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);  // XCC_ID[3:0]
}

// True when every barrier group of the launch is known to run on one XCC: all workgroups have
// recorded their XCC (each records its bit before it counts itself in) and every group's mask
// has one bit.  It can be false early in the launch (a workgroup not yet started); it is never
// true wrongly.  Thread 0.
__device__ __forceinline__ bool groups_single_xcc(KP& p) {
  auto ctrl = gl(p.ctrl);
  if (__hip_atomic_load(ctrl + kEntered, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)p.nwg) return false;
  const int ng_all = p.nwg < kBarGroups ? p.nwg : kBarGroups;
  bool ok = true;
  for (int g = 0; g < ng_all; ++g)
    ok &= __popc(__hip_atomic_load(ctrl + kXccMask + 32 * g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 1;
  return ok;
}

// Grid-wide barrier number b (1, 2, ... within one launch) of the persistent launch.
//
// Arrival is a two-level tree: workgroup w counts into group (w mod 8), whose counter lives
// on its own cache line; the last arrival of a group counts into the top counter; the last
// group leader publishes b in the release word, which every workgroup polls.  A single
// counter for all 256 workgroups serialises 256 same-address device-scope atomics when the
// workgroups arrive together.  All counters are monotonic within a launch (group g reads
// b * n_g after barrier b) and are reset by the last workgroup to leave the kernel.
//
// Ordering: every arrival is preceded by a release fence (the XCD's L2 is written back); a
// group leader and the final arrival run fences between their counter updates, and every
// waiter runs an acquire fence after seeing the release word, so each workgroup's stores
// before the barrier are visible to every workgroup after it.  One wave per workgroup runs
// the fences: the cache operations they issue act on the whole CU / XCD.
//
// Every wait is bounded: after ~0.5 s the status word records a timeout and the wait ends.
//
// Light release (`light`, decided after the launch's first barrier): when every group's
// workgroups run on one XCC -- each workgroup records its XCC in its group's mask word before
// the first barrier, which uses the full release -- a member's stores, complete in its XCC's L2
// once it counts in (vmcnt(0)), are written back by the group's last arrival, which runs on the
// same XCC: one L2 write-back per XCC and barrier instead of one per workgroup and two more on
// the leaders' path.
//
// drop_l2 (light releases only): the group's last arrival also drops its XCC's clean L2 lines
// (agent-scope acquire) before counting in.  Every other member of the group has counted in and
// waits for the release word, so nothing on that XCC loads again before the barrier ends, and
// every store of the barrier's other workgroups is written back before the word is set: after
// the barrier the XCC's L2 holds nothing from before it, at one invalidation per XCC.
//
// proven (thread 0, optional): set when this workgroup proved on arrival that every barrier group
// runs on one XCC (so the caller need not read the group masks again).
// The barrier in two halves, so that a workgroup can issue loads that do not depend on the
// barrier (data no workgroup writes before it) between its arrival and its wait.
__device__ __forceinline__ void grid_barrier_arrive(KP& p, unsigned b, bool light = false, bool drop_l2 = false,
                                                    bool* proven = nullptr) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int ng_all = p.nwg < kBarGroups ? p.nwg : kBarGroups;
    const int g = (int)blockIdx.x % ng_all;
    const unsigned n_g = (unsigned)((p.nwg - g + ng_all - 1) / ng_all);
    auto ctrl = gl(p.ctrl);
    // a member's release can be left to its group's last arrival (which releases in either
    // mode) once the groups are known to run on one XCC each
    const bool single = !light && groups_single_xcc(p);
    if (!light && !single) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (proven != nullptr) *proven = single;
    const unsigned prev = __hip_atomic_fetch_add(ctrl + kGroup + 32 * g, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == b * n_g) {
      if (light) {
        if (drop_l2) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent");  // write back, then drop
        else __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");          // the XCC's L2, all members
      }
      else acq_rel_fence(p.l2_coherent);
      const unsigned top = __hip_atomic_fetch_add(ctrl + kTop, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (top + 1 == b * (unsigned)ng_all) {
        if (!light) acq_rel_fence(p.l2_coherent);
        __hip_atomic_store(ctrl + kFlag, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}
__device__ __forceinline__ void grid_barrier_wait(KP& p, unsigned b) {
  if (threadIdx.x == 0) {
    auto ctrl = gl(p.ctrl);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(ctrl + kFlag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < b) {
      __builtin_amdgcn_s_sleep(1);
      if (__builtin_amdgcn_s_memrealtime() - t0 > 50000000ull) {
        __hip_atomic_store(ctrl + kStatus, (unsigned)MOEL_DEV_TIMEOUT, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    acquire_fence(p.l2_coherent);
  }
  __syncthreads();
}
__device__ __forceinline__ void grid_barrier(KP& p, unsigned b, bool light = false, bool drop_l2 = false,
                                             bool* proven = nullptr) {
  grid_barrier_arrive(p, b, light, drop_l2, proven);
  grid_barrier_wait(p, b);
}

__device__ __forceinline__ void stamp(KP& p, int slot) {
  if (p.dbg_ts != nullptr && threadIdx.x == 0)
    gl(p.dbg_ts)[blockIdx.x * MOEL_N_STAMPS_DEV + slot] = __builtin_amdgcn_s_memrealtime();
}

}  // namespace moel
