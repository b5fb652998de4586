// Kernels (persistent layer launch, one-kernel-per-step chain, weight packing) and the
// host side of the C ABI declared in include/moel.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/moel.h"
#include "moel_phases.h"

using namespace moel;

// =========================================================================================
// device: persistent launch
// =========================================================================================
// Each phase of the persistent launch is a separate (non-inlined) function so that the
// register allocator sizes each phase on its own instead of the union of all of them.
template <int PH, int D>
__device__ __forceinline__ void fused_phase(uint64_t ph, int wg_arg) {
  KP& p = params_from(ph);
  const int wg = uniform(wg_arg);
  char* smem = moel_lds;
  // step 0 (RMSNorm 1) has no work of its own: the QKV pass computes rstd from the rows it
  // reads anyway
  if constexpr (PH == kPhQkv) phase_qkv(p, wg, smem);
  if constexpr (PH == kPhAttnMerge) {
    if (p.attn_set_merge) phase_attn_merge_set(p, wg);
    else phase_attn_merge(p, wg);
  }
  if constexpr (PH == kPhOproj) phase_oproj(p, wg, smem);
  if constexpr (PH == kPhRouterPool) phase_router_pool(p, wg, smem);
  if constexpr (PH == kPhGemm1) {
    compute_routing(p, route_tables(smem), wg == 0);
    write_expert_hist(p, route_tables(smem), wg);
    phase_experts<true>(p, wg, smem);
  }
  if constexpr (PH == kPhGemm2) phase_experts<false>(p, wg, smem);
  if constexpr (PH == kPhCombine) phase_combine(p, wg, smem);
  if constexpr (PH == kPhUnpool) phase_unpool(p, wg, smem);
}

// A dense phase of the persistent launch (o-projection, router/pooler, unpooler), with the
// second half of the barrier before it run inside its first pass.
template <int PH>
__device__ __forceinline__ void fused_dense(uint64_t ph, int wg_arg, const BarWait& wait) {
  KP& p = params_from(ph);
  const int wg = uniform(wg_arg);
  if constexpr (PH == kPhOproj) phase_oproj(p, wg, moel_lds, wait);
  if constexpr (PH == kPhRouterPool) phase_router_pool(p, wg, moel_lds, wait);
  if constexpr (PH == kPhUnpool) phase_unpool(p, wg, moel_lds, wait);
}

// The down projection of the persistent launch, with the second half of barrier number bar run
// inside its first expert stream.
__device__ __forceinline__ void fused_down(uint64_t ph, int wg_arg, unsigned bar) {
  KP& p = params_from(ph);
  phase_experts<false>(p, uniform(wg_arg), moel_lds, (int)bar);
}

// The attention phase of the persistent launch, with the second half of the barrier before it
// (wait) called inside it.
template <int D, class Wait>
__device__ __forceinline__ void fused_attn(uint64_t ph, int wg_arg, Wait&& wait) {
  KP& p = params_from(ph);
  phase_attn<D>(p, uniform(wg_arg), moel_lds, wait);
}

// Barrier number ++bar of the launch, in two halves (see grid_barrier_arrive).  After the first
// one, every workgroup knows whether the barrier groups run on one XCC each; when they do, the
// rest of the launch's barriers and split-K fix-ups release per XCC (`light`, kept in
// RouteTables::light).
struct BarArrival {
  bool proven;  // thread 0: proved single-XCC groups on arrival
  bool lt;      // arrived with light release
};
__device__ __forceinline__ BarArrival launch_barrier_arrive(KP& p, unsigned& bar, bool light) {
  // before the first barrier a split-K fix-up of this workgroup may already have proven the
  // barrier groups single-XCC (RouteTables::light): the barrier then needs no proof of its own
  BarArrival a{false, light || (bar == 0 && route_tables(moel_lds).light != 0)};
  grid_barrier_arrive(p, ++bar, a.lt, false, &a.proven);
  return a;
}
__device__ __forceinline__ void launch_barrier_wait(KP& p, unsigned bar, bool& light, const BarArrival& a) {
  grid_barrier_wait(p, bar);
  if (bar == 1) {
    RouteTables& R = route_tables(moel_lds);
    if (threadIdx.x == 0) {
      // proven on arrival or before: the masks are final (every workgroup recorded its bit
      // before it counted itself in), so they need no second read
      int ok = 1;
      if (!a.proven && !a.lt) {
        const int ng_all = p.nwg < kBarGroups ? p.nwg : kBarGroups;
        for (int g = 0; g < ng_all; ++g)
          ok &= __popc(__hip_atomic_load(gl(p.ctrl) + kXccMask + 32 * g, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)) == 1;
      }
      R.light = ok;
    }
    __syncthreads();
    light = R.light != 0;
  }
}
__device__ __forceinline__ void launch_barrier(KP& p, unsigned& bar, bool& light) {
  const BarArrival a = launch_barrier_arrive(p, bar, light);
  launch_barrier_wait(p, bar, light, a);
}

// Launch entry: the abort word, and this workgroup's XCC into its barrier group's mask.
__device__ __forceinline__ bool launch_enter(KP& p) {
  __shared__ int s_abort;
  RouteTables& R = route_tables(moel_lds);
  if (threadIdx.x == 0) {
    s_abort = aborted(p) ? 1 : 0;
    R.light = 0;
    const int ng_all = p.nwg < kBarGroups ? p.nwg : kBarGroups;
    // the mask bit is recorded (the returning atomic has completed) before the entry count
    const unsigned m = __hip_atomic_fetch_or(gl(p.ctrl) + kXccMask + 32 * ((int)blockIdx.x % ng_all),
                                             1u << xcc_id(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" : : "v"(m) : "memory");
    __hip_atomic_fetch_add(gl(p.ctrl) + kEntered, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return s_abort == 0;
}

// Launch exit: the last workgroup out resets the barrier words for the next launch (and moves
// the status to the caller's word when one is given).
__device__ __forceinline__ void launch_exit(KP& p, bool run) {
  __syncthreads();
  if (threadIdx.x == 0) {
    if (!run && blockIdx.x == 0)
      __hip_atomic_store(gl(p.ctrl) + kStatus, MOEL_DEV_ABORTED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned prev =
        __hip_atomic_fetch_add(gl(p.ctrl) + kExit, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == (unsigned)p.nwg - 1) {
      auto ctrl = gl(p.ctrl);
      if (p.status_out != nullptr) {
        __hip_atomic_store(gl(p.status_out),
                           __hip_atomic_load(ctrl + kStatus, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctrl + kStatus, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(ctrl + kFlag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctrl + kTop, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int g = 0; g < kBarGroups; ++g)
        __hip_atomic_store(ctrl + kGroup + 32 * g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = 0; i < 2; ++i)
        __hip_atomic_store(ctrl + kWork + 32 * i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int g = 0; g < kBarGroups; ++g)
        __hip_atomic_store(ctrl + kXccMask + 32 * g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctrl + kEntered, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctrl + kExit, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The phases of one layer with a grid barrier between consecutive ones (the persistent
// launch's body; the stack launch runs it once per layer).
//
// qkv_wait (> 0): number of the grid barrier before the layer (between two layers of one
// launch), whose second half the QKV phase runs after its first weight loads; 0: none.
template <int D>
__device__ __forceinline__ void layer_phases(uint64_t ph, int wg, bool run, unsigned& bar, bool& light,
                                             unsigned qkv_wait = 0) {
  KP& p = params_from(ph);
  auto stamp = [&](int slot) {
    if (run) moel::stamp(p, slot);
  };
  auto sync = [&]() { launch_barrier(p, bar, light); };
  stamp(16 + kPhNorm1);
  stamp(kPhNorm1);
  if (qkv_wait > 0) {
    if (run) phase_qkv(p, wg, moel_lds, BarWait{ph, qkv_wait, 16 + kPhQkv});
    else grid_barrier_wait(p, qkv_wait);
  } else {
    stamp(16 + kPhQkv);
    if (run) fused_phase<kPhQkv, D>(ph, wg);
  }
  stamp(kPhQkv);
  {
    // the barrier before attention in two halves: attention items fetch their first cached key
    // rows between the arrival and the wait
    const BarArrival a = launch_barrier_arrive(p, bar, light);
    auto wait = [&]() {
      launch_barrier_wait(p, bar, light, a);
      stamp(16 + kPhAttn);
    };
    if (run) fused_attn<D>(ph, wg, wait);
    else wait();
  }
  stamp(kPhAttn);
  // with the merge per barrier group the merging workgroups wait for their group's items
  if (!p.attn_set_merge) sync();
  stamp(16 + kPhAttnMerge);
  if (run) fused_phase<kPhAttnMerge, D>(ph, wg);
  stamp(kPhAttnMerge);
  {
    // the barrier in two halves: the phase's first weight loads are issued before the wait
    const BarArrival a = launch_barrier_arrive(p, bar, light);
    if (run) fused_dense<kPhOproj>(ph, wg, BarWait{ph, bar, 16 + kPhOproj});
    else launch_barrier_wait(p, bar, light, a);
  }
  stamp(kPhOproj);
  {
    // the barrier in two halves: the phase's first weight loads are issued before the wait
    const BarArrival a = launch_barrier_arrive(p, bar, light);
    if (run) fused_dense<kPhRouterPool>(ph, wg, BarWait{ph, bar, 16 + kPhRouterPool});
    else launch_barrier_wait(p, bar, light, a);
  }
  stamp(kPhRouterPool);
  sync();
  stamp(16 + kPhGemm1);
  if (run) fused_phase<kPhGemm1, D>(ph, wg);
  stamp(kPhGemm1);
  {
    // the barrier in two halves: the down projection's first weight loads before the wait
    const BarArrival a = launch_barrier_arrive(p, bar, light);
    if (run) fused_down(ph, wg, bar);
    else launch_barrier_wait(p, bar, light, a);
  }
  stamp(kPhGemm2);
  sync();
  stamp(16 + kPhCombine);
  // the expert phases' work counters (and the attention groups' item counts) are free again
  // once both expert phases (the merge) have passed a barrier: cleared here for the next layer
  // of the launch (or the next launch)
  if (wg == 0 && threadIdx.x == 0) {
    for (int i = 0; i < 2; ++i)
      __hip_atomic_store(gl(p.ctrl) + kWork + 32 * i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int q = 0; q < kBarGroups; ++q)
      __hip_atomic_store(gl(p.ctrl) + kAttnDone + 32 * q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (run) fused_phase<kPhCombine, D>(ph, wg);
  stamp(kPhCombine);
  {
    // the barrier in two halves: the phase's first weight loads are issued before the wait
    const BarArrival a = launch_barrier_arrive(p, bar, light);
    if (run) fused_dense<kPhUnpool>(ph, wg, BarWait{ph, bar, 16 + kPhUnpool});
    else launch_barrier_wait(p, bar, light, a);
  }
  stamp(kPhUnpool);
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_layer_fused(LayerParams p_arg) {
  KP& p = kernel_params();
  const int wg = blockIdx.x;
  const uint64_t t_entry = __builtin_amdgcn_s_memrealtime();
  const bool run = launch_enter(p);
  // an aborted launch leaves every caller buffer untouched, the timestamps included
  if (run && p.dbg_ts != nullptr && threadIdx.x == 0)
    gl(p.dbg_ts)[blockIdx.x * MOEL_N_STAMPS_DEV + kNumPhases] = t_entry;  // entry
  unsigned bar = 0;
  bool light = false;
  layer_phases<D>(params_handle(p), wg, run, bar, light);
  launch_exit(p, run);
}

// Consecutive layers in one persistent launch: layer l's parameters (its weights, caches,
// window, and its input and output rows: layer l + 1 reads what layer l wrote) are kernel
// arguments like the single layer's, read through the constant cache; a grid barrier separates
// consecutive layers.  Kernel arguments, not a table in device memory: every launch gets a fresh
// argument buffer, so no cache can hold parameters of an earlier launch.
constexpr int kStackLayersPerLaunch = MOEL_STACK_LAYERS_PER_LAUNCH;  // 4 x 936 B fit the 4 KiB argument segment
struct StackArgs {
  LayerParams layer[kStackLayersPerLaunch];
  int n;
};
static_assert(sizeof(StackArgs) <= 4096, "stack launch arguments exceed the kernel argument segment");

// One layer of the stack launch, not inlined (the loop around it then holds only its counters
// and the register allocator sizes the layer's body on its own).  state: the launch's barrier
// count in bits 0..30, the light-release flag in bit 31; returns the state after the layer.
template <int D>
__device__ __noinline__ unsigned stack_layer(uint64_t ph_arg, int wg_arg, int run_arg, unsigned state_arg) {
  const uint64_t ph = ph_arg;  // params_from moves it to scalar registers
  const int wg = uniform(wg_arg);
  const bool run = uniform(run_arg) != 0;
  const unsigned state = (unsigned)uniform((int)state_arg);
  unsigned bar = state & 0x7fffffffu;
  bool light = (state >> 31) != 0;
  unsigned qkv_wait = 0;
  if (bar > 0) {
    // this layer's input is complete.  It rewrites the workspace lines of the layer before from
    // whichever XCD computes them, and an XCD's L2 can keep its own earlier copy past another
    // XCD's write, so every XCD drops its L2's clean lines here, as the boundary between two
    // launches would: with light releases once per XCC inside the barrier (its group's last
    // arrival), otherwise every workgroup after the barrier, whose release wrote every XCD's
    // dirty lines back
    KP& p = params_from(ph);
    if (light && p.l2_coherent) {
      // the barrier's second half runs in the layer's QKV phase, after the first weight loads:
      // the next layer's weights are in flight across the layer boundary.  They may be issued
      // before the group's last arrival drops the XCC's L2; weights are written by no one, so
      // the drop cannot leave them stale, and everything else is read after the wait
      grid_barrier_arrive(p, ++bar, true, true);
      qkv_wait = bar;
    } else {
      launch_barrier(p, bar, light);
      if (threadIdx.x == 0 && p.l2_coherent) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __syncthreads();
    }
  }
  layer_phases<D>(ph, wg, run, bar, light, qkv_wait);
  return bar | (light ? 0x80000000u : 0u);
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_stack_fused(StackArgs a_arg) {
  const uint64_t base = reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr());
  KP& p0 = params_from(base);
  const int nlayers = *reinterpret_cast<const __attribute__((address_space(4))) int*>(
      base + offsetof(StackArgs, n));
  const bool run = launch_enter(p0);
  unsigned state = 0;
  for (int l = 0; l < nlayers; ++l)
    state = stack_layer<D>(base + (uint64_t)l * sizeof(LayerParams), (int)blockIdx.x, run ? 1 : 0, state);
  launch_exit(p0, run);
}

// =========================================================================================
// device: streaming-read reference (moel_measure_read_bandwidth)
// =========================================================================================
// Every workgroup reads its share of `per_wg` 16-byte words, four loads per thread in flight.
// The xor of the loaded words is kept so that the loads stay; it is stored only if it equals
// a value no sum of the reads is meant to take (the store's condition is never relied on).
constexpr int kReadDepth = 4;
__device__ unsigned g_read_sink;
__global__ __launch_bounds__(kThreads) void k_stream_read(const u32x4* buf, size_t per_wg) {
  const u32x4* base = buf + (size_t)blockIdx.x * per_wg;
  unsigned acc = 0;
  for (size_t i = threadIdx.x; i < per_wg; i += (size_t)kThreads * kReadDepth) {
    u32x4 v[kReadDepth];
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) {
      const size_t j = i + (size_t)d * kThreads;
      v[d] = __builtin_nontemporal_load(base + (j < per_wg ? j : per_wg - 1));
    }
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) acc ^= v[d][0] ^ v[d][3];
  }
  if (acc == 0x9e3779b9u) g_read_sink = acc;
}

// =========================================================================================
// device: one kernel per step (ablation / fallback chain)
// =========================================================================================
template <int PH, int D>
__global__ __launch_bounds__(kThreads) void k_layer_phase(LayerParams p_arg) {
  KP& p = kernel_params();
  char* smem = moel_lds;
  __shared__ int s_abort;
  const int wg = blockIdx.x;
  // the expert phases' work counters are free again once both expert kernels have finished
  // (stream order): the combine kernel clears them for the next call, aborted or not
  if (PH == kPhCombine && wg == 0 && threadIdx.x == 0)
    for (int i = 0; i < 2; ++i)
      __hip_atomic_store(gl(p.ctrl) + kWork + 32 * i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0) {
    s_abort = aborted(p) ? 1 : 0;
    route_tables(smem).light = 0;  // no barriers here: split-K fix-ups use the full release
  }
  __syncthreads();
  if (s_abort) {
    if (wg == 0 && threadIdx.x == 0)
      __hip_atomic_store(gl(p.ctrl) + kStatus, MOEL_DEV_ABORTED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  stamp(p, 16 + PH);
  if constexpr (PH == kPhQkv) phase_qkv(p, wg, smem);
  if constexpr (PH == kPhAttn) phase_attn<D>(p, wg, smem, [] {});
  if constexpr (PH == kPhAttnMerge) phase_attn_merge(p, wg);
  if constexpr (PH == kPhOproj) phase_oproj(p, wg, smem);
  if constexpr (PH == kPhRouterPool) phase_router_pool(p, wg, smem);
  if constexpr (PH == kPhGemm1) {
    compute_routing(p, route_tables(smem), wg == 0);
    write_expert_hist(p, route_tables(smem), wg);
    phase_experts<true>(p, wg, smem);
  }
  if constexpr (PH == kPhGemm2) {
    compute_routing(p, route_tables(smem), false);
    phase_experts<false>(p, wg, smem);
  }
  if constexpr (PH == kPhCombine) {
    compute_routing(p, route_tables(smem), false);
    phase_combine(p, wg, smem);
  }
  if constexpr (PH == kPhUnpool) phase_unpool(p, wg, smem);
  stamp(p, PH);
}

// =========================================================================================
// device: weight packing and small utilities
// =========================================================================================
__global__ void k_pack_dense(const uint16_t* __restrict__ src, int N, int K, int rope_D,
                             uint8_t* __restrict__ dst, size_t nchunks) {
  const size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nchunks) return;
  const int S = K / 32;
  const int lane = (int)(c % 64);
  const size_t step = (c / 64) % S;
  const size_t tile = c / (64 * (size_t)S);
  const int R = (int)(tile * 16 + (lane & 15));
  int row = R;
  if (rope_D > 0) {
    const int head = R / rope_D, r = R % rope_D;
    row = head * rope_D + (r >> 1) + (r & 1) * (rope_D / 2);
  }
  // hardware k slot j of quarter q holds k = 4q + j (j < 4) or 16 + 4q + (j - 4) (j >= 4)
  const uint16_t* r = src + (size_t)row * K + step * 32 + 4 * (lane >> 4);
  const u32x2 lo = *reinterpret_cast<const u32x2*>(r);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(r + 16);
  *reinterpret_cast<u32x4*>(dst + c * 16) = u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// one thread per (expert, 64-row tile, k pair, lane)
__global__ void k_pack_nvfp4(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                             int N, int K, uint8_t* __restrict__ dst, size_t nthreads) {
  const size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= nthreads) return;
  const int lane = (int)(c % 64);
  const size_t pairs = K / 64;
  const size_t pp = (c / 64) % pairs;
  const size_t tile_all = c / (64 * pairs);  // expert * (N/64) + tile
  const size_t row_all = tile_all * 64 + lane;
  const uint8_t* crow = codes + row_all * (size_t)(K / 2);
  const uint8_t* srow = scales + row_all * (size_t)(K / 16);
  uint8_t* out = dst + tile_all * (size_t)(36 * K) + pp * 2304;
  *reinterpret_cast<u32x4*>(out + lane * 16) = *reinterpret_cast<const u32x4*>(crow + (2 * pp) * 16);
  *reinterpret_cast<u32x4*>(out + 1024 + lane * 16) =
      *reinterpret_cast<const u32x4*>(crow + (2 * pp + 1) * 16);
  *reinterpret_cast<uint32_t*>(out + 2048 + lane * 4) = *reinterpret_cast<const uint32_t*>(srow + pp * 4);
}

__global__ void k_set_word(unsigned* w, unsigned v) { *w = v; }

__global__ void k_fill_u32(unsigned* w, unsigned v, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = v;
}

// RoPE rows [pos0, pos0 + nrows) of the cos/sin table: angle = position * inv_freq[i] in
// double (inv_freq = theta^(-2i/D), evaluated on the host), cos and sin in double, stored as
// float -- the same values as the plan's host-computed table.
struct RopeFreq {
  double f[64];
};
__global__ void k_rope_rows(float* cos_out, float* sin_out, int pos0, int nrows, int half, RopeFreq fq) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= nrows * half) return;
  const int r = e / half, i = e - r * half;
  const double a = (double)(pos0 + r) * fq.f[i];
  cos_out[e] = (float)cos(a);
  sin_out[e] = (float)sin(a);
}

// Cross-XCD coherence check of the L2 caches for memory from hipMalloc (the plan's workspace
// and the caller's tensors).  Workgroups 1..15 (every XCD under round-robin dispatch, the
// writer's included) read a 64 KiB block, so that their XCDs' L2 hold copies of it; workgroup
// 0 then overwrites the block with `gen`, runs the grid barrier's release fence and raises a
// flag; each reader sees the flag, invalidates only its L1 (the barrier's L1-only acquire)
// and re-reads the block, counting words that are not `gen`.  Every spin is bounded; a
// timed-out spin counts as a failure.  out[0]: stale words, out[1]: timeouts.
constexpr int kCohWords = 16384;
constexpr int kCohBlocks = 16;
__device__ bool coh_spin(unsigned* f, unsigned v) {
  for (int it = 0; it < (1 << 22); ++it) {
    if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= v) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}
__global__ __launch_bounds__(256) void k_coherence_check(unsigned* buf, unsigned* flags, unsigned* out, unsigned gen) {
  __shared__ int ok;
  if (blockIdx.x > 0) {
    unsigned acc = 0;
    for (int i = threadIdx.x; i < kCohWords; i += 256) acc += buf[i];
    if (acc == 0x9e3779b9u) out[3] = acc;  // keeps the first read
    __syncthreads();
    if (threadIdx.x == 0) {
      __hip_atomic_fetch_add(flags + 0, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      ok = coh_spin(flags + 1, gen) ? 1 : 0;
      asm volatile("buffer_inv sc0" ::: "memory");
    }
    __syncthreads();
    unsigned stale = 0;
    for (int i = threadIdx.x; i < kCohWords; i += 256) stale += buf[i] != gen;
    atomicAdd(out, stale);
    if (threadIdx.x == 0 && !ok) atomicAdd(out + 1, 1u);
  } else {
    if (threadIdx.x == 0) ok = coh_spin(flags + 0, kCohBlocks - 1) ? 1 : 0;
    __syncthreads();
    for (int i = threadIdx.x; i < kCohWords; i += 256) buf[i] = gen;
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(flags + 1, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!ok) atomicAdd(out + 1, 1u);
    }
  }
}
__global__ void k_coherence_fill(unsigned* buf, unsigned v, unsigned* flags, unsigned* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < kCohWords) buf[i] = v;
  if (i < 4) {
    flags[i] = 0u;
    out[i] = 0u;
  }
}

// =========================================================================================
// host
// =========================================================================================
struct moel_stack {
  moel_plan* plan;
  int n;
  moel_weights* w;          // [n] (host copies of the caller's structs)
  void** k;                 // [n] caches
  void** v;
  int32_t* window;          // [n]
  float* act[2];            // device [16][H]: the rows passed between layers
};

struct moel_plan {
  moel_config cfg;
  int device;
  int nwg;
  int grp;
  void* ws;
  size_t ws_bytes;
  LayerParams base;  // shape + scratch pointers
  size_t lds_fused;
  size_t lds_phase[kNumPhases];
  int launch_mode;  // moel_launch_mode
  int acquire_mode;  // moel_acquire_mode
  int l2_coherent;   // result of the coherence check on the plan's device
};

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }


template <int D>
size_t attn_lds() { return sizeof(AttnLds<D>); }

constexpr size_t kLdsLimit = 160 * 1024;  // LDS of one CDNA4 compute unit
static_assert(kRouteBytes + sizeof(Fp4Lds) <= kLdsLimit, "expert-phase LDS exceeds one CU");
static_assert(kRouteBytes + sizeof(AttnLds<128>) <= kLdsLimit, "attention LDS exceeds one CU");

size_t lds_for_phase(int ph, int D) {
  size_t body = 0;
  switch (ph) {
    case kPhNorm1: case kPhAttnMerge: case kPhCombine: body = 0; break;
    case kPhAttn: body = D == 64 ? attn_lds<64>() : attn_lds<128>(); break;
    case kPhGemm1: case kPhGemm2: body = sizeof(Fp4Lds) > sizeof(DenseLds) ? sizeof(Fp4Lds) : sizeof(DenseLds); break;
    default: body = sizeof(DenseLds); break;
  }
  return kRouteBytes + body;
}

// LDS of the persistent launch: the largest phase
size_t lds_fused_bytes(int D) {
  size_t mx = 0;
  for (int ph = 0; ph < kNumPhases; ++ph) mx = std::max(mx, lds_for_phase(ph, D));
  return mx;
}

bool hip_ok(hipError_t e) {
  if (e != hipSuccess) {
    if (std::getenv("MOEL_LOG")) std::fprintf(stderr, "moel: HIP error %s\n", hipGetErrorString(e));
    return false;
  }
  return true;
}

// Runs the coherence check four times on `mem` (kCohMemWords words of device memory) on
// stream `s`; true when no stale word and no timeout was seen.
constexpr int kCohMemWords = kCohWords + 64;
bool coherence_check_on(unsigned* mem, hipStream_t s) {
  unsigned* buf = mem;
  unsigned* flags = mem + kCohWords;
  unsigned* out = mem + kCohWords + 32;
  bool good = true;
  for (unsigned rep = 0; good && rep < 4; ++rep) {
    const unsigned gen = 0x5a000001u + rep;
    hipLaunchKernelGGL(k_coherence_fill, dim3(kCohWords / 256), dim3(256), 0, s, buf, gen - 1, flags, out);
    hipLaunchKernelGGL(k_coherence_check, dim3(kCohBlocks), dim3(256), 0, s, buf, flags, out, gen);
    unsigned h[2] = {1u, 1u};
    good = hip_ok(hipGetLastError()) && hip_ok(hipStreamSynchronize(s)) &&
           hip_ok(hipMemcpy(h, out, sizeof(h), hipMemcpyDeviceToHost)) && h[0] == 0 && h[1] == 0;
  }
  return good;
}

// The coherence check's result for device `dev`, kept per device for the process.  The first
// query runs the check: on `mem` / `s` when given (memory the caller owns), else on memory and a
// stream allocated for it.
std::mutex g_coh_mu;
bool l2_coherent_device(int dev, unsigned* mem = nullptr, hipStream_t s = nullptr) {
  static int known[64];  // 0 unknown, 1 coherent, 2 not
  std::lock_guard<std::mutex> lock(g_coh_mu);
  if (dev >= 0 && dev < 64 && known[dev] != 0) return known[dev] == 1;
  bool good;
  if (mem != nullptr) {
    good = coherence_check_on(mem, s);
  } else {
    unsigned* own = nullptr;
    hipStream_t os = nullptr;
    good = hip_ok(hipMalloc(&own, kCohMemWords * sizeof(unsigned))) && hip_ok(hipStreamCreate(&os)) &&
           coherence_check_on(own, os);
    if (os != nullptr) (void)hipStreamDestroy(os);
    if (own != nullptr) (void)hipFree(own);
  }
  if (dev >= 0 && dev < 64) known[dev] = good ? 1 : 2;
  return good;
}

template <int D>
const void* fused_fn() { return reinterpret_cast<const void*>(&k_layer_fused<D>); }
template <int D>
const void* stack_fn() { return reinterpret_cast<const void*>(&k_stack_fused<D>); }

template <int D>
const void* phase_fn(int ph) {
  switch (ph) {
    case 0: return reinterpret_cast<const void*>(&k_layer_phase<0, D>);
    case 1: return reinterpret_cast<const void*>(&k_layer_phase<1, D>);
    case 2: return reinterpret_cast<const void*>(&k_layer_phase<2, D>);
    case 3: return reinterpret_cast<const void*>(&k_layer_phase<3, D>);
    case 4: return reinterpret_cast<const void*>(&k_layer_phase<4, D>);
    case 5: return reinterpret_cast<const void*>(&k_layer_phase<5, D>);
    case 6: return reinterpret_cast<const void*>(&k_layer_phase<6, D>);
    case 7: return reinterpret_cast<const void*>(&k_layer_phase<7, D>);
    case 8: return reinterpret_cast<const void*>(&k_layer_phase<8, D>);
    default: return reinterpret_cast<const void*>(&k_layer_phase<9, D>);
  }
}

// Split-K of a dense contraction of N rows over K on nwg workgroups: the number of K ranges.
// A workgroup of an unsplit phase reads the whole fp32 activation (16 x K x 4 B) beside its
// share of the weights (N x K x 2 B / nwg); split into S ranges, it reads 1/S of the activation
// for the same weight bytes, and the partial sums then cost a fix-up (arrival count, ordered
// sum by the block's last unit: ~5 us).  Measured on full-width and stack-share layers, the
// split pays only while the activation a workgroup reads exceeds its weights, i.e. while
// 32 nwg / (S N) > 1, and it is taken up to the smallest power of two that ends that (at most 8,
// each range at least 1,024 k so that every wave streams 4 or more steps).  The router/pooler
// (N = E + P rows, none of them a multiple of a workgroup's share) measured best one step
// further, while the activation exceeds half the weights (4 ranges instead of 2 at E 256,
// P 4096: 23.2-23.6 against 24.4-24.9 us on the full-width and the stack-share layers; QKV,
// o-projection and unpooler measured worse with any further split).
int choose_split(int N, int K, int nwg, double act_over_w = 1.0) {
  int ns = 1;
  while (ns < 8 && 32.0 * nwg / ((double)ns * N) > act_over_w + 1e-9 && (K / 32) % (2 * ns) == 0 &&
         K / (2 * ns) >= 1024)
    ns *= 2;
  return ns;
}

// The splits of the four dense phases (QKV, o-projection, router/pooler, unpooler).
// MOEL_DENSE_SPLITS = "q,o,r,u" (or one number for all) overrides the choice where the value is
// valid for the phase's shape (measurement of alternatives).
void dense_splits(const moel_config* cfg, int nwg, int out[4]) {
  const int N[4] = {(cfg->n_q_heads + 2 * cfg->n_kv_heads) * cfg->head_dim, cfg->hidden,
                    cfg->n_experts + cfg->pooled, cfg->hidden};
  const int K[4] = {cfg->hidden, cfg->n_q_heads * cfg->head_dim, cfg->hidden, cfg->pooled};
  int forced[4] = {0, 0, 0, 0};
  if (const char* env = std::getenv("MOEL_DENSE_SPLITS")) {
    int n = std::sscanf(env, "%d,%d,%d,%d", &forced[0], &forced[1], &forced[2], &forced[3]);
    if (n == 1) forced[1] = forced[2] = forced[3] = forced[0];
  }
  for (int i = 0; i < 4; ++i) {
    out[i] = choose_split(N[i], K[i], nwg, i == 2 ? 0.5 : 1.0);
    const int f = forced[i];
    if (f >= 1 && f <= 16 && (f & (f - 1)) == 0 && (K[i] / 32) % f == 0 && (K[i] / 32) / f >= 1 && nwg / f >= 1)
      out[i] = f;
  }
}

// Byte offsets of the workspace regions for a shape, a grid of nwg workgroups and a RoPE table
// of rope_rows rows.
struct WsLayout {
  size_t ctrl, q, qop, ao, aml, o, h, lg, pl, a, d, pls, as, aq, m, oop, hop, mop, part, part_ss, cos, sin, total;
};
WsLayout ws_layout(const moel_config* cfg, int nwg, int rope_rows) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t D = cfg->head_dim, Hq = cfg->n_q_heads, H = cfg->hidden, P = cfg->pooled, I = cfg->inter;
  const size_t E = cfg->n_experts, k = cfg->top_k, grp = Hq / cfg->n_kv_heads, T = kMaxT;
  L.ctrl = take((size_t)kCtrlWords * 4);
  L.q = take(T * Hq * D * 4);
  L.qop = take(T * Hq * 2 * D * 2);
  L.ao = take((size_t)nwg * grp * T * D * 4);
  L.aml = take((size_t)nwg * grp * T * 2 * 4);
  L.o = take(T * Hq * D * 4);
  L.h = take(T * H * 4);
  L.lg = take(T * E * 4);
  L.pl = take(T * P * 4);
  L.a = take(T * k * I * 4);
  L.d = take(T * k * P * 4);
  L.pls = take(T * P * 4);
  L.as = take(T * k * I * 4);
  L.aq = take(T * k * I * 4);
  L.m = take(T * P * 4);
  L.oop = take(T * Hq * D * 4);
  L.hop = take(T * H * 4);
  L.mop = take(T * P * 4);
  {
    int sk[4];
    dense_splits(cfg, nwg, sk);
    const size_t N[4] = {(Hq + 2 * (size_t)cfg->n_kv_heads) * D, H, E + P, H};
    size_t mx = 0;
    for (int i = 0; i < 4; ++i)
      if (sk[i] > 1) mx = std::max(mx, (size_t)sk[i] * N[i] * T * 4);
    L.part = take(mx);
    L.part_ss = take((size_t)nwg * T * 4);
  }
  L.cos = take((size_t)rope_rows * (D / 2) * 4);
  L.sin = take((size_t)rope_rows * (D / 2) * 4);
  L.total = off;
  return L;
}

// Shape fields of the launch parameters and their pointers into a workspace laid out by L.
void bind_base(LayerParams& b, const moel_config* cfg, int nwg, const WsLayout& L, char* ws) {
  std::memset(&b, 0, sizeof(b));
  b.H = cfg->hidden;
  b.Hq = cfg->n_q_heads;
  b.Hkv = cfg->n_kv_heads;
  b.D = cfg->head_dim;
  b.P = cfg->pooled;
  b.I = cfg->inter;
  b.E = cfg->n_experts;
  b.topk = cfg->top_k;
  b.n_shards = cfg->n_shards;
  b.rank = cfg->shard_rank;
  b.I_loc = cfg->inter / cfg->n_shards;
  b.P_loc = cfg->pooled / cfg->n_shards;
  b.kv_cap = cfg->kv_capacity;
  b.expert_dtype = cfg->expert_dtype;
  b.down_fp4 = cfg->down_input == MOEL_DOWN_INPUT_NVFP4 ? 1 : 0;
  b.eps = cfg->rms_eps;
  b.nwg = nwg;
  b.stride_gate = moel_packed_experts_bytes(cfg, 0) / (size_t)cfg->n_experts;
  b.stride_up = moel_packed_experts_bytes(cfg, 1) / (size_t)cfg->n_experts;
  b.stride_down = moel_packed_experts_bytes(cfg, 2) / (size_t)cfg->n_experts;
  b.ctrl = reinterpret_cast<unsigned*>(ws + L.ctrl);
  b.q_buf = reinterpret_cast<float*>(ws + L.q);
  b.q_op = reinterpret_cast<uint16_t*>(ws + L.qop);
  b.attn_o = reinterpret_cast<float*>(ws + L.ao);
  b.attn_ml = reinterpret_cast<float*>(ws + L.aml);
  b.o_buf = reinterpret_cast<float*>(ws + L.o);
  b.h_buf = reinterpret_cast<float*>(ws + L.h);
  b.logits = reinterpret_cast<float*>(ws + L.lg);
  b.pl = reinterpret_cast<float*>(ws + L.pl);
  b.a_buf = reinterpret_cast<float*>(ws + L.a);
  b.d_buf = reinterpret_cast<float*>(ws + L.d);
  b.pl_split = reinterpret_cast<uint16_t*>(ws + L.pls);
  b.a_split = reinterpret_cast<uint16_t*>(ws + L.as);
  b.aq_buf = reinterpret_cast<float*>(ws + L.aq);
  b.m_buf = reinterpret_cast<float*>(ws + L.m);
  b.o_op = reinterpret_cast<uint16_t*>(ws + L.oop);
  b.h_op = reinterpret_cast<float*>(ws + L.hop);
  b.m_op = reinterpret_cast<uint16_t*>(ws + L.mop);
  b.part = reinterpret_cast<float*>(ws + L.part);
  b.part_ss = reinterpret_cast<float*>(ws + L.part_ss);
  {
    int sk[4];
    dense_splits(cfg, nwg, sk);
    b.sk_qkv = sk[0];
    b.sk_oproj = sk[1];
    b.sk_rp = sk[2];
    b.sk_unpool = sk[3];
  }
  b.rope_cos = reinterpret_cast<const float*>(ws + L.cos);
  b.rope_sin = reinterpret_cast<const float*>(ws + L.sin);
  b.rope_row0 = 0;
}

// The per-call launch parameters from the shape's base parameters (validated arguments).
// Launch parameters of one step over n_req requests (one for the single-request calls, whose
// cache is the whole pool).  parents: the token tree of a single request (NULL = chains).
moel_status fill_call_batch(const moel_config* cfg, const LayerParams& base, int l2_coherent, const moel_weights* w,
                            void* k_cache, void* v_cache, const float* x, int32_t n_req, const moel_request* req,
                            int32_t window, const int32_t* parents, float* y, const moel_debug* dbg, LayerParams& p) {
  moel_status st = moel_validate_batch(cfg, n_req, req, base.nwg);
  if (st != MOEL_OK) return st;
  int32_t T = 0;
  for (int r = 0; r < n_req; ++r) T += req[r].T;
  // the single-request arguments check the rest (x, y, weights, caches, shapes); pos 0 stands
  // for the requests' positions, checked above
  st = moel_validate_call(cfg, w, k_cache, v_cache, x, T, 0, window, y);
  if (st != MOEL_OK) return st;
  if (parents != nullptr && n_req != 1) return MOEL_ERR_ARG;
  st = moel_validate_tree(parents, T);
  if (st != MOEL_OK) return st;
  p = base;
  p.l2_coherent = l2_coherent;
  p.T = T;
  p.ntt = (T + kTile - 1) / kTile;
  p.pos = req[0].pos;
  p.window = window;
  p.n_req = n_req;
  for (int t = 0; t < kMaxT; ++t) {
    p.tok_pos[t] = 0;
    p.tok_sees[t] = 0u;
  }
  int keys[MOEL_MAX_REQUESTS];
  int total_keys = 0, t0 = 0;
  for (int r = 0; r < n_req; ++r) {
    const moel_request& q = req[r];
    p.req_t0[r] = t0;
    p.req_pos[r] = q.pos;
    p.req_kvb[r] = q.kv_base;
    // the widest key range of the request is that of a depth-0 token
    p.req_lo[r] = window > 0 ? (q.pos - window + 1 > 0 ? q.pos - window + 1 : 0) : 0;
    keys[r] = q.pos + q.T - p.req_lo[r];
    total_keys += keys[r];
    // token positions and visibility (a chain when parents is NULL)
    int depth[MOEL_MAX_TOKENS];
    for (int i = 0; i < q.T; ++i) {
      const int t = t0 + i;
      const int par = parents ? parents[i] : i - 1;
      depth[i] = par < 0 ? 0 : depth[par] + 1;
      unsigned sees = 0u;
      for (int a = i; a >= 0; a = parents ? parents[a] : a - 1)
        if (window == 0 || depth[a] > depth[i] - window) sees |= 1u << (t0 + a);
      p.tok_pos[t] = q.pos + depth[i];
      p.tok_sees[t] = sees;
    }
    t0 += q.T;
  }
  p.req_t0[n_req] = t0;
  // key chunks: at least 128 keys, at most nwg / (Hkv ntt) of them over all requests; rounded up to
  // whole 128-key sub-chunks (a full sub-chunk inside every token's window needs no mask) where
  // that keeps their number
  int maxc = base.nwg / (cfg->n_kv_heads * p.ntt);  // one item per workgroup and token tile
  if (maxc < 1) maxc = 1;
  int nch = (total_keys + 127) / 128;
  if (nch > maxc) nch = maxc;
  if (nch < n_req) nch = n_req;
  int chunk = (total_keys + nch - 1) / nch;
  auto count = [&](int c) {
    int n = 0;
    for (int r = 0; r < n_req; ++r) n += (keys[r] + c - 1) / c;
    return n;
  };
  if (count(chunk) > maxc) {
    // each request rounds its last chunk up: the smallest chunk whose count fits (count does not
    // grow with the chunk, and the longest request's key count gives n_req <= maxc chunks)
    int hi = 1;
    for (int r = 0; r < n_req; ++r) hi = keys[r] > hi ? keys[r] : hi;
    int lo = chunk;  // count(lo) > maxc >= count(hi)
    while (hi - lo > 1) {
      const int mid = lo + (hi - lo) / 2;
      (count(mid) > maxc ? lo : hi) = mid;
    }
    chunk = hi;
  }
  const int chunk128 = (chunk + 127) / 128 * 128;
  if (count(chunk128) == count(chunk)) chunk = chunk128;
  p.attn_chunk = chunk;
  int ch = 0;
  for (int r = 0; r < n_req; ++r) {
    p.req_ch0[r] = ch;
    ch += (keys[r] + chunk - 1) / chunk;
  }
  p.req_ch0[n_req] = ch;
  p.attn_nchunks = ch;
  // the merge per barrier group: every attention group (kv head, token tile) on a barrier group
  // of its own, with one item per workgroup of it (MOEL_ATTN_SET_MERGE=0 turns it off, for
  // measurement)
  {
    static const int allow = [] {
      const char* e = std::getenv("MOEL_ATTN_SET_MERGE");
      return e == nullptr || std::atoi(e) != 0;
    }();
    const int ns = base.nwg < kBarGroups ? base.nwg : kBarGroups;
    p.attn_set_merge = allow && cfg->n_kv_heads * p.ntt <= ns && ch <= base.nwg / ns ? 1 : 0;
  }
  p.gamma1 = static_cast<const uint16_t*>(w->gamma1);
  p.gamma2 = static_cast<const uint16_t*>(w->gamma2);
  p.w_qkv = static_cast<const uint8_t*>(w->w_qkv);
  p.w_o = static_cast<const uint8_t*>(w->w_o);
  p.w_router = static_cast<const uint8_t*>(w->w_router);
  p.w_pool = static_cast<const uint8_t*>(w->w_pool);
  p.w_unpool = static_cast<const uint8_t*>(w->w_unpool);
  p.w_gate = static_cast<const uint8_t*>(w->w_gate);
  p.w_up = static_cast<const uint8_t*>(w->w_up);
  p.w_down = static_cast<const uint8_t*>(w->w_down);
  p.ts_gate = w->ts_gate;
  p.ts_up = w->ts_up;
  p.ts_down = w->ts_down;
  p.ts_act = p.down_fp4 ? w->ts_act : nullptr;
  p.expert_hist = w->expert_hist;
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.v_cache = static_cast<uint16_t*>(v_cache);
  p.x = x;
  p.y = y;
  p.dbg_idx = dbg ? dbg->expert_idx : nullptr;
  p.dbg_gates = dbg ? dbg->gates : nullptr;
  p.dbg_logits = dbg ? dbg->router_logits : nullptr;
  p.dbg_ts = dbg ? reinterpret_cast<unsigned long long*>(dbg->timestamps) : nullptr;
  // the fp32 copies the step does not read are written for calls that ask for routing outputs
  // (tests read them through moel_plan_scratch), not for timestamps alone
  p.debug_copies = dbg != nullptr && (dbg->expert_idx || dbg->gates || dbg->router_logits) ? 1 : 0;
  return MOEL_OK;
}

// ------------------------------------------------------------------------------------------
// Scratch of the allocation-free entry point (moel_layer_decode_noalloc): the workspace of one
// call -- control words, activation scratch, the call's RoPE rows -- in a file-scope device
// array, one copy per device for the life of the process.  Host code never uses the array's
// name as an address: the device address comes from hipGetSymbolAddress, once per device.
// ------------------------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)MOEL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr size_t kCohOffset = 64 * 1024;  // coherence check memory, behind the control words
static_assert(kCohOffset + kCohMemWords * 4 <= kStaticScratchBytes, "coherence check memory");

struct StaticDev {
  int state;        // 0 not set up, 1 ready, < 0 the moel_status of a failed set-up
  char* ptr;        // this device's address of `scratch`
  int nwg;          // workgroups of the persistent launch (compute units)
  int l2_coherent;  // coherence check result
};
StaticDev g_static[64];
std::mutex g_static_mu;

// Once per device, with the device current: the scratch address, the launch attributes, the
// coherence check (run on the scratch itself when no plan ran it before) and zeroed control
// words.  Synchronous on `s`; allocates nothing.
moel_status static_setup(int dev, hipStream_t s, StaticDev** out) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (dev < 0 || dev >= 64) return MOEL_ERR_UNSUPPORTED;
  StaticDev& sd = g_static[dev];
  if (sd.state < 0) return static_cast<moel_status>(sd.state);
  if (sd.state == 1) {
    *out = &sd;
    return MOEL_OK;
  }
  hipDeviceProp_t prop;
  if (!hip_ok(hipGetDeviceProperties(&prop, dev))) return MOEL_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    sd.state = MOEL_ERR_UNSUPPORTED;
    return MOEL_ERR_UNSUPPORTED;
  }
  void* ptr = nullptr;
  if (!hip_ok(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) || ptr == nullptr) return MOEL_ERR_HIP;
  int per_cu64 = 0, per_cu128 = 0;
  const bool attrs =
      hip_ok(hipFuncSetAttribute(fused_fn<64>(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_fused_bytes(64))) &&
      hip_ok(hipFuncSetAttribute(fused_fn<128>(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_fused_bytes(128))) &&
      hip_ok(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu64, fused_fn<64>(), kThreads, lds_fused_bytes(64))) &&
      hip_ok(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu128, fused_fn<128>(), kThreads, lds_fused_bytes(128)));
  if (!attrs) return MOEL_ERR_HIP;
  if (per_cu64 < 1 || per_cu128 < 1) {
    sd.state = MOEL_ERR_UNSUPPORTED;
    return MOEL_ERR_UNSUPPORTED;
  }
  char* base = static_cast<char*>(ptr);
  const bool coh = l2_coherent_device(dev, reinterpret_cast<unsigned*>(base + kCohOffset), s);
  hipLaunchKernelGGL(k_fill_u32, dim3((kCtrlWords + 255) / 256), dim3(256), 0, s, reinterpret_cast<unsigned*>(base), 0u,
                     (size_t)kCtrlWords);
  if (!hip_ok(hipGetLastError()) || !hip_ok(hipStreamSynchronize(s))) return MOEL_ERR_HIP;
  sd.ptr = base;
  sd.nwg = prop.multiProcessorCount;
  sd.l2_coherent = coh ? 1 : 0;
  sd.state = 1;
  *out = &sd;
  return MOEL_OK;
}

// the expert phases split their tile cost C (< tiles per expert * 17 * slots) over the
// workgroups in 32-bit arithmetic: C * workgroups must stay below 2^31
bool work_split_fits(const moel_config* cfg, int nwg) {
  const int64_t rows = std::max(cfg->inter, cfg->pooled) / cfg->n_shards;
  const int64_t tpe = rows / (cfg->expert_dtype == MOEL_EXPERT_NVFP4 ? 64 : 16);
  return tpe * 17 * MOEL_MAX_TOKENS * cfg->top_k * nwg < ((int64_t)1 << 31);
}

moel_status fill_call(const moel_config* cfg, const LayerParams& base, int l2_coherent, const moel_weights* w,
                      void* k_cache, void* v_cache, const float* x, int32_t T, int32_t pos, int32_t window,
                      const int32_t* parents, float* y, const moel_debug* dbg, LayerParams& p) {
  if (cfg == nullptr) return MOEL_ERR_ARG;
  if (T < 1 || T > MOEL_MAX_TOKENS || pos < 0 || window < 0) return MOEL_ERR_ARG;
  if ((int64_t)pos + T > cfg->kv_capacity) return MOEL_ERR_ARG;
  const moel_request one{T, pos, 0, cfg->kv_capacity};
  return fill_call_batch(cfg, base, l2_coherent, w, k_cache, v_cache, x, 1, &one, window, parents, y, dbg, p);
}

moel_status prepare_call(moel_plan* plan, const moel_weights* w, void* k_cache, void* v_cache,
                         const float* x, int32_t T, int32_t pos, int32_t window, const int32_t* parents,
                         float* y, const moel_debug* dbg, LayerParams& p) {
  if (plan == nullptr) return MOEL_ERR_ARG;
  const int l2c = plan->acquire_mode == MOEL_ACQUIRE_AUTO && plan->l2_coherent ? 1 : 0;
  return fill_call(&plan->cfg, plan->base, l2c, w, k_cache, v_cache, x, T, pos, window, parents, y, dbg, p);
}

// One step's launch: the persistent kernel, or one kernel per step.
moel_status launch_fused(moel_plan* plan, LayerParams& p, void* stream) {
  void* args[] = {&p};
  const void* fn = plan->cfg.head_dim == 64 ? fused_fn<64>() : fused_fn<128>();
  hipError_t e = plan->launch_mode == MOEL_LAUNCH_COOPERATIVE
                     ? hipLaunchCooperativeKernel(fn, dim3(plan->nwg), dim3(kThreads), args,
                                                  (unsigned)plan->lds_fused, static_cast<hipStream_t>(stream))
                     : hipLaunchKernel(fn, dim3(plan->nwg), dim3(kThreads), args, (unsigned)plan->lds_fused,
                                       static_cast<hipStream_t>(stream));
  return hip_ok(e) ? MOEL_OK : MOEL_ERR_HIP;
}
moel_status launch_unfused(moel_plan* plan, LayerParams& p_call, void* stream) {
  // the chain's kernels end at their own boundaries: the merge is a kernel of its own, and
  // nothing runs beside attention (no expert prefetch)
  LayerParams p = p_call;
  p.attn_set_merge = 0;
  p.pf_n = 0;
  void* args[] = {&p};
  for (int ph = kPhQkv; ph < kNumPhases; ++ph) {  // step 0 is part of step 1
    const void* fn = plan->cfg.head_dim == 64 ? phase_fn<64>(ph) : phase_fn<128>(ph);
    hipError_t e = hipLaunchKernel(fn, dim3(plan->nwg), dim3(kThreads), args, (unsigned)plan->lds_phase[ph],
                                   static_cast<hipStream_t>(stream));
    if (!hip_ok(e)) return MOEL_ERR_HIP;
  }
  return MOEL_OK;
}

}  // namespace

extern "C" {

moel_status moel_plan_create(const moel_config* cfg, moel_plan** out) {
  if (out == nullptr) return MOEL_ERR_ARG;
  moel_status st = moel_validate_config(cfg);
  if (st != MOEL_OK) return st;
  int dev = 0;
  if (!hip_ok(hipGetDevice(&dev))) return MOEL_ERR_UNSUPPORTED;
  hipDeviceProp_t prop;
  if (!hip_ok(hipGetDeviceProperties(&prop, dev))) return MOEL_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOEL_ERR_UNSUPPORTED;
  int coop = 0;
  if (!hip_ok(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev))) return MOEL_ERR_HIP;
  if (!coop) return MOEL_ERR_UNSUPPORTED;

  if (!work_split_fits(cfg, prop.multiProcessorCount)) return MOEL_ERR_SHAPE;
  moel_plan* plan = new (std::nothrow) moel_plan();
  if (plan == nullptr) return MOEL_ERR_HIP;
  plan->cfg = *cfg;
  plan->device = dev;
  plan->nwg = prop.multiProcessorCount;
  plan->grp = cfg->n_q_heads / cfg->n_kv_heads;
  const int nwg = plan->nwg, D = cfg->head_dim;

  // workspace: activation scratch, barrier words and the whole RoPE table of the cache
  const WsLayout L = ws_layout(cfg, nwg, cfg->kv_capacity);
  const size_t off = L.total;
  plan->ws_bytes = off;
  if (!hip_ok(hipMalloc(&plan->ws, off))) {
    delete plan;
    return MOEL_ERR_HIP;
  }
  char* ws = static_cast<char*>(plan->ws);
  if (!hip_ok(hipMemset(ws, 0, off))) {
    (void)hipFree(plan->ws);  // error path: the first error is the one reported
    delete plan;
    return MOEL_ERR_HIP;
  }
  // RoPE table: angle = position * theta^(-2i/D), evaluated in double, stored as float
  {
    const size_t n = (size_t)cfg->kv_capacity * (D / 2);
    float* hc = static_cast<float*>(std::malloc(n * 4));
    float* hs = static_cast<float*>(std::malloc(n * 4));
    if (hc == nullptr || hs == nullptr) {
      std::free(hc);
      std::free(hs);
      (void)hipFree(plan->ws);  // error path: the first error is the one reported
      delete plan;
      return MOEL_ERR_HIP;
    }
    for (int i = 0; i < D / 2; ++i) {
      const double f = std::pow((double)cfg->rope_theta, -(2.0 * i) / (double)D);
      for (int ps = 0; ps < cfg->kv_capacity; ++ps) {
        const double a = (double)ps * f;
        hc[(size_t)ps * (D / 2) + i] = (float)std::cos(a);
        hs[(size_t)ps * (D / 2) + i] = (float)std::sin(a);
      }
    }
    const bool ok = hip_ok(hipMemcpy(ws + L.cos, hc, n * 4, hipMemcpyHostToDevice)) &&
                    hip_ok(hipMemcpy(ws + L.sin, hs, n * 4, hipMemcpyHostToDevice));
    std::free(hc);
    std::free(hs);
    if (!ok) {
      (void)hipFree(plan->ws);  // error path: the first error is the one reported
      delete plan;
      return MOEL_ERR_HIP;
    }
  }
  bind_base(plan->base, cfg, nwg, L, ws);

  // LDS budgets
  size_t mx = 0;
  for (int ph = 0; ph < kNumPhases; ++ph) {
    plan->lds_phase[ph] = lds_for_phase(ph, D);
    if (plan->lds_phase[ph] > mx) mx = plan->lds_phase[ph];
  }
  plan->lds_fused = mx;
  bool ok = true;
  if (D == 64) {
    ok = ok && hip_ok(hipFuncSetAttribute(fused_fn<64>(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)mx));
    for (int ph = 0; ph < kNumPhases; ++ph)
      ok = ok && hip_ok(hipFuncSetAttribute(phase_fn<64>(ph), hipFuncAttributeMaxDynamicSharedMemorySize,
                                            (int)plan->lds_phase[ph]));
  } else {
    ok = ok && hip_ok(hipFuncSetAttribute(fused_fn<128>(), hipFuncAttributeMaxDynamicSharedMemorySize, (int)mx));
    for (int ph = 0; ph < kNumPhases; ++ph)
      ok = ok && hip_ok(hipFuncSetAttribute(phase_fn<128>(ph), hipFuncAttributeMaxDynamicSharedMemorySize,
                                            (int)plan->lds_phase[ph]));
  }
  // the plain launch relies on one resident workgroup per compute unit
  int per_cu = 0;
  if (ok)
    ok = hip_ok(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, D == 64 ? fused_fn<64>() : fused_fn<128>(),
                                                             kThreads, mx));
  if (!ok || per_cu < 1) {
    (void)hipFree(plan->ws);  // error path: the first error is the one reported
    delete plan;
    return ok ? MOEL_ERR_UNSUPPORTED : MOEL_ERR_HIP;
  }
  plan->launch_mode = MOEL_LAUNCH_PLAIN;
  plan->acquire_mode = MOEL_ACQUIRE_AUTO;
  plan->l2_coherent = l2_coherent_device(dev) ? 1 : 0;
  if (std::getenv("MOEL_LOG"))
    std::fprintf(stderr, "moel: plan H=%d Hq=%d Hkv=%d D=%d P=%d I=%d E=%d k=%d dtype=%d shards=%d nwg=%d ws=%zu lds=%zu l2_coherent=%d splits=%d,%d,%d,%d\n",
                 cfg->hidden, cfg->n_q_heads, cfg->n_kv_heads, D, cfg->pooled, cfg->inter, cfg->n_experts,
                 cfg->top_k, cfg->expert_dtype, cfg->n_shards, nwg, off, mx, plan->l2_coherent, plan->base.sk_qkv,
                 plan->base.sk_oproj, plan->base.sk_rp, plan->base.sk_unpool);
  *out = plan;
  return MOEL_OK;
}

moel_status moel_plan_destroy(moel_plan* plan) {
  if (plan == nullptr) return MOEL_ERR_ARG;
  hipError_t e = hipFree(plan->ws);
  delete plan;
  return e == hipSuccess ? MOEL_OK : MOEL_ERR_HIP;
}

int32_t moel_plan_workgroups(const moel_plan* plan) { return plan ? plan->nwg : 0; }

moel_status moel_plan_status(moel_plan* plan) {
  if (plan == nullptr) return MOEL_ERR_ARG;
  if (!hip_ok(hipDeviceSynchronize())) return MOEL_ERR_HIP;
  unsigned words[kCtrlWords];
  if (!hip_ok(hipMemcpy(words, plan->base.ctrl, sizeof(words), hipMemcpyDeviceToHost))) return MOEL_ERR_HIP;
  if (words[kStatus] == 0) return MOEL_OK;
  // a launch that timed out or was aborted may have left barrier words behind: clear every
  // word except the abort word
  const unsigned status = words[kStatus];
  const unsigned keep_abort = words[kAbort];
  for (int i = 0; i < kCtrlWords; ++i) words[i] = 0;
  words[kAbort] = keep_abort;
  if (!hip_ok(hipMemcpy(plan->base.ctrl, words, sizeof(words), hipMemcpyHostToDevice))) return MOEL_ERR_HIP;
  return status == MOEL_DEV_TIMEOUT ? MOEL_ERR_TIMEOUT : status == MOEL_DEV_ORDER ? MOEL_ERR_INTERNAL : MOEL_ERR_ABORTED;
}

moel_status moel_plan_scratch(const moel_plan* plan, int32_t which, void** ptr, size_t* bytes) {
  if (plan == nullptr || ptr == nullptr || bytes == nullptr) return MOEL_ERR_ARG;
  const LayerParams& b = plan->base;
  const size_t T = kMaxT, k = (size_t)b.topk;
  switch (which) {
    case 0: *ptr = b.q_buf; *bytes = T * b.Hq * b.D * 4; break;
    case 1: *ptr = b.o_buf; *bytes = T * b.Hq * b.D * 4; break;
    case 2: *ptr = b.h_buf; *bytes = T * b.H * 4; break;
    case 3: *ptr = b.logits; *bytes = T * b.E * 4; break;
    case 4: *ptr = b.pl; *bytes = T * b.P * 4; break;
    case 5: *ptr = b.a_buf; *bytes = T * k * b.I * 4; break;
    case 6: *ptr = b.d_buf; *bytes = T * k * b.P * 4; break;
    case 7: *ptr = b.m_buf; *bytes = T * b.P * 4; break;
    case 8: *ptr = b.aq_buf; *bytes = T * k * b.I * 4; break;
    default: return MOEL_ERR_ARG;
  }
  return MOEL_OK;
}

moel_status moel_plan_poison_scratch(moel_plan* plan, void* stream) {
  if (plan == nullptr) return MOEL_ERR_ARG;
  // the activation scratch: from the first activation region up to the RoPE table (the
  // control words before it and the table after it are kept)
  const LayerParams& b = plan->base;
  const char* lo = reinterpret_cast<const char*>(b.q_buf);
  const char* hi = reinterpret_cast<const char*>(b.rope_cos);
  const size_t n = (size_t)(hi - lo) / 4;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<unsigned*>(const_cast<char*>(lo)), 0xffffffffu, n);
  return hip_ok(hipGetLastError()) ? MOEL_OK : MOEL_ERR_HIP;
}

moel_status moel_plan_set_abort(moel_plan* plan, int32_t flag, void* stream) {
  if (plan == nullptr) return MOEL_ERR_ARG;
  hipLaunchKernelGGL(k_set_word, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream),
                     plan->base.ctrl + kAbort, flag ? 1u : 0u);
  return hip_ok(hipGetLastError()) ? MOEL_OK : MOEL_ERR_HIP;
}

moel_status moel_pack_dense(const void* src, int32_t N, int32_t K, int32_t rope_head_dim, void* dst,
                            void* stream) {
  if (src == nullptr || dst == nullptr || N <= 0 || K <= 0) return MOEL_ERR_ARG;
  if (N % 16 != 0 || K % 32 != 0) return MOEL_ERR_SHAPE;
  if (rope_head_dim < 0 || (rope_head_dim > 0 && (N % rope_head_dim != 0 || rope_head_dim % 2 != 0)))
    return MOEL_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return MOEL_ERR_ALIGN;
  const size_t n = (size_t)N * K / 8;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(k_pack_dense, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(src), N, K, rope_head_dim, static_cast<uint8_t*>(dst), n);
  return hip_ok(hipGetLastError()) ? MOEL_OK : MOEL_ERR_HIP;
}

moel_status moel_pack_experts(const moel_config* cfg, int32_t which, const void* src, const void* scales,
                              void* dst, void* stream) {
  moel_status st = moel_validate_config(cfg);
  if (st != MOEL_OK) return st;
  if (which < 0 || which > 2 || src == nullptr || dst == nullptr) return MOEL_ERR_ARG;
  const int E = cfg->n_experts;
  const int N = which < 2 ? cfg->inter / cfg->n_shards : cfg->pooled / cfg->n_shards;
  const int K = which < 2 ? cfg->pooled : cfg->inter;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) return MOEL_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cfg->expert_dtype == MOEL_EXPERT_BF16) {
    const size_t n = (size_t)E * N * K / 8;  // dense layout of the stacked [E*N, K] matrix
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(k_pack_dense, dim3(blocks), dim3(256), 0, s, static_cast<const uint16_t*>(src), E * N, K,
                       0, static_cast<uint8_t*>(dst), n);
  } else {
    if (scales == nullptr) return MOEL_ERR_ARG;
    if (reinterpret_cast<uintptr_t>(scales) & 3) return MOEL_ERR_ALIGN;
    const size_t n = (size_t)E * (N / 64) * (K / 64) * 64;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(k_pack_nvfp4, dim3(blocks), dim3(256), 0, s, static_cast<const uint8_t*>(src),
                       static_cast<const uint8_t*>(scales), N, K, static_cast<uint8_t*>(dst), n);
  }
  return hip_ok(hipGetLastError()) ? MOEL_OK : MOEL_ERR_HIP;
}

moel_status moel_layer_decode_tree(moel_plan* plan, const moel_weights* w, void* k_cache, void* v_cache,
                                   const float* x, int32_t T, int32_t pos, int32_t window,
                                   const int32_t* parents, float* y, const moel_debug* dbg, void* stream) {
  LayerParams p;
  moel_status st = prepare_call(plan, w, k_cache, v_cache, x, T, pos, window, parents, y, dbg, p);
  if (st != MOEL_OK) return st;
  return launch_fused(plan, p, stream);
}

moel_status moel_plan_set_launch(moel_plan* plan, int32_t mode) {
  if (plan == nullptr || (mode != MOEL_LAUNCH_PLAIN && mode != MOEL_LAUNCH_COOPERATIVE)) return MOEL_ERR_ARG;
  plan->launch_mode = mode;
  return MOEL_OK;
}

moel_status moel_plan_set_expert_prefetch(moel_plan* plan, int32_t n_experts) {
  if (plan == nullptr || n_experts < 0 || n_experts > 16) return MOEL_ERR_ARG;
  plan->base.pf_n = n_experts;
  return MOEL_OK;
}

moel_status moel_plan_set_acquire(moel_plan* plan, int32_t mode) {
  if (plan == nullptr || (mode != MOEL_ACQUIRE_AUTO && mode != MOEL_ACQUIRE_L2_INVALIDATE)) return MOEL_ERR_ARG;
  plan->acquire_mode = mode;
  return MOEL_OK;
}

int32_t moel_plan_l2_coherent(const moel_plan* plan) { return plan == nullptr ? -1 : plan->l2_coherent; }

moel_status moel_layer_decode_tree_unfused(moel_plan* plan, const moel_weights* w, void* k_cache,
                                           void* v_cache, const float* x, int32_t T, int32_t pos,
                                           int32_t window, const int32_t* parents, float* y,
                                           const moel_debug* dbg, void* stream) {
  LayerParams p;
  moel_status st = prepare_call(plan, w, k_cache, v_cache, x, T, pos, window, parents, y, dbg, p);
  if (st != MOEL_OK) return st;
  return launch_unfused(plan, p, stream);
}

moel_status moel_layer_decode_batch(moel_plan* plan, const moel_weights* w, void* k_pool, void* v_pool,
                                    const float* x, int32_t n_requests, const moel_request* requests,
                                    int32_t window, float* y, const moel_debug* dbg, void* stream) {
  if (plan == nullptr) return MOEL_ERR_ARG;
  LayerParams p;
  const int l2c = plan->acquire_mode == MOEL_ACQUIRE_AUTO && plan->l2_coherent ? 1 : 0;
  moel_status st = fill_call_batch(&plan->cfg, plan->base, l2c, w, k_pool, v_pool, x, n_requests, requests,
                                   window, nullptr, y, dbg, p);
  if (st != MOEL_OK) return st;
  return launch_fused(plan, p, stream);
}

moel_status moel_layer_decode_batch_unfused(moel_plan* plan, const moel_weights* w, void* k_pool,
                                            void* v_pool, const float* x, int32_t n_requests,
                                            const moel_request* requests, int32_t window, float* y,
                                            const moel_debug* dbg, void* stream) {
  if (plan == nullptr) return MOEL_ERR_ARG;
  LayerParams p;
  const int l2c = plan->acquire_mode == MOEL_ACQUIRE_AUTO && plan->l2_coherent ? 1 : 0;
  moel_status st = fill_call_batch(&plan->cfg, plan->base, l2c, w, k_pool, v_pool, x, n_requests, requests,
                                   window, nullptr, y, dbg, p);
  if (st != MOEL_OK) return st;
  return launch_unfused(plan, p, stream);
}

moel_status moel_layer_decode(moel_plan* plan, const moel_weights* w, void* k_cache, void* v_cache,
                              const float* x, int32_t T, int32_t pos, int32_t window, float* y,
                              const moel_debug* dbg, void* stream) {
  return moel_layer_decode_tree(plan, w, k_cache, v_cache, x, T, pos, window, nullptr, y, dbg, stream);
}

moel_status moel_layer_decode_unfused(moel_plan* plan, const moel_weights* w, void* k_cache, void* v_cache,
                                      const float* x, int32_t T, int32_t pos, int32_t window, float* y,
                                      const moel_debug* dbg, void* stream) {
  return moel_layer_decode_tree_unfused(plan, w, k_cache, v_cache, x, T, pos, window, nullptr, y, dbg,
                                        stream);
}

moel_status moel_stack_create(moel_plan* plan, int32_t n_layers, const moel_weights* weights, void* const* k_caches,
                              void* const* v_caches, const int32_t* windows, moel_stack** out) {
  if (plan == nullptr || out == nullptr || n_layers < 1 || n_layers > MOEL_MAX_STACK_LAYERS || weights == nullptr ||
      k_caches == nullptr || v_caches == nullptr || windows == nullptr)
    return MOEL_ERR_ARG;
  for (int l = 0; l < n_layers; ++l)
    if (windows[l] < 0) return MOEL_ERR_ARG;
  moel_stack* st = new (std::nothrow) moel_stack();
  if (st == nullptr) return MOEL_ERR_HIP;
  st->plan = plan;
  st->n = n_layers;
  st->w = new (std::nothrow) moel_weights[n_layers];
  st->k = new (std::nothrow) void*[n_layers];
  st->v = new (std::nothrow) void*[n_layers];
  st->window = new (std::nothrow) int32_t[n_layers];
  const size_t ab = sizeof(float) * kMaxT * (size_t)plan->cfg.hidden;
  bool ok = st->w && st->k && st->v && st->window;
  if (ok) {
    for (int l = 0; l < n_layers; ++l) {
      st->w[l] = weights[l];
      st->k[l] = k_caches[l];
      st->v[l] = v_caches[l];
      st->window[l] = windows[l];
    }
    ok = hip_ok(hipMalloc(&st->act[0], ab)) && hip_ok(hipMalloc(&st->act[1], ab));
    const int D = plan->cfg.head_dim;
    ok = ok && hip_ok(hipFuncSetAttribute(D == 64 ? stack_fn<64>() : stack_fn<128>(),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan->lds_fused));
  }
  if (!ok) {
    moel_stack_destroy(st);
    return MOEL_ERR_HIP;
  }
  *out = st;
  return MOEL_OK;
}

moel_status moel_stack_destroy(moel_stack* st) {
  if (st == nullptr) return MOEL_ERR_ARG;
  for (int i = 0; i < 2; ++i)
    if (st->act[i]) (void)hipFree(st->act[i]);
  delete[] st->w;
  delete[] st->k;
  delete[] st->v;
  delete[] st->window;
  delete st;
  return MOEL_OK;
}

moel_status moel_stack_decode(moel_stack* st, const float* x, int32_t T, int32_t pos, float* y, void* stream) {
  if (st == nullptr) return MOEL_ERR_ARG;
  moel_plan* plan = st->plan;
  const int n = st->n;
  if (T < 1 || T > kMaxT) return MOEL_ERR_ARG;
  const size_t ab = sizeof(float) * (size_t)T * (size_t)plan->cfg.hidden;  // the step's rows
  const uintptr_t xb = reinterpret_cast<uintptr_t>(x), yb = reinterpret_cast<uintptr_t>(y);
  if (xb < yb + ab && yb < xb + ab) return MOEL_ERR_ARG;  // y must not alias x
  // every layer's arguments are checked before anything is issued; the layers' rows go
  // x -> act[0] -> act[1] -> act[0] ... -> y
  const int nlaunch = (n + kStackLayersPerLaunch - 1) / kStackLayersPerLaunch;
  StackArgs* args = new (std::nothrow) StackArgs[nlaunch];
  if (args == nullptr) return MOEL_ERR_HIP;
  const float* xin = x;
  for (int l = 0; l < n; ++l) {
    float* yout = l == n - 1 ? y : st->act[l % 2];
    StackArgs& a = args[l / kStackLayersPerLaunch];
    moel_status s = prepare_call(plan, &st->w[l], st->k[l], st->v[l], xin, T, pos, st->window[l], nullptr, yout,
                                 nullptr, a.layer[l % kStackLayersPerLaunch]);
    if (s != MOEL_OK) {
      delete[] args;
      return s;
    }
    a.n = l % kStackLayersPerLaunch + 1;
    xin = yout;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* fn = plan->cfg.head_dim == 64 ? stack_fn<64>() : stack_fn<128>();
  hipError_t e = hipSuccess;
  for (int i = 0; i < nlaunch && e == hipSuccess; ++i) {
    void* kargs[] = {&args[i]};
    e = plan->launch_mode == MOEL_LAUNCH_COOPERATIVE
            ? hipLaunchCooperativeKernel(fn, dim3(plan->nwg), dim3(kThreads), kargs, (unsigned)plan->lds_fused, s)
            : hipLaunchKernel(fn, dim3(plan->nwg), dim3(kThreads), kargs, (unsigned)plan->lds_fused, s);
  }
  delete[] args;
  return hip_ok(e) ? MOEL_OK : MOEL_ERR_HIP;
}

moel_status moel_layer_decode_noalloc(const moel_config* cfg, const moel_weights* w, void* k_cache,
                                      void* v_cache, const float* x, int32_t T, int32_t pos, int32_t window,
                                      float* y, uint32_t* status, void* stream) {
  moel_status st = moel_validate_call(cfg, w, k_cache, v_cache, x, T, pos, window, y);
  if (st != MOEL_OK) return st;
  if (reinterpret_cast<uintptr_t>(status) & 3u) return MOEL_ERR_ALIGN;
  int dev = 0;
  if (!hip_ok(hipGetDevice(&dev))) return MOEL_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StaticDev* sd = nullptr;
  st = static_setup(dev, s, &sd);
  if (st != MOEL_OK) return st;
  if (!work_split_fits(cfg, sd->nwg)) return MOEL_ERR_SHAPE;
  // the call's workspace, with RoPE rows for the call's positions only
  const WsLayout L = ws_layout(cfg, sd->nwg, kMaxT);
  if (L.total > kStaticScratchBytes) {
    if (std::getenv("MOEL_LOG"))
      std::fprintf(stderr, "moel: noalloc workspace of %zu bytes exceeds the %zu-byte scratch\n", L.total,
                   kStaticScratchBytes);
    return MOEL_ERR_SHAPE;
  }
  LayerParams base;
  bind_base(base, cfg, sd->nwg, L, sd->ptr);
  LayerParams p;
  st = fill_call(cfg, base, sd->l2_coherent, w, k_cache, v_cache, x, T, pos, window, nullptr, y, nullptr, p);
  if (st != MOEL_OK) return st;
  p.rope_row0 = pos;  // rows pos .. pos + T - 1 (the chain's positions)
  p.status_out = status;
  RopeFreq fq;
  const int half = cfg->head_dim / 2;
  for (int i = 0; i < half; ++i) fq.f[i] = std::pow((double)cfg->rope_theta, -(2.0 * i) / (double)cfg->head_dim);
  hipLaunchKernelGGL(k_rope_rows, dim3((T * half + 255) / 256), dim3(256), 0, s,
                     reinterpret_cast<float*>(sd->ptr + L.cos), reinterpret_cast<float*>(sd->ptr + L.sin), pos, T,
                     half, fq);
  if (!hip_ok(hipGetLastError())) return MOEL_ERR_HIP;
  void* args[] = {&p};
  const int D = cfg->head_dim;
  const hipError_t e = hipLaunchKernel(D == 64 ? fused_fn<64>() : fused_fn<128>(), dim3(sd->nwg), dim3(kThreads),
                                       args, (unsigned)lds_fused_bytes(D), s);
  return hip_ok(e) ? MOEL_OK : MOEL_ERR_HIP;
}

moel_status moel_measure_read_bandwidth(const void* buf, size_t bytes, int32_t reps, float* gbps,
                                        void* stream) {
  if (buf == nullptr || gbps == nullptr || reps < 1 || reps > 1000) return MOEL_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return MOEL_ERR_ALIGN;
  int dev = 0;
  hipDeviceProp_t prop;
  if (!hip_ok(hipGetDevice(&dev)) || !hip_ok(hipGetDeviceProperties(&prop, dev))) return MOEL_ERR_HIP;
  const int nwg = prop.multiProcessorCount;
  if (nwg < 1 || bytes < (size_t)16 * kThreads * nwg) return MOEL_ERR_ARG;
  const size_t per_wg = bytes / 16 / (size_t)nwg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t a = nullptr, b = nullptr;
  moel_status st = MOEL_ERR_HIP;
  if (hip_ok(hipEventCreate(&a)) && hip_ok(hipEventCreate(&b))) {
    const u32x4* p = static_cast<const u32x4*>(buf);
    hipLaunchKernelGGL(k_stream_read, dim3(nwg), dim3(kThreads), 0, s, p, per_wg);  // untimed
    bool ok = hip_ok(hipGetLastError()) && hip_ok(hipEventRecord(a, s));
    for (int r = 0; ok && r < reps; ++r) {
      hipLaunchKernelGGL(k_stream_read, dim3(nwg), dim3(kThreads), 0, s, p, per_wg);
      ok = hip_ok(hipGetLastError());
    }
    float ms = 0.f;
    ok = ok && hip_ok(hipEventRecord(b, s)) && hip_ok(hipEventSynchronize(b)) && hip_ok(hipEventElapsedTime(&ms, a, b));
    if (ok && ms > 0.f) {
      *gbps = (float)((double)per_wg * 16.0 * nwg * reps / (ms * 1e-3) / 1e9);
      st = MOEL_OK;
    }
  }
  if (a != nullptr) (void)hipEventDestroy(a);
  if (b != nullptr) (void)hipEventDestroy(b);
  return st;
}

}  // extern "C"
