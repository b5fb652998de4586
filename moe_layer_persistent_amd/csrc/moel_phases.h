// The steps of one MoE decoder layer's verify pass as workgroup-level device functions.
//
// Every phase is written for a grid of `nwg` workgroups of 512 threads (8 wavefronts) and
// splits its work by workgroup index, so the same function serves both the persistent
// launch (phases separated by grid barriers) and the one-kernel-per-step chain.
//
// Precision: weights are bf16 or NVFP4 and the KV cache is bf16 (storage formats).  Every
// activation, the attention probabilities included, is kept in fp32 and enters the bf16 MFMAs
// as a pair of bf16 values (the nearest bf16 and the bf16 of the remainder, ~16 significant
// bits), so no activation is rounded to bf16 on the way through the layer.
//
// Packed weight layouts (produced by the pack kernels in moel_kernels.hip):
//   dense bf16 [N, K]  : 16-row tiles; per tile K/32 steps of 1 KiB; in a step, lane l holds
//                        8 bf16 of row (l % 16): k = 32*step + 4q + 0..3 and 32*step + 16 + 4q
//                        + 0..3 with q = l / 16 -- the B operand of one 16x16x32 MFMA.  The
//                        A operand takes the same k, so that the four lanes of a token read one
//                        contiguous 64-byte piece of the fp32 activation row per load.
//   NVFP4 expert [N, K]: 64-row tiles; per tile K/64 "pairs" of 2304 bytes: two 1 KiB code
//                        steps (lane l: 32 codes of row l, k = 32*step + 0..31, low nibble
//                        first) then 256 bytes of scales (lane l: the 4 E4M3 block scales of
//                        row l covering the pair's 64 k).
#pragma once
#include <type_traits>

#include "moel_device.h"

// Dynamic LDS of every layer kernel (sized at launch).
extern __shared__ __attribute__((aligned(16))) char moel_lds[];

namespace moel {

// ------------------------------------------------------------------------------------------
// LDS layout: routing tables at offset 0 (kept across the MoE phases of the persistent
// launch), phase scratch after them.
// ------------------------------------------------------------------------------------------
struct RouteTables {
  int idx[kMaxT * 8];          // [T][k] selected expert per slot (slot = t*k + kappa)
  float gate[kMaxT * 8];       // [T][k]
  // active entries: the experts hit by the step, ascending, each with its slots; an expert
  // with more than 16 slots takes one entry per 16 (the expert streams' largest token group)
  int n_active;
  int active_e[kMaxT * 8];
  int active_off[kMaxT * 8 + 1];
  int slots[kMaxT * 8];        // slots grouped by expert (ascending), slots ascending within
  int cnt[512];                // per expert: slots routed to it
  unsigned tmask[512];         // per expert: bit t set when token t selected it
  int off[512];                // per expert: first position in `slots`
  int wave_sum[2][kWaves];     // per-wave totals of the expert scans
  int next;                    // tile handed out by the work counter (bf16 expert phases)
  float ts[3][512];            // per expert: NVFP4 tensor scales of gate, up, down
  int dq[64];                  // NVFP4 expert phases: dynamic tiles handed to this workgroup,
                               // (sequence << 16) | tile, slot = sequence mod 64
  int light;                   // 1: every barrier group runs on one XCC (light releases)
};
constexpr int kRouteBytes = (sizeof(RouteTables) + 255) & ~255;

__device__ __forceinline__ RouteTables& route_tables(char* smem) {
  return *reinterpret_cast<RouteTables*>(smem);
}
__device__ __forceinline__ char* phase_smem(char* smem) { return smem + kRouteBytes; }

// 8 fp32 -> (hi, lo) bf16x8 operands
__device__ __forceinline__ void split8(const float4& a, const float4& b, u32x4& hi, u32x4& lo) {
  const u32x2 s0 = split_bf16(a.x, a.y), s1 = split_bf16(a.z, a.w);
  const u32x2 s2 = split_bf16(b.x, b.y), s3 = split_bf16(b.z, b.w);
  hi = u32x4{s0[0], s1[0], s2[0], s3[0]};
  lo = u32x4{s0[1], s1[1], s2[1], s3[1]};
}

// ------------------------------------------------------------------------------------------
// A-operand sources of the dense contractions: lane supplies A[token][k .. k+3] and
// A[token][k+16 .. k+19] (k = 32*step + 4q, the packed weights' k order) as hi + lo, for the
// token (lane mod 16) of 16-token tile g.  Rows of tokens t >= T read the row of token T-1
// (their products are computed and never read), so that no load in the streaming loops
// depends on a branch.
// ------------------------------------------------------------------------------------------
// gamma[k .. k+3] and gamma[k+16 .. k+19]
__device__ __forceinline__ u32x4 ldg_gamma(const uint16_t* g) {
  const u32x2 a = ldg8(g), b = ldg8(g + 16);
  return u32x4{a[0], a[1], b[0], b[1]};
}
// Rows of tokens t >= T read the row of token T-1 (their products are computed and never
// read), so that no load in the streaming loops depends on a branch.
// v * gamma from an fp32 row, plus the row's sum of squares: the contraction of an RMS-normed
// row is rstd * (W . (v * gamma)), so the pass that reads the row for the contraction also
// yields rstd (dense_pass leaves it in DenseLds::rstd) and the epilogue scales by it.
struct AGamma {
  static constexpr bool kStats = true;
  const float* v;
  int ld;
  const uint16_t* gamma;
  int T;
  float eps;
  struct Raw {
    float4 a, b;
    u32x4 g;
  };
  __device__ __forceinline__ AGamma scalar() const {
    return AGamma{uniform(v), uniform(ld), uniform(gamma), uniform(T), __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, eps)))};
  }
  __device__ __forceinline__ void fetch(int tok, int, int k, Raw& r) const {
    const float* src = v + (size_t)tok * ld + k;
    r.a = ldgf4(src);
    r.b = ldgf4(src + 16);
    r.g = ldg_gamma(gamma + k);
  }
  __device__ __forceinline__ void finish(const Raw& r, u32x4& hi, u32x4& lo) const {
    float4 a = r.a, b = r.b;
    a.x *= bf_lo(r.g[0]);
    a.y *= bf_hi(r.g[0]);
    a.z *= bf_lo(r.g[1]);
    a.w *= bf_hi(r.g[1]);
    b.x *= bf_lo(r.g[2]);
    b.y *= bf_hi(r.g[2]);
    b.z *= bf_lo(r.g[3]);
    b.w *= bf_hi(r.g[3]);
    split8(a, b, hi, lo);
  }
  __device__ __forceinline__ float sq(const Raw& r) const {
    float s = r.a.x * r.a.x;
    s = fmaf(r.a.y, r.a.y, s);
    s = fmaf(r.a.z, r.a.z, s);
    s = fmaf(r.a.w, r.a.w, s);
    s = fmaf(r.b.x, r.b.x, s);
    s = fmaf(r.b.y, r.b.y, s);
    s = fmaf(r.b.z, r.b.z, s);
    return fmaf(r.b.w, r.b.w, s);
  }
};
// Index (in floats) of element (t, k) of a [32][K] fp32 activation stored in operand order:
// per 16-token tile a [K/32] run of 2 KiB blocks, one per 32-element k step, in which lane
// l = t % 16 + 16 q of the contraction finds its 8 values k = 4q + 0..3 at float 4 l and
// k = 16 + 4q + 0..3 at float 256 + 4 l.  A wave's load of a step is then two contiguous
// 1 KiB reads, where the row-major layout spreads each over 16 rows.  Rows t >= T are left as
// they are (their products are never read).
__device__ __forceinline__ size_t op_index(int t, int k, int K) {
  const int r = k & 31;
  return (size_t)(t >> 4) * 16 * K + (size_t)(k >> 5) * 512 + ((r >> 4) << 8) + (((r & 15) >> 2) << 6) +
         4 * (t & 15) + (r & 3);
}
// Index (in bf16 elements) of the nearest-value half of element (t, k) of a [32][K] activation
// stored as ready-made A operands: per 16-token tile a [K/32] run of 2 KiB blocks, one per
// 32-element k step, in which lane l = t % 16 + 16 q finds the nearest bf16 values of its 8
// elements (k = 4q + 0..3, 16 + 4q + 0..3, the word order of split8) at element 8 l and the
// bf16 of their remainders 512 elements later.  A wave's load of a step is two contiguous
// 1 KiB reads and the contraction does no splitting: the producer splits each value once
// (4 B per element, as in fp32).
__device__ __forceinline__ size_t opsplit_index(int t, int k, int K) {
  const int r = k & 31;
  return (size_t)(t >> 4) * 32 * K + (size_t)(k >> 5) * 1024 + 8 * ((t & 15) + 16 * ((r & 15) >> 2)) +
         ((r >> 4) << 2) + (r & 3);
}
__device__ __forceinline__ void store_opsplit(__attribute__((address_space(1))) uint16_t* base, int t, int k,
                                              int K, float v) {
  const size_t i = opsplit_index(t, k, K);
  const uint16_t h = f2bf(v);
  base[i] = h;
  base[i + 512] = f2bf(v - bf2f(h));
}
// An activation stored as ready-made A operands (lane l reads its own token slot l % 16 of
// tile g).
struct AOp {
  static constexpr bool kStats = false;
  const uint16_t* v;
  int T;
  int K;  // row length
  struct Raw {
    u32x4 hi, lo;
  };
  __device__ __forceinline__ AOp scalar() const { return AOp{uniform(v), uniform(T), uniform(K)}; }
  __device__ __forceinline__ void fetch(int, int g, int k, Raw& r) const {
    const uint16_t* src = v + (size_t)g * 32 * K + (size_t)(k >> 5) * 1024 + 8 * lane_id();
    r.hi = ldg16(src);
    r.lo = ldg16(src + 512);
  }
  __device__ __forceinline__ void finish(const Raw& r, u32x4& hi, u32x4& lo) const {
    hi = r.hi;
    lo = r.lo;
  }
};
// v * gamma from an fp32 activation in operand order, plus the sums of squares (as AGamma).
struct AGammaOp {
  static constexpr bool kStats = true;
  const float* v;
  const uint16_t* gamma;
  int T;
  float eps;
  int K;  // row length
  struct Raw {
    float4 a, b;
    u32x4 g;
  };
  __device__ __forceinline__ AGammaOp scalar() const {
    return AGammaOp{uniform(v), uniform(gamma), uniform(T), __builtin_bit_cast(float, uniform(__builtin_bit_cast(int, eps))),
                    uniform(K)};
  }
  __device__ __forceinline__ void fetch(int, int g, int k, Raw& r) const {
    const float* src = v + (size_t)g * 16 * K + (size_t)(k >> 5) * 512 + 4 * lane_id();
    r.a = ldgf4(src);
    r.b = ldgf4(src + 256);
    r.g = ldg_gamma(gamma + k);
  }
  __device__ __forceinline__ void finish(const Raw& r, u32x4& hi, u32x4& lo) const {
    float4 a = r.a, b = r.b;
    a.x *= bf_lo(r.g[0]);
    a.y *= bf_hi(r.g[0]);
    a.z *= bf_lo(r.g[1]);
    a.w *= bf_hi(r.g[1]);
    b.x *= bf_lo(r.g[2]);
    b.y *= bf_hi(r.g[2]);
    b.z *= bf_lo(r.g[3]);
    b.w *= bf_hi(r.g[3]);
    split8(a, b, hi, lo);
  }
  __device__ __forceinline__ float sq(const Raw& r) const {
    float s = r.a.x * r.a.x;
    s = fmaf(r.a.y, r.a.y, s);
    s = fmaf(r.a.z, r.a.z, s);
    s = fmaf(r.a.w, r.a.w, s);
    s = fmaf(r.b.x, r.b.x, s);
    s = fmaf(r.b.y, r.b.y, s);
    s = fmaf(r.b.z, r.b.z, s);
    return fmaf(r.b.w, r.b.w, s);
  }
};

// ------------------------------------------------------------------------------------------
// Dense contraction over a workgroup's rows: out[tok][row] = sum_k A[tok][k] * W[row][k] over a
// range of k steps.  Rows are assigned in octets (8 rows = four 128-byte lines of every 1 KiB
// step), so that workgroups never share a cache line.  NT tiles of 16 rows per pass (NT * NTT
// <= 8) against NTT tiles of 16 tokens, each weight word used by every token tile; the k-waves
// split the pass's steps evenly and stream them through a ring of DEPTH steps; partials meet
// in LDS.  Lanes of an octet outside the workgroup's range load their partner octet's line
// instead (the same line another lane fetches; the products are never read), so no load sits
// behind a branch.  On return `fin` holds [tile j][row r][tok] sums for tiles t_first ..
// t_first+NT-1 over steps ks0 .. ks0+ksn-1, and (sources with stats) `sumsq` the sum of squares
// of each token's A elements over those steps, `rstd` 1/rms over the full K when the pass
// covers all of it.
// ------------------------------------------------------------------------------------------
constexpr int kDenseMaxNT = 8;
constexpr int kMaxSplit = 16;  // split-K ranges of a dense phase at most
struct DenseLds {
  f32x4 red[kWaves * kDenseMaxNT * 64];   // 64 KiB
  float fin[kDenseMaxNT * 16 * kMaxT];    // 16 KiB
  float ss[kMaxTiles * kWaves * 64];  // per-lane sums of squares of the A rows (sources with stats)
  float sumsq[kMaxT];           // per token: sum of squares over the pass's k steps
  float rstd[kMaxT];            // 1 / rms of each token's A row (sources with stats)
  int last;                     // split-K: this workgroup reduces its block
};

// Largest divisor of n that is <= 8: the number of waves that split a reduction of n units
// so that every one of them gets the same count.
__device__ __forceinline__ int kwaves_for(int n) {
  int w = n < kWaves ? n : kWaves;
  while (n % w) --w;
  return w;
}

// The second half of the grid barrier before a dense phase of the persistent launch, run by a
// dense pass after it has issued the weight loads of its first steps (weights are not written
// by any phase, the activation is): the barrier's number and, when the phase start is stamped,
// its timestamp slot.  NoWait: a phase without a barrier before it (or a pass after the first).
struct NoWait {
  __device__ void operator()() const {}
};
struct BarWait {
  uint64_t ph;
  unsigned bar;
  int slot;  // < 0: no timestamp
  __device__ void operator()() const {
    KP& p = params_from(ph);
    grid_barrier_wait(p, (unsigned)uniform((int)bar));
    const int sl = uniform(slot);
    if (sl >= 0) stamp(p, sl);
  }
};

// Not inlined (one body per NT); the arguments arrive in vector registers and are moved to
// scalar registers first.  wait() is called once by every thread; with a BarWait the weight
// loads of the ring's first steps are issued before it and their activation loads after it.
template <int NT, int NTT, class ASrc, class Wait = NoWait>
__device__ __noinline__ void dense_pass(const uint8_t* w0_arg, int tiles0_arg, const uint8_t* w1_arg,
                                        int K_arg, int ks0_arg, int ksn_arg, int t_first_arg, int oct_lo_arg,
                                        int oct_hi_arg, const ASrc A_arg, const Wait wait = Wait{}) {
  // k steps in flight per wave: 2 keeps ~100 KB per CU in flight, which measured faster than
  // deeper rings (more outstanding requests per CU lowered the achieved bandwidth)
  constexpr int DEPTH = 2;
  static_assert(NT * NTT <= kDenseMaxNT && NTT <= kMaxTiles, "reduction scratch");
  // the phase scratch of the dynamic LDS, addressed through the LDS symbol (a pointer argument
  // would arrive as a generic address and turn every access into a flat one)
  DenseLds& L = *reinterpret_cast<DenseLds*>(phase_smem(moel_lds));
  const uint8_t* w0 = uniform(w0_arg);
  const uint8_t* w1 = uniform(w1_arg);
  const int tiles0 = uniform(tiles0_arg), K = uniform(K_arg), t_first = uniform(t_first_arg);
  const int ks0 = uniform(ks0_arg), ksn = uniform(ksn_arg);
  const int oct_lo = uniform(oct_lo_arg), oct_hi = uniform(oct_hi_arg);
  const ASrc A = A_arg.scalar();
  const int lane = lane_id(), wv = wave_id();
  const int S = K >> 5;  // steps per tile row (the packed tile's stride)
  const int nkw = kwaves_for(ksn);
  f32x4 acc[NTT][NT];
  float ssum[NTT];  // sums of squares of this lane's A elements (sources with stats)
#pragma unroll
  for (int g = 0; g < NTT; ++g) {
    ssum[g] = 0.f;
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  constexpr bool kSplitWait = !std::is_same<Wait, NoWait>::value;
  const bool kwave = wv < nkw;
  {
    // k-wave wv takes the steps ks0 + wv, ks0 + wv + nkw, ... so that the workgroup's loads in
    // flight cover one contiguous stretch of each tile
    const int ns = ksn / nkw;
    int tok[NTT];
#pragma unroll
    for (int g = 0; g < NTT; ++g) tok[g] = kTile * g + (lane & 15) < A.T ? kTile * g + (lane & 15) : A.T - 1;
    const int kq = 4 * (lane >> 4) + 32 * (ks0 + wv);
    const uint8_t* base[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int t = t_first + j;
      const int oct = 2 * t + ((lane & 15) >> 3);
      const int src_lane = (oct >= oct_lo && oct < oct_hi) ? lane : (lane ^ 8);
      base[j] = (t < tiles0 ? w0 + (size_t)t * S * 1024 : w1 + (size_t)(t - tiles0) * S * 1024) +
                (size_t)(ks0 + wv) * 1024 + src_lane * 16;
    }
    typename ASrc::Raw ra[DEPTH][NTT];
    u32x4 rw[DEPTH][NT];
    auto issue = [&](int d, int i) {
#pragma unroll
      for (int g = 0; g < NTT; ++g) A.fetch(tok[g], g, kq + 32 * nkw * i, ra[d][g]);
#pragma unroll
      for (int j = 0; j < NT; ++j) rw[d][j] = ldg_stream(base[j] + (size_t)i * nkw * 1024);
    };
    auto compute = [&](int d) {
#pragma unroll
      for (int g = 0; g < NTT; ++g) {
        u32x4 a_hi, a_lo;
        A.finish(ra[d][g], a_hi, a_lo);
        if constexpr (ASrc::kStats) ssum[g] += A.sq(ra[d][g]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          acc[g][j] = mfma16x16x32(a_hi, rw[d][j], acc[g][j]);
          acc[g][j] = mfma16x16x32(a_lo, rw[d][j], acc[g][j]);
        }
      }
    };
    // straight-line prologue (steps past the end repeat the last one and are never used), so
    // that the ring registers enter the loop in issue order; with a barrier before the pass the
    // weights of these steps go first, the activation after the barrier's wait
    if constexpr (kSplitWait) {
      if (kwave) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
#pragma unroll
          for (int j = 0; j < NT; ++j) rw[d][j] = ldg_stream(base[j] + (size_t)(d < ns ? d : ns - 1) * nkw * 1024);
      }
      wait();
      if (kwave) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
          for (int g = 0; g < NTT; ++g) A.fetch(tok[g], g, kq + 32 * nkw * (d < ns ? d : ns - 1), ra[d][g]);
          sched_fence();
        }
      }
    } else if (kwave) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        issue(d, d < ns ? d : ns - 1);
        sched_fence();
      }
    }
    if (kwave) {
    int i0 = 0;
    for (; i0 + 2 * DEPTH <= ns; i0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        compute(d);
        issue(d, i0 + DEPTH + d);
        sched_fence();
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (i0 + d < ns) {
        compute(d);
        if (i0 + DEPTH + d < ns) issue(d, i0 + DEPTH + d);
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (i0 + DEPTH + d < ns) compute(d);
#pragma unroll
    for (int g = 0; g < NTT; ++g)
#pragma unroll
      for (int j = 0; j < NT; ++j) L.red[(wv * kDenseMaxNT + g * NT + j) * 64 + lane] = acc[g][j];
    }
  }
  // every (token, k) of the A rows is fetched by exactly one lane of the k-waves (lanes whose
  // token is >= T repeat token T-1 and are left out)
  if constexpr (ASrc::kStats) {
#pragma unroll
    for (int g = 0; g < NTT; ++g)
      L.ss[(g * kWaves + wv) * 64 + lane] = (wv < nkw && kTile * g + (lane & 15) < A.T) ? ssum[g] : 0.f;
  }
  lds_barrier();
  if constexpr (ASrc::kStats) {
    if (threadIdx.x < kTile * NTT) {
      const int g = threadIdx.x >> 4, tt = threadIdx.x & 15;
      float s = 0.f;
      for (int w = 0; w < nkw; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) s += L.ss[(g * kWaves + w) * 64 + 16 * q + tt];
      L.sumsq[threadIdx.x] = s;
      L.rstd[threadIdx.x] = 1.0f / sqrtf(s / (float)K + A.eps);
    }
  }
  for (int e = threadIdx.x; e < NTT * NT * 256; e += kThreads) {
    const int g = NTT == 1 ? 0 : e / (NT * 256), eg = e - g * NT * 256;
    const int j = eg >> 8, ln = (eg >> 2) & 63, r = eg & 3;
    float s = 0.f;
    for (int w = 0; w < nkw; ++w) s += L.red[(w * kDenseMaxNT + g * NT + j) * 64 + ln][r];
    const int tok = kTile * g + 4 * (ln >> 4) + r, row = ln & 15;
    L.fin[(j * 16 + row) * kMaxT + tok] = s;
  }
  lds_barrier();
}

// Octet range of a workgroup (or a split-K block) for a contraction with `tiles` 16-row tiles.
__device__ __forceinline__ void octet_range(int tiles, int wg, int nwg, int& lo, int& hi) {
  const int n = 2 * tiles;
  // 32-bit: n * nwg < 2^32 for every accepted shape (n <= N / 8)
  lo = (int)((unsigned)wg * (unsigned)n / (unsigned)nwg);
  hi = (int)((unsigned)(wg + 1) * (unsigned)n / (unsigned)nwg);
}

// nt row tiles against ntt token tiles (nt * ntt <= 8)
template <class ASrc, class Wait = NoWait>
__device__ __forceinline__ void dense_pass_nt(int nt, int ntt, const uint8_t* w0, int tiles0, const uint8_t* w1,
                                              int K, int ks0, int ksn, int t, int lo, int hi, const ASrc& A,
                                              const Wait& wait = Wait{}) {
  if (ntt == 1) {
    switch (nt) {
      case 1: dense_pass<1, 1, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      case 2: dense_pass<2, 1, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      case 3: dense_pass<3, 1, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      case 4: dense_pass<4, 1, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      case 5: dense_pass<5, 1, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      case 6: dense_pass<6, 1, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      case 7: dense_pass<7, 1, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      default: dense_pass<8, 1, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
    }
  } else {
    switch (nt) {
      case 1: dense_pass<1, 2, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      case 2: dense_pass<2, 2, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      case 3: dense_pass<3, 2, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
      default: dense_pass<4, 2, ASrc, Wait>(w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait); break;
    }
  }
}

// A dense phase: the output rows of `tiles0 + tiles1` tiles (two stacked matrices) over the full
// K, with epi(L, t_first, ntiles, oct_lo, oct_hi) called on every group of <= 8 finished tiles.
//
// nsplit == 1: each workgroup owns an octet range over the whole K.
// nsplit > 1 (split-K): the rows form nwg / nsplit blocks and K nsplit equal step ranges; each
// workgroup owns one (block, range) unit, so it reads the activation only over its range.  The
// units write their partial sums (and, for sources with stats, their sums of squares) to `part`,
// count their arrival on the block's counter, and the last of a block's units to arrive sums the
// partials in range order -- a fixed order, so the result does not depend on which unit came
// last -- and runs the epilogue.  Where nwg is a multiple of 8 nsplit, the units of a block sit
// on one XCD (workgroup w runs on XCD w mod 8), so the partials it reads are in that XCD's L2.
// No unit waits for another.
//
// wait: the second half of the grid barrier before the phase (BarWait), or NoWait; run once by
// every workgroup, inside its first pass (after the pass has issued its first weight loads) or
// before it leaves without work.
template <class ASrc, class Epi, class Wait = NoWait>
__device__ __forceinline__ void dense_phase(KP& p, int fix_id, int nsplit, const uint8_t* w0, int tiles0,
                                            const uint8_t* w1, int tiles1, int K, int wg, const ASrc& A,
                                            DenseLds& L, Epi&& epi, const Wait& wait = Wait{}) {
  const int nwg = p.nwg;
  const int tiles = tiles0 + tiles1;
  const int S = K >> 5;
  const int ntt = p.ntt;
  const int gs = kDenseMaxNT / ntt;  // row tiles per pass
  const int lgT = ntt == 1 ? 4 : 5;  // log2 of the tokens the passes cover (16 per tile)
  if (nsplit <= 1) {
    int lo, hi;
    octet_range(tiles, wg, nwg, lo, hi);
    if (lo >= hi) {
      wait();
      return;
    }
    const int tf = lo >> 1, tl = (hi - 1) >> 1;
    for (int t = tf; t <= tl; t += gs) {
      const int nt = (tl - t + 1) < gs ? (tl - t + 1) : gs;
      if (t == tf) dense_pass_nt(nt, ntt, w0, tiles0, w1, K, 0, S, t, lo, hi, A, wait);
      else dense_pass_nt(nt, ntt, w0, tiles0, w1, K, 0, S, t, lo, hi, A);
      epi(L, t, nt, lo, hi);
      lds_barrier();
    }
    return;
  }
  const int nblk = nwg / nsplit;
  if (wg >= nblk * nsplit) {
    wait();
    return;
  }
  int b, js;
  if (nwg % (8 * nsplit) == 0) {
    const int x = wg & 7, i = wg >> 3;  // XCD and index within it
    b = x + 8 * (i / nsplit);
    js = i % nsplit;
  } else {
    b = wg / nsplit;
    js = wg % nsplit;
  }
  int lo, hi;
  octet_range(tiles, b, nblk, lo, hi);
  if (lo >= hi) {  // an empty block: none of its units takes part
    wait();
    return;
  }
  const int tf = lo >> 1, tl = (hi - 1) >> 1;
  const int ksn = S / nsplit, ks0 = js * ksn;
  const int ntot = tiles * 16;
  auto part = gl(p.part);
  for (int t = tf; t <= tl; t += gs) {
    const int nt = (tl - t + 1) < gs ? (tl - t + 1) : gs;
    if (t == tf) dense_pass_nt(nt, ntt, w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A, wait);
    else dense_pass_nt(nt, ntt, w0, tiles0, w1, K, ks0, ksn, t, lo, hi, A);
    for (int e = threadIdx.x; e < (nt * 16) << lgT; e += kThreads) {
      const int j = e >> (lgT + 4), r = (e >> lgT) & 15, tok = e & ((1 << lgT) - 1);
      const int n = (t + j) * 16 + r;
      if (tok < p.T && (n >> 3) >= lo && (n >> 3) < hi)
        part[((size_t)js * ntot + n) * kMaxT + tok] = L.fin[(j * 16 + r) * kMaxT + tok];
    }
    lds_barrier();
  }
  if constexpr (ASrc::kStats) {
    if (threadIdx.x < kMaxT) gl(p.part_ss)[(b * nsplit + js) * kMaxT + threadIdx.x] = L.sumsq[threadIdx.x];
  }
  // arrival: the partials are written back before the count (release), and the last unit of
  // the block reads them after it (acquire).  With light releases the block's units share one
  // XCC (they belong to one barrier group), so the partials, complete in its L2 once counted in
  // (vmcnt(0)), need no write-back, and the last unit invalidates only its L1.  Otherwise the
  // units may sit on several XCDs, and the address of a partial belongs to another block (often
  // on another XCD) in each phase: the last unit's L2 may still hold a copy of it from an
  // earlier phase, which the L2 coherence of the device does not cover (a line that this XCD
  // wrote earlier in the launch), so it takes the agent-scope acquire, which drops the L2's
  // clean lines.
  // a block's units share a barrier group (hence, once the groups are known to run on one XCC
  // each, one L2) when nwg is a multiple of 8 nsplit.  Before the launch's first barrier has
  // settled that, a unit proves it itself (groups_single_xcc) and counts in with bit 16 set: if
  // any unit of the block proved it, every unit's partials are in the last unit's L2.  The
  // proof's loads are issued before the wait for the partials' stores, so that the two
  // overlap; a proof also holds for the rest of the launch (kept in RouteTables::light).
  const bool known = route_tables(moel_lds).light != 0;
  const bool one_group = nwg % (8 * nsplit) == 0;
  bool proven = false;
  if (threadIdx.x == 0 && !known && one_group) proven = groups_single_xcc(p);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    auto cnt = gl(p.ctrl) + kFix + kFixPerPhase * fix_id + b;
    if (proven) route_tables(moel_lds).light = 1;
    const bool light = (known && one_group) || proven;
    if (!light) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned inc = proven ? 0x10001u : 1u;
    const unsigned prev = __hip_atomic_fetch_add(cnt, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (prev & 0xffffu) == (unsigned)nsplit - 1;
    if (last) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next launch
      const bool any_light = light || ((prev + inc) >> 16) != 0;
      if (any_light) asm volatile("buffer_inv sc0" ::: "memory");
      else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    L.last = last;
  }
  __syncthreads();
  if (!L.last) return;
  // the partials of every output this thread sums are loaded together (all in flight at once),
  // then summed in split order
  if constexpr (ASrc::kStats) {
    if (threadIdx.x < kMaxT) {
      float v[kMaxSplit];
#pragma unroll
      for (int q = 0; q < kMaxSplit; ++q)
        v[q] = q < nsplit ? gl(p.part_ss)[(b * nsplit + q) * kMaxT + threadIdx.x] : 0.f;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kMaxSplit; ++q)
        if (q < nsplit) s += v[q];
      L.rstd[threadIdx.x] = 1.0f / sqrtf(s / (float)K + A.eps);
    }
  }
  constexpr int kPer = 4;  // outputs per thread and round
  for (int t = tf; t <= tl; t += gs) {
    const int nt = (tl - t + 1) < gs ? (tl - t + 1) : gs;
    const int ne = (nt * 16) << lgT;
    for (int e0 = 0; e0 < ne; e0 += kPer * kThreads) {
      float v[kPer][kMaxSplit];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = e0 + threadIdx.x + i * kThreads;
        const int j = e >> (lgT + 4), r = (e >> lgT) & 15, tok = e & ((1 << lgT) - 1);
        const int n = (t + j) * 16 + r;
        const bool ok = e < ne && tok < p.T && (n >> 3) >= lo && (n >> 3) < hi;
#pragma unroll
        for (int q = 0; q < kMaxSplit; ++q)
          v[i][q] = (ok && q < nsplit) ? part[((size_t)q * ntot + n) * kMaxT + tok] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = e0 + threadIdx.x + i * kThreads;
        const int j = e >> (lgT + 4), r = (e >> lgT) & 15, tok = e & ((1 << lgT) - 1);
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < kMaxSplit; ++q)
          if (q < nsplit) sum += v[i][q];
        if (e < ne) L.fin[(j * 16 + r) * kMaxT + tok] = sum;
      }
    }
    lds_barrier();
    epi(L, t, nt, lo, hi);
    lds_barrier();
  }
}

__device__ __forceinline__ bool octet_in(int row, int lo, int hi) {
  const int o = row >> 3;
  return o >= lo && o < hi;
}

// ------------------------------------------------------------------------------------------
// QKV projection + RoPE + q store + KV-cache write.  w_qkv rows are packed with the
// rotation partners (i, i + D/2) of every head interleaved: packed row 2i <-> canonical i,
// packed row 2i+1 <-> canonical i + D/2.  The cache stores bf16 (nearest); q stays fp32.
// ------------------------------------------------------------------------------------------
template <class Wait = NoWait>
__device__ __forceinline__ void phase_qkv(KP& p, int wg, char* smem, const Wait& wait = Wait{}) {
  DenseLds& L = *reinterpret_cast<DenseLds*>(phase_smem(smem));
  AGamma A{p.x, p.H, p.gamma1, p.T, p.eps};  // RMSNorm 1 folded in: rstd from the same pass
  const int tiles = (p.Hq + 2 * p.Hkv) * p.D / 16;
  const int half = p.D >> 1;
  dense_phase(p, 0, p.sk_qkv, p.w_qkv, tiles, nullptr, 0, p.H, wg, A, L,
              [&](DenseLds& L, int tf, int nt, int lo, int hi) {
                const int lgT = p.ntt == 1 ? 4 : 5;  // tokens covered: 16 per tile
                for (int e = threadIdx.x; e < (nt * 8) << lgT; e += kThreads) {
                  const int j = e >> (lgT + 3), pr = (e >> lgT) & 7, t = e & ((1 << lgT) - 1);
                  const int R = (tf + j) * 16 + 2 * pr;  // packed row (even)
                  if (t >= p.T || !octet_in(R, lo, hi)) continue;
                  const float a = L.fin[(j * 16 + 2 * pr) * kMaxT + t] * L.rstd[t];
                  const float b = L.fin[(j * 16 + 2 * pr + 1) * kMaxT + t] * L.rstd[t];
                  const int head = R / p.D, i = (R % p.D) >> 1;
                  // pool slot of the token: its request's base + position + index in the request
                  int ps = 0;
                  for (int r = 0; r < p.n_req; ++r)
                    if (t >= p.req_t0[r]) ps = p.req_kvb[r] + p.req_pos[r] - p.req_t0[r] + t;
                  const int rp = p.tok_pos[t];  // position (RoPE)
                  if (head < p.Hq + p.Hkv) {
                    const float c = gl(p.rope_cos)[(size_t)(rp - p.rope_row0) * half + i];
                    const float s = gl(p.rope_sin)[(size_t)(rp - p.rope_row0) * half + i];
                    const float ra = a * c - b * s, rb = b * c + a * s;
                    if (head < p.Hq) {
                      auto q = gl(p.q_buf + (size_t)t * p.Hq * p.D + head * p.D);
                      q[i] = ra;
                      q[i + half] = rb;
                      // the attention's operand: scaled to base-2 score units, as hi + lo
                      const float qscale = 1.4426950408889634f / sqrtf((float)p.D);
                      const float sa = ra * qscale, sb = rb * qscale;
                      const uint16_t ha = f2bf(sa), hb = f2bf(sb);
                      auto qo = gl(p.q_op + ((size_t)t * p.Hq + head) * 2 * p.D);
                      qo[i] = ha;
                      qo[i + half] = hb;
                      qo[p.D + i] = f2bf(sa - bf2f(ha));
                      qo[p.D + i + half] = f2bf(sb - bf2f(hb));
                    } else {
                      auto k = gl(p.k_cache + ((size_t)(head - p.Hq) * p.kv_cap + ps) * p.D);
                      k[i] = f2bf(ra);
                      k[i + half] = f2bf(rb);
                    }
                  } else {
                    auto v = gl(p.v_cache + ((size_t)(head - p.Hq - p.Hkv) * p.kv_cap + ps) * p.D);
                    v[i] = f2bf(a);
                    v[i + half] = f2bf(b);
                  }
                }
              }, wait);
}

// ------------------------------------------------------------------------------------------
// Attention partials.  Item = (kv head g, key chunk c, 16-token tile); each wave is one q head
// of the group.
// Keys go in sub-chunks of SK = 128: while one sub-chunk is in LDS and being used, the next
// one's K/V rows are already in flight into registers.  S^T = K Q^T on MFMA (keys as rows;
// q as hi + lo, pre-multiplied by log2(e)/sqrt(D) so that scores come out in base-2 units),
// softmax in fp32 with exp2, the exact max of each sub-chunk and an online rescale between
// sub-chunks, O += P V on MFMA (P as a pair of bf16 values, hi + lo, like every other
// activation; V transposed in LDS).  The partials' running maxima stay in base-2 units for the
// merge.
// ------------------------------------------------------------------------------------------
// ------------------------------------------------------------------------------------------
// Previous-step expert prefetch.  From the layer's routing history (tokens per expert of the
// last step) the pf_n experts that most tokens chose (ties to the lower index, unused experts
// left out) are ranked the same way in every prefetching workgroup; their packed gate, up and
// down weights, as one list of 16-byte words, are split evenly over the np prefetching
// workgroups, which read their share once with ordinary loads (so that the memory-side cache
// keeps the lines) and discard it.  Runs on workgroups with no attention work while attention
// runs; changes no result.
// ------------------------------------------------------------------------------------------
__device__ unsigned g_prefetch_sink;
__device__ __noinline__ void expert_prefetch(uint64_t ph, int idx_arg, int np_arg) {
  KP& p = params_from(ph);
  const int idx = uniform(idx_arg), np = uniform(np_arg);
  int* hist = reinterpret_cast<int*>(phase_smem(moel_lds));  // [E] history, then [16] selection
  int* sel = hist + 512;
  const int E = p.E, n = p.pf_n;
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = (int)gl(p.expert_hist)[e];
  if (threadIdx.x < 16) sel[threadIdx.x] = -1;
  __syncthreads();
  // rank of an expert the last step used: the used experts before it (more tokens, or as many
  // and a lower index); every used expert ranks before every unused one
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const int c = hist[e];
    if (c > 0) {
      int rank = 0;
      for (int f = 0; f < E; ++f) {
        const int cf = hist[f];
        rank += (cf > c) | ((cf == c) & (f < e));
      }
      if (rank < n) sel[rank] = e;
    }
  }
  __syncthreads();
  int nsel = 0;
  for (int k = 0; k < n; ++k) nsel += uniform(sel[k]) >= 0 ? 1 : 0;
  const unsigned wn0 = (unsigned)(p.stride_gate >> 4), wn1 = (unsigned)(p.stride_up >> 4),
                 wn2 = (unsigned)(p.stride_down >> 4);
  const unsigned W = (unsigned)nsel * (wn0 + wn1 + wn2);  // 16-byte words in all
  const unsigned lo = (unsigned)((uint64_t)W * (unsigned)idx / (unsigned)np);
  const unsigned hi = (unsigned)((uint64_t)W * (unsigned)(idx + 1) / (unsigned)np);
  unsigned acc = 0;
  constexpr int kIn = 8;  // 16-byte loads in flight per thread
  // the segments (expert slot k, matrix m) in list order, each intersected with [lo, hi)
  unsigned base = 0;
  for (int k = 0; k < nsel; ++k) {
    const size_t e = (size_t)uniform(sel[k]);
#pragma unroll 1
    for (int m = 0; m < 3; ++m) {
      const unsigned wm = m == 0 ? wn0 : m == 1 ? wn1 : wn2;
      const unsigned s0 = lo > base ? lo : base, s1 = hi < base + wm ? hi : base + wm;
      if (s0 < s1) {
        const uint8_t* src = (m == 0 ? p.w_gate + e * p.stride_gate
                              : m == 1 ? p.w_up + e * p.stride_up : p.w_down + e * p.stride_down) +
                             (size_t)(s0 - base) * 16;
        const unsigned cnt = s1 - s0;
        // two batches of kIn loads: a batch is consumed only after the next one is issued, so
        // the loads stay in flight across iterations
        u32x4 v[2][kIn];
        auto issue = [&](int b, unsigned i) {
#pragma unroll
          for (int d = 0; d < kIn; ++d) {
            const unsigned j = i + d * kThreads < cnt ? i + d * kThreads : cnt - 1;
            v[b][d] = ldg16(src + (size_t)j * 16);  // cacheable: non-temporal reads leave nothing behind
          }
        };
        auto consume = [&](int b) {
#pragma unroll
          for (int d = 0; d < kIn; ++d) acc ^= v[b][d][0] ^ v[b][d][3];
        };
        const unsigned step = kIn * kThreads;
        unsigned i = threadIdx.x;
        issue(0, i);
        for (; i + step < cnt; i += 2 * step) {
          issue(1, i + step);
          sched_fence();
          consume(0);
          if (i + 2 * step < cnt) issue(0, i + 2 * step);
          sched_fence();
          consume(1);
        }
        if (i < cnt) consume(0);
      }
      base += wm;
    }
  }
  // keeps the loads: the xor of the words read is stored only if it equals a constant that no
  // step relies on
  if (acc == 0x9e3779b9u) g_prefetch_sink = acc;
}

template <int D>
struct AttnLds {
  static constexpr int SK = 128;          // keys per sub-chunk
  static constexpr int KS = D + 8;        // Ks row stride (bf16 elements)
  static constexpr int VS = SK + 8;       // Vt row stride
  uint16_t Ks[SK * KS];
  uint16_t Vt[D * VS];
  // V^T element (d, key): 4-key groups XOR-swizzled by d / 8, so that the transposing stores
  // of one wave (16 d-octets x 4 keys) spread over the banks; a 4-key group stays contiguous
  // for the 8-byte operand reads.
  __device__ static __forceinline__ int vt_index(int d, int key) {
    return d * VS + ((((key >> 2) ^ ((d >> 3) & 15)) << 2) | (key & 3));
  }
};

//
// wait(): the second half of the grid barrier before the phase (or nothing, in a kernel of its
// own), called exactly once.  A workgroup whose first key sub-chunk holds cached keys only (rows
// this step does not write) fetches those rows first, so that they arrive during the wait.
template <int D, class Wait>
__device__ __forceinline__ void phase_attn(KP& p, int wg, char* smem, Wait&& wait) {
  using L_t = AttnLds<D>;
  L_t& L = *reinterpret_cast<L_t*>(phase_smem(smem));
  constexpr int SK = L_t::SK, KS = L_t::KS;
  constexpr int NS = D / 32;              // MFMA k-steps over the head dim
  constexpr int ND = D / 16;              // output d tiles
  constexpr int NKT = SK / 16;            // key tiles per sub-chunk
  constexpr int NCH = SK * (D / 8) / kThreads;  // 16-byte K (and V) chunks per thread per sub-chunk
  static_assert(NCH * kThreads == SK * (D / 8), "sub-chunk staging must divide evenly");
  const int lane = lane_id(), wv = wave_id();
  const int grp = p.Hq / p.Hkv;
  // items: (kv head, key chunk) x 16-token tile, the tiles of one (head, chunk) adjacent
  const int nitems = p.Hkv * p.attn_nchunks * p.ntt;
  const float NEG = -__builtin_inff();
  const int gq = lane >> 4, tq = lane & 15;
  // this thread's place in a sub-chunk's staging: 16-byte column c8 of rows row0 + i * RSTEP
  constexpr int RSTEP = kThreads / (D / 8);
  const int row0 = threadIdx.x / (D / 8), c8 = (threadIdx.x % (D / 8)) * 8;
  // this workgroup's items: every nwg-th from wg; with the merge per barrier group, chunk j of
  // group q = wg mod 8 (kv head q mod Hkv, token tile q / Hkv) on the group's j-th workgroup
  int it0 = wg, istep = p.nwg, q_set = -1;
  if (p.attn_set_merge) {
    const int ns = p.nwg < kBarGroups ? p.nwg : kBarGroups;
    const int q = wg % ns, j = wg / ns;
    it0 = istep = nitems;
    if (q < p.Hkv * p.ntt && j < p.attn_nchunks) {
      it0 = (j * p.Hkv + q % p.Hkv) * p.ntt + q / p.Hkv;
      q_set = q;
    }
  }
  bool waited = false;
  for (int it = it0; it < nitems; it += istep) {
    const int ib = it / p.ntt, tile = it - ib * p.ntt;  // (head, chunk) item and token tile
    const int g = ib % p.Hkv, cc = ib / p.Hkv;  // kv head, flat chunk
    // the chunk's request rq and its chunk c within the request (uniform)
    int rq = 0;
    while (rq + 1 < p.n_req && cc >= p.req_ch0[rq + 1]) ++rq;
    const int c = cc - p.req_ch0[rq];
    const int pos_r = p.req_pos[rq], t0_r = p.req_t0[rq], T_r = p.req_t0[rq + 1] - t0_r;
    const int kb = p.req_lo[rq] + c * p.attn_chunk;  // keys are the request's positions
    int ke = kb + p.attn_chunk;
    if (ke > pos_r + T_r) ke = pos_r + T_r;
    const bool act = wv < grp;
    const int hw = wv;  // query head within the group
    const int h = g * grp + hw;
    const uint16_t* kg = p.k_cache + ((size_t)g * p.kv_cap + p.req_kvb[rq]) * D + c8;
    const uint16_t* vg = p.v_cache + ((size_t)g * p.kv_cap + p.req_kvb[rq]) * D + c8;
    // K/V rows of a sub-chunk into registers; in the last, partial sub-chunk rows past the
    // chunk end repeat its last key (never visible, so never weighted)
    u32x4 kr[NCH], vr[NCH];
    auto fetch = [&](int sb) {
      if (sb + SK <= ke) {
        const size_t r = (size_t)(sb + row0) * D;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          kr[i] = ldg16(kg + r + (size_t)i * RSTEP * D);
          vr[i] = ldg16(vg + r + (size_t)i * RSTEP * D);
        }
      } else {
        const int last = ke - 1;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int key = sb + row0 + i * RSTEP <= last ? sb + row0 + i * RSTEP : last;
          kr[i] = ldg16(kg + (size_t)key * D);
          vr[i] = ldg16(vg + (size_t)key * D);
        }
      }
    };
    // q of this wave's head for the lane's token of the tile, scaled and split by the QKV
    // phase (tokens past T repeat token T-1; their rows are never read).  Issued before the
    // first K/V rows: the wait for those at the first LDS fill then covers q too (loads
    // complete in order), so no wait for q is left inside the key loop, where it would also
    // drain the next sub-chunk's rows in flight.
    const int tk = kTile * tile + tq;
    const int tqc = tk < p.T ? tk : p.T - 1;
    u32x4 qh[NS], ql[NS];
    auto load_q = [&]() {
      const uint16_t* qs = p.q_op + ((size_t)tqc * p.Hq + (act ? h : 0)) * 2 * D + 8 * gq;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qh[s] = ldg16(qs + 32 * s);
        ql[s] = ldg16(qs + D + 32 * s);
      }
    };
    const int first_end = kb + SK <= ke ? kb + SK : ke;  // keys of the first sub-chunk: [kb, first_end)
    if (!waited && first_end <= pos_r) {
      // cached keys only: their rows are in flight across the barrier's wait; q (written before
      // the barrier) follows it and is waited for here, so that no wait for q is left inside
      // the key loop
      fetch(kb);
      wait();
      waited = true;
      load_q();
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    } else {
      if (!waited) {
        wait();
        waited = true;
      }
      load_q();
      fetch(kb);
    }
    float m_run = NEG, l_run = 0.f;
    f32x4 O[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) O[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this lane's token: its position, which of the step's keys it sees, and the first cached
    // key inside its window
    const int ptok = p.tok_pos[tqc];
    const unsigned sees = p.tok_sees[tqc];
    const int lo_t = p.window == 0 ? -0x7fffffff - 1 : ptok - p.window + 1;
    // this lane's token takes part in the item: a token of the step, of the item's request
    const bool tok_ok = tk >= t0_r && tk < t0_r + T_r;
    const bool multi = p.n_req > 1;
    for (int sb = kb; sb < ke; sb += SK) {
      lds_barrier();  // the previous sub-chunk's LDS reads are done
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int row = row0 + i * RSTEP;
        *reinterpret_cast<u32x4*>(&L.Ks[row * KS + c8]) = kr[i];
        // V^T: the 8 values of this chunk go to rows c8 .. c8 + 7 of one swizzled key column
        uint16_t* vt = &L.Vt[L_t::vt_index(c8, row)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vt[(2 * j) * L_t::VS] = (uint16_t)(vr[i][j] & 0xffffu);
          vt[(2 * j + 1) * L_t::VS] = (uint16_t)(vr[i][j] >> 16);
        }
      }
      lds_barrier();
      if (sb + SK < ke) fetch(sb + SK);  // in flight while this sub-chunk is used
      if (act) {
        f32x4 S[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(&L.Ks[(kt * 16 + tq) * KS + 32 * s + 8 * gq]);
            S[kt] = mfma16x16x32(ka, qh[s], S[kt]);
            S[kt] = mfma16x16x32(ka, ql[s], S[kt]);
          }
        }
        // mask; lane holds keys kt*16 + 4*gq + r of the tile's token tq.  A whole sub-chunk of cached
        // keys inside every token's window needs none (rows of tokens past T are never read).
        // Otherwise key j is visible iff j is in the chunk and, for a cached key, inside the
        // token's window, for a key of the step, bit j - pos of the token's set; computed
        // without branches (selects on every element)
        float mx = NEG;
        const bool all_vis = sb + SK <= ke && sb + SK <= pos_r && (p.window == 0 || sb > pos_r + T_r - 1 - p.window);
        if (all_vis && !multi) {
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[kt][r]);
        } else if (all_vis) {  // every key visible to the request's tokens, none to the others
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = tok_ok ? S[kt][r] : NEG;
              S[kt][r] = v;
              mx = fmaxf(mx, v);
            }
        } else {
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = sb + kt * 16 + 4 * gq + r;
              const int js = j - pos_r;  // < 0: cached; else the request's token t0_r + js
              const unsigned in_win = (unsigned)(j >= lo_t);
              const unsigned seen = (sees >> ((t0_r + js) & 31)) & 1u;
              const unsigned vis = (unsigned)tok_ok & (unsigned)(j < ke) & (js < 0 ? in_win : seen);
              const float v = vis ? S[kt][r] : NEG;
              S[kt][r] = v;
              mx = fmaxf(mx, v);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const bool none = (m_new == NEG);
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = none ? 0.f : __builtin_amdgcn_exp2f(S[kt][r] - m_new);
            S[kt][r] = e;
            ls += e;
          }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        l_run = l_run * alpha + ls;
        m_run = m_new;
        float ao[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ao[r] = __shfl(alpha, 4 * gq + r);
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int r = 0; r < 4; ++r) O[d][r] *= ao[r];
#pragma unroll
        for (int kp = 0; kp < NKT / 2; ++kp) {
          // P as (hi, lo): the nearest bf16 and the bf16 of the remainder (~16 significant bits)
          const u32x2 p0 = split_bf16(S[2 * kp][0], S[2 * kp][1]), p1 = split_bf16(S[2 * kp][2], S[2 * kp][3]);
          const u32x2 p2 = split_bf16(S[2 * kp + 1][0], S[2 * kp + 1][1]);
          const u32x2 p3 = split_bf16(S[2 * kp + 1][2], S[2 * kp + 1][3]);
          const u32x4 ph = {p0[0], p1[0], p2[0], p3[0]};
          const u32x4 pl = {p0[1], p1[1], p2[1], p3[1]};
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            // k slots of this lane: keys 32kp + 4gq + 0..3 and 32kp + 16 + 4gq + 0..3
            const int dd = 16 * d + tq;
            const u32x2 v0 = *reinterpret_cast<const u32x2*>(&L.Vt[L_t::vt_index(dd, 32 * kp + 4 * gq)]);
            const u32x2 v1 = *reinterpret_cast<const u32x2*>(&L.Vt[L_t::vt_index(dd, 32 * kp + 16 + 4 * gq)]);
            const u32x4 vb = {v0[0], v0[1], v1[0], v1[1]};
            O[d] = mfma16x16x32(ph, vb, O[d]);
            O[d] = mfma16x16x32(pl, vb, O[d]);
          }
        }
      }
    }
    if (act) {
      // the tile's 16 token rows of the (head, chunk) item's partial
      auto op = gl(p.attn_o + ((size_t)(ib * grp + hw) * kMaxT + kTile * tile) * D);
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) op[(4 * gq + r) * D + 16 * d + tq] = O[d][r];
      if (lane < 16) {
        auto ml = gl(p.attn_ml + ((size_t)(ib * grp + hw) * kMaxT + kTile * tile + lane) * 2);
        ml[0] = m_run;
        ml[1] = l_run;
      }
    }
  }
  if (!waited) wait();
  if (q_set >= 0) {
    // count the item in on its group: its partial is complete in this XCC's L2 (vmcnt(0)), which
    // the group's merging workgroups share when the barrier groups run on one XCC each
    // (otherwise the release writes it back)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      if (route_tables(moel_lds).light == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_add(gl(p.ctrl) + kAttnDone + 32 * q_set, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the previous-step expert prefetch, on the workgroups that have neither an attention item nor
  // (with the merge per barrier group) merge work: barrier groups past the attention groups, or
  // the workgroups past the items
  if (p.pf_n > 0 && p.expert_hist != nullptr) {
    int idx = -1, np = 0;
    if (p.attn_set_merge) {
      const int ns = p.nwg < kBarGroups ? p.nwg : kBarGroups, ng = p.Hkv * p.ntt;
      const int r = p.nwg % ns;
      np = (p.nwg / ns) * (ns - ng) + (r > ng ? r - ng : 0);
      if (wg % ns >= ng) idx = (wg / ns) * (ns - ng) + (wg % ns - ng);
    } else if (nitems < p.nwg) {
      np = p.nwg - nitems;
      if (wg >= nitems) idx = wg - nitems;
    }
    if (idx >= 0) expert_prefetch(params_handle(p), idx, np);
  }
}

// Merge the key-chunk partials of one (token t, q head h, head-dim d) element -> o (fp32).  A
// chunk with no visible key for a token has m = -inf, weight exp(-inf) = 0 and O = l = 0.
// Chunks go in groups of 16 whose loads are all in flight together, merged into a running
// (max, numerator, denominator) with the usual rescale between groups.
__device__ __forceinline__ void merge_element(KP& p, int t, int h, int d) {
  const int grp = p.Hq / p.Hkv;
  const int nch = p.attn_nchunks;
  constexpr int U = 16;
  const float NEG = -__builtin_inff();
  const int g = h / grp, w = h % grp;
  // row (item it, head w, token t) of the partials, item it = c * Hkv + g
  const size_t row0 = (size_t)(g * grp + w) * kMaxT + t;  // chunk 0
  const size_t rstep = (size_t)p.Hkv * grp * kMaxT;       // next chunk
  float M = NEG, num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < nch; c0 += U) {
    f32x2 ml[U];
    float ov[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = c0 + j < nch ? c0 + j : nch - 1;
      const size_t row = row0 + (size_t)c * rstep;
      ml[j] = *gl(reinterpret_cast<const f32x2*>(p.attn_ml + row * 2));
      ov[j] = gl(p.attn_o)[row * p.D + d];
    }
    float Mg = M;
#pragma unroll
    for (int j = 0; j < U; ++j) Mg = fmaxf(Mg, ml[j][0]);
    const float r = M == NEG ? 0.f : __builtin_amdgcn_exp2f(M - Mg);  // rescale of the earlier groups (base 2)
    num *= r;
    den *= r;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const float wgt = (c0 + j < nch && ml[j][0] != NEG) ? __builtin_amdgcn_exp2f(ml[j][0] - Mg) : 0.f;
      num = fmaf(wgt, ov[j], num);
      den = fmaf(wgt, ml[j][1], den);
    }
    M = Mg;
  }
  const float o = num / den;
  if (p.debug_copies) gl(p.o_buf)[(size_t)t * p.Hq * p.D + h * p.D + d] = o;
  store_opsplit(gl(p.o_op), t, h * p.D + d, p.Hq * p.D, o);
}

// Merge of every (token, q head) row over all workgroups, one thread per head-dim value (after
// a grid barrier, or in its own kernel).
__device__ __forceinline__ void phase_attn_merge(KP& p, int wg) {
  const int total = p.T * p.Hq * p.D;
  for (int e = wg * kThreads + threadIdx.x; e < total; e += p.nwg * kThreads) {
    const int d = e % p.D, h = (e / p.D) % p.Hq, t = e / (p.D * p.Hq);
    merge_element(p, t, h, d);
  }
}

// Merge per barrier group (attn_set_merge): the workgroups of barrier group q merge the rows of
// attention group q (kv head q mod Hkv, token tile q / Hkv) once its items have counted in, with
// no grid barrier between the items and the merge.  The same arithmetic per element as
// phase_attn_merge, so the results are bitwise those of the barrier-separated merge.
__device__ __forceinline__ void phase_attn_merge_set(KP& p, int wg) {
  const int ns = p.nwg < kBarGroups ? p.nwg : kBarGroups;
  const int q = wg % ns, j = wg / ns, nq = (p.nwg - q + ns - 1) / ns;
  if (q >= p.Hkv * p.ntt) return;
  const int grp = p.Hq / p.Hkv, g = q % p.Hkv, tile = q / p.Hkv;
  const int t0 = kTile * tile;
  const int tn = p.T - t0 < kTile ? p.T - t0 : kTile;
  const int total = tn * grp * p.D;
  if (j * kThreads >= total) return;  // no element here: nothing to wait for
  if (threadIdx.x == 0) {
    auto cnt = gl(p.ctrl) + kAttnDone + 32 * q;
    const unsigned need = (unsigned)p.attn_nchunks;
    const uint64_t ts0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
      __builtin_amdgcn_s_sleep(1);
      if (__builtin_amdgcn_s_memrealtime() - ts0 > 50000000ull) {
        __hip_atomic_store(gl(p.ctrl) + kStatus, (unsigned)MOEL_DEV_TIMEOUT, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    // the items' partials: in this XCC's L2 (light: invalidate the L1 only), else written back
    // by their releases (drop the L2's clean lines too)
    if (route_tables(moel_lds).light != 0) asm volatile("buffer_inv sc0" ::: "memory");
    else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  for (int e = j * kThreads + threadIdx.x; e < total; e += nq * kThreads) {
    const int d = e % p.D, hw = (e / p.D) % grp, tt = e / (p.D * grp);
    merge_element(p, t0 + tt, g * grp + hw, d);
  }
}

// ------------------------------------------------------------------------------------------
// o-projection + residual -> h (fp32).
// ------------------------------------------------------------------------------------------
template <class Wait = NoWait>
__device__ __forceinline__ void phase_oproj(KP& p, int wg, char* smem, const Wait& wait = Wait{}) {
  DenseLds& L = *reinterpret_cast<DenseLds*>(phase_smem(smem));
  AOp A{p.o_op, p.T, p.Hq * p.D};
  dense_phase(p, 1, p.sk_oproj, p.w_o, p.H / 16, nullptr, 0, p.Hq * p.D, wg, A, L,
              [&](DenseLds& L, int tf, int nt, int lo, int hi) {
                const int lgT = p.ntt == 1 ? 4 : 5;  // tokens covered: 16 per tile
                for (int e = threadIdx.x; e < (nt * 16) << lgT; e += kThreads) {
                  const int j = e >> (lgT + 4), r = (e >> lgT) & 15, t = e & ((1 << lgT) - 1);
                  const int n = (tf + j) * 16 + r;
                  if (t < p.T && octet_in(n, lo, hi)) {
                    const float h = gl(p.x)[(size_t)t * p.H + n] + L.fin[(j * 16 + r) * kMaxT + t];
                    gl(p.h_buf)[(size_t)t * p.H + n] = h;
                    gl(p.h_op)[op_index(t, n, p.H)] = h;
                  }
                }
              }, wait);
}

// ------------------------------------------------------------------------------------------
// Router logits and pooler from hn = h * rstd2 * gamma2, one contraction over the stacked
// rows [router; pooler].  RMSNorm 2 is folded in as for RMSNorm 1: the pass contracts
// h * gamma2, yields rstd2 from the h it reads, and the epilogue scales by it.
// ------------------------------------------------------------------------------------------
template <class Wait = NoWait>
__device__ __forceinline__ void phase_router_pool(KP& p, int wg, char* smem, const Wait& wait = Wait{}) {
  DenseLds& L = *reinterpret_cast<DenseLds*>(phase_smem(smem));
  AGammaOp A{p.h_op, p.gamma2, p.T, p.eps, p.H};
  const int te = p.E / 16;
  dense_phase(p, 2, p.sk_rp, p.w_router, te, p.w_pool, p.P / 16, p.H, wg, A, L,
              [&](DenseLds& L, int tf, int nt, int lo, int hi) {
                const int lgT = p.ntt == 1 ? 4 : 5;  // tokens covered: 16 per tile
                for (int e = threadIdx.x; e < (nt * 16) << lgT; e += kThreads) {
                  const int j = e >> (lgT + 4), r = (e >> lgT) & 15, t = e & ((1 << lgT) - 1);
                  const int n = (tf + j) * 16 + r;
                  if (t >= p.T || !octet_in(n, lo, hi)) continue;
                  const float v = L.fin[(j * 16 + r) * kMaxT + t] * L.rstd[t];
                  if (n < p.E) {
                    gl(p.logits)[t * p.E + n] = v;
                    if (p.dbg_logits) gl(p.dbg_logits)[t * p.E + n] = v;
                  } else {
                    if (p.debug_copies) gl(p.pl)[(size_t)t * p.P + (n - p.E)] = v;
                    store_split(gl(p.pl_split) + (size_t)t * p.P * 2, n - p.E, v);
                  }
                }
              }, wait);
}

// ------------------------------------------------------------------------------------------
// Routing: top-k per token (logit descending, ties to the lower expert index), gates =
// softmax over the selected logits, and per-expert slot lists.  Computed redundantly by
// every workgroup from the same logits, so all agree bit for bit.
// ------------------------------------------------------------------------------------------
// (v, i) <- the better of (v, i) and (ov, oi): larger logit, lower expert index on ties
// (bitwise operators: short-circuit || / && would become exec-mask branches)
__device__ __forceinline__ void kv_better(float& v, int& i, float ov, int oi) {
  const bool take = (ov > v) | ((ov == v) & (oi < i));
  v = take ? ov : v;
  i = take ? oi : i;
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void kv_dpp_step(float& v, int& i) {
  const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                                          __builtin_bit_cast(int, v), CTRL,
                                                                          ROW_MASK, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xF, false);
  kv_better(v, i, ov, oi);
}
// Arg-max over each 32-lane half of the wave by DPP (VALU only, no LDS round trips): xor 1 and
// xor 2 within quads, half-row and row mirrors (row maximum in every lane of the row), then a
// row-15 broadcast into rows 1 and 3, which leaves the maximum of lanes 0-31 in lane 31 and of
// lanes 32-63 in lane 63.
// Sorts a lane's (value, expert) pairs best first (larger value; lower expert on ties) with a
// bitonic network; branch-free compare-exchanges.
template <int NV>
__device__ __forceinline__ void kv_sort_desc(float (&v)[NV], int (&ix)[NV]) {
#pragma unroll
  for (int k = 2; k <= NV; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const bool l_better = (v[l] > v[i]) | ((v[l] == v[i]) & (ix[l] < ix[i]));
          const bool sw = ((i & k) == 0) ? l_better : !l_better;
          const float a = v[i], b = v[l];
          const int ia = ix[i], ib = ix[l];
          v[i] = sw ? b : a;
          v[l] = sw ? a : b;
          ix[i] = sw ? ib : ia;
          ix[l] = sw ? ia : ib;
        }
      }
}

__device__ __forceinline__ void half_argmax(float& v, int& i, float& v_lo, int& i_lo, float& v_hi, int& i_hi) {
  kv_dpp_step<0xB1, 0xF>(v, i);   // quad_perm [1,0,3,2]
  kv_dpp_step<0x4E, 0xF>(v, i);   // quad_perm [2,3,0,1]
  kv_dpp_step<0x141, 0xF>(v, i);  // row_half_mirror
  kv_dpp_step<0x140, 0xF>(v, i);  // row_mirror
  kv_dpp_step<0x142, 0xA>(v, i);  // row_bcast15 into rows 1 and 3
  v_lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  i_lo = __builtin_amdgcn_readlane(i, 31);
  v_hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  i_hi = __builtin_amdgcn_readlane(i, 63);
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP: shifts 1, 2, 4, 8 within each row of
// 16 lanes, then the row-15 broadcast into rows 1 and 3 and the row-31 broadcast into rows 2
// and 3 carry the row totals forward.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void scan_dpp_step(int& v) {
  v += __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ void wave_inclusive_scan(int& v) {
  scan_dpp_step<0x111, 0xF>(v);  // row_shr 1
  scan_dpp_step<0x112, 0xF>(v);  // row_shr 2
  scan_dpp_step<0x114, 0xF>(v);  // row_shr 4
  scan_dpp_step<0x118, 0xF>(v);  // row_shr 8
  scan_dpp_step<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  scan_dpp_step<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
}

__device__ __forceinline__ void compute_routing(KP& p, RouteTables& R, bool write_debug) {
  const int lane = lane_id(), wv = wave_id();
  const int nslot = p.T * p.topk;
  const float NEG = -__builtin_inff();
  const int BIG = 0x7fffffff;
  static_assert(kThreads == 512, "one thread per expert table entry");
  R.cnt[threadIdx.x] = 0;
  R.tmask[threadIdx.x] = 0u;
  if (p.expert_dtype == 0) {  // weights, independent of the step: issued beside the logits
    for (int i = threadIdx.x; i < 3 * p.E; i += kThreads) {
      const int m = i / p.E, e = i - m * p.E;
      float ts = gl(m == 0 ? p.ts_gate : m == 1 ? p.ts_up : p.ts_down)[e];
      if (m == 2 && p.down_fp4) ts *= gl(p.ts_act)[e];  // the fp4 gather's tensor scale
      R.ts[m][e] = ts;
    }
  }
  // top-k: wave w takes tokens 16 th + 2w (lanes 0-31) and 16 th + 2w + 1 (lanes 32-63) at the
  // same time, th over the token tiles; lane l of a half holds experts (l mod 32) + 32 j,
  // j < NV = ceil(E / 32)
  auto topk = [&](auto nv_tag, int th) {
    constexpr int NV = decltype(nv_tag)::value;
    const int t = kTile * th + 2 * wv + (lane >> 5);
    const bool tok_ok = t < p.T;
    const int tc = tok_ok ? t : 0;
    float v[NV];
    int ix[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = (lane & 31) + 32 * j;
      const bool ok = tok_ok && e < p.E;
      v[j] = ok ? gl(p.logits)[tc * p.E + (e < p.E ? e : 0)] : NEG;
      ix[j] = ok ? e : BIG;
    }
    // each lane's list best first: a round's candidates are the list heads, and the lane that
    // owns the winner pops its head
    kv_sort_desc<NV>(v, ix);
    float sel0_lo = 0.f, sel0_hi = 0.f, esum = 0.f, ex_r = 0.f;
    for (int r = 0; r < p.topk; ++r) {
      float bv = v[0];
      int bi = ix[0];
      float v_lo, v_hi;
      int i_lo, i_hi;
      half_argmax(bv, bi, v_lo, i_lo, v_hi, i_hi);
      const float wv_ = lane < 32 ? v_lo : v_hi;
      const int wi = lane < 32 ? i_lo : i_hi;
      const bool pop = ix[0] == wi;
#pragma unroll
      for (int j = 0; j < NV - 1; ++j) {
        v[j] = pop ? v[j + 1] : v[j];
        ix[j] = pop ? ix[j + 1] : ix[j];
      }
      v[NV - 1] = pop ? NEG : v[NV - 1];
      ix[NV - 1] = pop ? BIG : ix[NV - 1];
      if (r == 0) {
        sel0_lo = v_lo;
        sel0_hi = v_hi;
      }
      const float ex = __expf(wv_ - (lane < 32 ? sel0_lo : sel0_hi));
      esum += ex;
      if ((lane & 31) == r) ex_r = ex;  // lane r of each half keeps the r-th numerator
      if ((lane & 31) == 0 && tok_ok) R.idx[t * p.topk + r] = wi;
    }
    if ((lane & 31) < p.topk && tok_ok) R.gate[t * p.topk + (lane & 31)] = ex_r / esum;
  };
  for (int th = 0; th < p.ntt; ++th) {
    if (p.E <= 256) topk(std::integral_constant<int, 8>{}, th);
    else topk(std::integral_constant<int, 16>{}, th);
  }
  lds_barrier();
  // slot lists, expert-major with slots ascending within an expert.  Per expert: the count of
  // its slots and the mask of tokens that chose it (LDS integer atomics, order-independent);
  // an exclusive scan over the experts gives each expert's first position and, over the
  // experts' entry counts (one per 16 slots, rounded up), the rank of its first active entry;
  // a slot's position is its expert's first position plus the number of earlier tokens that
  // chose the same expert (one token picks an expert at most once, so token order is slot
  // order).
  const int s = threadIdx.x;
  if (s < nslot) {
    const int e = R.idx[s];
    atomicAdd(&R.cnt[e], 1);
    atomicOr(&R.tmask[e], 1u << (s / p.topk));
  }
  lds_barrier();
  const int e = threadIdx.x;  // kThreads >= E (E <= 512)
  const int c = e < p.E ? R.cnt[e] : 0;
  const int na = (c + kTile - 1) / kTile;  // the expert's active entries
  int incl_c = c, incl_a = na;
  wave_inclusive_scan(incl_c);
  wave_inclusive_scan(incl_a);
  if (lane == 63) {
    R.wave_sum[0][wv] = incl_c;
    R.wave_sum[1][wv] = incl_a;
  }
  lds_barrier();
  int base_c = 0, base_a = 0;
  for (int w = 0; w < wv; ++w) {
    base_c += R.wave_sum[0][w];
    base_a += R.wave_sum[1][w];
  }
  const int off_e = base_c + incl_c - c;
  if (e < p.E) {
    R.off[e] = off_e;
    for (int i = 0; i < na; ++i) {
      const int ra = base_a + incl_a - na + i;
      R.active_e[ra] = e;
      R.active_off[ra] = off_e + kTile * i;
    }
  }
  if (e == kThreads - 1) {
    R.n_active = base_a + incl_a;
    R.active_off[base_a + incl_a] = base_c + incl_c;  // == nslot
  }
  lds_barrier();
  if (s < nslot) {
    const int es = R.idx[s];
    const int t = s / p.topk;
    R.slots[R.off[es] + __popc(R.tmask[es] & ((1u << t) - 1u))] = s;
  }
  if (write_debug) {
    for (int s3 = threadIdx.x; s3 < nslot; s3 += kThreads) {
      if (p.dbg_idx) gl(p.dbg_idx)[s3] = R.idx[s3];
      if (p.dbg_gates) gl(p.dbg_gates)[s3] = R.gate[s3];
    }
  }
  lds_barrier();
}

// The layer's routing history for the next step: tokens per expert of this step (workgroup 0,
// from the routing tables every workgroup holds).
__device__ __forceinline__ void write_expert_hist(KP& p, const RouteTables& R, int wg) {
  if (wg != 0 || p.expert_hist == nullptr) return;
  for (int e = threadIdx.x; e < p.E; e += kThreads) gl(p.expert_hist)[e] = (unsigned)R.cnt[e];
}

// ------------------------------------------------------------------------------------------
// NVFP4 experts on 4x4x4 MFMA: a wavefront lane owns one weight row.  The 4 A rows of each
// 4x4x4 block carry 2 tokens as (hi, hi', lo, lo') and are broadcast from one 4-lane block
// to all 16 blocks (CBSZ=4, ABID selects the 4-element k slice); row sums hi + lo give the
// fp32-accurate product.  The E4M3 block scale multiplies each 16-k partial in fp32.
// G = token pairs (1, 2, 4, 8), NM = matrices sharing the activation (2 gate+up, 1 down).
// ------------------------------------------------------------------------------------------
// LDS of the NVFP4 expert phases.  red: per-wave partial sums of a tile, [wave][lane][RW]
// floats with RW = NM*2*G; double-buffered by tile parity when two buffers fit (RW <= 16),
// so that one barrier per tile suffices.  stage: finished outputs of the stream's tiles in
// stream order, 64 rows x 2G slots per tile, written to global memory when the stream ends
// (no global store sits between the weight loads); st_tile: the tile of each stage entry.
constexpr int kFp4RedPer = 32;        // floats per (wave, lane): NM*2*G for NM = 2, G = 8
constexpr int kFp4Stage = 8192;       // floats (32 KiB): 64 tiles of one token pair
constexpr int kFp4MaxStaged = kFp4Stage / 128;
struct Fp4Lds {
  float red[kWaves * 64 * kFp4RedPer];
  float stage[kFp4Stage];
  int st_tile[kFp4MaxStaged];
};

template <int NM, int G>
struct Fp4Pair {
  u32x4 c[NM][2];   // codes of the pair's two 32-k steps
  uint32_t sc[NM];  // 4 block scales of the pair
  u32x2 a[G];       // activation operand: 4 bf16 (hi or lo) of lane 4b+i's token slot
};

// Activation operands come from the split-operand copy of the activation (per 4-element
// quad: 4 bf16 nearest values, then 4 bf16 remainders).  row0[g]: split row of token slot 2g,
// dr[g]: offset (bf16 units) of slot 2g+1's row from it, both uniform; lane 4b+i reads quad
// b of the pair from the row of slot 2g + (i & 1), the nearest half for i < 2 and the
// remainder half for i >= 2.  Plain arithmetic, so that no per-lane choice between registers
// is made through memory.
template <int NM, int G>
__device__ __forceinline__ void fp4_pair_load_w(Fp4Pair<NM, G>& f, const uint8_t* const (&wt)[NM]) {
  const int lane = lane_id();
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    f.c[m][0] = ldg_stream(wt[m] + lane * 16);
    f.c[m][1] = ldg_stream(wt[m] + 1024 + lane * 16);
    f.sc[m] = ldg_stream32(wt[m] + 2048 + 4 * lane);
  }
}
template <int NM, int G>
__device__ __forceinline__ void fp4_pair_load_a(Fp4Pair<NM, G>& f, const uint16_t* const (&row0)[G],
                                                const long (&dr)[G], int k0) {
  const int lane = lane_id();
  const int lane_off = 8 * (lane >> 2) + 4 * ((lane >> 1) & 1);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const long off = (lane & 1) ? dr[g] : 0l;
    f.a[g] = ldg8(row0[g] + off + 2 * k0 + lane_off);
  }
}
template <int NM, int G>
__device__ __forceinline__ void fp4_pair_load(Fp4Pair<NM, G>& f, const uint8_t* const (&wt)[NM],
                                              const uint16_t* const (&row0)[G], const long (&dr)[G], int k0) {
  fp4_pair_load_w<NM, G>(f, wt);
  fp4_pair_load_a<NM, G>(f, row0, dr, k0);
}

template <int H, int J, int NM, int G>
__device__ __forceinline__ void fp4_mfma_block(const Fp4Pair<NM, G>& f, const u32x2 (&a)[G],
                                               f32x4 (&acc)[NM][G]) {
  // block q = 2*H + J (16 k): MFMAs with ABID = 8*H + 4*J + u, u = 0..3
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const uint32_t w0 = f.c[m][H][2 * J], w1 = f.c[m][H][2 * J + 1];
    u32x2 b[4];
    b[0] = u32x2{fp4x2_to_bf16x2<0>(w0), fp4x2_to_bf16x2<1>(w0)};
    b[1] = u32x2{fp4x2_to_bf16x2<2>(w0), fp4x2_to_bf16x2<3>(w0)};
    b[2] = u32x2{fp4x2_to_bf16x2<0>(w1), fp4x2_to_bf16x2<1>(w1)};
    b[3] = u32x2{fp4x2_to_bf16x2<2>(w1), fp4x2_to_bf16x2<3>(w1)};
    const float s = e4m3_to_f32<2 * H + J>(f.sc[m]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      f32x4 P = f32x4{0.f, 0.f, 0.f, 0.f};
      P = mfma4x4x4_bcast<8 * H + 4 * J + 0>(a[g], b[0], P);
      P = mfma4x4x4_bcast<8 * H + 4 * J + 1>(a[g], b[1], P);
      P = mfma4x4x4_bcast<8 * H + 4 * J + 2>(a[g], b[2], P);
      P = mfma4x4x4_bcast<8 * H + 4 * J + 3>(a[g], b[3], P);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][g][r] = fmaf(s, P[r], acc[m][g][r]);
    }
  }
}

// rows of a 4-lane block: (hi t0, hi t1, lo t0, lo t1)
template <int NM, int G>
__device__ __forceinline__ void fp4_pair_compute(const Fp4Pair<NM, G>& f, f32x4 (&acc)[NM][G]) {
  const u32x2 (&a)[G] = f.a;
  fp4_mfma_block<0, 0>(f, a, acc);
  fp4_mfma_block<0, 1>(f, a, acc);
  fp4_mfma_block<1, 0>(f, a, acc);
  fp4_mfma_block<1, 1>(f, a, acc);
}

// NVFP4 encoding of the SwiGLU output for the fp4 gather before the down projection: the
// nearest representable value, ties to the even code, saturating; decided in fp32.
__device__ __forceinline__ float e4m3_nearest(float v) {  // v >= 0
  if (!(v < 448.0f)) return 448.0f;
  // v in [2^ex, 2^(ex+1)) keeps 4 significant bits: quantum 2^(ex-3), never below 2^-9
  const int ex = (int)((__float_as_uint(v) >> 23) & 0xffu) - 127;
  const int q = ex - 3 > -9 ? ex - 3 : -9;
  const float r = ldexpf(rintf(ldexpf(v, -q)), q);
  return r < 448.0f ? r : 448.0f;
}
__device__ __forceinline__ float e2m1_nearest(float m) {  // m >= 0
  // decision points: the midpoints of 0, 0.5, 1, 1.5, 2, 3, 4, 6, each tie to the even code
  return m <= 0.25f ? 0.0f : m < 0.75f ? 0.5f : m <= 1.25f ? 1.0f : m < 1.75f ? 1.5f
       : m <= 2.5f ? 2.0f : m < 3.5f ? 3.0f : m <= 5.0f ? 4.0f : 6.0f;
}
// Encodes the value v held by this lane as part of the 16-element block held by its 16-lane
// group (all 64 lanes active): returns E2M1 value x E4M3 block scale (exact in bf16), the
// tensor scale ts left to the down projection's sums.
__device__ __forceinline__ float fp4_gather_value(float v, float ts) {
  float amax = fabsf(v);
  amax = fmaxf(amax, __shfl_xor(amax, 8));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  const float s = e4m3_nearest(amax / (6.0f * ts));
  const float den = s * ts;
  const float mag = den > 0.0f ? e2m1_nearest(fabsf(v / den)) : 0.0f;
  return copysignf(mag * s, v);
}

// token-pair group that an expert with n_e slots needs
__device__ __forceinline__ int fp4_group(int n_e) { return n_e <= 2 ? 1 : n_e <= 4 ? 2 : n_e <= 8 ? 4 : 8; }

constexpr int kDqEnd = 0xffff;  // tile field of a hand-out past the last tile
// Hand-outs stay in the ring until every k-wave has read them (at most two are live).
constexpr int kDqSlots = 64;
static_assert(sizeof(RouteTables::dq) == kDqSlots * sizeof(int), "hand-out ring size");

// Tile stream of an NVFP4 expert phase.  The workgroup computes, in order, the 64-row tiles
// of the stream's positions: static positions 0 .. te-ts-1 are tiles ts .. te-1 (global tile
// order: active expert major), later positions are dynamic tiles k0, k0+1, ... handed to the
// workgroup by the device-wide work counter.  One ring of DEPTH register buffers runs over the
// whole stream, across tile and expert boundaries: the k-waves split each tile's K/64 pairs
// evenly (npt each; wave wv takes pairs wv, wv + nkw, ...), and the ring holds the next
// DEPTH pairs of every k-wave, so no tile or hand-out boundary drains it.  The k-waves meet
// at one LDS barrier per tile, where the tile is reduced.  Wave 0 requests the hand-out of
// position s+1 when its loads enter position s and publishes it in the LDS ring `dq` before
// the next barrier; every wave passes that barrier before its loads reach s+1 (the stream's
// start barrier covers s = 1), so a hand-out is always published before it is read.
// The stream ends before a tile that needs a larger token group than G, when the stage is
// full, or at the end of the work.  Return: -1 when the work is done; a static tile to resume
// from (>= 0); or -(2 + k) to resume at dynamic position k (handed out and published in dq).
//
// wait_bar (> 0): number of the grid barrier before the phase, whose second half the stream
// runs after the weight loads of its first pairs and before their activation loads (the
// activation is written by the phase before the barrier, the weights by none); 0: none.
template <bool GATEUP, int G, int DEPTH>
__device__ __noinline__ int fp4_expert_stream(uint64_t ph, int ts_arg, int te_arg, int k0_arg, int tdyn_arg,
                                              int wait_bar_arg) {
  KP& p = params_from(ph);
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int RW = NM * 2 * G;  // red floats per lane
  constexpr bool DB = 2 * RW <= kFp4RedPer;
  constexpr int SPT = 64 * 2 * G;          // stage floats per tile
  constexpr int MAXT = kFp4Stage / SPT;    // tiles per stream
  RouteTables& R = route_tables(moel_lds);
  Fp4Lds& L = *reinterpret_cast<Fp4Lds*>(phase_smem(moel_lds));
  const int ts = uniform(ts_arg), k0 = uniform(k0_arg), t_dyn = uniform(tdyn_arg);
  const int n_st = uniform(te_arg) - ts;
  const int lane = lane_id(), wv = wave_id();
  const int tpe = (GATEUP ? p.I_loc : p.P_loc) >> 6;
  const int t_end = uniform(R.n_active) * tpe;
  const int K = GATEUP ? p.P : p.I;
  const int Sp = K >> 6;  // 64-k pairs (K % 128 == 0)
  const int nkw = kwaves_for(Sp);
  const int npt = Sp / nkw;
  const bool kw = wv < nkw;
  const size_t tile_bytes = (size_t)36 * K;  // 64 rows of K/2 + K/16 bytes

  // Tile of position s.  A hand-out found missing (it cannot be, see above) ends the stream
  // with an error status instead of waiting.
  auto tile_at = [&](int s) -> int {
    if (s < n_st) return ts + s;
    const int k = k0 + s - n_st;
    const int v = uniform(R.dq[k & (kDqSlots - 1)]);
    if ((v >> 16) != k) {
      if (threadIdx.x == 0)
        __hip_atomic_store(gl(p.ctrl) + kStatus, (unsigned)MOEL_DEV_ORDER, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return kDqEnd;
    }
    return v & 0xffff;
  };

  // ---- hand-outs (wave 0): requested when the loads enter a position, published later
  bool gpend = false;
  unsigned gv = 0u;
  int is = 0;  // position whose pairs are being issued
  auto request = [&]() {  // for position is + 1
    if (wv == 0 && is + 1 >= n_st) {
      if (lane == 0) gv = __hip_atomic_fetch_add(gl(p.ctrl) + kWork + 32 * (GATEUP ? 0 : 1), 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      gpend = true;
    }
  };
  auto publish = [&]() {
    if (gpend) {
      if (lane == 0) {
        const int k = k0 + is + 1 - n_st;
        const unsigned t = (unsigned)t_dyn + gv;
        R.dq[k & (kDqSlots - 1)] = (k << 16) | (t < (unsigned)t_end ? (int)t : kDqEnd);
      }
      gpend = false;
    }
  };

  // ---- issue side: the position's expert (u, e, slots) and tile j within it, all uniform.
  // Moving to the next static tile of the same expert is a pointer increment; the expert's
  // tables are read only when the expert changes.
  int iu = -1, ij = 0, ie = 0, ine = 1;
  const uint8_t* wb[NM];
  const uint16_t* row0[G];
  long dr[G];
  auto set_expert = [&](int u) {
    iu = u;
    ie = uniform(R.active_e[u]);
    const int s_lo = uniform(R.active_off[u]);
    ine = uniform(R.active_off[u + 1]) - s_lo;
    const int rstride = GATEUP ? p.P : p.I;
    // slots past n_e repeat the last one (their products are computed and never read)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int j0 = 2 * g < ine ? 2 * g : ine - 1, j1 = 2 * g + 1 < ine ? 2 * g + 1 : ine - 1;
      const int s0 = uniform(R.slots[s_lo + j0]), s1 = uniform(R.slots[s_lo + j1]);
      const int r0 = GATEUP ? s0 / p.topk : s0, r1 = GATEUP ? s1 / p.topk : s1;
      row0[g] = uniform((GATEUP ? p.pl_split : p.a_split) + (size_t)r0 * 2 * rstride + wv * 128);
      dr[g] = (long)(r1 - r0) * 2 * rstride;
    }
  };
  auto set_tile = [&]() {  // weights of tile ij of expert ie
    const size_t toff = (size_t)ij * tile_bytes + (size_t)wv * 2304;
    wb[0] = uniform((GATEUP ? p.w_gate + (size_t)ie * p.stride_gate : p.w_down + (size_t)ie * p.stride_down) + toff);
    if (GATEUP) wb[NM - 1] = uniform(p.w_up + (size_t)ie * p.stride_up + toff);
  };
  // position 0
  {
    const int t0 = tile_at(0);  // the caller guarantees that the stream takes it
    const int u = t0 / tpe;
    set_expert(u);
    ij = t0 - u * tpe;
    set_tile();
  }
  int it_e = ie, it_ne = ine;  // expert and slot count of the tile being issued

  // ---- compute side: reduction of the stream's n-th tile (expert e, ne slots) into the stage
  f32x4 acc[NM][G];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[m][g] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto tile_end = [&](int n, int e, int ne, int t) {
    publish();  // before the barrier: the hand-out of the position after the next
    float* red = L.red + (DB ? (n & 1) * (kWaves * 64 * RW) : 0);
    if (kw) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          red[(wv * 64 + lane) * RW + m * 2 * G + 2 * g] = acc[m][g][0] + acc[m][g][2];
          red[(wv * 64 + lane) * RW + m * 2 * G + 2 * g + 1] = acc[m][g][1] + acc[m][g][3];
          acc[m][g] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    lds_barrier();
    const float ts0 = GATEUP ? R.ts[0][e] : R.ts[2][e];
    const float ts1 = GATEUP ? R.ts[1][e] : 0.f;
    float* out = L.stage + n * SPT;
    for (int x = threadIdx.x; x < 64 * ne; x += kThreads) {
      const int ln = x & 63, j = x >> 6;
      if (GATEUP) {
        float gs = 0.f, us = 0.f;
        for (int w = 0; w < nkw; ++w) {
          gs += red[(w * 64 + ln) * RW + j];
          us += red[(w * 64 + ln) * RW + 2 * G + j];
        }
        gs *= ts0;
        us *= ts1;
        out[x] = gs / (1.0f + __expf(-gs)) * us;
      } else {
        float ds = 0.f;
        for (int w = 0; w < nkw; ++w) ds += red[(w * 64 + ln) * RW + j];
        out[x] = ds * ts0;
      }
    }
    if (threadIdx.x == 0) L.st_tile[n] = t;
    if (!DB) lds_barrier();  // red is rewritten at the next tile end
  };

  // the loads move on to position is + 1: end the stream there, or set it up.  Returns false
  // at the end of the stream.
  int it = tile_at(0);
  auto advance = [&]() -> bool {
    publish();  // wave 0 never reads its own hand-out unpublished
    const int s = is + 1;
    if (s >= MAXT) return false;
    int t;
    if (s < n_st) {
      t = ts + s;
      if (++ij == tpe) {
        ij = 0;
        set_expert(iu + 1);
      }
    } else {
      t = tile_at(s);
      if (t >= t_end) return false;
      const int u = t / tpe;
      if (u != iu) set_expert(u);
      ij = t - u * tpe;
    }
    if (fp4_group(ine) > G) return false;
    set_tile();
    is = s;
    it = t;
    it_e = ie;
    it_ne = ine;
    request();
    return true;
  };

  Fp4Pair<NM, G> ring[DEPTH];
  auto issue = [&](Fp4Pair<NM, G>& f, int pr) {
    const uint8_t* wt[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) wt[m] = wb[m] + (size_t)pr * nkw * 2304;
    fp4_pair_load<NM, G>(f, wt, row0, dr, 64 * nkw * pr);
  };
  bool more = true;
  const int wait_bar = uniform(wait_bar_arg);
  if (wait_bar > 0) {
    // the first pairs' weights, the barrier's wait, then their activations
    if (kw) {
      request();
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const uint8_t* wt[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) wt[m] = wb[m] + (size_t)d * nkw * 2304;
        fp4_pair_load_w<NM, G>(ring[d], wt);
      }
    }
    grid_barrier_wait(p, (unsigned)wait_bar);
    stamp(p, 16 + (GATEUP ? kPhGemm1 : kPhGemm2));
    if (kw) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        fp4_pair_load_a<NM, G>(ring[d], row0, dr, 64 * nkw * d);
        sched_fence();
      }
      publish();
    }
  } else if (kw) {
    request();
    // DEPTH <= npt: the first DEPTH pairs all lie in the first tile
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      issue(ring[d], d);
      sched_fence();
    }
    publish();
  }
  lds_barrier();  // position 1's hand-out is published
  if (kw) {
    int ct = it, ce = it_e, cne = it_ne, cn = 0, cp = 0;  // tile being computed
    int ip = DEPTH;
    if (ip == npt) {
      more = advance();
      ip = 0;
    }
    while (more) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        fp4_pair_compute<NM, G>(ring[d], acc);
        issue(ring[d], ip + d);
        sched_fence();
      }
      cp += DEPTH;
      if (cp == npt) {
        tile_end(cn, ce, cne, ct);
        ct = it;
        ce = it_e;
        cne = it_ne;
        ++cn;
        cp = 0;
      }
      ip += DEPTH;
      if (ip == npt) {
        more = advance();
        ip = 0;
      }
    }
    // the ring holds the last DEPTH pairs of tile ct
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) fp4_pair_compute<NM, G>(ring[d], acc);
    tile_end(cn, ce, cne, ct);
    publish();
  } else {
    // waves without k work take part in the reductions, following the same positions
    for (int n = 0;; ++n) {
      const int t = it, e = it_e, ne = it_ne;
      more = advance();
      tile_end(n, e, ne, t);
      if (!more) break;
    }
  }
  // write the stream's outputs (positions 0 .. is).  SPT and kThreads are multiples of 64,
  // so every wave runs the same iterations with all lanes, and the 16 elements of a row
  // block (16 consecutive x) sit in 16 consecutive lanes.
  lds_barrier();
  for (int x = threadIdx.x; x < (is + 1) * SPT; x += kThreads) {
    const int n = x / SPT, r = x - n * SPT, j = r >> 6;
    const int t = L.st_tile[n];
    const int u = t / tpe;
    const int s_lo = R.active_off[u];
    float v = L.stage[x];
    if (GATEUP && p.down_fp4) v = fp4_gather_value(v, gl(p.ts_act)[R.active_e[u]]);
    if (j < R.active_off[u + 1] - s_lo) {
      const int slot = R.slots[s_lo + j];
      const int row = (t - u * tpe) * 64 + (r & 63);
      if (GATEUP) {
        const size_t ai = (size_t)slot * p.I + p.rank * p.I_loc + row;
        if (p.debug_copies) {
          gl(p.a_buf)[ai] = L.stage[x];
          if (p.down_fp4) gl(p.aq_buf)[ai] = v;
        }
        store_split(gl(p.a_split) + (size_t)slot * p.I * 2, p.rank * p.I_loc + row, v);
      } else {
        gl(p.d_buf)[(size_t)slot * p.P + p.rank * p.P_loc + row] = L.stage[x];
      }
    }
  }
  lds_barrier();  // the stage and st_tile are rewritten by the next stream
  const int stop = is + 1;
  if (stop >= n_st && tile_at(stop) >= t_end) return -1;
  return stop < n_st ? ts + stop : -(2 + k0 + stop - n_st);
}

// ------------------------------------------------------------------------------------------
// bf16 experts on 16x16x32 MFMA.  The 16 A rows carry up to 8 slots as (hi x8, lo x8); a
// second row tile takes slots 8..15, read ready-made from the split-operand copies of pl and
// a (each lane loads only its row's half: 16 bytes per step).  Tiles ta..tb-1 of one expert
// run as one stream: the k-waves split each tile's K/32 steps evenly, and a ring of RD steps
// (weight and activation words) per wave runs across tile boundaries, so a tile's reduction
// never waits for the next tile's first loads.  Every step carries two weight words per lane:
// gate and up of one tile, or (down projection) two adjacent tiles sharing the activation.
// ------------------------------------------------------------------------------------------
template <bool GATEUP>
__device__ __forceinline__ void bf16_expert_tiles(KP& p, const RouteTables& R, int u, int ta, int tb,
                                  DenseLds& L) {
  constexpr int NM = 2;  // weight words per step: gate and up, or two adjacent down tiles
  constexpr int TPS = GATEUP ? 1 : 2;  // tiles per step
  constexpr int RD = 2;  // steps in flight per wave
  const int lane = lane_id(), wv = wave_id();
  const int e = R.active_e[u];
  const int s_lo = R.active_off[u], n_e = R.active_off[u + 1] - s_lo;
  const int K = GATEUP ? p.P : p.I;
  const int S = K >> 5;
  const int nkw = kwaves_for(S);
  const int nst = S / nkw;  // steps per k-wave and tile
  const int sa = wv * nst;
  const int nrt = n_e > 8 ? 2 : 1;  // row tiles
  const uint8_t* wb[NM];
  if (GATEUP) {
    wb[0] = p.w_gate + (size_t)e * p.stride_gate;
    wb[NM - 1] = p.w_up + (size_t)e * p.stride_up;
  } else {
    wb[0] = wb[1] = p.w_down + (size_t)e * p.stride_down;
  }
  // split row of this lane's slot, at its half (nearest values for A rows 0-7, remainders
  // for rows 8-15); the lane's 8 k of a step (the packed weights' order, 32s + 4q + 0..3 and
  // 32s + 16 + 4q + 0..3) are quads 8s + q and 8s + 4 + q
  const uint16_t* arow[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int j = 8 * rt + (lane & 7);
    arow[rt] = nullptr;
    if (j < n_e) {
      const int slot = R.slots[s_lo + j];
      arow[rt] = (GATEUP ? p.pl_split + (size_t)(slot / p.topk) * p.P * 2 : p.a_split + (size_t)slot * p.I * 2) +
                 ((lane & 15) >= 8 ? 4 : 0) + 8 * (lane >> 4);
    }
  }
  struct Step {
    u32x4 w[NM];
    u32x2 a[2][2];
  };
  // flattened position i of this wave: tile group ta + TPS (i / nst), step sa + i % nst; the
  // last group of an odd down range has one tile (its second word is not loaded or stored)
  const int ngrp = (tb - ta + TPS - 1) / TPS;
  const int total = wv < nkw ? ngrp * nst : 0;
  auto issue = [&](Step& st, int i) {
    const int tr = i / nst, s = sa + i - tr * nst;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int ti = ta + TPS * tr + (GATEUP ? 0 : m);
      if (GATEUP || ti < tb) st.w[m] = ldg_stream(wb[m] + ((size_t)ti * S + s) * 1024 + lane * 16);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      if (rt < nrt && arow[rt] != nullptr) {
        st.a[rt][0] = ldg8(arow[rt] + 64 * s);
        st.a[rt][1] = ldg8(arow[rt] + 64 * s + 32);
      }
    }
  };
  f32x4 acc[2][NM];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[rt][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  // reduction of tile group tg: tiles ta + TPS tg .. (all waves take part)
  auto tile_end = [&](int tg) {
    const int ti = ta + TPS * tg;
    const int nt = GATEUP ? 1 : (ti + 1 < tb ? 2 : 1);
    if (wv < nkw) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          L.red[(wv * 4 + rt * 2 + m) * 64 + lane] = acc[rt][m];
          acc[rt][m] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    lds_barrier();
    // slot j = 8*rt + jj: hi at A row jj, lo at row 8 + jj; row i lives in lane 16*(i/4)+r, comp i%4
    for (int x = threadIdx.x; x < 16 * n_e * nt; x += kThreads) {
      const int r = x & 15, j = (x >> 4) % n_e, m = (x >> 4) / n_e;  // m: tile of the group (down)
      const int rt = j >> 3, jj = j & 7;
      const int l_hi = 16 * (jj >> 2) + r, l_lo = 16 * ((8 + jj) >> 2) + r, c = jj & 3;
      const int slot = R.slots[s_lo + j];
      float s0 = 0.f, s1 = 0.f;
      for (int w = 0; w < nkw; ++w) {
        s0 += L.red[(w * 4 + rt * 2 + m) * 64 + l_hi][c] + L.red[(w * 4 + rt * 2 + m) * 64 + l_lo][c];
        if (GATEUP)
          s1 += L.red[(w * 4 + rt * 2 + 1) * 64 + l_hi][c] + L.red[(w * 4 + rt * 2 + 1) * 64 + l_lo][c];
      }
      if (GATEUP) {
        const float a = s0 / (1.0f + __expf(-s0)) * s1;
        const int c = p.rank * p.I_loc + ti * 16 + r;
        if (p.debug_copies) gl(p.a_buf)[(size_t)slot * p.I + c] = a;
        store_split(gl(p.a_split) + (size_t)slot * p.I * 2, c, a);
      } else {
        gl(p.d_buf)[(size_t)slot * p.P + p.rank * p.P_loc + (ti + m) * 16 + r] = s0;
      }
    }
    lds_barrier();  // red is rewritten at the next tile end
  };
  if (wv >= nkw) {
    for (int tg = 0; tg < ngrp; ++tg) tile_end(tg);
    return;
  }
  Step ring[RD];
#pragma unroll
  for (int d = 0; d < RD; ++d)
    if (d < total) issue(ring[d], d);
  for (int i0 = 0; i0 < total; i0 += RD) {
#pragma unroll
    for (int d = 0; d < RD; ++d) {
      const int i = i0 + d;
      if (i < total) {
        const Step cur = ring[d];
        if (i + RD < total) issue(ring[d], i + RD);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          if (rt < nrt) {
            u32x4 a = {0u, 0u, 0u, 0u};
            if (arow[rt] != nullptr) a = u32x4{cur.a[rt][0][0], cur.a[rt][0][1], cur.a[rt][1][0], cur.a[rt][1][1]};
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[rt][m] = mfma16x16x32(a, cur.w[m], acc[rt][m]);
          }
        }
        const int tr = i / nst;
        if (i - tr * nst == nst - 1) tile_end(tr);
      }
    }
  }
}

// Expert GEMM phase: the flattened list (active expert u, tile) split evenly over workgroups.
// wait_bar (> 0): number of the grid barrier before the phase, whose second half the phase runs
// itself, in its first stream after that stream's first weight loads (NVFP4 experts), or first
// (bf16 experts, or a workgroup without tiles); 0: none.
template <bool GATEUP>
__device__ __forceinline__ void phase_experts(KP& p, int wg, char* smem, int wait_bar = 0) {
  RouteTables& R = route_tables(smem);
  const int rows = GATEUP ? p.I_loc : p.P_loc;
  const bool fp4 = p.expert_dtype == 0;
  const int tpe = fp4 ? rows / 64 : rows / 16;
  const int U = uniform(R.n_active);
  // Tiles are split by estimated cost, not by count: a tile of expert u costs A + n_e(u)
  // units (its weight bytes, plus the per-token work), with A fitted to measured tile times.
  // Tile (u, j) covers [P_u + j c_u, P_u + (j+1) c_u) with P_u = tpe (A u + sum_{v<u} n_e(v))
  // = tpe (A u + active_off[u]); a workgroup takes the tiles whose cost interval starts in
  // its share [wg C / nwg, (wg+1) C / nwg).
  // 32-bit: C * nwg < 2^31 for every accepted shape (checked at plan creation)
  const int A = GATEUP ? 16 : 9;
  const int C = tpe * (A * U + uniform(R.active_off[U]));
  auto first_tile = [&](int c) -> int {  // first tile whose cost interval starts at or after c
    if (c >= C) return U * tpe;
    int lo = 0, hi = U - 1;  // largest u with P_u <= c (P_0 = 0 <= c)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tpe * (A * mid + uniform(R.active_off[mid])) <= c) lo = mid;
      else hi = mid - 1;
    }
    const int Pu = tpe * (A * lo + uniform(R.active_off[lo]));
    const int cu = A + uniform(R.active_off[lo + 1]) - uniform(R.active_off[lo]);
    return lo * tpe + (int)((unsigned)(c - Pu + cu - 1) / (unsigned)cu);
  };
  // Static part: the first 7/8 of the cost, split evenly.  Dynamic part: the remaining tiles,
  // one per hand-out from a device-wide counter, so that workgroups that run slower (for any
  // reason: more tokens per tile, a busier XCD) take fewer of them.  Which workgroup computes
  // a tile does not change its arithmetic, so results stay bitwise reproducible.
  const int Cs = C - C / 8;
  const int t0 = first_tile((int)((unsigned)wg * (unsigned)Cs / (unsigned)p.nwg));
  const int t1 = first_tile((int)((unsigned)(wg + 1) * (unsigned)Cs / (unsigned)p.nwg));
  const int t_dyn = first_tile(Cs), t_end = U * tpe;
  auto ctr = gl(p.ctrl) + kWork + 32 * (GATEUP ? 0 : 1);
  if (fp4) {
    if (threadIdx.x < kDqSlots) R.dq[threadIdx.x] = -1;
    lds_barrier();
    const int Sp = (GATEUP ? p.P : p.I) >> 6;
    const int npt = Sp / kwaves_for(Sp);
    int ts = t0, k = 0;
    int wb = wait_bar;  // passed to the first stream only
    for (;;) {
      int t = ts;
      if (ts >= t1) {  // next position is dynamic: hand it out unless a stream already did
        if (uniform(R.dq[k & (kDqSlots - 1)]) >> 16 != k) {
          if (threadIdx.x == 0) {
            const unsigned v = (unsigned)t_dyn + __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            R.dq[k & (kDqSlots - 1)] = (k << 16) | (v < (unsigned)t_end ? (int)v : kDqEnd);
          }
          lds_barrier();
        }
        t = uniform(R.dq[k & (kDqSlots - 1)]) & 0xffff;
        if (t >= t_end) break;
      }
      const int G = fp4_group(uniform(R.active_off[t / tpe + 1]) - uniform(R.active_off[t / tpe]));
      const uint64_t h = params_handle(p);
      // Ring depth 2: with every workgroup streaming all the time, two pairs in flight per wave
      // (~74 KB per CU for gate/up) measured faster than 4 or 8 (more outstanding requests per
      // CU lowered the achieved bandwidth), and 1 no faster.  Depth 1 for G = 8 (registers)
      // and for shapes with an odd pair count per wave (K < 1024).
      int r;
      const bool d2 = npt % 2 == 0;
      if (G == 1) r = d2 ? fp4_expert_stream<GATEUP, 1, 2>(h, ts, t1, k, t_dyn, wb)
                         : fp4_expert_stream<GATEUP, 1, 1>(h, ts, t1, k, t_dyn, wb);
      else if (G == 2) r = d2 ? fp4_expert_stream<GATEUP, 2, 2>(h, ts, t1, k, t_dyn, wb)
                              : fp4_expert_stream<GATEUP, 2, 1>(h, ts, t1, k, t_dyn, wb);
      else if (G == 4) r = d2 ? fp4_expert_stream<GATEUP, 4, 2>(h, ts, t1, k, t_dyn, wb)
                              : fp4_expert_stream<GATEUP, 4, 1>(h, ts, t1, k, t_dyn, wb);
      else r = fp4_expert_stream<GATEUP, 8, 1>(h, ts, t1, k, t_dyn, wb);
      wb = 0;
      r = uniform(r);
      if (r == -1) break;
      if (r >= 0) {
        ts = r;
      } else {
        ts = t1;
        k = -r - 2;
      }
    }
    if (wb > 0) {  // no stream ran: the barrier's second half still
      grid_barrier_wait(p, (unsigned)wb);
      stamp(p, 16 + (GATEUP ? kPhGemm1 : kPhGemm2));
    }
    return;
  }
  if (wait_bar > 0) {
    grid_barrier_wait(p, (unsigned)wait_bar);
    stamp(p, 16 + (GATEUP ? kPhGemm1 : kPhGemm2));
  }
  DenseLds& L = *reinterpret_cast<DenseLds*>(phase_smem(smem));
  for (int t = t0; t < t1;) {
    const int u = t / tpe;
    const int ta = t % tpe;
    int tb = tpe;
    if ((u + 1) * tpe > t1) tb = t1 - u * tpe;
    bf16_expert_tiles<GATEUP>(p, R, u, ta, tb, L);
    t = u * tpe + tb;
  }
  for (;;) {
    if (threadIdx.x == 0)
      R.next = t_dyn + (int)__hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
    const int t = uniform(R.next);
    lds_barrier();  // R.next is rewritten by the next grab
    if (t >= t_end) break;
    bf16_expert_tiles<GATEUP>(p, R, t / tpe, t % tpe, t % tpe + 1, L);
  }
}

// m[t] = sum over the token's slots, in selection order, of gate * d
__device__ __forceinline__ void phase_combine(KP& p, int wg, char* smem) {
  const RouteTables& R = route_tables(smem);
  const int total = p.T * p.P_loc;
  for (int x = wg * kThreads + threadIdx.x; x < total; x += p.nwg * kThreads) {
    const int t = x / p.P_loc, pc = p.rank * p.P_loc + x % p.P_loc;
    float s = 0.f;
    for (int k = 0; k < p.topk; ++k)
      s = fmaf(R.gate[t * p.topk + k], gl(p.d_buf)[(size_t)(t * p.topk + k) * p.P + pc], s);
    if (p.debug_copies) gl(p.m_buf)[(size_t)t * p.P + pc] = s;
    store_opsplit(gl(p.m_op), t, pc, p.P, s);
  }
}

// y = h + m W_unpool^T
template <class Wait = NoWait>
__device__ __forceinline__ void phase_unpool(KP& p, int wg, char* smem, const Wait& wait = Wait{}) {
  DenseLds& L = *reinterpret_cast<DenseLds*>(phase_smem(smem));
  AOp A{p.m_op, p.T, p.P};
  dense_phase(p, 3, p.sk_unpool, p.w_unpool, p.H / 16, nullptr, 0, p.P, wg, A, L,
              [&](DenseLds& L, int tf, int nt, int lo, int hi) {
                const int lgT = p.ntt == 1 ? 4 : 5;  // tokens covered: 16 per tile
                for (int e = threadIdx.x; e < (nt * 16) << lgT; e += kThreads) {
                  const int j = e >> (lgT + 4), r = (e >> lgT) & 15, t = e & ((1 << lgT) - 1);
                  const int n = (tf + j) * 16 + r;
                  if (t >= p.T || !octet_in(n, lo, hi)) continue;
                  gl(p.y)[(size_t)t * p.H + n] = gl(p.h_buf)[(size_t)t * p.H + n] + L.fin[(j * 16 + r) * kMaxT + t];
                }
              }, wait);
}

}  // namespace moel
