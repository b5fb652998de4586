/*
 * moel.h -- C ABI of the MI355X (gfx950) MoE decoder-layer verify step.
 *
 * One call runs one decoder layer of a mixture-of-experts model for the batch-1
 * speculative-verify step: T draft tokens of one request (the pages verify 16; the library
 * takes up to MOEL_MAX_TOKENS = 32, as two 16-token tiles) go through
 *   RMSNorm -> QKV projection + rotate-half RoPE + KV-cache write -> GQA attention
 *   (sliding window or global) -> o-projection + residual -> RMSNorm -> top-k router
 *   and pooler -> SwiGLU experts (NVFP4 or bf16) -> weighted combine -> unpooler +
 *   residual
 * as a single persistent launch (orcarouter.ai English post, "Where the kernel boundary
 * sits": one launch per decoder layer covering attention, the dense GEMMs, the expert
 * GEMMs and the combine; "The draft model got faster too": 16 tokens verified in one
 * pass; aicoder.com news item, "Key Takeaways": batch 1 only).  The same computation is
 * also available as a chain of one kernel per step (moel_layer_decode_unfused), kept as
 * an ablation and as the fallback target.
 *
 * Conventions (all entry points):
 *   - Tensor pointers are DEVICE pointers (HIP global memory) owned by the caller unless
 *     stated otherwise.  The library keeps no reference to them after a call returns.
 *   - Every call validates its arguments on the host first.  On any error nothing is
 *     launched and no caller buffer is touched; the return code says why.
 *   - Launching calls are asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *   - Floating point: weights and the KV cache are bf16 (or NVFP4 for experts); the
 *     residual stream x / y is fp32.  No float atomics are used: results are bitwise
 *     reproducible for identical inputs.
 *   - No C++ exceptions cross this boundary.
 */
#ifndef MOEL_H
#define MOEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEL_MAX_TOKENS 32
#define MOEL_ABI_VERSION 7

typedef enum moel_status {
  MOEL_OK = 0,
  MOEL_ERR_ARG = -1,         /* null pointer, bad count, T/pos/window out of range      */
  MOEL_ERR_SHAPE = -2,       /* config shape the kernels do not support                 */
  MOEL_ERR_ALIGN = -3,       /* pointer not 16-byte aligned                             */
  MOEL_ERR_HIP = -4,         /* a HIP runtime call failed                               */
  MOEL_ERR_TIMEOUT = -5,     /* a device-side wait exceeded its bound (plan status)     */
  MOEL_ERR_ABORTED = -6,     /* the plan's abort word was set (plan status)             */
  MOEL_ERR_UNSUPPORTED = -7, /* no suitable device (not gfx950 / no cooperative launch) */
  MOEL_ERR_INTERNAL = -8     /* a device-side consistency check failed (plan status)     */
} moel_status;

typedef enum moel_expert_dtype {
  MOEL_EXPERT_NVFP4 = 0,     /* E2M1 codes, E4M3 scale per 16 elements, fp32 per matrix */
  MOEL_EXPERT_BF16 = 1
} moel_expert_dtype;

/* What the down projection reads (orcarouter.ai English post, "Where the kernel boundary
 * sits": with both expert GEMMs N-sharded, the SwiGLU output is all-gathered in fp4 between
 * them).  EXACT: the SwiGLU output as computed (fp32, carried as a bf16 pair).  NVFP4: that
 * output encoded in the experts' own NVFP4 format, the payload such a gather carries: per
 * 16 consecutive elements an E4M3 scale, the value nearest to amax / (6 ts), and E2M1
 * elements nearest to v / (scale ts), both ties to even and saturating (448, 6), decided
 * in fp32; ts = the expert's activation tensor scale (moel_weights.ts_act).  NVFP4 experts
 * only. */
typedef enum moel_down_input {
  MOEL_DOWN_INPUT_EXACT = 0,
  MOEL_DOWN_INPUT_NVFP4 = 1
} moel_down_input;

/* Shape of one layer.  Sharded configurations hold one GPU's share of the experts'
 * N dimension: gate/up keep inter/n_shards rows, down keeps pooled/n_shards rows (the
 * slice of rank shard_rank); the missing slices are zero, standing in for the cross-GPU
 * gathers (orcarouter.ai English post, "Where the kernel boundary sits": both MoE GEMMs
 * sharded on N).  Head counts are the GPU's own (e.g. 8 q / 1 kv for a TP8 share). */
typedef struct moel_config {
  int32_t hidden;         /* H; multiple of 256                                          */
  int32_t n_q_heads;      /* Hq; multiple of n_kv_heads                                  */
  int32_t n_kv_heads;     /* Hkv                                                         */
  int32_t head_dim;       /* D; 64 or 128                                                */
  int32_t pooled;         /* P; multiple of 128 (and of 64 * n_shards)                   */
  int32_t inter;          /* I (SwiGLU width, K of the down projection); multiple of 128 */
  int32_t n_experts;      /* E; multiple of 16, <= 512                                   */
  int32_t top_k;          /* k; 1..8, <= E                                               */
  int32_t expert_dtype;   /* moel_expert_dtype                                           */
  int32_t n_shards;       /* 1 = whole layer                                             */
  int32_t shard_rank;     /* 0 <= shard_rank < n_shards                                  */
  int32_t kv_capacity;    /* slots per kv head in the caller's cache                     */
  float rms_eps;          /* RMSNorm epsilon                                             */
  float rope_theta;       /* RoPE base                                                   */
  int32_t down_input;     /* moel_down_input                                             */
} moel_config;

/* Layer weights in the kernels' packed layouts (see the moel_pack_* calls).  All device
 * pointers, 16-byte aligned, caller-owned. */
typedef struct moel_weights {
  const void* gamma1;     /* bf16 [H]            attention RMSNorm gain                  */
  const void* gamma2;     /* bf16 [H]            MoE RMSNorm gain                        */
  const void* w_qkv;      /* packed dense, QKV   [(Hq+2Hkv)*D, H] (pack with rope heads) */
  const void* w_o;        /* packed dense        [H, Hq*D]                               */
  const void* w_router;   /* packed dense        [E, H]                                  */
  const void* w_pool;     /* packed dense        [P, H]                                  */
  const void* w_unpool;   /* packed dense        [H, P]                                  */
  const void* w_gate;     /* packed experts      [E][inter/n_shards, P]                  */
  const void* w_up;       /* packed experts      [E][inter/n_shards, P]                  */
  const void* w_down;     /* packed experts      [E][pooled/n_shards, I]                 */
  const float* ts_gate;   /* fp32 [E] tensor scales (NVFP4 only, else NULL)              */
  const float* ts_up;
  const float* ts_down;
  const float* ts_act;    /* fp32 [E] activation tensor scales, > 0 (down_input NVFP4,
                           * else ignored)                                              */
  uint32_t* expert_hist;  /* uint32 [E] this layer's routing history, caller-owned device
                           * memory, 4-byte aligned (NULL: none).  Every step of the layer
                           * writes, per expert, how many of its tokens chose it; with the
                           * plan's expert prefetch on (moel_plan_set_expert_prefetch) a step
                           * first reads what the previous step wrote.  Zero it before the
                           * layer's first step.  Steps of one layer on different streams
                           * race on it.                                                  */
} moel_weights;

/* Optional outputs for tests and profiling; any member may be NULL. */
typedef struct moel_debug {
  int32_t* expert_idx;    /* [T, k] selected experts, selection order                    */
  float* gates;           /* [T, k] softmax over the selected logits                     */
  float* router_logits;   /* [T, E] fp32                                                 */
  uint64_t* timestamps;   /* [n_workgroups, MOEL_N_STAMPS] s_memrealtime ticks (100 MHz):
                           * slot i < 10 end of step i, slot 10 entry, slot 16 + i start of
                           * step i (after the grid barrier that precedes it)          */
} moel_debug;

#define MOEL_N_STAMPS 32

typedef struct moel_plan moel_plan;

/* --- host-only helpers (no GPU needed) ------------------------------------------- */

const char* moel_status_string(int32_t status);
int32_t moel_abi_version(void);

/* Checks that `cfg` is a shape the kernels support.  Pure host code. */
moel_status moel_validate_config(const moel_config* cfg);

/* Checks the per-call arguments of moel_layer_decode against `cfg`: 1 <= T <= MOEL_MAX_TOKENS,
 * pos >= 0, pos + T <= kv_capacity, window >= 0, non-NULL 16-byte-aligned pointers,
 * y not aliasing x.  Pure host code (pointers are only compared, never dereferenced). */
moel_status moel_validate_call(const moel_config* cfg, const moel_weights* w,
                               const void* k_cache, const void* v_cache, const float* x,
                               int32_t T, int32_t pos, int32_t window, const float* y);

/* Bytes of the packed layouts: exactly the canonical bytes of the same matrices (bf16
 * elements; for NVFP4 the codes plus the E4M3 block scales), with no padding. */
size_t moel_packed_dense_bytes(int32_t N, int32_t K);
size_t moel_packed_experts_bytes(const moel_config* cfg, int32_t which /*0 gate,1 up,2 down*/);

/* --- plan ------------------------------------------------------------------------- */

/* Validates cfg, selects the current HIP device, allocates the plan's workspace once
 * (activation scratch, barrier words, status word, RoPE cos/sin table computed on the
 * host in fp64 and stored fp32) and chooses the work decomposition.  *out is set only
 * on success.  Not for the hot path.
 *
 * Environment variables (for diagnostics and for measuring alternatives; none changes a
 * result beyond the summation order of a split contraction):
 *   MOEL_LOG            set: one line per plan (shape, workgroups, workspace and LDS bytes,
 *                       the L2 coherence check, the dense K-splits) and every HIP error on
 *                       stderr.
 *   MOEL_DENSE_SPLITS   "q,o,r,u" or one number for all: the K-split of the QKV,
 *                       o-projection, router/pooler and unpooler contractions, read when a
 *                       plan is created; a value is used where it is a power of two <= 16
 *                       that divides the phase's 32-element k steps, 0 keeps the plan's choice.
 *   MOEL_ATTN_SET_MERGE 0: the attention merge always runs as a phase of its own after a
 *                       grid barrier (otherwise each attention group merges on its own
 *                       barrier group where it fits); read once per process. */
moel_status moel_plan_create(const moel_config* cfg, moel_plan** out);
moel_status moel_plan_destroy(moel_plan* plan);

/* Number of workgroups of the persistent launch (one per compute unit). */
int32_t moel_plan_workgroups(const moel_plan* plan);

/* Reads the device-side status word (blocks until `plan`'s work on the device is done):
 * MOEL_OK, MOEL_ERR_TIMEOUT, MOEL_ERR_ABORTED or MOEL_ERR_INTERNAL.  A non-OK status is cleared (and the
 * plan's barrier words reset) by this call. */
moel_status moel_plan_status(moel_plan* plan);

/* How moel_layer_decode launches the persistent kernel (plan default: plain).
 *   MOEL_LAUNCH_PLAIN: an ordinary launch of one workgroup per compute unit.  Its grid
 *     barriers need every workgroup resident at once; moel_plan_create checks that one
 *     workgroup fits per compute unit, so on a device running nothing else they all are.
 *     Kernels of other streams holding compute units delay the barriers until they end; a
 *     barrier that waits ~0.5 s ends with MOEL_ERR_TIMEOUT (plan status) instead of hanging.
 *     Consecutive calls on one stream are serialised by the stream.
 *   MOEL_LAUNCH_COOPERATIVE: a cooperative launch, which guarantees residency on a shared
 *     device; the runtime leaves a gap of ~20 us between consecutive such launches.
 * Returns MOEL_ERR_ARG for another mode. */
typedef enum { MOEL_LAUNCH_PLAIN = 0, MOEL_LAUNCH_COOPERATIVE = 1 } moel_launch_mode;
moel_status moel_plan_set_launch(moel_plan* plan, int32_t mode);

/* Acquire side of the persistent launch's grid barriers.  Not a step of the layer: a
 * property of how the workgroups of one launch see each other's stores.
 *   MOEL_ACQUIRE_AUTO (default): when the plan's device keeps a clean copy in one XCD's L2
 *     coherent with a later write from another XCD for hipMalloc memory (checked once per
 *     device and process when a plan is created, see moel_plan_l2_coherent), a barrier
 *     invalidates only the L1 caches; otherwise it runs the memory model's agent-scope
 *     acquire, which also invalidates the L2 and with it the code and weights held there.
 *     Within one layer every line read across XCDs is written once, which is what the L1-only
 *     acquire relies on (a line that an XCD itself wrote earlier in the launch is not kept
 *     coherent); between the layers of a stack launch every XCD drops its L2's clean lines.
 *   MOEL_ACQUIRE_L2_INVALIDATE: always the agent-scope acquire.
 * Results are bitwise identical in both modes.  Returns MOEL_ERR_ARG for another mode. */
typedef enum { MOEL_ACQUIRE_AUTO = 0, MOEL_ACQUIRE_L2_INVALIDATE = 1 } moel_acquire_mode;
moel_status moel_plan_set_acquire(moel_plan* plan, int32_t mode);

/* 1 if the coherence check passed on the plan's device (a workgroup's stores, written back by
 * a release fence, were seen by readers on every XCD after an L1-only invalidation, with no
 * stale word in four trials), 0 if not, -1 for a null plan. */
int32_t moel_plan_l2_coherent(const moel_plan* plan);

/* Previous-step expert prefetch (orcarouter.ai English post, "Three bills a kernel this big has
 * to pay": while the layer runs, one warp reads which experts the previous step routed to and
 * pulls this GPU's slices of the most-used ones into the last-level cache, betting that
 * consecutive steps route alike).  n_experts = 0 (default) turns it off; 1..16 enables it for
 * layers whose moel_weights.expert_hist is set: the step reads the history, takes the
 * n_experts experts that most of the previous step's tokens chose (ties to the lower index;
 * experts no token chose are left out), and the workgroups that have no attention work read
 * those experts' packed gate, up and down weights once with ordinary loads while attention
 * runs, so that the memory-side cache holds them when the expert phases stream them.  It
 * changes no result (bitwise).  Persistent launches only (moel_layer_decode, the tree and batch
 * variants, moel_stack_decode); the one-kernel-per-step chain still writes the history but
 * does not prefetch.  Returns MOEL_ERR_ARG for a null plan or n_experts outside 0..16. */
moel_status moel_plan_set_expert_prefetch(moel_plan* plan, int32_t n_experts);

/* Fills the plan's activation scratch (every intermediate buffer of a step; not its control
 * words or RoPE table) with all-ones words, a NaN in fp32 and in bf16, on `stream`.  For
 * tests: a step that reads a scratch word before the phase that produces it has written it
 * then carries a NaN into its outputs, where a step on unpoisoned scratch would silently reuse
 * an earlier step's value.  A step after it runs as usual (it writes everything it reads). */
moel_status moel_plan_poison_scratch(moel_plan* plan, void* stream);

/* Sets (1) or clears (0) the plan's abort word.  While set, launched kernels skip all
 * work, leave every caller buffer untouched and report MOEL_ERR_ABORTED. */
moel_status moel_plan_set_abort(moel_plan* plan, int32_t abort_flag, void* stream);

/* Intermediate activations of the last completed step, for tests and profiling tools
 * (all fp32, row-major, rows = tokens or token slots):
 * (R = MOEL_MAX_TOKENS rows; the step's T come first)
 *   0 q [R][Hq*D] after RoPE       1 o [R][Hq*D] attention output    2 h [R][H]
 *   3 router logits [R][E]         4 pl [R][P] pooled vector         5 a [R*k][I] SwiGLU out
 *   6 d [R*k][P] expert outputs    7 m [R][P] combined vector
 *   8 aq [R*k][I] with down_input NVFP4: the down projection's input as E2M1 value times
 *     E4M3 block scale (its tensor scale multiplies the projection's sums)
 * *ptr receives a device pointer into the plan's workspace (owned by the plan; valid until
 * moel_plan_destroy; overwritten by the next step), *bytes its size.  o, m, pl, a and aq
 * are fp32 copies the step itself does not read (the experts read pl and a as split bf16
 * operand words): a step writes them only when its moel_debug asks for routing outputs
 * (expert_idx, gates or router_logits; they hold the last such step's values). */
moel_status moel_plan_scratch(const moel_plan* plan, int32_t which, void** ptr, size_t* bytes);

/* --- weight packing (one-time, not on the hot path) --------------------------------- */

/* Dense bf16 matrix [N, K] row-major -> packed layout (16-row tiles, 32-element k steps,
 * one 1 KiB block per (tile, step); in a block, lane l's 16 bytes hold row l % 16 at
 * k = 4q + 0..3 and 16 + 4q + 0..3 of the step, q = l / 16).  rope_head_dim > 0 interleaves the rows of every
 * rope_head_dim-row head pairwise (i, i + D/2) so that rotation partners are adjacent;
 * pass head_dim for w_qkv and 0 otherwise.  N % 16 == 0, K % 32 == 0. */
moel_status moel_pack_dense(const void* src, int32_t N, int32_t K, int32_t rope_head_dim,
                            void* dst, void* stream);

/* Experts of one matrix kind (0 gate, 1 up, 2 down) -> packed layout.
 *   NVFP4: codes uint8 [E, N, K/2] (even k in the low nibble) and scales uint8 E4M3
 *          [E, N, K/16] -> 64-row tiles; per tile K/64 pairs of 2304 bytes: two 1 KiB code
 *          steps (lane l: the 32 codes of row l for one 32-element k step, even k in the low
 *          nibble), then 256 bytes of scales (lane l: row l's 4 block scales of the pair's
 *          64 k).  K % 128 == 0.
 *   bf16:  src [E, N, K] (scales NULL) -> the dense layout per expert. */
moel_status moel_pack_experts(const moel_config* cfg, int32_t which, const void* src,
                              const void* scales, void* dst, void* stream);

/* --- the layer step -------------------------------------------------------------- */

/* One verify step of one layer, as ONE persistent launch (see moel_plan_set_launch).
 *   k_cache, v_cache: bf16 [Hkv, kv_capacity, D]; slots [pos, pos+T) of every kv head
 *                     are overwritten with the new (rotated, rounded) keys / values;
 *                     every other byte is left untouched.
 *   x: fp32 [T, H] input residual stream;  y: fp32 [T, H] output (must not alias x).
 *   pos: tokens already in the cache (token t sits at position pos + t).
 *   window: 0 = global attention; W > 0: token at position p sees keys j with
 *           p - W < j <= p.
 *   dbg: optional outputs (NULL = none). */
moel_status moel_layer_decode(moel_plan* plan, const moel_weights* w, void* k_cache,
                              void* v_cache, const float* x, int32_t T, int32_t pos,
                              int32_t window, float* y, const moel_debug* dbg, void* stream);

/* Same arguments and results, as a chain of one kernel per step. */
moel_status moel_layer_decode_unfused(moel_plan* plan, const moel_weights* w, void* k_cache,
                                      void* v_cache, const float* x, int32_t T, int32_t pos,
                                      int32_t window, float* y, const moel_debug* dbg,
                                      void* stream);

/* --- token-tree verify -------------------------------------------------------------- */

/* Checks a token tree of T nodes given by parent indices: parents[t] in [-1, t) for every
 * t < T (-1: a root, attached to the cached prefix).  `parents` is a HOST array; a NULL
 * array is the chain.  Pure host code. */
moel_status moel_validate_tree(const int32_t* parents, int32_t T);

/* The verify step over a tree of candidate tokens instead of a chain (orcarouter.ai English
 * post, "The draft model got faster too": the verify pass checks a tree of draft tokens;
 * the pages give neither its mask nor its positions, so the plainest reading is taken).
 * Token t is the tree node with parent parents[t] (HOST array of T entries, checked by
 * moel_validate_tree): it sits at position pos + depth(t) (RoPE), its key and value are
 * written to cache slot pos + t (exactly slots [pos, pos+T) are written, as for the chain),
 * and it attends to the cached keys j < pos with p - W < j (p its position, W = window, no
 * limit for W == 0) and to the step's tokens that are itself or its ancestors (the same rule
 * on their positions).  Everything after attention is per token, as for the chain.  The
 * chain parents[t] = t - 1 gives exactly moel_layer_decode's results; parents == NULL is
 * the chain.  Other arguments, results and errors as moel_layer_decode. */
moel_status moel_layer_decode_tree(moel_plan* plan, const moel_weights* w, void* k_cache,
                                   void* v_cache, const float* x, int32_t T, int32_t pos,
                                   int32_t window, const int32_t* parents, float* y,
                                   const moel_debug* dbg, void* stream);

/* Same arguments and results, as a chain of one kernel per step. */
moel_status moel_layer_decode_tree_unfused(moel_plan* plan, const moel_weights* w, void* k_cache,
                                           void* v_cache, const float* x, int32_t T, int32_t pos,
                                           int32_t window, const int32_t* parents, float* y,
                                           const moel_debug* dbg, void* stream);

/* --- several requests in one step (batch > 1) ---------------------------------------------- */

#define MOEL_MAX_REQUESTS 8

/* One request of a batched verify step (aicoder.com news item, "Key Takeaways", and orcarouter.ai
 * English post, "What this number is, and what it is not": the measured path is batch 1, larger
 * batches are the next step).  Its T tokens are consecutive rows of the step's x and y, the
 * requests in order.  Its KV cache is slots [kv_base, kv_base + kv_slots) of every kv head of a
 * pool shared by the batch (a [Hkv, kv_capacity, D] bf16 pair, kv_capacity the plan's); the
 * request's slot i holds its position i. */
typedef struct moel_request {
  int32_t T;         /* >= 1 tokens (a chain: token i attends to the request's tokens 0..i)   */
  int32_t pos;       /* >= 0 positions already in the request's cache; pos + T <= kv_slots     */
  int32_t kv_base;   /* >= 0 first pool slot of the request; kv_base + kv_slots <= kv_capacity  */
  int32_t kv_slots;  /* slots of the request's cache                                            */
} moel_request;

/* Checks a batch on the host: 1 <= n_requests <= MOEL_MAX_REQUESTS, every request as described
 * above, the requests' slot ranges pairwise disjoint, the sum of T at most MOEL_MAX_TOKENS, and
 * n_requests * n_kv_heads * (16-token tiles of the step) attention items no more than the
 * workgroups (workgroups = 0 skips that check).  MOEL_ERR_ARG on any violation (MOEL_ERR_SHAPE
 * for the last one). */
moel_status moel_validate_batch(const moel_config* cfg, int32_t n_requests, const moel_request* requests,
                                int32_t workgroups);

/* One verify step for n_requests requests at once: every request's tokens go through the layer
 * together (the weights are read once for all of them); attention reads each request's own
 * cache and writes its new keys and values at pool slots kv_base + pos + i.  Every row's result
 * is that of moel_layer_decode for its request alone, up to the rounding order of attention
 * (the key chunks are sized for the whole batch).  window: the layer's, for every request.
 * k_pool, v_pool: the shared caches; x, y: fp32 [sum of T, hidden] (y must not alias x).
 * dbg: as for moel_layer_decode, over the step's rows.  Errors: as moel_layer_decode and
 * moel_validate_batch; nothing is launched and no buffer touched on error. */
moel_status moel_layer_decode_batch(moel_plan* plan, const moel_weights* w, void* k_pool, void* v_pool,
                                    const float* x, int32_t n_requests, const moel_request* requests,
                                    int32_t window, float* y, const moel_debug* dbg, void* stream);
moel_status moel_layer_decode_batch_unfused(moel_plan* plan, const moel_weights* w, void* k_pool,
                                            void* v_pool, const float* x, int32_t n_requests,
                                            const moel_request* requests, int32_t window, float* y,
                                            const moel_debug* dbg, void* stream);

/* --- a stack of layers in one launch ------------------------------------------------ */

#define MOEL_MAX_STACK_LAYERS 256
#define MOEL_STACK_LAYERS_PER_LAUNCH 4

typedef struct moel_stack moel_stack;

/* Registers n_layers layers of the plan's shape to be run one after another with persistent
 * launches that each cover up to MOEL_STACK_LAYERS_PER_LAUNCH layers (moel_stack_decode): layer
 * l + 1 takes layer l's output rows as its input, with a grid barrier instead of a launch boundary
 * between the layers of one launch (orcarouter.ai English post, "Where the kernel boundary sits": the pages move
 * the launch boundary off the layer boundary; "What the 5.9 ms is still spent on": a launch per
 * layer is a fixed cost).  Nothing of one layer overlaps the next: at each layer boundary every
 * XCD drops its L2's clean lines, as a launch boundary does.  The layers' launch parameters
 * travel as kernel arguments, MOEL_STACK_LAYERS_PER_LAUNCH layers' worth per launch.
 *   weights[l], k_caches[l], v_caches[l], windows[l]: layer l as for moel_layer_decode (HOST
 *     arrays of n_layers entries, copied; the device buffers they point to stay caller-owned and
 *     must outlive the stack).
 * Allocates two [MOEL_MAX_TOKENS, hidden] fp32 device buffers for the rows between layers.  *out is set only
 * on success.  Not for the hot path.  The stack uses the plan's workspace: steps of a plan's
 * stack and of the plan itself must not overlap (they are ordered when issued on one stream). */
moel_status moel_stack_create(moel_plan* plan, int32_t n_layers, const moel_weights* weights,
                              void* const* k_caches, void* const* v_caches, const int32_t* windows,
                              moel_stack** out);

/* One verify step through every layer of the stack: x fp32 [T, hidden] into the first layer, y
 * fp32 [T, hidden] out of the last (must not alias x), every layer's KV cache written at slots
 * [pos, pos+T) as by moel_layer_decode.  Results are bitwise those of moel_layer_decode called
 * layer by layer.  Every layer's arguments are validated on the host before anything is issued;
 * device status through moel_plan_status.  Asynchronous on `stream`. */
moel_status moel_stack_decode(moel_stack* stack, const float* x, int32_t T, int32_t pos, float* y,
                              void* stream);

moel_status moel_stack_destroy(moel_stack* stack);

/* --- allocation-free step -------------------------------------------------------- */

/* Bytes of device memory the allocation-free step uses on each GPU it runs on (held until the
 * process ends). */
#define MOEL_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moel_layer_decode without a plan.  Nothing is
 * allocated, by this call or by the library on its behalf.  The step's workspace (control
 * words, activation scratch, the RoPE rows of positions pos .. pos+T-1) lives in a device array
 * of MOEL_NOALLOC_SCRATCH_BYTES owned by the library, one per GPU; the size a shape needs is
 *   ~ 4 KiB + 4 B * (32 * (3 Hq D + 2 H + E + 4 P + 3 k I + k P + D) + CUs * (Hq/Hkv) * 32 * (D + 2))
 * (about 59 MiB for H 8192, 64/8 heads of 128, P = I = 4096, E 256, k 8 on 256 compute units),
 * and a shape that needs more is rejected with MOEL_ERR_SHAPE before anything is launched.
 * The first call on a device sets that device up (synchronously, on `stream`): it looks the
 * array up, runs the L2 coherence check on it (unless a plan already did on that device) and
 * clears its control words.
 *   cfg: the layer's shape, as for moel_plan_create (any config it accepts within the size).
 *   w, k_cache, v_cache, x, T, pos, window, y: as for moel_layer_decode (the chain verify).
 *   status: optional caller-owned DEVICE word (4-byte aligned; NULL = not reported) that the
 *     launch sets to 0 or, after a device-side wait timed out or a consistency check failed, to
 *     a nonzero code.  No abort word exists for this call.
 * Results are those of moel_layer_decode (same kernels; RoPE rows computed on the device in
 * double precision, as the plan computes its table on the host).  All calls on one GPU share
 * its array and each call leaves its contents behind: calls that overlap on one GPU (on
 * different streams) race and must not be issued; calls in one stream are ordered.  Errors:
 * as moel_layer_decode, plus MOEL_ERR_SHAPE for a workspace beyond the array and
 * MOEL_ERR_ALIGN for a misaligned status word. */
moel_status moel_layer_decode_noalloc(const moel_config* cfg, const moel_weights* w, void* k_cache,
                                      void* v_cache, const float* x, int32_t T, int32_t pos,
                                      int32_t window, float* y, uint32_t* status, void* stream);

/* --- measurement reference ---------------------------------------------------------- */

/* Streaming-read bandwidth of the device, the practical reference beside the nominal HBM peak
 * for the layer's roofline fraction (not a step of the layer).  One 512-thread workgroup per CU
 * reads an equal share of buf[0, bytes) in 16-byte non-temporal loads, four per thread in
 * flight, reps times back to back on `stream` after one untimed pass; *gbps receives
 * (bytes read per pass) * reps / elapsed, timed with HIP events.  The share of each workgroup
 * is bytes / (16 * n_CU) 16-byte words, rounded down; the bytes beyond are not read.
 *   buf: DEVICE pointer, caller-owned, 16-byte aligned; bytes >= 16 * 512 * n_CU.
 *   reps: 1 .. 1000.  gbps: HOST pointer.
 * Waits for `stream`.  Errors: MOEL_ERR_ARG (null pointers, reps out of range, too few bytes),
 * MOEL_ERR_ALIGN, MOEL_ERR_HIP. */
moel_status moel_measure_read_bandwidth(const void* buf, size_t bytes, int32_t reps, float* gbps,
                                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEL_H */
