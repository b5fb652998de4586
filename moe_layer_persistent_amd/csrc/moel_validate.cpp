// Host-only argument validation and size queries of the C ABI (no HIP calls: these run
// and are tested on machines without a GPU).
#include <stdint.h>

#include "../../include/moel.h"

extern "C" {

const char* moel_status_string(int32_t s) {
  switch (s) {
    case MOEL_OK: return "ok";
    case MOEL_ERR_ARG: return "invalid argument";
    case MOEL_ERR_SHAPE: return "unsupported shape";
    case MOEL_ERR_ALIGN: return "misaligned pointer";
    case MOEL_ERR_HIP: return "HIP runtime error";
    case MOEL_ERR_TIMEOUT: return "device wait timed out";
    case MOEL_ERR_ABORTED: return "aborted";
    case MOEL_ERR_UNSUPPORTED: return "unsupported device";
    case MOEL_ERR_INTERNAL: return "device consistency check failed";
    default: return "unknown status";
  }
}

int32_t moel_abi_version(void) { return MOEL_ABI_VERSION; }

moel_status moel_validate_config(const moel_config* c) {
  if (c == nullptr) return MOEL_ERR_ARG;
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->pooled <= 0 ||
      c->inter <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->n_shards <= 0 || c->kv_capacity <= 0)
    return MOEL_ERR_ARG;
  if (!(c->rms_eps > 0.0f) || !(c->rope_theta > 0.0f)) return MOEL_ERR_ARG;
  if (c->shard_rank < 0 || c->shard_rank >= c->n_shards) return MOEL_ERR_ARG;
  if (c->expert_dtype != MOEL_EXPERT_NVFP4 && c->expert_dtype != MOEL_EXPERT_BF16) return MOEL_ERR_ARG;
  if (c->down_input != MOEL_DOWN_INPUT_EXACT && c->down_input != MOEL_DOWN_INPUT_NVFP4) return MOEL_ERR_ARG;
  if (c->down_input == MOEL_DOWN_INPUT_NVFP4 && c->expert_dtype != MOEL_EXPERT_NVFP4) return MOEL_ERR_SHAPE;
  if (c->top_k > c->n_experts || c->top_k > 8) return MOEL_ERR_SHAPE;
  if (c->hidden % 256 != 0) return MOEL_ERR_SHAPE;
  // bounds that keep the dense phases' row splits in 32-bit arithmetic
  if (c->hidden > 65536 || c->pooled > 65536 || c->inter > 131072 || c->n_q_heads * c->head_dim > 65536)
    return MOEL_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return MOEL_ERR_SHAPE;
  if (c->n_q_heads % c->n_kv_heads != 0 || c->n_q_heads / c->n_kv_heads > 8) return MOEL_ERR_SHAPE;
  if (c->n_experts % 16 != 0 || c->n_experts > 512) return MOEL_ERR_SHAPE;
  if (c->pooled % 128 != 0 || c->inter % 128 != 0) return MOEL_ERR_SHAPE;
  const int row_unit = c->expert_dtype == MOEL_EXPERT_NVFP4 ? 64 : 16;
  if (c->inter % (row_unit * c->n_shards) != 0 || c->pooled % (row_unit * c->n_shards) != 0)
    return MOEL_ERR_SHAPE;
  if ((int64_t)c->kv_capacity * c->head_dim > ((int64_t)1 << 31) / c->n_kv_heads) return MOEL_ERR_SHAPE;
  // the NVFP4 expert phases hand tiles out as (sequence << 16) | tile with 0xffff marking the
  // end of the work: every tile number of a step (active entries x 64-row tiles per expert;
  // an expert takes one entry per 16 of its slots, so at most min(2 E, 32 top_k) entries)
  // and every sequence number must fit 15 bits
  if (c->expert_dtype == MOEL_EXPERT_NVFP4) {
    const int64_t rows = (c->inter > c->pooled ? c->inter : c->pooled) / c->n_shards;
    const int64_t e2 = 2 * (int64_t)c->n_experts, slots = (int64_t)MOEL_MAX_TOKENS * c->top_k;
    const int64_t active = e2 < slots ? e2 : slots;
    if ((rows / 64) * active >= 0x7fff) return MOEL_ERR_SHAPE;
  }
  return MOEL_OK;
}

static bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

moel_status moel_validate_call(const moel_config* cfg, const moel_weights* w, const void* k_cache,
                               const void* v_cache, const float* x, int32_t T, int32_t pos, int32_t window,
                               const float* y) {
  moel_status st = moel_validate_config(cfg);
  if (st != MOEL_OK) return st;
  if (w == nullptr || k_cache == nullptr || v_cache == nullptr || x == nullptr || y == nullptr)
    return MOEL_ERR_ARG;
  if (T < 1 || T > MOEL_MAX_TOKENS) return MOEL_ERR_ARG;
  if (pos < 0 || window < 0) return MOEL_ERR_ARG;
  if ((int64_t)pos + T > cfg->kv_capacity) return MOEL_ERR_ARG;
  const void* ptrs[] = {w->gamma1, w->gamma2, w->w_qkv, w->w_o, w->w_router, w->w_pool, w->w_unpool,
                        w->w_gate, w->w_up, w->w_down};
  for (const void* p : ptrs) {
    if (p == nullptr) return MOEL_ERR_ARG;
    if (misaligned(p)) return MOEL_ERR_ALIGN;
  }
  if (cfg->expert_dtype == MOEL_EXPERT_NVFP4 && (w->ts_gate == nullptr || w->ts_up == nullptr || w->ts_down == nullptr))
    return MOEL_ERR_ARG;
  if (cfg->down_input == MOEL_DOWN_INPUT_NVFP4 && w->ts_act == nullptr) return MOEL_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(w->expert_hist) & 3u) != 0) return MOEL_ERR_ALIGN;
  if (misaligned(k_cache) || misaligned(v_cache) || misaligned(x) || misaligned(y)) return MOEL_ERR_ALIGN;
  const uintptr_t xb = reinterpret_cast<uintptr_t>(x), yb = reinterpret_cast<uintptr_t>(y);
  const uintptr_t n = (uintptr_t)T * (uintptr_t)cfg->hidden * 4u;
  if (xb < yb + n && yb < xb + n) return MOEL_ERR_ARG;  // y must not alias x
  return MOEL_OK;
}

size_t moel_packed_dense_bytes(int32_t N, int32_t K) {
  if (N <= 0 || K <= 0) return 0;
  return (size_t)N * (size_t)K * 2u;
}

size_t moel_packed_experts_bytes(const moel_config* cfg, int32_t which) {
  if (cfg == nullptr || which < 0 || which > 2 || cfg->n_shards <= 0) return 0;
  const size_t N = which < 2 ? (size_t)(cfg->inter / cfg->n_shards) : (size_t)(cfg->pooled / cfg->n_shards);
  const size_t K = which < 2 ? (size_t)cfg->pooled : (size_t)cfg->inter;
  const size_t E = (size_t)cfg->n_experts;
  if (cfg->expert_dtype == MOEL_EXPERT_BF16) return E * N * K * 2u;
  return E * N * (K / 2 + K / 16);
}

}  // extern "C"

moel_status moel_validate_tree(const int32_t* parents, int32_t T) {
  if (T < 1 || T > MOEL_MAX_TOKENS) return MOEL_ERR_ARG;
  if (parents == nullptr) return MOEL_OK;
  for (int32_t t = 0; t < T; ++t)
    if (parents[t] < -1 || parents[t] >= t) return MOEL_ERR_ARG;
  return MOEL_OK;
}

extern "C" moel_status moel_validate_batch(const moel_config* cfg, int32_t n_requests, const moel_request* requests,
                                           int32_t workgroups) {
  if (cfg == nullptr || requests == nullptr || n_requests < 1 || n_requests > MOEL_MAX_REQUESTS) return MOEL_ERR_ARG;
  int64_t total = 0;
  for (int32_t r = 0; r < n_requests; ++r) {
    const moel_request& q = requests[r];
    if (q.T < 1 || q.pos < 0 || q.kv_base < 0 || q.kv_slots < 1) return MOEL_ERR_ARG;
    if ((int64_t)q.pos + q.T > q.kv_slots) return MOEL_ERR_ARG;
    if ((int64_t)q.kv_base + q.kv_slots > cfg->kv_capacity) return MOEL_ERR_ARG;
    total += q.T;
    for (int32_t s = 0; s < r; ++s) {  // slot ranges pairwise disjoint
      const moel_request& o = requests[s];
      if (q.kv_base < (int64_t)o.kv_base + o.kv_slots && o.kv_base < (int64_t)q.kv_base + q.kv_slots)
        return MOEL_ERR_ARG;
    }
  }
  if (total > MOEL_MAX_TOKENS) return MOEL_ERR_ARG;
  const int64_t tiles = (total + 15) / 16;  // 16-token tiles: one attention item per request, kv head and tile
  if (workgroups > 0 && (int64_t)n_requests * cfg->n_kv_heads * tiles > workgroups) return MOEL_ERR_SHAPE;
  return MOEL_OK;
}
