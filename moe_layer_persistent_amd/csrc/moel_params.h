// Kernel argument block shared by the host launcher and the device phases.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "moel.h"  // MOEL_MAX_TOKENS, MOEL_MAX_REQUESTS

#define MOEL_N_STAMPS_DEV 32
#define MOEL_DEV_TIMEOUT 1u
#define MOEL_DEV_ABORTED 2u
#define MOEL_DEV_ORDER 3u    /* a workgroup-internal hand-out was read before it was published */

namespace moel {

// Phase ids: index of the timestamp slot written at the end of each phase, and of the
// unfused chain's kernels.
enum Phase {
  kPhNorm1 = 0,     // RMSNorm 1: no work of its own (the QKV pass computes rstd)
  kPhQkv = 1,       // RMSNorm 1 + QKV projection + RoPE + q store + KV-cache write
  kPhAttn = 2,      // attention partials per (kv head, key chunk)
  kPhAttnMerge = 3, // merge of the key-chunk partials -> o (bf16)
  kPhOproj = 4,     // o-projection + residual -> h
  kPhRouterPool = 5,// RMSNorm 2 + router logits and pooler
  kPhGemm1 = 6,     // routing tables + expert gate/up + SwiGLU -> a (bf16)
  kPhGemm2 = 7,     // expert down projection -> d (fp32)
  kPhCombine = 8,   // gate-weighted combine over a token's slots -> m (bf16)
  kPhUnpool = 9,    // unpooler + residual -> y
  kNumPhases = 10
};

struct LayerParams {
  // shape
  int H, Hq, Hkv, D, P, I, E, topk;
  int n_shards, rank, I_loc, P_loc, kv_cap, expert_dtype;
  // 1: the down projection reads the SwiGLU output encoded as NVFP4 (the fp4 gather)
  int down_fp4;
  float eps;
  // call: T tokens in ntt = ceil(T / 16) token tiles of 16
  int T, ntt, pos, window;
  int nwg;
  // 1: the XCDs' L2 caches are kept coherent for the plan's memory (checked when the plan is
  // created), so a barrier's acquire invalidates only the L1; 0: it also invalidates the L2
  int l2_coherent;
  // 1 when the call passes debug outputs: also write the fp32 copies of o, m, pl, a and aq
  // that the step itself does not read (plan scratch export)
  int debug_copies;
  // split-K of the dense phases (1 = none): QKV, o-projection, router/pooler, unpooler
  int sk_qkv, sk_oproj, sk_rp, sk_unpool;
  // the step's requests (one for moel_layer_decode): request r owns tokens req_t0[r] ..
  // req_t0[r+1]-1 (req_t0[n_req] = T), has req_pos[r] positions cached at pool slots
  // req_kvb[r] + 0 .. req_pos[r] - 1, and attends to its keys req_lo[r] .. req_pos[r] + T_r - 1
  int n_req;
  int req_t0[MOEL_MAX_REQUESTS + 1];
  int req_pos[MOEL_MAX_REQUESTS];
  int req_kvb[MOEL_MAX_REQUESTS];
  int req_lo[MOEL_MAX_REQUESTS];
  // attention decomposition (per call): chunks of attn_chunk keys, request r's being the flat
  // chunks req_ch0[r] .. req_ch0[r+1]-1 (attn_nchunks = req_ch0[n_req] in all)
  int attn_chunk, attn_nchunks;
  int req_ch0[MOEL_MAX_REQUESTS + 1];
  // 1: the persistent launch merges the key-chunk partials without a grid barrier in between:
  // group q = (kv head q mod Hkv, token tile q / Hkv) has its attn_nchunks items and its merge
  // on the workgroups of barrier group q (q < 8, at most nwg / 8 items each); its items count
  // in on a control word and its merging workgroups wait for that count
  int attn_set_merge;
  // the step's tokens as the nodes of token trees (a chain per request for the linear verify):
  // token t of request r (req_t0[r] <= t < req_t0[r+1]) is at position tok_pos[t] (RoPE) and
  // writes its key and value at pool slot req_kvb[r] + req_pos[r] + t - req_t0[r]; bit i of
  // tok_sees[t] is set iff t attends to token i's key: i is t or an ancestor of t in the same
  // request and within the window of t
  int tok_pos[MOEL_MAX_TOKENS];
  unsigned tok_sees[MOEL_MAX_TOKENS];
  // weights (packed)
  const uint16_t* gamma1;
  const uint16_t* gamma2;
  const uint8_t* w_qkv;
  const uint8_t* w_o;
  const uint8_t* w_router;
  const uint8_t* w_pool;
  const uint8_t* w_unpool;
  const uint8_t* w_gate;
  const uint8_t* w_up;
  const uint8_t* w_down;
  const float* ts_gate;
  const float* ts_up;
  const float* ts_down;
  const float* ts_act;  // [E] activation tensor scales of the fp4 gather
  // the layer's routing history: [E] tokens per expert of the last step (NULL: none); with
  // pf_n > 0 the step first prefetches the pf_n experts that the last step used most
  unsigned* expert_hist;
  int pf_n;
  size_t stride_gate, stride_up, stride_down;  // packed bytes per expert
  // caches and io
  uint16_t* k_cache;
  uint16_t* v_cache;
  const float* x;
  float* y;
  const float* rope_cos;  // [rows][D/2], row r holds position rope_row0 + r
  const float* rope_sin;
  int rope_row0;
  // scratch (plan workspace)
  float* q_buf;     // [32][Hq*D]
  // q again as the attention's MFMA operand: per (token, head), q * log2(e) / sqrt(D) as the
  // nearest bf16 values [D], then the bf16 of the remainders [D]
  uint16_t* q_op;   // [32][Hq][2][D]
  float* attn_o;    // [items][grp][32][D]
  float* attn_ml;   // [items][grp][32][2]
  float* o_buf;     // [32][Hq*D]
  float* h_buf;     // [32][H]
  float* logits;    // [32][E]
  float* pl;        // [32][P]
  float* a_buf;     // [32*topk][I]
  // pl and a_buf again as the hi/lo bf16 operands of the NVFP4 expert MFMAs: per 4-element
  // quad, 4 bf16 of the nearest values then 4 bf16 of the remainders (16 bytes)
  uint16_t* pl_split;  // [32][P/4][8]
  uint16_t* a_split;   // [32*topk][I/4][8]
  float* aq_buf;    // [32*topk][I] fp4-gathered SwiGLU output (E2M1 x E4M3), debug copy
  float* d_buf;     // [32*topk][P]
  float* m_buf;     // [32][P]
  // o and m again as the ready-made A operands of the dense contractions that read them (see
  // opsplit_index): per 32-element k step and 16-token tile one 2 KiB block, lane l's 8 nearest
  // bf16 values at byte 16 l and the 8 bf16 of their remainders at 1024 + 16 l; h (read with
  // gamma 2 and its sums of squares) as fp32 in the same operand order (op_index): lane l's 8
  // values at 16 l and 1024 + 16 l
  uint16_t* o_op;
  float* h_op;
  uint16_t* m_op;
  // split-K partial sums of a dense phase: [split][row][32 tokens], and each unit's sums of
  // squares of its A rows (sources with stats): [unit][32 tokens]
  float* part;
  float* part_ss;
  unsigned* ctrl;   // barrier counter, exit counter, status, abort
  // when set, the last workgroup to leave the persistent launch moves the device status here
  // (0 = ok) and clears it in the control block
  unsigned* status_out;
  // debug (optional)
  int* dbg_idx;
  float* dbg_gates;
  float* dbg_logits;
  unsigned long long* dbg_ts;
};

// The launch parameters as seen by device code: a reference into the kernel-argument segment
// (constant address space), so every field read is a scalar load through the constant cache.
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
typedef const __attribute__((address_space(4))) LayerParams KP;
#endif

}  // namespace moel
