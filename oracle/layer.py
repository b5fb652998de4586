"""Vectorised fp64 oracle of one MoE decoder layer's batch-1 speculative-verify step.

Test infrastructure only (see the package docstring).

What the step computes (orcarouter.ai English post, "Where the kernel boundary
sits" and "The draft model got faster too"; aicoder.com news item, "Key
Takeaways"): one decoder layer of a mixture-of-experts model verifying T <= 16
draft tokens of one request in a single pass.  The launch covers the QKV
projection and the KV-cache write, attention (sliding window over the last
2,048 tokens, or global), the dense GEMMs, routing of each token to 8 of 256
experts, a down-projection of every token to a narrower width ahead of the
experts (the pooler), the expert GEMMs and a projection back to the model width
after them (the unpooler).

Where the pages are silent the plainest reading is taken (each one is listed
with its rationale in the design notes):
  * pre-norm block: h = x + Attn(RMSNorm1(x)); y = h + MoE(RMSNorm2(h)); no biases
  * RMSNorm: v * (mean(v^2) + eps)^-1/2 * gamma
  * RoPE, rotate-half pairing (i, i + D/2), theta = 10000, position pos + t,
    on q and k of every layer
  * key j visible to the token at position p iff j <= p and (W == 0 or j > p - W)
  * token-tree verify (the verify pass checks a tree of candidate tokens rather than
    a chain; the pages give neither its mask nor its positions): node t with parent
    p(t) (-1: a root, attached to the cached prefix) sits at position pos + depth(t),
    its key and value are written to cache slot pos + t, and it sees the cached keys
    by the window rule at its own position and, among the step's nodes, exactly its
    ancestors and itself (by the same rule on their positions).  The chain
    p(t) = t - 1 is the linear verify above.
  * GQA: q head h reads kv head floor(h * Hkv / Hq); score scale 1/sqrt(D)
  * router on the normalised hidden state (the pooler's input): top-k by logit
    descending with ties to the lower expert index, gates = softmax over the k
    selected logits, in selection order
  * SwiGLU expert: a = silu(x Wg^T) * (x Wu^T); d = a Wd^T
  * combine: m_t = sum over the token's k slots, in selection order, of gate * d
  * expert N-sharding (one GPU's share): gate/up keep rows
    [rank*I/S, (rank+1)*I/S) of the intermediate width, the SwiGLU output is
    zero outside that slice; down keeps rows [rank*P/S, ...) of the pooled
    width and its output is zero elsewhere (zero padding stands in for the
    cross-GPU gathers).
  * fp4 gather of the SwiGLU output (optional; the pages gather it in fp4 after the first
    expert GEMM and fix no encoding): a is encoded in the weights' own NVFP4 format, E2M1
    elements with an E4M3 scale per 16 consecutive elements and a static fp32 tensor scale
    per expert, each scale and code the nearest value (ties to even, saturating), decided in
    fp32; the down projection reads the decoded values.
Precision: the layer in exact (fp64) arithmetic on its given inputs.  Weights
are bf16 or NVFP4 and the KV cache is bf16: those are storage formats, so the
new keys and values are rounded to bf16 (nearest even) when written to the
cache and attention reads them from the cache.  No activation is rounded.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, Optional, Tuple

import numpy as np

from .formats import bf16_round, nvfp4_dequant, nvfp4_quantize, nvfp4_values


@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    pooled: int
    inter: int
    n_experts: int
    top_k: int
    n_shards: int = 1
    shard_rank: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0


# --------------------------------------------------------------------------------------------
# the steps, one function each
# --------------------------------------------------------------------------------------------
def rmsnorm(v: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row, before rounding: v * (mean(v^2) + eps)^-1/2 * gamma."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * gamma[None, :]


def rope(vec: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE: vec [T, nh, D], positions [T] -> rotated [T, nh, D].

    Pair (i, i + D/2) is rotated by angle position * theta^(-2i/D).
    """
    D = vec.shape[-1]
    half = D // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / D)
    ang = positions.astype(np.float64)[:, None] * inv_freq[None, :]       # [T, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = vec[..., :half], vec[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def visible_range(p: int, window: int) -> Tuple[int, int]:
    """Half-open range [lo, p+1) of key positions visible to the token at position p."""
    lo = 0 if window == 0 else max(0, p - window + 1)
    return lo, p + 1


def attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos: int,
              window: int) -> np.ndarray:
    """GQA attention of the T new tokens over the (already updated) cache.

    q [T, Hq, D], caches [Hkv, C, D] (bf16 values) -> o [T, Hq, D].
    Full score vector per query, its global max, exact normaliser.
    """
    T, Hq, D = q.shape
    Hkv = k_cache.shape[0]
    grp = Hq // Hkv
    o = np.zeros((T, Hq, D))
    scale = 1.0 / np.sqrt(D)
    for t in range(T):
        lo, hi = visible_range(pos + t, window)
        for g in range(Hkv):
            heads = slice(g * grp, (g + 1) * grp)
            K = k_cache[g, lo:hi]                     # [nk, D]
            V = v_cache[g, lo:hi]
            s = (q[t, heads] @ K.T) * scale           # [grp, nk]
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o[t, heads] = p @ V
    return o


def tree_depths(parents) -> np.ndarray:
    """Depth of every node of a token tree given by parent indices (-1: root; parents[t] < t)."""
    depth = np.zeros(len(parents), dtype=np.int64)
    for t, par in enumerate(parents):
        if not (-1 <= par < t):
            raise ValueError(f"parent of node {t} must lie in [-1, {t})")
        depth[t] = 0 if par < 0 else depth[par] + 1
    return depth


def tree_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, pos: int,
                   window: int, parents) -> np.ndarray:
    """GQA attention of the T tree nodes over the (already updated) cache.

    Node t at position pos + depth(t) sees cached key j < pos by the window rule at its
    position, and the step's node i (slot pos + i, position pos + depth(i)) iff i is t or
    an ancestor of t and the same rule holds for depth(i).
    """
    T, Hq, D = q.shape
    Hkv = k_cache.shape[0]
    grp = Hq // Hkv
    depth = tree_depths(parents)
    o = np.zeros((T, Hq, D))
    scale = 1.0 / np.sqrt(D)
    for t in range(T):
        pt = pos + depth[t]
        lo, _ = visible_range(pt, window)
        slots = list(range(lo, pos))
        anc, i = [], t
        while i >= 0:
            anc.append(i)
            i = parents[i]
        slots += [pos + i for i in sorted(anc) if window == 0 or pos + depth[i] > pt - window]
        for g in range(Hkv):
            heads = slice(g * grp, (g + 1) * grp)
            K = k_cache[g, slots]
            V = v_cache[g, slots]
            s_ = (q[t, heads] @ K.T) * scale
            s_ = s_ - s_.max(axis=1, keepdims=True)
            p_ = np.exp(s_)
            p_ /= p_.sum(axis=1, keepdims=True)
            o[t, heads] = p_ @ V
    return o


def route(logits: np.ndarray, k: int):
    """Top-k per token by logit descending, ties to the lower expert index.

    Returns idx [T, k] (selection order), gates [T, k] (softmax over the selected
    logits) and gap [T] = k-th selected logit - (k+1)-th (inf when k == E).
    """
    T, E = logits.shape
    idx = np.zeros((T, k), dtype=np.int64)
    gap = np.full(T, np.inf)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))      # primary: -logit, then index
        idx[t] = order[:k]
        if k < E:
            gap[t] = logits[t, order[k - 1]] - logits[t, order[k]]
    sel = np.take_along_axis(logits, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    gates = z / z.sum(axis=1, keepdims=True)
    return idx, gates, gap


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def nvfp4_experts(get_raw: Callable[[int], dict]) -> ExpertFn:
    """Expert accessor from raw NVFP4 storage.

    get_raw(e) returns {"gate": (codes, scales, ts), "up": (...), "down": (...)}.
    """
    def fn(e: int):
        raw = get_raw(e)
        return tuple(nvfp4_dequant(*raw[m]) for m in ("gate", "up", "down"))
    return fn


def bf16_experts(get_raw: Callable[[int], dict]) -> ExpertFn:
    """get_raw(e) returns {"gate": W, "up": W, "down": W} as fp64 arrays of bf16 values."""
    def fn(e: int):
        raw = get_raw(e)
        return tuple(np.asarray(raw[m], dtype=np.float64) for m in ("gate", "up", "down"))
    return fn


def down_input_nvfp4(a: np.ndarray, ts: float) -> np.ndarray:
    """The SwiGLU output as the down projection reads it when it is gathered in fp4 (orcarouter.ai
    English post, "Where the kernel boundary sits": an fp4 all-gather after the first expert
    GEMM): the fp32 row encoded as NVFP4 with the expert's activation tensor scale ts, decoded
    back (exact, fp64)."""
    codes, scales = nvfp4_quantize(np.asarray(a, dtype=np.float32)[None, :], ts)
    return nvfp4_values(codes, scales)[0] * float(np.float32(ts))


def expert_out(pl_t: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
               dims: Dims, act_ts: Optional[float] = None,
               a_in: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One token through one expert (this GPU's shard).  Returns (a [inter], the down
    projection's input [inter], d [pooled]); with act_ts the input is a encoded as NVFP4
    (down_input_nvfp4), else a itself; a given a_in replaces it."""
    il = dims.inter // dims.n_shards
    plc = dims.pooled // dims.n_shards
    r = dims.shard_rank
    g = Wg @ pl_t
    u = Wu @ pl_t
    a = np.zeros(dims.inter)
    a[r * il:(r + 1) * il] = silu(g) * u
    if a_in is None:
        a_in = a if act_ts is None else down_input_nvfp4(a, act_ts)
    d = np.zeros(dims.pooled)
    d[r * plc:(r + 1) * plc] = Wd @ a_in
    return a, a_in, d


# --------------------------------------------------------------------------------------------
# the whole step
# --------------------------------------------------------------------------------------------
def layer_step(inp: Dict[str, np.ndarray], dims: Dims, pos: int, window: int, experts: ExpertFn,
               force_idx: Optional[np.ndarray] = None, moe_tokens=None,
               parents=None, act_scales=None, force_down_input=None,
               force_kv=None) -> Dict[str, np.ndarray]:
    """One layer step.  `inp` holds fp64 arrays (bf16-valued weights):
    x [T,H], gamma1 [H], w_qkv [(Hq+2Hkv)D, H], w_o [H, Hq*D], gamma2 [H], w_router [E,H],
    w_pool [P,H], w_unpool [H,P], k_cache/v_cache [Hkv, C, D].

    force_idx [T, k] replaces the router's choice (gates are then the softmax over those
    logits).  moe_tokens limits the expert and unpooler work to a subset of tokens (y rows of
    the other tokens are returned as NaN); everything else is computed for all tokens.
    parents [T] makes the tokens the nodes of a token tree (see the module docstring); None
    is the chain.  act_scales [E] (fp32 activation tensor scale per expert) makes the down
    projection read its input encoded as NVFP4 (down_input_nvfp4); None reads a itself.
    force_down_input [T, k, inter] replaces the down projection's input of every slot, as
    force_idx replaces the routing (the caller checks that the replacement is a valid encoding
    of a, e.g. a device's encoding of its own SwiGLU output).
    force_kv = (k_rows, v_rows), each [T, Hkv, D] of bf16 values, replaces the rows written to
    the cache (the new keys after RoPE and the new values, rounded), as force_idx replaces the
    routing: the caller checks that every value is a bf16 neighbour of the exact one (a device
    may round a value that sits within its arithmetic error of a rounding boundary the other
    way); everything after the write then reads those rows.
    Returns y, the written K/V rows, routing and every intermediate.
    """
    x = np.asarray(inp["x"], dtype=np.float64)
    T, H = x.shape
    Hq, Hkv, D = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    out: Dict[str, np.ndarray] = {}

    # attention block
    xn = rmsnorm(x, inp["gamma1"], dims.rms_eps)
    qkv = xn @ inp["w_qkv"].T
    q = qkv[:, :Hq * D].reshape(T, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(T, Hkv, D)
    positions = pos + (np.arange(T) if parents is None else tree_depths(parents))
    q_r = rope(q, positions, dims.rope_theta)
    k_exact = rope(k, positions, dims.rope_theta)
    k_r = bf16_round(k_exact)
    v_r = bf16_round(v)
    if force_kv is not None:
        k_r = np.asarray(force_kv[0], dtype=np.float64).reshape(T, Hkv, D)
        v_r = np.asarray(force_kv[1], dtype=np.float64).reshape(T, Hkv, D)
    k_cache = np.array(inp["k_cache"], dtype=np.float64, copy=True)
    v_cache = np.array(inp["v_cache"], dtype=np.float64, copy=True)
    for t in range(T):
        k_cache[:, pos + t] = k_r[t]
        v_cache[:, pos + t] = v_r[t]
    o = (attention(q_r, k_cache, v_cache, pos, window) if parents is None
         else tree_attention(q_r, k_cache, v_cache, pos, window, parents))
    h = x + o.reshape(T, Hq * D) @ inp["w_o"].T

    # MoE block
    hn = rmsnorm(h, inp["gamma2"], dims.rms_eps)
    logits = hn @ inp["w_router"].T
    idx, gates, gap = route(logits, dims.top_k)
    if force_idx is not None:
        idx = np.asarray(force_idx, dtype=np.int64)
        sel = np.take_along_axis(logits, idx, axis=1)
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
        gates = z / z.sum(axis=1, keepdims=True)
    pl = hn @ inp["w_pool"].T

    toks = range(T) if moe_tokens is None else list(moe_tokens)
    m = np.full((T, dims.pooled), np.nan)
    a_all = np.full((T, dims.top_k, dims.inter), np.nan)
    aq_all = np.full((T, dims.top_k, dims.inter), np.nan)
    d_all = np.full((T, dims.top_k, dims.pooled), np.nan)
    needed = sorted({int(idx[t, kk]) for t in toks for kk in range(dims.top_k)})
    for e in needed:                              # one expert's weights resident at a time
        Wg, Wu, Wd = experts(e)
        for t in toks:
            for kk in range(dims.top_k):
                if idx[t, kk] == e:
                    a_all[t, kk], aq_all[t, kk], d_all[t, kk] = expert_out(
                        pl[t], Wg, Wu, Wd, dims, None if act_scales is None else float(act_scales[e]),
                        None if force_down_input is None else np.asarray(force_down_input[t, kk], np.float64))
    for t in toks:
        acc = np.zeros(dims.pooled)
        for kk in range(dims.top_k):              # selection order
            acc = acc + gates[t, kk] * d_all[t, kk]
        m[t] = acc
    y = np.full((T, H), np.nan)
    tl = list(toks)
    y[tl] = h[tl] + m[tl] @ inp["w_unpool"].T

    out.update(y=y, xn=xn, q=q_r, k_new=k_r, v_new=v_r, k_exact=k_exact, v_exact=v, o=o, h=h, hn=hn,
               logits=logits,
               idx=idx, gates=gates, gap=gap, pl=pl, a=a_all, a_in=aq_all, d=d_all, m=m,
               k_cache=k_cache, v_cache=v_cache)
    return out
