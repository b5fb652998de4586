"""Loop-only oracle of the same layer step, for tiny shapes.

Test infrastructure only (see the package docstring).

Every quantity is a Python float (IEEE binary64) computed with explicit loops:
per token, per head, per key, per output feature, per reduction index.  It
re-derives each definition (bf16 rounding of the cache writes, E2M1 / E4M3
decoding and, for the fp4 gather of the SwiGLU output, encoding, RMSNorm,
rotate-half RoPE, windowed causal attention, top-k routing with the lower index
winning ties, SwiGLU experts, combine, residuals) from the written rules and
does not call into ``layer.py`` or ``formats.py``, so that the vectorised
oracle can be checked against it.
"""
from __future__ import annotations

import math
import struct
from typing import Dict, List


def r_bf16(v: float) -> float:
    """Nearest bf16 value, ties to even (8 significant bits, min exponent -126)."""
    if v == 0.0 or math.isinf(v) or math.isnan(v):
        return v
    mant, ex = math.frexp(v)          # v = mant * 2**ex, 0.5 <= |mant| < 1
    # value = mant * 2**ex; keep 8 significant bits -> step 2**(ex-8), not below 2**-133
    step_exp = max(ex - 8, -133)
    n = v / (2.0 ** step_exp)
    n_r = round(n)                    # Python round(): ties to even
    out = n_r * (2.0 ** step_exp)
    if abs(out) >= 2.0 ** 128:
        return math.copysign(math.inf, v)
    return out


def fp4_elem(code: int) -> float:
    negative = (code >> 3) & 1
    exp_field = (code >> 1) & 3
    man = code & 1
    if exp_field == 0:
        mag = 0.5 * man
    else:
        mag = (2.0 ** (exp_field - 1)) * (1.0 + 0.5 * man)
    return -mag if negative else mag


def fp8_scale(b: int) -> float:
    negative = (b >> 7) & 1
    exp_field = (b >> 3) & 15
    man = b & 7
    if exp_field == 15 and man == 7:
        return math.nan
    if exp_field == 0:
        mag = (man / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp_field - 7)
    return -mag if negative else mag


def _nvfp4_row_elem(codes_row, scales_row, ts: float, k: int) -> float:
    byte = int(codes_row[k // 2])
    code = (byte & 15) if k % 2 == 0 else (byte >> 4)
    return fp4_elem(code) * fp8_scale(int(scales_row[k // 16])) * ts


def _f32(v: float) -> float:
    """Nearest binary32 value (ties to even).  A binary32 product or quotient rounded once
    equals the binary64 result rounded again to binary32 (53 >= 2 * 24 + 2 bits)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _e4m3_round(v: float) -> float:
    """Nearest E4M3 value to v >= 0 (4 significant bits, quantum 2^-9 below 2^-6), ties to an
    even significand, saturating at 448."""
    if v >= 448.0:
        return 448.0
    if v == 0.0:
        return 0.0
    _, ex = math.frexp(v)             # v = m 2^ex, 0.5 <= m < 1: quantum 2^(ex - 4)
    q = 2.0 ** max(ex - 4, -9)
    r = round(v / q) * q              # Python round(): ties to even
    return min(r, 448.0)


def _e2m1_round(v: float) -> float:
    """Nearest E2M1 magnitude to v >= 0, ties to the even code, saturating at 6: the decision
    points are the midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5 of the grid
    0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7)."""
    if v <= 0.25:
        return 0.0
    if v < 0.75:
        return 0.5
    if v <= 1.25:
        return 1.0
    if v < 1.75:
        return 1.5
    if v <= 2.5:
        return 2.0
    if v < 3.5:
        return 3.0
    if v <= 5.0:
        return 4.0
    return 6.0


def _fp4_gather(a: List[float], ts: float) -> List[float]:
    """a as the down projection reads it after an fp4 gather: per 16-element block an E4M3
    scale for amax / (6 ts), each element an E2M1 multiple of scale * ts (fp32 decisions)."""
    t32 = _f32(ts)
    six_ts = _f32(6.0 * t32)
    out = []
    for b in range(0, len(a), 16):
        blk = [_f32(v) for v in a[b:b + 16]]
        amax = max(abs(v) for v in blk)
        s = _e4m3_round(_f32(amax / six_ts))
        den = _f32(s * t32)
        for v in blk:
            if den == 0.0:
                out.append(0.0)
                continue
            mag = _e2m1_round(abs(_f32(v / den)))
            out.append(math.copysign(mag, v) * s * t32 if mag != 0.0 else 0.0)
    return out


def _dot(a, b) -> float:
    s = 0.0
    for i in range(len(a)):
        s += a[i] * b[i]
    return s


def _norm(vec: List[float], gamma: List[float], eps: float) -> List[float]:
    n = len(vec)
    ss = 0.0
    for v in vec:
        ss += v * v
    inv = 1.0 / math.sqrt(ss / n + eps)
    return [vec[i] * inv * gamma[i] for i in range(n)]


def _rotate(vec: List[float], position: int, theta: float) -> List[float]:
    D = len(vec)
    half = D // 2
    out = [0.0] * D
    for i in range(half):
        angle = position * theta ** (-(2.0 * i) / D)
        c, s = math.cos(angle), math.sin(angle)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i + half] * c + vec[i] * s
    return out


def layer_step(inp: Dict, dims, pos: int, window: int, expert_raw, nvfp4: bool = True,
               parents=None, act_scales=None) -> Dict:
    """Same contract as layer.layer_step on tiny inputs given as nested lists / arrays.

    expert_raw(e) returns {"gate": (codes, scales, ts) | W, "up": ..., "down": ...}.
    parents: token-tree parent of every token (-1 for a root), None for the chain; a token's
    position is pos plus its number of ancestors, and it sees the step's tokens that are
    itself or its ancestors.
    act_scales: per-expert activation tensor scales; given, the down projection reads the
    SwiGLU output after an fp4 gather (_fp4_gather).
    """
    x = [[float(v) for v in row] for row in inp["x"]]
    T, H = len(x), len(x[0])
    Hq, Hkv, D = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    E, K = dims.n_experts, dims.top_k
    w_qkv = inp["w_qkv"]
    C = len(inp["k_cache"][0])
    kc = [[[float(inp["k_cache"][g][j][d]) for d in range(D)] for j in range(C)] for g in range(Hkv)]
    vc = [[[float(inp["v_cache"][g][j][d]) for d in range(D)] for j in range(C)] for g in range(Hkv)]

    # token positions and, per token, the step's tokens it may see (itself and its ancestors)
    par = [t - 1 for t in range(T)] if parents is None else [int(v) for v in parents]
    posn, sees = [], []
    for t in range(T):
        chain, i = [], t
        while i != -1:
            chain.append(i)
            i = par[i]
        posn.append(pos + len(chain) - 1)
        sees.append(set(chain))

    # RMSNorm 1, QKV projection, RoPE, rounding, cache write
    q_all, k_all, v_all = [], [], []
    for t in range(T):
        xn = _norm(x[t], [float(v) for v in inp["gamma1"]], dims.rms_eps)
        row = [_dot(xn, [float(v) for v in w_qkv[n]]) for n in range(len(w_qkv))]
        qh = [_rotate(row[h * D:(h + 1) * D], posn[t], dims.rope_theta) for h in range(Hq)]
        kh = [_rotate(row[(Hq + g) * D:(Hq + g + 1) * D], posn[t], dims.rope_theta) for g in range(Hkv)]
        vh = [row[(Hq + Hkv + g) * D:(Hq + Hkv + g + 1) * D] for g in range(Hkv)]
        q_all.append([list(qv) for qv in qh])
        k_all.append([[r_bf16(v) for v in kv] for kv in kh])
        v_all.append([[r_bf16(v) for v in vv] for vv in vh])
        for g in range(Hkv):
            kc[g][pos + t] = list(k_all[t][g])
            vc[g][pos + t] = list(v_all[t][g])

    # attention, o-projection, residual
    group = Hq // Hkv
    h_all = []
    for t in range(T):
        p = posn[t]
        o_flat = []
        for hh in range(Hq):
            g = hh // group
            # cached keys by position; the step's slot pos + i holds token i at position posn[i]
            keys = [j for j in range(0, pos) if j <= p and (window == 0 or j > p - window)]
            keys += [pos + i for i in range(T)
                     if i in sees[t] and (window == 0 or posn[i] > p - window)]
            scores = [_dot(q_all[t][hh], kc[g][j]) / math.sqrt(D) for j in keys]
            mx = max(scores)
            ws = [math.exp(s - mx) for s in scores]
            tot = sum(ws)
            for d in range(D):
                acc = 0.0
                for i, j in enumerate(keys):
                    acc += ws[i] / tot * vc[g][j][d]
                o_flat.append(acc)
        h_row = []
        for n in range(H):
            h_row.append(x[t][n] + _dot(o_flat, [float(v) for v in inp["w_o"][n]]))
        h_all.append(h_row)

    # MoE block
    il = dims.inter // dims.n_shards
    plc = dims.pooled // dims.n_shards
    rk = dims.shard_rank
    y, idx_all, gate_all, logit_all = [], [], [], []
    for t in range(T):
        hn = _norm(h_all[t], [float(v) for v in inp["gamma2"]], dims.rms_eps)
        logits = [_dot(hn, [float(v) for v in inp["w_router"][e]]) for e in range(E)]
        remaining = list(range(E))
        chosen = []
        for _ in range(K):
            best = remaining[0]
            for e in remaining[1:]:
                if logits[e] > logits[best]:      # strict: equal logits keep the lower index
                    best = e
            chosen.append(best)
            remaining.remove(best)
        mx = max(logits[e] for e in chosen)
        ex = [math.exp(logits[e] - mx) for e in chosen]
        gates = [v / sum(ex) for v in ex]
        pl = [_dot(hn, [float(v) for v in inp["w_pool"][pp]]) for pp in range(dims.pooled)]
        m_acc = [0.0] * dims.pooled
        for slot, e in enumerate(chosen):
            raw = expert_raw(e)
            a = [0.0] * dims.inter
            for i in range(il):
                if nvfp4:
                    gsum = 0.0
                    usum = 0.0
                    gc, gs, gts = raw["gate"]
                    uc, us, uts = raw["up"]
                    for kk in range(dims.pooled):
                        gsum += pl[kk] * _nvfp4_row_elem(gc[i], gs[i], float(gts), kk)
                        usum += pl[kk] * _nvfp4_row_elem(uc[i], us[i], float(uts), kk)
                else:
                    gsum = _dot(pl, [float(v) for v in raw["gate"][i]])
                    usum = _dot(pl, [float(v) for v in raw["up"][i]])
                sig = gsum / (1.0 + math.exp(-gsum)) if gsum > -700 else 0.0
                a[rk * il + i] = sig * usum
            if act_scales is not None:
                a = _fp4_gather(a, float(act_scales[e]))
            for pp in range(plc):
                if nvfp4:
                    dc, ds, dts = raw["down"]
                    dsum = 0.0
                    for kk in range(dims.inter):
                        dsum += a[kk] * _nvfp4_row_elem(dc[pp], ds[pp], float(dts), kk)
                else:
                    dsum = _dot(a, [float(v) for v in raw["down"][pp]])
                m_acc[rk * plc + pp] += gates[slot] * dsum
        m = m_acc
        y.append([h_all[t][n] + _dot(m, [float(v) for v in inp["w_unpool"][n]]) for n in range(H)])
        idx_all.append(chosen)
        gate_all.append(gates)
        logit_all.append(logits)
    return dict(y=y, idx=idx_all, gates=gate_all, logits=logit_all, k_new=k_all, v_new=v_all,
                h=h_all)
