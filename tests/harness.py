"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on seeded
inputs, run the oracle on the same inputs, compare to the stated bar.

Bar (per token): y max-abs <= 2e-2 and cosine >= 0.999 against the oracle; written K/V
values each a bf16 neighbour of the exact value; every cache byte outside the written slots
bit-identical; router logits within half the 1e-3 exemption gap, so the selected expert set
is bit-exact wherever the oracle's k-th/(k+1)-th logit gap exceeds 1e-3, and the selection
order consistent with the oracle's logits up to the logit error; q, o, h and the pooled
vector within fixed relative bounds.  Everything after the cache write is compared against
the oracle reading the device's written K/V rows (a valid rounding, as the device's expert
choice is valid within the exemption), y also against the free-running oracle on a few
tokens.  y is compared against the oracle re-run with the device's chosen experts in the
device's order, so the exempt tokens are checked too.  With the fp4 gather of the SwiGLU output the encoding is a
decision taken in fp32 on values the device and the oracle compute with different rounding,
so it is checked the same way: the device's SwiGLU output within 1e-3 of the oracle's (of
the row's largest magnitude; it inherits the attention's bf16 probabilities through h), its encoded down input bit-exact against the oracle's encoder
applied to that device output, the expert outputs within 1e-4 of the down projection of that
input, and y against the oracle re-run with that input.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from moe_layer_persistent_amd import binding, synth
from oracle import formats as oformats
from oracle import layer as olayer

Y_MAX_ABS = 2e-2
Y_MIN_COS = 0.999
GAP_EXEMPT = 1e-3
# router logits within half the exemption gap, so that the selected set is unique by
# construction wherever the gap exceeds the exemption
LOGIT_MAX_ABS = GAP_EXEMPT / 2
# the same logits against the oracle that rounds the written K/V itself: a new key or value the
# device rounded to the other bf16 neighbour moves later logits by up to ~1e-3 at full width
LOGIT_MAX_ABS_FREE = 5e-3
# intermediate activations, max error relative to the largest exact value: every activation is
# carried with ~16 significant bits (a bf16 pair) and summed in fp32, so errors sit near 1e-6
REL_ERR_MAX = {"q": 3e-5, "o": 3e-5, "h": 3e-5, "pl": 3e-5}


def dims_of(w: synth.Workload) -> olayer.Dims:
    return olayer.Dims(w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.pooled, w.inter,
                       w.n_experts, w.top_k, w.n_shards, w.shard_rank, w.rms_eps, w.rope_theta)


class GpuRun:
    """Inputs of one layer on the GPU, packed weights, a plan and the outputs of a step."""

    def __init__(self, w: synth.Workload, layer: int = 0, routing: str = "iid", plan=None,
                 tensors=None, lw=None):
        self.w = w
        self.layer = layer
        self.window = w.layer_window(layer)
        self.t = tensors if tensors is not None else synth.make_layer(w, layer, "cuda", routing=routing)
        self.cfg = binding.config_from_workload(w)
        self.plan = plan if plan is not None else binding.Plan(self.cfg)
        self.lw = lw if lw is not None else self.plan.pack_layer(self.t)
        self.k0 = self.t["k_cache"].clone()
        self.v0 = self.t["v_cache"].clone()
        torch.cuda.synchronize()

    def fresh_caches(self):
        return self.k0.clone(), self.v0.clone()

    def run(self, fused=True, T=None, pos=None, stamps=False, x=None, parents=None):
        w = self.w
        T = w.T if T is None else T
        pos = w.pos if pos is None else pos
        x = self.t["x"][:T].contiguous() if x is None else x
        kc, vc = self.fresh_caches()
        y = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
        dbg = {
            "expert_idx": torch.full((T, w.top_k), -1, dtype=torch.int32, device="cuda"),
            "gates": torch.zeros((T, w.top_k), dtype=torch.float32, device="cuda"),
            "router_logits": torch.zeros((T, w.n_experts), dtype=torch.float32, device="cuda"),
        }
        if stamps:
            dbg["timestamps"] = torch.zeros((self.plan.workgroups, binding.MOEL_N_STAMPS),
                                            dtype=torch.int64, device="cuda")
        self.plan.layer_decode(self.lw, kc, vc, x, pos, self.window, y, dbg=dbg, fused=fused, parents=parents)
        torch.cuda.synchronize()
        st = self.plan.status()
        assert st == binding.MOEL_OK, binding.status_string(st)
        return dict(y=y, k_cache=kc, v_cache=vc, T=T, pos=pos, x=x, parents=parents, **dbg)


class RequestView:
    """One request of a batched step, seen as a single-request run: its cache is its slot range
    of the pool and its rows of the step's scratch start at row0."""

    def __init__(self, run: GpuRun, req, row0: int):
        T, pos, kvb, slots = req
        self.w = run.w
        self.t = run.t
        self.window = run.window
        self.plan = run.plan
        self.k0 = run.k0[:, kvb:kvb + slots].contiguous()
        self.v0 = run.v0[:, kvb:kvb + slots].contiguous()
        self.row0 = row0

    @staticmethod
    def out_of(out: Dict, req, row0: int) -> Dict:
        T, pos, kvb, slots = req
        rows = slice(row0, row0 + T)
        o = {k: out[k][rows] for k in ("y", "x", "expert_idx", "gates", "router_logits")}
        o["k_cache"] = out["k_cache"][:, kvb:kvb + slots].contiguous()
        o["v_cache"] = out["v_cache"][:, kvb:kvb + slots].contiguous()
        o.update(T=T, pos=pos, parents=None)
        return o


def run_batch(run: GpuRun, reqs, fused: bool = True, x: Optional[torch.Tensor] = None) -> Dict:
    """One batched step over (T, pos, kv_base, kv_slots) requests on fresh copies of the pool."""
    w = run.w
    T = sum(r[0] for r in reqs)
    x = run.t["x"][:T].contiguous() if x is None else x
    kc, vc = run.fresh_caches()
    y = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
    dbg = {
        "expert_idx": torch.full((T, w.top_k), -1, dtype=torch.int32, device="cuda"),
        "gates": torch.zeros((T, w.top_k), dtype=torch.float32, device="cuda"),
        "router_logits": torch.zeros((T, w.n_experts), dtype=torch.float32, device="cuda"),
    }
    run.plan.layer_decode_batch(run.lw, kc, vc, x, reqs, run.window, y, dbg=dbg, fused=fused)
    torch.cuda.synchronize()
    st = run.plan.status()
    assert st == binding.MOEL_OK, binding.status_string(st)
    return dict(y=y, k_cache=kc, v_cache=vc, x=x, **dbg)


def check_batch_against_oracle(run: GpuRun, out: Dict, reqs, moe_tokens=None) -> List[dict]:
    """Every request of a batched step against the oracle run on that request alone, and the
    pool outside every request's slot range bit-identical.  moe_tokens: per request, as for
    check_against_oracle (None = all)."""
    keep = torch.ones(run.k0.shape[1], dtype=torch.bool, device=run.k0.device)
    for (T, pos, kvb, slots) in reqs:
        keep[kvb:kvb + slots] = False
    for name, c_out, c_in in (("k", out["k_cache"], run.k0), ("v", out["v_cache"], run.v0)):
        assert torch.equal(c_out[:, keep].view(torch.int16), c_in[:, keep].view(torch.int16)), \
            f"{name} pool changed outside the requests' slots"
    reps, row0 = [], 0
    for r in reqs:
        view = RequestView(run, r, row0)
        rep = {}
        check_against_oracle(view, RequestView.out_of(out, r, row0), moe_tokens=moe_tokens, report=rep)
        reps.append(rep)
        row0 += r[0]
    return reps


def _f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def oracle_inputs(run: GpuRun, T: int, x: torch.Tensor) -> Dict[str, np.ndarray]:
    t = run.t
    inp = {k: _f64(t[k]) for k in ("gamma1", "gamma2", "w_qkv", "w_o", "w_router", "w_pool", "w_unpool")}
    inp["x"] = _f64(x[:T])
    inp["k_cache"] = _f64(run.k0)
    inp["v_cache"] = _f64(run.v0)
    return inp


def expert_fn(run: GpuRun):
    t, w = run.t, run.w
    if w.expert_dtype == synth.NVFP4:
        def raw(e):
            return {m: (t[m + "_codes"][e].cpu().numpy(), t[m + "_scales"][e].cpu().numpy(),
                        float(t[m + "_ts"][e].item())) for m in ("gate", "up", "down")}
        return olayer.nvfp4_experts(raw)

    def rawb(e):
        return {m: _f64(t[m][e]) for m in ("gate", "up", "down")}
    return olayer.bf16_experts(rawb)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(np.dot(a, b) / (na * nb))


def device_down_input(run: GpuRun, gpu_idx: np.ndarray, T: int) -> np.ndarray:
    """[T, k, inter] the device's fp4-gathered down input of every slot (value x tensor scale)."""
    w = run.w
    k, I = w.top_k, w.inter
    r0 = getattr(run, "row0", 0)
    aq = run.plan.scratch("aq").view(binding.MOEL_MAX_TOKENS * k, I).cpu().numpy().astype(np.float64)
    act = run.t["act_ts"].cpu().numpy()
    out = np.empty((T, k, I))
    for t in range(T):
        for kk in range(k):
            out[t, kk] = aq[(r0 + t) * k + kk] * float(np.float32(act[int(gpu_idx[t, kk])]))
    return out


def check_fp4_gather(run: GpuRun, gpu_idx: np.ndarray, ref: Dict, toks: Sequence[int]) -> dict:
    """The SwiGLU output, its fp4-gathered encoding and the expert outputs of the given tokens'
    slots (ref: the oracle run with the device's down input)."""
    w = run.w
    k, I = w.top_k, w.inter
    a_dev = run.plan.scratch("a").view(binding.MOEL_MAX_TOKENS * k, I).cpu().numpy()
    aq_dev = run.plan.scratch("aq").view(binding.MOEL_MAX_TOKENS * k, I).cpu().numpy().astype(np.float64)
    d_dev = run.plan.scratch("d").view(binding.MOEL_MAX_TOKENS * k, w.pooled).cpu().numpy().astype(np.float64)
    act = run.t["act_ts"].cpu().numpy()
    ex = expert_fn(run)
    plc, r = w.pooled // w.n_shards, w.shard_rank
    r0 = getattr(run, "row0", 0)
    agree, d_err, a_err = [], 0.0, 0.0
    for t in toks:
        for kk in range(k):
            slot, e = (r0 + t) * k + kk, int(gpu_idx[t, kk])
            a_ref = ref["a"][t, kk]
            err = float(np.abs(a_dev[slot] - a_ref).max() / (np.abs(a_ref).max() + 1e-30))
            assert err <= 1e-3, ("SwiGLU output vs oracle", t, kk, err)
            a_err = max(a_err, err)
            ts = float(np.float32(act[e]))
            codes, scales = oformats.nvfp4_quantize(a_dev[slot][None, :], float(act[e]))
            want = oformats.nvfp4_values(codes, scales)[0]
            bad = np.nonzero(aq_dev[slot] != want)[0]
            assert bad.size == 0, ("encoded down input differs", t, kk, bad[:8], aq_dev[slot][bad[:8]], want[bad[:8]])
            _, _, Wd = ex(e)
            d_want = np.zeros(w.pooled)
            d_want[r * plc:(r + 1) * plc] = Wd @ (want * ts)
            err = float(np.abs(d_dev[slot] - d_want).max() / (np.abs(d_want).max() + 1e-30))
            assert err <= 1e-4, ("expert output vs the down projection of its input", t, kk, err)
            d_err = max(d_err, err)
            # the oracle's own encoding of its exact SwiGLU output: equal except where a value
            # sits within the device's arithmetic error of a decision point (reported)
            agree.append(float(np.mean(olayer.down_input_nvfp4(a_ref, float(act[e])) == want * ts)))
    return {"a_rel_err": a_err, "d_rel_err": d_err, "encoded_equal_frac_vs_oracle_own": min(agree)}


def check_against_oracle(run: GpuRun, out: Dict, moe_tokens: Optional[Sequence[int]] = None,
                         report: Optional[dict] = None,
                         free_tokens: Optional[Sequence[int]] = None) -> dict:
    """Compares one device step with the oracle; raises AssertionError on any miss.

    Every statistic is gathered first and the misses are raised together at the end, so that
    one failing run reports all of them.  moe_tokens: tokens whose MoE block and y are compared
    (default all); free_tokens: tokens whose y is also compared with the free-running oracle
    (its own KV rounding; default the first and the last of moe_tokens).
    """
    w = run.w
    T, pos = out["T"], out["pos"]
    dims = dims_of(w)
    inp = oracle_inputs(run, T, out["x"])
    gpu_idx = out["expert_idx"].cpu().numpy().astype(np.int64)
    toks = list(range(T)) if moe_tokens is None else sorted(set(int(t) for t in moe_tokens if t < T))
    if free_tokens is None:
        free_tokens = sorted({toks[0], toks[-1]})
    parents = out.get("parents")
    fp4g = getattr(w, "down_input", synth.DOWN_EXACT) == synth.DOWN_NVFP4
    act = _f64(run.t["act_ts"]) if fp4g else None
    misses: List[str] = []

    def need(cond, msg):
        if not cond:
            misses.append(msg)

    # ---- KV cache.  The written (head, slot) set is exact and every other byte untouched; a
    # written value is the bf16 nearest the exact value or, when the exact value lies within the
    # device's arithmetic error of a rounding boundary, the other neighbour (< 1 ulp away).
    ref0 = olayer.layer_step(inp, dims, pos, run.window, expert_fn(run), moe_tokens=[], parents=parents,
                             act_scales=act)
    k_out, v_out = out["k_cache"], out["v_cache"]
    kv_eq, dev_kv = [], []
    for name, c_out, c_in, new, xv in (("k", k_out, run.k0, ref0["k_new"], ref0["k_exact"]),
                                        ("v", v_out, run.v0, ref0["v_new"], ref0["v_exact"])):
        keep = torch.ones(c_in.shape[1], dtype=torch.bool, device=c_in.device)
        keep[pos:pos + T] = False
        assert torch.equal(c_out[:, keep].view(torch.int16), c_in[:, keep].view(torch.int16)), \
            f"{name} cache changed outside the written slots"
        got = _f64(c_out[:, pos:pos + T]).transpose(1, 0, 2)          # [T, Hkv, D]
        dev_kv.append(got)
        ulp = np.ldexp(1.0, np.frexp(np.abs(xv))[1] - 8)             # bf16 spacing at |exact|
        # the device's own error on a value is relative to the magnitude of its row, not to the
        # value (a small result of a long sum carries the absolute error of the sum)
        scale = np.abs(xv).max(axis=-1, keepdims=True)
        off = np.abs(got - xv) / (ulp + 2.0 ** -13 * scale)
        need(off.max() < 1.0, f"{name} written value further than 1 ulp from exact ({off.max()})")
        eq = float(np.mean(got == new))
        need(eq >= 0.9, f"{name} bitwise-equal fraction {eq}")   # reported; a sanity floor only
        kv_eq.append(eq)
        for t in range(T):
            need(cosine(got[t].ravel(), new[t].ravel()) >= Y_MIN_COS, f"{name} row {t} cosine")
    # ---- everything after the cache write, against the oracle reading the device's written
    # rows (a valid rounding, checked above): what remains is the kernels' arithmetic error
    ref1 = olayer.layer_step(inp, dims, pos, run.window, expert_fn(run), moe_tokens=[], parents=parents,
                             act_scales=act, force_kv=tuple(dev_kv))
    dev_logits = out["router_logits"].cpu().numpy()
    lg_err = float(np.abs(dev_logits - ref1["logits"]).max())
    lg_err_free = float(np.abs(dev_logits - ref0["logits"]).max())
    # a logit error below half the exemption gap cannot swap the k-th and (k+1)-th expert of a
    # token whose gap exceeds the exemption: the set is then unique and must match bit for bit
    need(lg_err <= LOGIT_MAX_ABS, f"router logits max-abs {lg_err} > {LOGIT_MAX_ABS}")
    sets_equal = np.array([sorted(gpu_idx[t]) == sorted(ref1["idx"][t]) for t in range(T)])
    exact = ref1["gap"] > GAP_EXEMPT
    need(sets_equal[exact].all(), f"expert sets differ at tokens {np.nonzero(exact & ~sets_equal)[0]}")
    # against the free-running oracle (its own rounding of the written K/V) the logits also
    # carry the effect of the values rounded the other way (each within 1 ulp, checked above):
    # the set must match wherever that gap exceeds the exemption by twice this error
    need(lg_err_free <= LOGIT_MAX_ABS_FREE,
         f"router logits (free-running) max-abs {lg_err_free} > {LOGIT_MAX_ABS_FREE}")
    sets_equal0 = np.array([sorted(gpu_idx[t]) == sorted(ref0["idx"][t]) for t in range(T)])
    exact0 = ref0["gap"] > max(GAP_EXEMPT, 2 * lg_err_free)
    need(sets_equal0[exact0].all(),
         f"expert sets differ from the free-running oracle at tokens {np.nonzero(exact0 & ~sets_equal0)[0]}")
    for t in range(T):
        need(len(set(gpu_idx[t])) == w.top_k and gpu_idx[t].min() >= 0 and gpu_idx[t].max() < w.n_experts,
             f"token {t}: selection not {w.top_k} distinct experts")
        sel = ref1["logits"][t, gpu_idx[t]]
        need(np.all(np.diff(sel) <= 2 * lg_err + 1e-6), f"token {t}: selection order invalid {sel}")
    gsel = out["gates"].cpu().numpy()
    need(np.abs(gsel.sum(axis=1) - 1.0).max() <= 1e-5, "gates do not sum to 1")
    ref = olayer.layer_step(inp, dims, pos, run.window, expert_fn(run), force_idx=gpu_idx, moe_tokens=toks,
                            parents=parents, act_scales=act, force_kv=tuple(dev_kv),
                            force_down_input=device_down_input(run, gpu_idx, T) if fp4g else None)
    gate_err = float(np.abs(gsel - ref["gates"]).max())
    need(gate_err <= 2 * lg_err + 1e-5, f"gates max-abs {gate_err} (logits {lg_err})")
    stats = {"max_abs": 0.0, "min_cos": 1.0, "exempt_tokens": int((~exact).sum()),
             "min_gap": float(ref1["gap"].min()),
             "order_equal_frac": float(np.mean(np.all(gpu_idx == ref1["idx"], axis=1))),
             "logit_err": lg_err, "logit_err_free": lg_err_free, "gate_err": gate_err,
             "free_band_tokens": int((~exact0 & (ref0["gap"] > GAP_EXEMPT)).sum()),
             "kv_bitwise_frac": min(kv_eq), "tokens_checked": len(toks)}
    # intermediate activations (max error relative to the largest exact value)
    inter = {}
    for name, key in (("q", "q"), ("o", "o"), ("h", "h"), ("pl", "pl")):
        r0 = getattr(run, "row0", 0)
        got_i = run.plan.scratch(name).view(binding.MOEL_MAX_TOKENS, -1)[r0:r0 + T].cpu().numpy().astype(np.float64)
        want = ref[key].reshape(T, -1)
        inter[name] = float(np.abs(got_i - want).max() / (np.abs(want).max() + 1e-30))
        need(inter[name] <= REL_ERR_MAX[name], f"{name} relative error {inter[name]} > {REL_ERR_MAX[name]}")
    stats["rel_err"] = inter
    if fp4g:
        stats["fp4_gather"] = check_fp4_gather(run, gpu_idx, ref, toks)
    y = out["y"].cpu().numpy().astype(np.float64)
    for t in toks:
        err = float(np.abs(y[t] - ref["y"][t]).max())
        cs = cosine(y[t], ref["y"][t])
        stats["max_abs"] = max(stats["max_abs"], err)
        stats["min_cos"] = min(stats["min_cos"], cs)
        need(err <= Y_MAX_ABS and cs >= Y_MIN_COS, f"token {t}: y max-abs {err} cos {cs}")
    # the same bar against the free-running oracle (its own KV rounding) on a few tokens
    if not fp4g:
        ft = [t for t in free_tokens if t < T]
        reff = olayer.layer_step(inp, dims, pos, run.window, expert_fn(run), force_idx=gpu_idx, moe_tokens=ft,
                                 parents=parents, act_scales=act)
        stats["max_abs_free"] = 0.0
        for t in ft:
            err = float(np.abs(y[t] - reff["y"][t]).max())
            cs = cosine(y[t], reff["y"][t])
            stats["max_abs_free"] = max(stats["max_abs_free"], err)
            need(err <= Y_MAX_ABS and cs >= Y_MIN_COS, f"token {t} (free-running): y max-abs {err} cos {cs}")
    if report is not None:
        report.update(stats)
    assert not misses, f"{misses} | stats {stats}"
    return stats
