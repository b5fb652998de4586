"""Benchmark of one MoE decoder layer's batch-1 verify step (T = 16) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload swa_fp4] [--routing iid|shared]

A step is one persistent launch of the whole layer over one batch of 16 synthetic verify
tokens.  Inputs are resident in HBM before timing starts.  To keep the 256 MB Infinity
Cache from serving weights across steps, consecutive steps alternate between two packed
copies of the layer's weights (so each step's weights were last touched two steps ago and
>7 GB have streamed in between).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

PEAK_HBM_GBPS = 8000.0


def algorithmic_bytes(w, idx, pos, window, T):
    """Bytes the step must move at least once: every weight byte it uses (dense weights, the
    routed experts' matrices), the visible KV window, x, y and the KV writes."""
    H, D, Hq, Hkv, P, I = w.hidden, w.head_dim, w.n_q_heads, w.n_kv_heads, w.pooled, w.inter
    dense = 2 * (w.qkv_rows * H + H * Hq * D + w.n_experts * H + P * H + H * P + 2 * H)
    if w.expert_dtype == 0:
        per_elem = 0.5 + 1.0 / 16.0
    else:
        per_elem = 2.0
    expert = per_elem * (2 * w.inter_local * P + w.pooled_local * I)
    U = len(set(int(e) for e in idx.reshape(-1)))
    lo = max(0, pos - window + 1) if window > 0 else 0
    kv_read = (pos + T - lo) * Hkv * D * 2 * 2
    io = T * H * 4 * 2 + T * Hkv * D * 2 * 2
    return dense + U * expert + kv_read + io, U


def kernel_source_digest() -> str:
    """sha256 over the HIP sources of the library (the counters below belong to one version)."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "moe_layer_persistent_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".h", ".hip", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


# a 16-node token tree: node t's parent (-1: root)
TREE16 = [-1, 0, 1, 2, 0, 4, 5, 1, 7, 3, 9, 4, 11, 12, 2, 14]


def measured_traffic(workload: str):
    """HBM bytes per launch of the fused kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by the same counters on a copy of known size), or None
    when the summary belongs to another version of the kernel sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"k_layer_fused_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_digest() or "traffic_bytes_per_launch" not in kv:
        return None
    return {"bytes_per_launch": float(kv["traffic_bytes_per_launch"]), "source": os.path.relpath(path)}


def cpu_baseline(w, t, idx, window, budget_s=25.0):
    """The oracle, timed on this host's cores on a bounded sample of the same step: the
    whole attention block and routing for all 16 tokens, plus the expert block for as many
    tokens as fit the budget; scaled to one full layer by the distinct experts used."""
    import numpy as np
    import torch
    from oracle import layer as olayer

    dims = olayer.Dims(w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.pooled, w.inter,
                       w.n_experts, w.top_k, w.n_shards, 0, w.rms_eps, w.rope_theta)
    f64 = lambda x: x.detach().to("cpu").double().numpy()
    inp = {k: f64(t[k]) for k in ("x", "gamma1", "gamma2", "w_qkv", "w_o", "w_router", "w_pool", "w_unpool",
                                  "k_cache", "v_cache")}
    if w.expert_dtype == 0:
        raw = lambda e: {m: (t[m + "_codes"][e].cpu().numpy(), t[m + "_scales"][e].cpu().numpy(),
                             float(t[m + "_ts"][e].item())) for m in ("gate", "up", "down")}
        ex = olayer.nvfp4_experts(raw)
    else:
        ex = olayer.bf16_experts(lambda e: {m: f64(t[m][e]) for m in ("gate", "up", "down")})
    gi = idx.astype(np.int64)
    t0 = time.perf_counter()
    olayer.layer_step(inp, dims, w.pos, window, ex, force_idx=gi, moe_tokens=[])
    t_attn = time.perf_counter() - t0
    toks, used = [], set()
    t_moe = 0.0
    for tok in range(w.T):
        t1 = time.perf_counter()
        olayer.layer_step(inp, dims, w.pos, window, ex, force_idx=gi, moe_tokens=[tok])
        dt = time.perf_counter() - t1 - t_attn
        t_moe += max(dt, 0.0)
        toks.append(tok)
        used |= set(int(e) for e in gi[tok])
        if t_attn + t_moe > budget_s:
            break
    U = len(set(int(e) for e in gi.reshape(-1)))
    per_expert = t_moe / max(len(used), 1)
    est = t_attn + per_expert * U
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": est * 1e6, "unit": "us/layer", "cores": threads, "kind": "oracle",
            "sample": f"attention+routing for all {w.T} tokens ({t_attn:.2f}s) + expert block for tokens "
                      f"{toks[0]}..{toks[-1]} ({len(used)} distinct experts, {t_moe:.2f}s), scaled to the "
                      f"{U} distinct experts of the step; fp64 NumPy"}


ACCEPTED_PER_STEP = 6.6  # tokens accepted per verify step of 16 (the pages' acceptance length)


def stack_bench(steps: int, warmup: int):
    """One GPU's TP8 share of the 62-layer stack, timed as 62 back-to-back layer launches per
    verify step (distinct weights per layer, so nothing is warm in the 256 MB last-level cache;
    each layer's y is the next layer's x).  Returns a dict for the JSON line."""
    import torch
    from moe_layer_persistent_amd import binding, synth

    w = synth.WORKLOADS["stack_tp8"]
    dev = torch.device("cuda")
    plan = binding.Plan(binding.config_from_workload(w))
    layers, caches = [], []
    t_gen = time.perf_counter()
    x0 = None
    for l in range(w.n_layers):
        t = synth.make_layer(w, l, dev)
        layers.append(plan.pack_layer(t))
        caches.append((t["k_cache"], t["v_cache"]))
        if l == 0:
            x0 = t["x"].contiguous()
        del t
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    stream = torch.cuda.current_stream()
    bufs = [x0.clone(), torch.empty_like(x0)]

    def step():
        bufs[0].copy_(x0)
        for l in range(w.n_layers):
            xin, yout = bufs[l % 2], bufs[(l + 1) % 2]
            plan.layer_decode(layers[l], caches[l][0], caches[l][1], xin, w.pos, w.layer_window(l), yout,
                              stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    st = plan.status()
    assert st == 0, binding.status_string(st)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    st = plan.status()
    assert st == 0, binding.status_string(st)
    step_us = a.elapsed_time(b) * 1e3 / steps
    out = {"workload": w.name, "layers": w.n_layers, "global_layers": sum(w.layer_window(l) == 0 for l in range(w.n_layers)),
           "kv_history": w.pos, "T": w.T, "verify_step_us": round(step_us, 1),
           "us_per_layer": round(step_us / w.n_layers, 2),
           "tokens_per_s": round(ACCEPTED_PER_STEP / (step_us * 1e-6), 1),
           "tokens_per_s_note": f"{ACCEPTED_PER_STEP} accepted tokens per verify step / the 62-layer verify time "
                                "(one GPU's share; no draft, embedding, LM head or collectives)",
           "weights_GB": round(sum(lw.nbytes() for lw in layers) / 1e9, 1), "setup_s": round(t_gen, 1),
           "steps": steps}
    del layers, caches, bufs
    plan.close()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="swa_fp4")
    ap.add_argument("--routing", default="iid")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 62-layer stack timing")
    ap.add_argument("--dump-stamps", default=None, help="write the per-workgroup timestamps (.npy)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU sharding is a design note, not a measured path)"}))
        sys.exit(2)

    import numpy as np
    import torch
    from moe_layer_persistent_amd import binding, synth

    w = synth.WORKLOADS[args.workload]
    assert w.n_layers == 1, "stack workloads are timed by bench_stack"
    window = w.layer_window(0)
    dev = torch.device("cuda")
    t = synth.make_layer(w, 0, dev, routing=args.routing)
    plan = binding.Plan(binding.config_from_workload(w))
    # a second plan for the same weights with the SwiGLU output gathered in fp4 (created beside
    # the first, before the weights are packed, so that both workspaces are allocated alike)
    plan_a4 = None
    if w.expert_dtype == synth.NVFP4 and w.down_input == synth.DOWN_EXACT:
        plan_a4 = binding.Plan(binding.config_from_workload(w.with_(down_input=synth.DOWN_NVFP4)))
    copies = [plan.pack_layer(t), plan.pack_layer(t)]
    T = w.T
    x = t["x"].contiguous()
    kc = t["k_cache"].clone()
    vc = t["v_cache"].clone()
    y = torch.empty((T, w.hidden), dtype=torch.float32, device=dev)
    dbg = {"expert_idx": torch.zeros((T, w.top_k), dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream()
    plan.layer_decode(copies[0], kc, vc, x, w.pos, window, y, dbg=dbg, stream=stream)
    torch.cuda.synchronize()
    assert plan.status() == 0
    idx = dbg["expert_idx"].cpu().numpy()
    alg_bytes, U = algorithmic_bytes(w, idx, w.pos, window, T)

    def timed(fused, steps, warmup, parents=None, pl=None, cps=None):
        """Back-to-back launches between two events on the launch stream: the average launch
        duration (us) over the timed region, and the host wall time (s)."""
        pl = plan if pl is None else pl
        cps = copies if cps is None else cps
        for i in range(warmup):
            pl.layer_decode(cps[i % 2], kc, vc, x, w.pos, window, y, fused=fused, stream=stream,
                            parents=parents)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(stream)
        for i in range(steps):
            pl.layer_decode(cps[i % 2], kc, vc, x, w.pos, window, y, fused=fused, stream=stream,
                            parents=parents)
        b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return a.elapsed_time(b) * 1e3 / steps, wall

    def per_launch(fused, steps):
        """Event pairs around single launches (spread of launch times; includes dispatch gaps)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record(stream)
            plan.layer_decode(copies[i % 2], kc, vc, x, w.pos, window, y, fused=fused, stream=stream)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]

    mean_us, wall = timed(True, args.steps, args.warmup)
    st = plan.status()
    assert st == 0, binding.status_string(st)
    ms_per_step = wall * 1e3 / args.steps
    durs = per_launch(True, max(5, args.steps // 2))
    # the same weights with the SwiGLU output gathered in fp4 before the down projection (the
    # payload of the N-sharded layout's first all-gather), through a plan configured for it
    a4_us = None
    if plan_a4 is not None:
        cps_a4 = [binding.LayerWeights(c.packed, dict(c.ts, act=t["act_ts"].contiguous())) for c in copies]
        a4_us, _ = timed(True, args.steps, args.warmup, pl=plan_a4, cps=cps_a4)
        st = plan_a4.status()
        assert st == 0, binding.status_string(st)
        plan_a4.close()
    # the same launches through the cooperative launch API (guaranteed residency on a shared
    # device), for comparison: the runtime adds a gap between consecutive cooperative launches
    plan.set_launch(binding.MOEL_LAUNCH_COOPERATIVE)
    coop_us, _ = timed(True, max(5, args.steps // 2), 2)
    plan.set_launch(binding.MOEL_LAUNCH_PLAIN)
    # and with barriers whose acquire also invalidates the L2 (the memory model's agent-scope
    # acquire), for comparison with the L1-only acquire taken where the L2s are coherent
    plan.set_acquire(binding.MOEL_ACQUIRE_L2_INVALIDATE)
    inv_us, _ = timed(True, max(5, args.steps // 2), 2)
    plan.set_acquire(binding.MOEL_ACQUIRE_AUTO)
    # the same step as a token-tree verify (16 nodes: two branches off the root, one branching
    # again), which moves only positions and the attention mask
    tree_us, _ = timed(True, max(5, args.steps // 2), 2, parents=TREE16)
    gbps = alg_bytes / (mean_us * 1e-6) / 1e9
    traffic = measured_traffic(w.name)
    result = {
        "metric": "us per decoder layer at T=16 verify + achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(mean_us, 2),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4-e2m1/e4m3 experts, bf16 weights+KV, fp32 accumulate" if w.expert_dtype == 0
        else "bf16 weights+KV, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) activations / KV history, N(0,0.02) weights)",
        "config": {"workload": w.name, "T": T, "hidden": w.hidden, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "window": window, "kv_history": w.pos,
                   "experts": w.n_experts, "top_k": w.top_k, "pooled": w.pooled, "inter": w.inter,
                   "routing": args.routing, "distinct_experts": U, "weight_copies_rotated": 2,
                   "launch": "plain",
                   "barrier_acquire": "L1 only (XCD L2s coherent)" if plan.l2_coherent else "L1 + L2 invalidate"},
        "latency_us": {"mean_back_to_back": round(mean_us, 2),
                       "single_launch_median": round(statistics.median(durs), 2),
                       "single_launch_p10": round(float(np.percentile(durs, 10)), 2),
                       "single_launch_p90": round(float(np.percentile(durs, 90)), 2),
                       "cooperative_launch_back_to_back": round(coop_us, 2),
                       "l2_invalidating_acquire_back_to_back": round(inv_us, 2),
                       "token_tree_verify_back_to_back": round(tree_us, 2),
                       "fp4_gathered_down_input_back_to_back": None if a4_us is None else round(a4_us, 2)},
        "achieved_GBps": round(gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else int(traffic["bytes_per_launch"]),
                     "algorithmic_bytes_per_launch": int(alg_bytes),
                     "kernel": "k_layer_fused (one launch per layer, one workgroup per CU)"},
    }
    # per-phase timeline of one fused launch (workgroup timestamps, 100 MHz clock): slot i is
    # the end of step i, slot 16 + i its start (after the preceding grid barrier)
    names = ["norm1", "qkv_rope_kv", "attention", "attn_merge", "o_proj", "router_pool", "experts_gate_up",
             "experts_down", "combine", "unpool"]
    ts = torch.zeros((plan.workgroups, binding.MOEL_N_STAMPS), dtype=torch.int64, device=dev)
    plan.layer_decode(copies[0], kc, vc, x, w.pos, window, y, dbg={"timestamps": ts}, stream=stream)
    torch.cuda.synchronize()
    tsn = ts.cpu().numpy().astype(np.float64)
    if args.dump_stamps:
        np.save(args.dump_stamps + "_fused.npy", ts.cpu().numpy())
        ts.zero_()
        plan.layer_decode(copies[1], kc, vc, x, w.pos, window, y, dbg={"timestamps": ts}, fused=False,
                          stream=stream)
        torch.cuda.synchronize()
        np.save(args.dump_stamps + "_unfused.npy", ts.cpu().numpy())
        np.save(args.dump_stamps + "_idx.npy", idx)
    t0 = tsn[:, 10].min()
    ends = [(tsn[:, i].max() - t0) / 100.0 for i in range(10)]
    result["phase_end_us"] = {n: round(e, 1) for n, e in zip(names, ends)}
    result["phase_us"] = {n: round(e - (ends[i - 1] if i else 0.0), 1) for i, (n, e) in enumerate(zip(names, ends))}
    work = (tsn[:, :10] - tsn[:, 16:26]) / 100.0
    result["phase_work_us"] = {n: {"median": round(float(np.median(work[:, i])), 1),
                                   "max": round(float(work[:, i].max()), 1)} for i, n in enumerate(names)}
    # grid barrier before step i: last arrival -> first / last departure
    result["barrier_us"] = {names[i]: {"first_out": round((tsn[:, 16 + i].min() - tsn[:, i - 1].max()) / 100.0, 2),
                                       "last_out": round((tsn[:, 16 + i].max() - tsn[:, i - 1].max()) / 100.0, 2)}
                            for i in range(1, 10)}
    if traffic is not None:
        result["roofline"]["traffic_source"] = traffic["source"]
    if not args.no_unfused:
        u_us, _ = timed(False, max(5, args.steps // 2), 2)
        result["unfused_chain_us"] = {"mean_back_to_back": round(u_us, 2), "launches": 10}
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    del copies
    torch.cuda.empty_cache()
    if not args.no_stack:
        result["stack"] = stack_bench(steps=3, warmup=1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, t, idx, window)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
