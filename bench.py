"""Benchmark of one MoE decoder layer's batch-1 verify step (T = 16) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload swa_fp4] [--routing iid|shared|pages]

A step is one persistent launch of the whole layer over one batch of 16 synthetic verify
tokens.  Inputs are resident in HBM before timing starts.  To keep the 256 MB Infinity
Cache from serving weights across steps, consecutive steps alternate between two packed
copies of the layer's weights (so each step's weights were last touched two steps ago and
>7 GB have streamed in between).  Prints one JSON line.

Beside the headline workload (`value`, `roofline`), the line carries every other layer
configuration timed the same way, each with its own algorithmic bytes and fraction of the
HBM peak (`configs`), the 62-layer stack share (`stack`, fused and one kernel per step),
the headline layer with the pages' routing concentration (`routing_pages`, about 49 distinct
experts), the same 16 rows as four requests of four tokens in one batched step
(`batched_verify`), a 32-token step (`verify_32_tokens`), and the CPU oracle timed on
a bounded sample of the headline step (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

PEAK_HBM_GBPS = 8000.0
ACCEPTED_PER_STEP = 6.6  # tokens accepted per verify step of 16 (the pages' acceptance length)
# a 16-node token tree: node t's parent (-1: root)
TREE16 = [-1, 0, 1, 2, 0, 4, 5, 1, 7, 3, 9, 4, 11, 12, 2, 14]
PHASES = ["norm1", "qkv_rope_kv", "attention", "attn_merge", "o_proj", "router_pool", "experts_gate_up",
          "experts_down", "combine", "unpool"]


def algorithmic_bytes(w, idx, pos, window, T, requests=None):
    """Bytes the step must move at least once: every weight byte it uses (dense weights, the
    routed experts' matrices), the visible KV window, x, y and the KV writes.  requests: the
    (T, pos, kv_base, kv_slots) requests of a batched step, each reading its own window (pos and
    T are then ignored)."""
    H, D, Hq, Hkv, P, I = w.hidden, w.head_dim, w.n_q_heads, w.n_kv_heads, w.pooled, w.inter
    dense = 2 * (w.qkv_rows * H + H * Hq * D + w.n_experts * H + P * H + H * P + 2 * H)
    if w.expert_dtype == 0:
        per_elem = 0.5 + 1.0 / 16.0
    else:
        per_elem = 2.0
    expert = per_elem * (2 * w.inter_local * P + w.pooled_local * I)
    U = len(set(int(e) for e in idx.reshape(-1)))
    reqs = [(T, pos)] if requests is None else [(r[0], r[1]) for r in requests]
    kv_read = 0
    for T_r, pos_r in reqs:
        lo = max(0, pos_r - window + 1) if window > 0 else 0
        kv_read += (pos_r + T_r - lo) * Hkv * D * 2 * 2
    T = sum(r[0] for r in reqs)
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, t, idx, window, repeats=3):
    """The oracle, timed on this host's cores on a bounded sample of the same step: the whole
    attention block and routing for all 16 tokens, plus the expert block of token 0 (its
    experts dequantised and applied), scaled to one full layer by the distinct experts of the
    step.  Median of `repeats` runs with every core available to the BLAS, and again with one
    thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import layer as olayer

    dims = olayer.Dims(w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.pooled, w.inter,
                       w.n_experts, w.top_k, w.n_shards, w.shard_rank, w.rms_eps, w.rope_theta)
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
    U = len(set(int(e) for e in gi.reshape(-1)))
    n0 = len(set(int(e) for e in gi[0]))

    def one():
        t0 = time.perf_counter()
        olayer.layer_step(inp, dims, w.pos, window, ex, force_idx=gi, moe_tokens=[])
        t_attn = time.perf_counter() - t0
        t1 = time.perf_counter()
        olayer.layer_step(inp, dims, w.pos, window, ex, force_idx=gi, moe_tokens=[0])
        t_moe = max(time.perf_counter() - t1 - t_attn, 0.0)
        return t_attn + t_moe / n0 * U, t_attn, t_moe

    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    with threadpool_limits(threads):
        all_runs = [one() for _ in range(repeats)]
    with threadpool_limits(1):
        one_runs = [one() for _ in range(repeats)]
    med = lambda runs: statistics.median(r[0] for r in runs)
    return {"value": round(med(all_runs) * 1e6, 1), "unit": "us/layer", "cores": threads, "kind": "oracle",
            "value_1_thread": round(med(one_runs) * 1e6, 1),
            "cpu_model": cpu_model(), "repeats": repeats,
            "sample": f"fp64 NumPy oracle of the {w.name} step: attention block and routing for all {w.T} tokens "
                      f"({statistics.median(r[1] for r in all_runs):.2f}s) + the expert block of token 0 "
                      f"({n0} experts, {statistics.median(r[2] for r in all_runs):.2f}s), scaled to the {U} distinct "
                      f"experts of the step; median of {repeats} runs with {threads} BLAS threads (value) and with 1 "
                      f"thread (value_1_thread)"}


class LayerBench:
    """One layer workload on the GPU: inputs, two packed weight copies, a plan; times launches."""

    def __init__(self, w, routing="iid", layer=0, copies=2):
        import torch
        from moe_layer_persistent_amd import binding, synth
        self.torch, self.binding, self.synth = torch, binding, synth
        self.w = w
        self.window = w.layer_window(layer)
        self.dev = torch.device("cuda")
        self.t = synth.make_layer(w, layer, self.dev, routing=routing)
        self.plan = binding.Plan(binding.config_from_workload(w))
        self.extra_plans = []
        self.copies = [self.plan.pack_layer(self.t) for _ in range(copies)]
        self.x = self.t["x"].contiguous()
        self.kc = self.t["k_cache"].clone()
        self.vc = self.t["v_cache"].clone()
        self.y = torch.empty((w.T, w.hidden), dtype=torch.float32, device=self.dev)
        self.stream = torch.cuda.current_stream()

    def settle(self, seconds=0.3):
        """Untimed launches for a fixed time before the first measurement, so that the device's
        clocks and power state have settled (the first launches on a fresh box run slower)."""
        torch = self.torch
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(8):
                self.plan.layer_decode(self.copies[i % len(self.copies)], self.kc, self.vc, self.x, self.w.pos,
                                       self.window, self.y, stream=self.stream)
                i += 1
            torch.cuda.synchronize()

    def route(self, x=None, requests=None, pos=None):
        """Runs one step with debug outputs; returns the selected experts [T, k]."""
        torch = self.torch
        x = self.x if x is None else x
        T = x.shape[0] if requests is None else sum(r[0] for r in requests)
        idx = torch.zeros((T, self.w.top_k), dtype=torch.int32, device=self.dev)
        y = torch.empty((T, self.w.hidden), dtype=torch.float32, device=self.dev)
        if requests is None:
            self.plan.layer_decode(self.copies[0], self.kc, self.vc, x, self.w.pos if pos is None else pos,
                                   self.window, y, dbg={"expert_idx": idx}, stream=self.stream)
        else:
            self.plan.layer_decode_batch(self.copies[0], self.kc, self.vc, x, requests, self.window, y,
                                         dbg={"expert_idx": idx}, stream=self.stream)
        torch.cuda.synchronize()
        st = self.plan.status()
        assert st == 0, self.binding.status_string(st)
        return idx.cpu().numpy()

    def timed(self, steps, warmup, fused=True, parents=None, pl=None, cps=None, x=None, requests=None, pos=None):
        """Back-to-back launches between two events on the launch stream: the average launch
        duration (us) over the timed region, and the host wall time (s).  requests: time the
        batched step over these (T, pos, kv_base, kv_slots) requests instead; x, pos: another
        step's rows (T = its row count) and history."""
        torch = self.torch
        pl = self.plan if pl is None else pl
        cps = self.copies if cps is None else cps
        x = self.x if x is None else x
        w = self.w
        pos = w.pos if pos is None else pos
        y = self.y if x.shape[0] == self.y.shape[0] else torch.empty((x.shape[0], w.hidden), dtype=torch.float32,
                                                                       device=self.dev)

        def launch(i):
            if requests is None:
                pl.layer_decode(cps[i % len(cps)], self.kc, self.vc, x, pos, self.window, y, fused=fused,
                                stream=self.stream, parents=parents)
            else:
                pl.layer_decode_batch(cps[i % len(cps)], self.kc, self.vc, x, requests, self.window, y,
                                      fused=fused, stream=self.stream)
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record(self.stream)
        for i in range(steps):
            launch(i)
        b.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        st = pl.status()
        assert st == 0, self.binding.status_string(st)
        return a.elapsed_time(b) * 1e3 / steps, wall

    def per_launch(self, steps):
        """Event pairs around single launches (spread of launch times; includes dispatch gaps)."""
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            evs[i][0].record(self.stream)
            self.plan.layer_decode(self.copies[i % 2], self.kc, self.vc, self.x, self.w.pos, self.window, self.y,
                                   stream=self.stream)
            evs[i][1].record(self.stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]

    def phases(self, dump=None, idx=None):
        """Per-phase timeline of one fused launch (workgroup timestamps, 100 MHz clock): slot i is
        the end of step i, slot 16 + i its start (after the preceding grid barrier)."""
        import numpy as np
        torch = self.torch
        ts = torch.zeros((self.plan.workgroups, self.binding.MOEL_N_STAMPS), dtype=torch.int64, device=self.dev)
        self.plan.layer_decode(self.copies[0], self.kc, self.vc, self.x, self.w.pos, self.window, self.y,
                               dbg={"timestamps": ts}, stream=self.stream)
        torch.cuda.synchronize()
        tsn = ts.cpu().numpy().astype(np.float64)
        if dump:
            np.save(dump + "_fused.npy", ts.cpu().numpy())
            ts.zero_()
            self.plan.layer_decode(self.copies[1], self.kc, self.vc, self.x, self.w.pos, self.window, self.y,
                                   dbg={"timestamps": ts}, fused=False, stream=self.stream)
            torch.cuda.synchronize()
            np.save(dump + "_unfused.npy", ts.cpu().numpy())
            if idx is not None:
                np.save(dump + "_idx.npy", idx)
        t0 = tsn[:, 10].min()
        ends = [(tsn[:, i].max() - t0) / 100.0 for i in range(10)]
        work = (tsn[:, :10] - tsn[:, 16:26]) / 100.0
        return {
            "phase_end_us": {n: round(e, 1) for n, e in zip(PHASES, ends)},
            "phase_us": {n: round(e - (ends[i - 1] if i else 0.0), 1) for i, (n, e) in enumerate(zip(PHASES, ends))},
            "phase_work_us": {n: {"median": round(float(np.median(work[:, i])), 1), "max": round(float(work[:, i].max()), 1)}
                              for i, n in enumerate(PHASES)},
            # grid barrier before step i: last arrival -> first / last departure
            "barrier_us": {PHASES[i]: {"first_out": round((tsn[:, 16 + i].min() - tsn[:, i - 1].max()) / 100.0, 2),
                                       "last_out": round((tsn[:, 16 + i].max() - tsn[:, i - 1].max()) / 100.0, 2)}
                           for i in range(1, 10)},
        }

    def close(self):
        for p in [self.plan] + self.extra_plans:
            p.close()
        self.copies = []
        self.t = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def stamp_table(tsn, fused=True):
    """Phase timeline from workgroup timestamps [nwg, 32] (100 MHz): slot i the end of step i,
    slot 16 + i its start.  Fused: each phase's time runs from the previous phase's last end (the
    grid barrier included) to its own last end.  One kernel per step: each kernel's own span
    (first start to last end), and the gap from the previous kernel's last end to its first
    start."""
    import numpy as np
    if fused:
        t0 = tsn[:, 10].min()
        ends = [(tsn[:, i].max() - t0) / 100.0 for i in range(10)]
        return {n: round(e - (ends[i - 1] if i else 0.0), 1) for i, (n, e) in enumerate(zip(PHASES, ends))}
    out, prev_end = {}, None
    for i in range(1, 10):
        st, en = tsn[:, 16 + i].min(), tsn[:, i].max()
        out[PHASES[i]] = round((en - st) / 100.0, 1)
        if prev_end is not None:
            out["gap_before_" + PHASES[i]] = round((st - prev_end) / 100.0, 1)
        prev_end = en
    return out


def roofline_entry(w, alg_bytes, U, us, traffic=None):
    gbps = alg_bytes / (us * 1e-6) / 1e9
    out = {"us_per_layer": round(us, 2), "algorithmic_bytes_per_launch": int(alg_bytes), "distinct_experts": U,
           "achieved_GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
           "traffic": None if traffic is None else int(traffic["bytes_per_launch"])}
    if traffic is not None:
        out["traffic_source"] = traffic["source"]
    return out


def config_bench(name, steps, warmup, unfused=False):
    """Another layer configuration, timed like the headline one: µs per layer and its roofline."""
    from moe_layer_persistent_amd import synth
    w = synth.WORKLOADS[name]
    lb = LayerBench(w)
    idx = lb.route()
    alg, U = algorithmic_bytes(w, idx, w.pos, lb.window, w.T)
    lb.settle()
    us, _ = lb.timed(steps, warmup)
    out = roofline_entry(w, alg, U, us, measured_traffic(name))
    out.update(window=lb.window, kv_history=w.pos, experts=("nvfp4" if w.expert_dtype == 0 else "bf16"))
    if unfused:
        out["unfused_chain_us"] = round(lb.timed(max(3, steps // 2), 2, fused=False)[0], 2)
    lb.close()
    return out


def progress(msg):
    """A progress line on stderr (the JSON result is the only stdout line)."""
    print(msg, file=sys.stderr, flush=True)


def copy_calibration_run(dev):
    """Three plain 1 GiB device-to-device copies: the reference that the HBM counters of a
    profiling run are scaled by."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def stack_bench(steps: int, warmup: int, copy_calibration: bool = False, unfused: bool = True,
                extras: bool = True):
    """One GPU's TP8 share of the 62-layer stack, timed as 62 back-to-back layer launches per
    verify step (distinct weights per layer, so nothing is warm in the 256 MB last-level cache;
    each layer's y is the next layer's x), fused and as the one-kernel-per-step chain.  The
    algorithmic bytes are summed over the layers, each with the experts its own routing used.
    unfused / extras: also time the one-kernel-per-step chain / the multi-layer launch and the
    phase timelines.  Progress goes to stderr."""
    import numpy as np
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
        if l % 8 == 7:
            progress(f"stack: {l + 1} layers generated")
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    progress(f"stack: {w.n_layers} layers generated and packed in {t_gen:.1f} s")
    stream = torch.cuda.current_stream()
    bufs = [x0.clone(), torch.empty_like(x0)]

    def step(fused=True, idx=None, x=None):
        bufs[0].copy_(x0 if x is None else x)
        for l in range(w.n_layers):
            xin, yout = bufs[l % 2], bufs[(l + 1) % 2]
            dbg = None if idx is None else {"expert_idx": idx[l]}
            plan.layer_decode(layers[l], caches[l][0], caches[l][1], xin, w.pos, w.layer_window(l), yout,
                              fused=fused, stream=stream, dbg=dbg)

    # one step with the routing of every layer recorded, for the algorithmic bytes
    idx = [torch.zeros((w.T, w.top_k), dtype=torch.int32, device=dev) for _ in range(w.n_layers)]
    step(idx=idx)
    torch.cuda.synchronize()
    alg, us_l = 0, []
    for l in range(w.n_layers):
        b, U = algorithmic_bytes(w, idx[l].cpu().numpy(), w.pos, w.layer_window(l), w.T)
        alg += b
        us_l.append(U)

    def timed(fused, n, wu):
        for _ in range(wu):
            step(fused)
        torch.cuda.synchronize()
        st = plan.status()
        assert st == 0, binding.status_string(st)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            step(fused)
        b.record(stream)
        torch.cuda.synchronize()
        st = plan.status()
        assert st == 0, binding.status_string(st)
        return a.elapsed_time(b) * 1e3 / n

    timed(True, max(2, min(10, 2 * steps)), 0)  # untimed: settles clocks and power state
    progress("stack: settled")
    step_us = timed(True, steps, warmup)
    progress(f"stack: fused {step_us / w.n_layers:.1f} us/layer")
    unfused_us = None
    if unfused:
        unfused_us = timed(False, max(2, steps // 2), 1)
        progress(f"stack: one kernel per step {unfused_us / w.n_layers:.1f} us/layer")
    stack_us, phases, prefetch = None, {}, None
    if extras:
        # previous-step expert prefetch (the 14 experts each layer's previous step used most,
        # ~50 MB per layer at this share): every step with the same input rows (the routing the
        # prefetch bets on repeats exactly), and steps alternating between two inputs (the bet
        # is lost more often)
        hists = [torch.zeros(w.n_experts, dtype=torch.int32, device=dev) for _ in range(w.n_layers)]
        for lw, h in zip(layers, hists):
            lw.set_history(h)
        plan.set_expert_prefetch(14)
        same_us = timed(True, steps, warmup)
        x_alt = (0.5 * x0.flip(0)).contiguous()

        def timed_alt(n):
            for i in range(2):
                step(True, x=x0 if i % 2 else x_alt)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(n):
                step(True, x=x0 if i % 2 else x_alt)
            b.record(stream)
            torch.cuda.synchronize()
            st = plan.status()
            assert st == 0, binding.status_string(st)
            return a.elapsed_time(b) * 1e3 / n
        alt_us = timed_alt(max(2, steps))
        plan.set_expert_prefetch(0)
        off_alt_us = timed_alt(max(2, steps))
        for lw in layers:
            lw.set_history(None)
        del hists
        prefetch = {"experts": 14, "us_per_layer_same_routing": round(same_us / w.n_layers, 2),
                    "us_per_layer_alternating_inputs": round(alt_us / w.n_layers, 2),
                    "us_per_layer_alternating_inputs_off": round(off_alt_us / w.n_layers, 2),
                    "us_per_layer_off": round(step_us / w.n_layers, 2)}
        progress(f"stack: expert prefetch {prefetch}")
        # the stack through moel_stack_decode: binding.STACK_LAYERS_PER_LAUNCH layers per persistent
        # launch (grid barriers between them)
        stk = binding.Stack(plan, layers, [c[0] for c in caches], [c[1] for c in caches],
                            [w.layer_window(l) for l in range(w.n_layers)])
        ys = torch.empty_like(x0)
        for _ in range(warmup + 2):
            stk.decode(x0, w.pos, ys, stream=stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            stk.decode(x0, w.pos, ys, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        st = plan.status()
        assert st == 0, binding.status_string(st)
        stack_us = a.elapsed_time(b) * 1e3 / steps
        stk.close()
        progress(f"stack: multi-layer launch {stack_us / w.n_layers:.1f} us/layer")
        # per-phase timelines of a global layer (0) and a sliding-window layer (1), fused and as
        # one kernel per step
        for l in (0, 1):
            for fused in (True, False):
                ts = torch.zeros((plan.workgroups, binding.MOEL_N_STAMPS), dtype=torch.int64, device=dev)
                plan.layer_decode(layers[l], caches[l][0], caches[l][1], bufs[0], w.pos, w.layer_window(l),
                                  bufs[1], fused=fused, stream=stream, dbg={"timestamps": ts})
                torch.cuda.synchronize()
                key = f"layer{l}_{'global' if w.layer_window(l) == 0 else 'swa'}_{'fused' if fused else 'unfused'}"
                phases[key] = stamp_table(ts.cpu().numpy().astype(np.float64), fused)
    gbps = alg / (step_us * 1e-6) / 1e9
    traffic = measured_traffic("stack_tp8")
    out = {"workload": w.name, "layers": w.n_layers,
           "global_layers": sum(w.layer_window(l) == 0 for l in range(w.n_layers)),
           "kv_history": w.pos, "T": w.T, "verify_step_us": round(step_us, 1),
           "us_per_layer": round(step_us / w.n_layers, 2),
           "tokens_per_s": round(ACCEPTED_PER_STEP / (step_us * 1e-6), 1),
           "tokens_per_s_note": f"{ACCEPTED_PER_STEP} accepted tokens per verify step / the 62-layer verify time "
                                "(one GPU's share; no draft, embedding, LM head or collectives)",
           "algorithmic_bytes_per_step": int(alg), "algorithmic_bytes_per_layer": int(alg / w.n_layers),
           "distinct_experts_mean": round(sum(us_l) / len(us_l), 1),
           "achieved_GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4),
           "traffic_per_launch": None if traffic is None else int(traffic["bytes_per_launch"]),
           "weights_GB": round(sum(lw.nbytes() for lw in layers) / 1e9, 1), "setup_s": round(t_gen, 1),
           "steps": steps}
    if unfused_us is not None:
        out["unfused_chain"] = {"verify_step_us": round(unfused_us, 1),
                                "us_per_layer": round(unfused_us / w.n_layers, 2), "launches_per_layer": 10}
    if prefetch is not None:
        out["expert_prefetch"] = prefetch
    if stack_us is not None:
        out["stack_launches"] = {"verify_step_us": round(stack_us, 1), "us_per_layer": round(stack_us / w.n_layers, 2),
                                 "tokens_per_s": round(ACCEPTED_PER_STEP / (stack_us * 1e-6), 1),
                                 "achieved_GBps": round(alg / (stack_us * 1e-6) / 1e9, 1),
                                 "frac": round(alg / (stack_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                                 "note": f"moel_stack_decode: {binding.STACK_LAYERS_PER_LAUNCH} layers per persistent launch "
                                         f"({-(-w.n_layers // binding.STACK_LAYERS_PER_LAUNCH)} launches per step)"}
        out["phase_us"] = phases
    del layers, caches, bufs
    plan.close()
    torch.cuda.empty_cache()
    if copy_calibration:
        copy_calibration_run(dev)
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
    ap.add_argument("--no-configs", action="store_true", help="skip the other full-width layer configurations")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline launches (no launch-mode, tree, fp4-gather or routing variants)")
    ap.add_argument("--dump-stamps", default=None, help="write the per-workgroup timestamps (.npy)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer step runs on one GPU only; --gpus must be 1 "
                                   "(sharding over several GPUs is described, not built)"}))
        sys.exit(2)

    import numpy as np
    import torch
    from moe_layer_persistent_amd import binding, synth

    w = synth.WORKLOADS[args.workload]
    if w.n_layers != 1:
        stack = stack_bench(steps=max(1, args.steps // 5), warmup=1, copy_calibration=args.copy_calibration,
                            unfused=not args.no_unfused, extras=not args.no_extras)
        print(json.dumps({"metric": "us per decoder layer at T=16 verify + achieved HBM GB/s (% of peak), 1 GPU",
                          "value": stack["us_per_layer"], "unit": "us/layer", "n_gpus": 1, "stack": stack}))
        return
    lb = LayerBench(w, routing=args.routing)
    # a second plan for the same weights with the SwiGLU output gathered in fp4 (created beside
    # the first, before timing, so that both workspaces are allocated alike)
    plan_a4 = None
    if not args.no_extras and w.expert_dtype == synth.NVFP4 and w.down_input == synth.DOWN_EXACT:
        plan_a4 = binding.Plan(binding.config_from_workload(w.with_(down_input=synth.DOWN_NVFP4)))
        lb.extra_plans.append(plan_a4)
    T = w.T
    idx = lb.route()
    alg_bytes, U = algorithmic_bytes(w, idx, w.pos, lb.window, T)
    lb.settle()

    mean_us, wall = lb.timed(args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    durs = lb.per_launch(max(5, args.steps // 2))
    gbps = alg_bytes / (mean_us * 1e-6) / 1e9
    traffic = measured_traffic(w.name)
    latency = {"mean_back_to_back": round(mean_us, 2),
               "single_launch_median": round(statistics.median(durs), 2),
               "single_launch_p10": round(float(np.percentile(durs, 10)), 2),
               "single_launch_p90": round(float(np.percentile(durs, 90)), 2)}
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
        "dtype": "bf16",  # the MFMA operand type of every contraction (fp32 accumulation)
        "dtype_detail": "NVFP4 (E2M1 codes, E4M3 block scales) experts decoded to bf16 in registers; bf16 "
                        "weights and KV cache; fp32 accumulation, softmax and residual stream" if w.expert_dtype == 0
        else "bf16 experts, weights and KV cache; fp32 accumulation, softmax and residual stream",
        "data": "synthetic (seeded N(0,1) activations / KV history, N(0,0.02) weights)",
        "config": {"workload": w.name, "T": T, "hidden": w.hidden, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "window": lb.window, "kv_history": w.pos,
                   "experts": w.n_experts, "top_k": w.top_k, "pooled": w.pooled, "inter": w.inter,
                   "routing": args.routing, "distinct_experts": U, "weight_copies_rotated": 2,
                   "launch": "plain",
                   "barrier_acquire": "L1 only (L2 coherence check passed)" if lb.plan.l2_coherent else "L1 + L2 invalidate"},
        "latency_us": latency,
        "achieved_GBps": round(gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else int(traffic["bytes_per_launch"]),
                     "algorithmic_bytes_per_launch": int(alg_bytes),
                     "kernel": "k_layer_fused (one launch per layer, one workgroup per CU)"},
    }
    if traffic is not None:
        result["roofline"]["traffic_source"] = traffic["source"]
    if not args.no_extras:
        # the same weights with the SwiGLU output gathered in fp4 before the down projection (the
        # payload of the N-sharded layout's first all-gather), through a plan configured for it
        if plan_a4 is not None:
            cps_a4 = [binding.LayerWeights(c.packed, dict(c.ts, act=lb.t["act_ts"].contiguous())) for c in lb.copies]
            latency["fp4_gathered_down_input_back_to_back"] = round(
                lb.timed(args.steps, args.warmup, pl=plan_a4, cps=cps_a4)[0], 2)
        # the cooperative launch API (guaranteed residency on a shared device): the runtime adds a
        # gap between consecutive cooperative launches
        lb.plan.set_launch(binding.MOEL_LAUNCH_COOPERATIVE)
        latency["cooperative_launch_back_to_back"] = round(lb.timed(max(5, args.steps // 2), 2)[0], 2)
        lb.plan.set_launch(binding.MOEL_LAUNCH_PLAIN)
        # barriers whose acquire also invalidates the L2 (the memory model's agent-scope acquire)
        lb.plan.set_acquire(binding.MOEL_ACQUIRE_L2_INVALIDATE)
        latency["l2_invalidating_acquire_back_to_back"] = round(lb.timed(max(5, args.steps // 2), 2)[0], 2)
        lb.plan.set_acquire(binding.MOEL_ACQUIRE_AUTO)
        # the same step as a token-tree verify, which moves only positions and the attention mask
        latency["token_tree_verify_back_to_back"] = round(lb.timed(max(5, args.steps // 2), 2, parents=TREE16)[0], 2)
        # several requests in one step: the 16 rows as 4 requests of 4 tokens, each with its own
        # history in a quarter of the cache pool (the same weights read once for all of them)
        quarter = w.kv_capacity // 4
        hist = min(w.pos, quarter - 4)
        reqs_b = [(4, hist, r * quarter, quarter) for r in range(4)]
        idx_b = lb.route(requests=reqs_b)
        alg_b, U_b = algorithmic_bytes(w, idx_b, 0, lb.window, 0, requests=reqs_b)
        us_b, _ = lb.timed(max(5, args.steps // 2), 2, requests=reqs_b)
        result["batched_verify"] = dict(roofline_entry(w, alg_b, U_b, us_b),
                                        requests="4 x (T 4, history %d, %d-slot pool quarter)" % (hist, quarter))
        # 32 tokens in one step (two 16-token tiles): the same weights, 32 synthetic rows drawn
        # like the 16, history 16 shorter so that the cache holds the step
        x32 = synth.make_x(w.with_(T=32), 0, lb.dev)
        pos32 = w.pos - 16
        idx_32 = lb.route(x32, pos=pos32)
        alg_32, U_32 = algorithmic_bytes(w, idx_32, pos32, lb.window, 32)
        us_32, _ = lb.timed(max(5, args.steps // 2), 2, x=x32, pos=pos32)
        result["verify_32_tokens"] = dict(roofline_entry(w, alg_32, U_32, us_32), T=32, kv_history=pos32)
        # the pages' routing concentration (a shared component in every token, tuned so that the
        # 16 tokens use about 49 distinct experts): the same weights and caches, other input rows
        if args.routing == "iid":
            xs = synth.make_x(w, 0, lb.dev, routing="pages")
            idx_s = lb.route(xs)
            alg_s, U_s = algorithmic_bytes(w, idx_s, w.pos, lb.window, T)
            us_s, _ = lb.timed(args.steps, args.warmup, x=xs)
            result["routing_pages"] = roofline_entry(w, alg_s, U_s, us_s)
    result.update(lb.phases(args.dump_stamps, idx))
    if not args.no_unfused:
        u_us, _ = lb.timed(max(5, args.steps // 2), 2, fused=False)
        result["unfused_chain_us"] = {"mean_back_to_back": round(u_us, 2), "launches": 10}
    if args.copy_calibration:
        copy_calibration_run(lb.dev)
    t_cpu = lb.t
    lb.close()
    if not args.no_extras:
        # the device's streaming-read bandwidth (16-byte non-temporal loads over 4 GiB, one
        # workgroup per CU): the practical reference beside the nominal peak
        buf = torch.empty(4 << 30, dtype=torch.uint8, device=lb.dev)
        sr = binding.measure_read_bandwidth(buf, reps=10)
        del buf
        torch.cuda.empty_cache()
        result["roofline"]["stream_read_GBps"] = round(sr, 1)
        result["roofline"]["frac_of_stream_read"] = round(gbps / sr, 4)
    if not args.no_configs and w.name == "swa_fp4":
        result["configs"] = {"swa_fp4": roofline_entry(w, alg_bytes, U, mean_us, traffic)}
        for name in ("global_fp4", "swa_bf16"):
            result["configs"][name] = config_bench(name, max(5, args.steps // 2), 2)
    if not args.no_stack:
        result["stack"] = stack_bench(steps=3, warmup=1)
    if not args.no_cpu_baseline:
        lb_t = synth.make_layer(w, 0, "cuda", routing=args.routing) if t_cpu is None else t_cpu
        result["cpu_baseline"] = cpu_baseline(w, lb_t, idx, lb.window)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
