"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Small shapes are compared on every token; the full-width workloads run at their real
sizes in the same launch configuration the benchmark times, with every token's routing
and KV writes checked and the MoE output checked on sampled tokens (the oracle
dequantises only the experts those tokens use).
"""
import numpy as np
import pytest
import torch

from moe_layer_persistent_amd import binding, synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import harness  # noqa: E402  (imports the oracle: tests only)


def _log(msg):
    print(msg, flush=True)


def _same_bytes(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.fixture(scope="module")
def tiny_run():
    return harness.GpuRun(synth.WORKLOADS["tiny"])


@pytest.mark.parametrize("fused", [True, False])
def test_tiny_matches_oracle(tiny_run, fused):
    _log(f"tiny fused={fused}")
    out = tiny_run.run(fused=fused)
    rep = {}
    harness.check_against_oracle(tiny_run, out, report=rep)
    _log(f"tiny fused={fused}: {rep}")


SMALL = [
    dict(),                                                    # T=5, window 40, pos 70, NVFP4
    dict(T=16, pos=300, window=0, expert_dtype=synth.NVFP4),
    dict(T=1, pos=0, window=0),
    dict(T=16, pos=20, window=7, head_dim=128, n_q_heads=4, n_kv_heads=1, hidden=768),
    dict(T=9, pos=600, window=256, expert_dtype=synth.BF16, inter=256),
    dict(T=12, pos=33, window=0, n_shards=2, inter=512, pooled=256),
    dict(T=16, pos=1000, window=300, n_experts=32, top_k=8, pooled=512, inter=512),
    dict(T=16, pos=300, window=0, down_input=synth.DOWN_NVFP4),                 # fp4 gather
    dict(T=7, pos=33, window=20, n_shards=2, inter=512, pooled=256, down_input=synth.DOWN_NVFP4),
    # degenerate and extreme cases: a window of one key (each token sees only itself), a
    # single expert per token, the largest expert count, the smallest widths
    dict(T=16, pos=100, window=1),
    dict(T=8, pos=50, window=0, top_k=1),
    dict(T=16, pos=64, window=0, n_experts=512, top_k=8, pooled=256, inter=256),
    dict(T=3, pos=5, window=0, hidden=256, n_q_heads=2, n_kv_heads=1, pooled=128, inter=128),
    # one GPU's share of N-sharded experts at other ranks than 0 (output slices placed at the
    # rank's offset in the SwiGLU output, the expert outputs and the combine)
    dict(T=16, pos=100, window=32, n_experts=32, top_k=8, n_shards=8, shard_rank=7, inter=512, pooled=512),
    dict(T=11, pos=60, window=0, n_experts=32, top_k=8, n_shards=8, shard_rank=1, inter=512, pooled=512,
         down_input=synth.DOWN_NVFP4),
]


@pytest.mark.parametrize("kw", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_small_matches_oracle(kw):
    w = synth.small_workload(**kw)
    _log(f"small {kw}")
    run = harness.GpuRun(w)
    rep = {}
    harness.check_against_oracle(run, run.run(fused=True), report=rep)
    _log(f"small {kw}: {rep}")


@pytest.mark.parametrize("kw", [dict(), dict(expert_dtype=synth.BF16), dict(down_input=synth.DOWN_NVFP4)],
                         ids=["nvfp4", "bf16", "fp4_gather"])
def test_concentrated_routing_matches_oracle(kw):
    """Routing concentrated on few experts (shared component in every token): experts that
    hold all 16 tokens, i.e. the largest token groups of the expert streams."""
    w = synth.small_workload(T=16, pos=100, window=0, n_experts=32, top_k=8, pooled=512, inter=512, **kw)
    _log(f"concentrated {kw}")
    run = harness.GpuRun(w, routing="shared")
    rep = {}
    out = run.run(fused=True)
    counts = np.bincount(out["expert_idx"].cpu().numpy().ravel(), minlength=w.n_experts)
    assert counts.max() > 8, counts
    harness.check_against_oracle(run, out, report=rep)
    _log(f"concentrated {kw}: {rep}")


@pytest.mark.parametrize("splits", ["2,2,2,2", "4,4,4,4", "8,8,8,8", "16,16,16,16"])
def test_split_k_dense_phases_match_oracle(splits, monkeypatch):
    """Dense phases with their K split over workgroups (partial sums per range, summed in range
    order by the block's last unit), forced for every dense phase (MOEL_DENSE_SPLITS, read when
    the plan is created): against the oracle, deterministic, and fused = unfused bitwise.  16
    ranges give blocks of 12 QKV tiles, two passes of 8 and 4."""
    monkeypatch.setenv("MOEL_DENSE_SPLITS", splits)
    w = synth.small_workload(T=16, pos=300, window=0, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
                             pooled=1024, inter=1024, n_experts=64, top_k=8)
    _log(f"split-K {splits}")
    run = harness.GpuRun(w)
    monkeypatch.delenv("MOEL_DENSE_SPLITS")
    rep = {}
    a = run.run(fused=True)
    harness.check_against_oracle(run, a, report=rep)
    _log(f"split-K {splits}: {rep}")
    b = run.run(fused=True)
    c = run.run(fused=False)
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(a[k], b[k]), k
        assert _same_bytes(a[k], c[k]), k


def test_fused_equals_unfused_and_is_deterministic():
    w = synth.small_workload(T=16, pos=500, window=100, n_experts=32, top_k=8, pooled=512, inter=512)
    run = harness.GpuRun(w)
    a = run.run(fused=True)
    b = run.run(fused=True)
    c = run.run(fused=False)
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(a[k], b[k]), k
        assert _same_bytes(a[k], c[k]), k


# (id, workload overrides, call T, call pos, forced dense splits)
POISON = [
    ("nvfp4", dict(T=5), 5, 70, None),
    ("split_k", dict(T=16, pos=300, window=0, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
                     pooled=1024, inter=1024, n_experts=64, top_k=8), 16, 300, "4,4,4,4"),
    ("two_token_tiles", dict(T=32, pos=200, window=64, head_dim=128, n_q_heads=4, n_kv_heads=1, hidden=768),
     32, 184, None),
    ("bf16", dict(T=16, pos=150, window=0, expert_dtype=synth.BF16), 16, 150, None),
    ("fp4_gather", dict(T=16, pos=200, window=64, n_experts=32, top_k=8, pooled=512, inter=512,
                        down_input=synth.DOWN_NVFP4), 16, 200, None),
]


@pytest.mark.parametrize("case", POISON, ids=[c[0] for c in POISON])
def test_poisoned_scratch_changes_nothing(case, monkeypatch):
    """Every scratch word a step reads is written earlier in the same step (no consumer reads
    before its producer): with the plan's activation scratch filled with NaN before the call,
    fused and unfused steps give bitwise the outputs (and expert activations) of the same step
    on a scratch that holds an earlier step's values."""
    name, kw, T, pos, splits = case
    if splits:
        monkeypatch.setenv("MOEL_DENSE_SPLITS", splits)
    w = synth.small_workload(**kw)
    _log(f"poison {name} {kw} T {T} pos {pos} splits {splits}")
    run = harness.GpuRun(w)
    if splits:
        monkeypatch.delenv("MOEL_DENSE_SPLITS")
    rows = T * w.top_k
    for fused in (True, False):
        ref = run.run(fused=fused, T=T, pos=pos)
        ref_act = {n: run.plan.scratch(n).view(binding.MOEL_MAX_TOKENS * w.top_k, -1)[:rows].clone() for n in ("a", "d")}
        run.plan.poison_scratch()
        out = run.run(fused=fused, T=T, pos=pos)
        for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
            assert _same_bytes(ref[k], out[k]), (fused, k)
        for n, v in ref_act.items():
            assert _same_bytes(v, run.plan.scratch(n).view(binding.MOEL_MAX_TOKENS * w.top_k, -1)[:rows]), (fused, n)
        assert bool(torch.isfinite(out["y"]).all()), fused


def test_fp4_gather_fused_equals_unfused():
    w = synth.small_workload(T=16, pos=200, window=64, n_experts=32, top_k=8, pooled=512, inter=512,
                             down_input=synth.DOWN_NVFP4)
    run = harness.GpuRun(w)
    a = run.run(fused=True)
    aq = run.plan.scratch("aq").clone()
    c = run.run(fused=False)
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates"):
        assert _same_bytes(a[k], c[k]), k
    assert _same_bytes(aq, run.plan.scratch("aq"))


def test_plain_and_cooperative_launches_agree():
    w = synth.small_workload(T=16, pos=300, window=0, n_experts=32, top_k=8, pooled=512, inter=512)
    run = harness.GpuRun(w)
    a = run.run(fused=True)
    run.plan.set_launch(binding.MOEL_LAUNCH_COOPERATIVE)
    b = run.run(fused=True)
    run.plan.set_launch(binding.MOEL_LAUNCH_PLAIN)
    c = run.run(fused=True)
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(a[k], b[k]), k
        assert _same_bytes(a[k], c[k]), k
    with pytest.raises(binding.MoelError):
        run.plan.set_launch(7)


def test_l1_only_and_l2_invalidating_acquire_agree():
    """The grid barriers' L1-only acquire (taken where the device keeps its XCDs' L2 caches
    coherent) gives the same bytes as the agent-scope acquire that also invalidates the L2,
    and as the one-kernel-per-step chain, whose kernel boundaries order everything."""
    w = synth.small_workload(T=16, pos=1500, window=0, hidden=2048, n_q_heads=16, n_kv_heads=4,
                             head_dim=128, n_experts=64, top_k=8, pooled=1024, inter=1024)
    run = harness.GpuRun(w)
    _log(f"l2_coherent {run.plan.l2_coherent}")
    a = run.run(fused=True)
    run.plan.set_acquire(binding.MOEL_ACQUIRE_L2_INVALIDATE)
    b = run.run(fused=True)
    run.plan.set_acquire(binding.MOEL_ACQUIRE_AUTO)
    c = run.run(fused=False)
    d = run.run(fused=True)
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(a[k], b[k]), k
        assert _same_bytes(a[k], c[k]), k
        assert _same_bytes(a[k], d[k]), k
    with pytest.raises(binding.MoelError):
        run.plan.set_acquire(3)


# token-tree verify: a 16-node tree (two branches off the root, one branching again), a
# forest of two roots, and the chain given as a tree
TREE16 = [-1, 0, 1, 2, 0, 4, 5, 1, 7, 3, 9, 4, 11, 12, 2, 14]
FOREST = [-1, -1, 0, 1, 2, 3, 0, 6]


@pytest.mark.parametrize("case", [
    dict(parents=TREE16, window=0, pos=500),
    dict(parents=TREE16, window=64, pos=300),
    dict(parents=TREE16, window=6, pos=40),
    dict(parents=FOREST, window=0, pos=200),
], ids=["tree_global", "tree_window", "tree_short_window", "forest"])
def test_tree_verify_matches_oracle(case):
    par = case["parents"]
    w = synth.small_workload(T=len(par), pos=case["pos"], window=case["window"], n_experts=32, top_k=8,
                             pooled=512, inter=512)
    _log(f"tree {case}")
    run = harness.GpuRun(w)
    rep = {}
    out = run.run(fused=True, parents=par)
    harness.check_against_oracle(run, out, report=rep)
    _log(f"tree {case}: {rep}")
    # the one-kernel-per-step chain gives the same bytes
    b = run.run(fused=False, parents=par)
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(out[k], b[k]), k


def test_chain_given_as_a_tree_is_the_chain():
    w = synth.small_workload(T=16, pos=700, window=128, n_experts=32, top_k=8, pooled=512, inter=512)
    run = harness.GpuRun(w)
    a = run.run(fused=True)
    b = run.run(fused=True, parents=list(range(-1, 15)))
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(a[k], b[k]), k
    with pytest.raises(binding.MoelError):
        run.run(fused=True, parents=[-1, 1] + list(range(1, 15)))   # parent not before its child


def test_timestamps_leave_outputs_bit_identical():
    w = synth.small_workload(T=8, pos=200, window=64)
    run = harness.GpuRun(w)
    a = run.run(fused=True, stamps=False)
    b = run.run(fused=True, stamps=True)
    assert torch.equal(a["y"], b["y"])
    assert torch.equal(a["k_cache"].view(torch.int16), b["k_cache"].view(torch.int16))
    ts = b["timestamps"].cpu().numpy()
    assert (ts[:, :10] > 0).all()
    assert (np.diff(ts[:, :10].astype(np.int64), axis=1) >= 0).all()


def test_rewind_rewrites_only_the_step_slots():
    """Calling again at the same pos with different x (a rejected draft) rewrites exactly
    slots [pos, pos+T) and leaves earlier slots untouched."""
    w = synth.small_workload(T=6, pos=50, window=0)
    run = harness.GpuRun(w)
    kc, vc = run.fresh_caches()
    y = torch.empty((w.T, w.hidden), dtype=torch.float32, device="cuda")
    run.plan.layer_decode(run.lw, kc, vc, run.t["x"], w.pos, 0, y)
    k1 = kc.clone()
    x2 = torch.randn_like(run.t["x"])
    run.plan.layer_decode(run.lw, kc, vc, x2, w.pos, 0, y)
    torch.cuda.synchronize()
    assert torch.equal(kc[:, :w.pos].view(torch.int16), k1[:, :w.pos].view(torch.int16))
    assert not torch.equal(kc[:, w.pos:w.pos + w.T].view(torch.int16), k1[:, w.pos:w.pos + w.T].view(torch.int16))
    out = run.run(fused=True, x=x2)
    assert torch.equal(out["k_cache"][:, w.pos:w.pos + w.T].view(torch.int16),
                       kc[:, w.pos:w.pos + w.T].view(torch.int16))


def test_abort_leaves_buffers_untouched():
    w = synth.small_workload(T=4, pos=30, window=0)
    run = harness.GpuRun(w)
    kc, vc = run.fresh_caches()
    y = torch.full((w.T, w.hidden), 7.0, dtype=torch.float32, device="cuda")
    dbg = {"expert_idx": torch.full((w.T, w.top_k), 7, dtype=torch.int32, device="cuda"),
           "timestamps": torch.full((run.plan.workgroups, binding.MOEL_N_STAMPS), 7, dtype=torch.int64,
                                    device="cuda")}
    for fused in (True, False):
        run.plan.set_abort(True)
        run.plan.layer_decode(run.lw, kc, vc, run.t["x"], w.pos, 0, y, dbg=dbg, fused=fused)
        torch.cuda.synchronize()
        assert run.plan.status() == binding.MOEL_ERR_ABORTED
        run.plan.set_abort(False)
        torch.cuda.synchronize()
        assert torch.all(y == 7.0)
        assert torch.equal(kc.view(torch.int16), run.k0.view(torch.int16))
        assert torch.all(dbg["expert_idx"] == 7) and torch.all(dbg["timestamps"] == 7)
    assert run.plan.status() == binding.MOEL_OK


def test_invalid_calls_launch_nothing():
    w = synth.small_workload(T=4, pos=30, window=0)
    run = harness.GpuRun(w)
    kc, vc = run.fresh_caches()
    y = torch.full((w.T, w.hidden), 7.0, dtype=torch.float32, device="cuda")
    for T, pos, window in ((0, 30, 0), (33, 30, 0), (4, w.kv_capacity - 3, 0), (4, -1, 0), (4, 30, -2)):
        with pytest.raises(binding.MoelError) as ei:
            run.plan.layer_decode(run.lw, kc, vc, run.t["x"], pos, window, y, T=T)
        assert ei.value.code == binding.MOEL_ERR_ARG
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    assert torch.equal(kc.view(torch.int16), run.k0.view(torch.int16))


# ---------------------------------------------------------------- batched verify
# (T, pos, kv_base, kv_slots) per request: three requests of 16 tokens in all over an 800-slot
# pool, with different depths and bases
BATCH3 = [(5, 100, 0, 300), (7, 250, 300, 400), (4, 30, 700, 100)]
# eight requests of one to three tokens
BATCH8 = [(t, 10 + 11 * i, 100 * i, 100) for i, t in enumerate([1, 2, 3, 1, 2, 3, 2, 2])]


def _batch_workload(**kw):
    base = dict(T=16, pos=784, n_experts=32, top_k=8, pooled=512, inter=512)
    base.update(kw)
    return synth.small_workload(**base)


@pytest.mark.parametrize("reqs,window", [(BATCH3, 0), (BATCH3, 40), (BATCH3, 6), (BATCH8, 0), (BATCH8, 5)],
                         ids=["three_global", "three_window", "three_short_window", "eight_global",
                              "eight_window"])
def test_batch_matches_oracle_per_request(reqs, window):
    run = harness.GpuRun(_batch_workload(window=window))
    _log(f"batch {reqs} window {window}")
    out = harness.run_batch(run, reqs)
    reps = harness.check_batch_against_oracle(run, out, reqs)
    _log(f"batch: {[{k: r[k] for k in ('max_abs', 'min_cos', 'logit_err')} for r in reps]}")
    # the one-kernel-per-step chain gives the same bytes
    b = harness.run_batch(run, reqs, fused=False)
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(out[k], b[k]), k


def test_poisoned_scratch_changes_nothing_in_trees_batches_and_stacks():
    """The poisoned-scratch check (see test_poisoned_scratch_changes_nothing) on the other entry
    points: a token tree, a batch of three requests (fused and unfused), and three layers of one
    shape in one launch."""
    run = harness.GpuRun(synth.small_workload(T=16, pos=300, window=64, n_experts=32, top_k=8, pooled=512,
                                              inter=512))
    for fused in (True, False):
        ref = run.run(fused=fused, parents=TREE16)
        run.plan.poison_scratch()
        out = run.run(fused=fused, parents=TREE16)
        for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
            assert _same_bytes(ref[k], out[k]), ("tree", fused, k)
    run = harness.GpuRun(_batch_workload(window=40))
    for fused in (True, False):
        ref = harness.run_batch(run, BATCH3, fused=fused)
        run.plan.poison_scratch()
        out = harness.run_batch(run, BATCH3, fused=fused)
        for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
            assert _same_bytes(ref[k], out[k]), ("batch", fused, k)
    w = synth.small_workload(T=32, pos=300, window=64, n_experts=32, top_k=8, pooled=512, inter=512, hidden=1024,
                             n_q_heads=8, n_kv_heads=2, head_dim=128)
    plan = binding.Plan(binding.config_from_workload(w))
    windows = [0, 64, 7]
    ts = [synth.make_layer(w, l, "cuda") for l in range(3)]
    lws = [plan.pack_layer(t) for t in ts]
    k0, v0 = [t["k_cache"] for t in ts], [t["v_cache"] for t in ts]
    kc, vc = [k.clone() for k in k0], [v.clone() for v in v0]
    st = binding.Stack(plan, lws, kc, vc, windows)
    outs = []
    for poison in (False, True):
        for l in range(3):
            kc[l].copy_(k0[l])
            vc[l].copy_(v0[l])
        if poison:
            plan.poison_scratch()
        x = ts[0]["x"][:16].contiguous()
        y = torch.full_like(x, float("nan"))
        st.decode(x, 300, y)
        torch.cuda.synchronize()
        assert plan.status() == binding.MOEL_OK
        outs.append((y, [k.clone() for k in kc], [v.clone() for v in vc]))
    (y0, ka, va), (y1, kb, vb) = outs
    assert _same_bytes(y0, y1)
    for l in range(3):
        assert _same_bytes(ka[l], kb[l]) and _same_bytes(va[l], vb[l]), l
    st.close()
    plan.close()


def test_batch_key_chunks_sized_for_the_whole_batch():
    # 8 kv heads leave 32 key chunks for the batch: three requests of ~1600 keys split into
    # chunks of 151 keys (150 would give 33 chunks)
    w = _batch_workload(hidden=512, n_q_heads=16, n_kv_heads=8, head_dim=64, pos=4784, window=0)
    reqs = [(5, 1590, 0, 1600), (6, 1500, 1600, 1600), (5, 1580, 3200, 1600)]
    run = harness.GpuRun(w)
    out = harness.run_batch(run, reqs)
    reps = harness.check_batch_against_oracle(run, out, reqs)
    _log(f"batch chunks: {[{k: r[k] for k in ('max_abs', 'min_cos', 'logit_err')} for r in reps]}")


def test_single_request_batch_is_layer_decode():
    w = _batch_workload(pos=700, window=128)
    run = harness.GpuRun(w)
    a = run.run(fused=True)
    b = harness.run_batch(run, [(w.T, w.pos, 0, w.kv_capacity)])
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(a[k], b[k]), k


def test_batch_rows_do_not_depend_on_the_other_requests():
    """A request's rows and cache writes are those it gets when the other requests' tokens
    change (their inputs, their caches' contents), up to attention's rounding order: its rows
    meet the oracle bar either way and its written K/V are bitwise equal."""
    run = harness.GpuRun(_batch_workload(window=40))
    a = harness.run_batch(run, BATCH3)
    x2 = run.t["x"][:16].clone()
    x2[5:] = torch.randn_like(x2[5:])          # requests 1 and 2 change, request 0 keeps its rows
    b = harness.run_batch(run, BATCH3, x=x2)
    T0, pos0, kvb0, _ = BATCH3[0]
    assert _same_bytes(a["k_cache"][:, kvb0 + pos0:kvb0 + pos0 + T0], b["k_cache"][:, kvb0 + pos0:kvb0 + pos0 + T0])
    assert _same_bytes(a["expert_idx"][:T0], b["expert_idx"][:T0])
    d = float((a["y"][:T0] - b["y"][:T0]).abs().max())
    assert d <= 1e-5, d


def test_invalid_batches_launch_nothing():
    run = harness.GpuRun(_batch_workload(window=0))
    kc, vc = run.fresh_caches()
    y = torch.full((16, run.w.hidden), 7.0, dtype=torch.float32, device="cuda")
    for reqs in ([], [(4, 0, 0, 100), (4, 0, 50, 100)], [(4, 98, 0, 100)], [(17, 0, 0, 100), (16, 0, 100, 100)]):
        with pytest.raises(binding.MoelError) as ei:
            run.plan.layer_decode_batch(run.lw, kc, vc, run.t["x"], reqs, 0, y)
        assert ei.value.code == binding.MOEL_ERR_ARG
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    assert torch.equal(kc.view(torch.int16), run.k0.view(torch.int16))


def test_full_width_batch_matches_oracle():
    # swa_fp4 with its 8208-slot pool shared by three requests of 4, 4 and 8 tokens
    w = synth.WORKLOADS["swa_fp4"]
    reqs = [(4, 2500, 0, 2600), (4, 1900, 2600, 2000), (8, 3500, 4600, 3608)]
    _log(f"full batch {reqs}: generating")
    run = harness.GpuRun(w)
    out = harness.run_batch(run, reqs)
    _log("full batch: oracle")
    reps = harness.check_batch_against_oracle(run, out, reqs)
    _log(f"full batch: {reps}")


# ---------------------------------------------------------------- two 16-token tiles (T up to 32)
# (workload overrides, call T, call pos): the workload's cache holds pos + 16 slots, so a call of
# more than 16 tokens starts earlier
TILES2 = [
    (dict(T=32, pos=300, window=0), 32, 284),
    (dict(T=32, pos=300, window=40), 32, 284),
    (dict(T=20, pos=60, window=7), 20, 56),
    (dict(T=32, pos=200, window=64, head_dim=128, n_q_heads=4, n_kv_heads=1, hidden=768), 32, 184),
    (dict(T=32, pos=150, window=0, expert_dtype=synth.BF16), 32, 134),
    (dict(T=17, pos=100, window=32, n_experts=32, top_k=8, pooled=512, inter=512), 17, 99),
    (dict(T=32, pos=100, window=0, n_experts=32, top_k=8, n_shards=8, shard_rank=3, inter=512, pooled=512,
          down_input=synth.DOWN_NVFP4), 32, 84),
]


@pytest.mark.parametrize("case", TILES2, ids=[str(i) for i in range(len(TILES2))])
def test_two_token_tiles_match_oracle(case):
    kw, T, pos = case
    w = synth.small_workload(**kw)
    _log(f"tiles2 {kw} T {T} pos {pos}")
    run = harness.GpuRun(w)
    out = run.run(fused=True, T=T, pos=pos)
    rep = {}
    harness.check_against_oracle(run, out, report=rep)
    _log(f"tiles2: {rep}")
    b = run.run(fused=False, T=T, pos=pos)
    for k in ("y", "k_cache", "v_cache", "expert_idx", "gates", "router_logits"):
        assert _same_bytes(out[k], b[k]), k


@pytest.mark.parametrize("kw", [dict(), dict(expert_dtype=synth.BF16)], ids=["nvfp4", "bf16"])
def test_two_token_tiles_with_experts_over_16_slots(kw):
    """Concentrated routing at 32 tokens: experts chosen by more than 16 tokens, which the
    expert streams take as one entry per 16 slots."""
    w = synth.small_workload(T=32, pos=116, window=0, n_experts=32, top_k=8, pooled=512, inter=512, **kw)
    run = harness.GpuRun(w, routing="shared")
    out = run.run(fused=True, T=32, pos=100)
    counts = np.bincount(out["expert_idx"].cpu().numpy().ravel(), minlength=w.n_experts)
    _log(f"tiles2 shared: slots per expert max {counts.max()}")
    assert counts.max() > 16
    rep = {}
    harness.check_against_oracle(run, out, report=rep)
    _log(f"tiles2 shared: {rep}")


@pytest.mark.parametrize("splits", ["2,2,2,2", "8,8,8,8"])
def test_two_token_tiles_split_k(splits, monkeypatch):
    monkeypatch.setenv("MOEL_DENSE_SPLITS", splits)
    w = synth.small_workload(T=32, pos=316, window=0, hidden=2048, n_q_heads=16, n_kv_heads=4, head_dim=128,
                             n_experts=32, top_k=8, pooled=1024, inter=1024)
    run = harness.GpuRun(w)
    out = run.run(fused=True, T=32, pos=300)
    harness.check_against_oracle(run, out)
    b = run.run(fused=False, T=32, pos=300)
    for k in ("y", "k_cache", "v_cache", "expert_idx"):
        assert _same_bytes(out[k], b[k]), k


def test_two_token_tiles_tree_and_batch():
    # a 32-node tree (two branches off a chain), and a batch of three requests of 32 tokens
    par = [-1] + list(range(0, 15)) + [3] + list(range(16, 26)) + [20, 27, 28, 29, 30]
    assert len(par) == 32 and all(-1 <= v < i for i, v in enumerate(par))
    w = synth.small_workload(T=32, pos=516, window=48, n_experts=32, top_k=8, pooled=512, inter=512)
    run = harness.GpuRun(w)
    out = run.run(fused=True, T=32, pos=500, parents=par)
    harness.check_against_oracle(run, out)
    wb = _batch_workload(T=32, pos=784, window=40)
    runb = harness.GpuRun(wb)
    reqs = [(12, 100, 0, 300), (11, 250, 300, 400), (9, 30, 700, 100)]
    outb = harness.run_batch(runb, reqs)
    harness.check_batch_against_oracle(runb, outb, reqs)
    b = harness.run_batch(runb, reqs, fused=False)
    for k in ("y", "k_cache", "v_cache", "expert_idx"):
        assert _same_bytes(outb[k], b[k]), k


def test_two_token_tiles_full_width():
    # swa_fp4 verifying 32 tokens (history 8,176): every token against the oracle
    w = synth.WORKLOADS["swa_fp4"].with_(T=32)
    _log("tiles2 full: generating")
    run = harness.GpuRun(w)
    out = run.run(fused=True, T=32, pos=w.pos - 16)
    rep = {}
    _log("tiles2 full: oracle")
    harness.check_against_oracle(run, out, report=rep)
    _log(f"tiles2 full: {rep}")


# ---------------------------------------------------------------- full-width workloads
FULL = ["swa_fp4", "global_fp4", "swa_bf16", "swa_fp4_a4"]


@pytest.mark.parametrize("name", FULL)
def test_full_width_matches_oracle(name):
    w = synth.WORKLOADS[name]
    _log(f"full {name}: generating")
    run = harness.GpuRun(w)
    _log(f"full {name}: running")
    out = run.run(fused=True)
    rep = {}
    _log(f"full {name}: oracle")
    harness.check_against_oracle(run, out, report=rep)
    _log(f"full {name}: {rep}")


@pytest.mark.parametrize("layer,rank", [(0, 0), (1, 0), (2, 7)], ids=["global_r0", "swa_r0", "swa_r7"])
def test_stack_share_layer_matches_oracle(layer, rank):
    w = synth.WORKLOADS["stack_tp8"].with_(shard_rank=rank)
    _log(f"stack layer {layer} rank {rank}: generating")
    run = harness.GpuRun(w, layer=layer)
    out = run.run(fused=True)
    rep = {}
    harness.check_against_oracle(run, out, report=rep)
    _log(f"stack layer {layer} rank {rank}: {rep}")


@pytest.mark.parametrize("down", [synth.DOWN_EXACT, synth.DOWN_NVFP4], ids=["exact", "fp4_gather"])
def test_expert_n_shards_equal_full_width_rows(down):
    """N-sharding the expert GEMMs splits no K reduction (orcarouter.ai English post, "Where the
    kernel boundary sits": the sharded MoE GEMMs can be made bitwise identical to expert
    parallelism): with the same weights, one GPU's share of the SwiGLU output (its gate/up rows,
    and with the fp4 gather their encoding) is bitwise equal to the same rows of the full-width
    layer, at every rank."""
    full = synth.small_workload(T=16, pos=200, window=64, n_experts=32, top_k=8, pooled=512, inter=1024,
                                down_input=down)
    run_f = harness.GpuRun(full)
    out_f = run_f.run(fused=True)
    k, I = full.top_k, full.inter
    a_f = run_f.plan.scratch("a").view(binding.MOEL_MAX_TOKENS * k, I).clone()
    aq_f = run_f.plan.scratch("aq").view(binding.MOEL_MAX_TOKENS * k, I).clone() if down else None
    S = 8
    il, plc = full.inter // S, full.pooled // S
    for rank in (0, 3, 7):
        sh = full.with_(n_shards=S, shard_rank=rank)
        t = dict(run_f.t)
        for m in ("gate", "up"):
            for part in ("_codes", "_scales"):
                t[m + part] = run_f.t[m + part][:, rank * il:(rank + 1) * il].contiguous()
        for part in ("_codes", "_scales"):
            t["down" + part] = run_f.t["down" + part][:, rank * plc:(rank + 1) * plc].contiguous()
        run_s = harness.GpuRun(sh, tensors=t)
        out_s = run_s.run(fused=True)
        assert torch.equal(out_s["expert_idx"], out_f["expert_idx"])
        cols = slice(rank * il, (rank + 1) * il)
        a_s = run_s.plan.scratch("a").view(binding.MOEL_MAX_TOKENS * k, I)
        assert _same_bytes(a_s[:, cols], a_f[:, cols]), rank
        if down:
            aq_s = run_s.plan.scratch("aq").view(binding.MOEL_MAX_TOKENS * k, I)
            assert _same_bytes(aq_s[:, cols], aq_f[:, cols]), rank
        run_s.plan.close()
        _log(f"n-shard rank {rank}: gate/up rows bitwise equal to the full-width layer's")


def _layer_by_layer(plan, lws, k0, v0, windows, x, pos):
    kc, vc = [k.clone() for k in k0], [v.clone() for v in v0]
    cur = x
    for l, lw in enumerate(lws):
        y = torch.empty_like(x)
        plan.layer_decode(lw, kc[l], vc[l], cur, pos, windows[l], y)
        cur = y
    torch.cuda.synchronize()
    assert plan.status() == binding.MOEL_OK
    return cur, kc, vc


def test_read_bandwidth_reference():
    """The streaming-read reference the bench reports beside the nominal peak: a positive rate
    below the nominal 8 TB/s over 1 GiB, and the too-small buffer rejected."""
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    gbps = binding.measure_read_bandwidth(buf, reps=3)
    _log(f"streaming read: {gbps:.0f} GB/s")
    assert 500.0 < gbps < 8000.0
    with pytest.raises(RuntimeError):
        binding.measure_read_bandwidth(buf[:4096], reps=1)
    del buf


def test_stack_launch_equals_layer_by_layer():
    """Layers of one shape in one persistent launch (moel_stack_decode; grid barriers between the
    layers) give bitwise the rows and caches of moel_layer_decode called layer by layer: a global
    layer and two sliding-window ones, several calls in a row with 16, 5, 1, 9 and 32 tokens (with
    few tokens the expert tiles of consecutive layers land on different XCDs, the case where an
    XCD's L2 keeps its own copy of a rewritten workspace line unless the layer boundary drops it);
    and a stack of 8 layers, which takes two launches, its input and output rows adjacent in one
    buffer."""
    w = synth.small_workload(T=32, pos=300, window=64, n_experts=32, top_k=8, pooled=512, inter=512, hidden=1024,
                             n_q_heads=8, n_kv_heads=2, head_dim=128)
    plan = binding.Plan(binding.config_from_workload(w))
    windows = [0, 64, 7]
    ts = [synth.make_layer(w, l, "cuda") for l in range(3)]
    lws = [plan.pack_layer(t) for t in ts]
    k0 = [t["k_cache"] for t in ts]
    v0 = [t["v_cache"] for t in ts]
    kc, vc = [k.clone() for k in k0], [v.clone() for v in v0]
    st = binding.Stack(plan, lws, kc, vc, windows)
    for T, pos in ((16, 300), (5, 120), (5, 120), (1, 77), (9, 200), (32, 284)):
        x = ts[0]["x"][:T].contiguous()
        y_ref, k_ref, v_ref = _layer_by_layer(plan, lws, k0, v0, windows, x, pos)
        for l in range(3):
            kc[l].copy_(k0[l])
            vc[l].copy_(v0[l])
        y = torch.full_like(x, float("nan"))
        st.decode(x, pos, y)
        torch.cuda.synchronize()
        assert plan.status() == binding.MOEL_OK
        assert _same_bytes(y, y_ref), T
        for l in range(3):
            assert _same_bytes(kc[l], k_ref[l]) and _same_bytes(vc[l], v_ref[l]), (T, l)
    st.close()
    # 8 layers (two launches): the windows cycle global, 64, 7
    lws8 = [lws[l % 3] for l in range(8)]
    k8, v8 = [k0[l % 3].clone() for l in range(8)], [v0[l % 3].clone() for l in range(8)]
    win8 = [windows[l % 3] for l in range(8)]
    rows = torch.full((32, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
    x, y = rows[:16], rows[16:]  # adjacent, not overlapping
    x.copy_(ts[0]["x"][:16])
    y_ref, k_ref, v_ref = _layer_by_layer(plan, lws8, k8, v8, win8, x, 300)
    kc8, vc8 = [k.clone() for k in k8], [v.clone() for v in v8]
    st8 = binding.Stack(plan, lws8, kc8, vc8, win8)
    st8.decode(x, 300, y)
    torch.cuda.synchronize()
    assert plan.status() == binding.MOEL_OK
    assert _same_bytes(y, y_ref)
    for l in range(8):
        assert _same_bytes(kc8[l], k_ref[l]) and _same_bytes(vc8[l], v_ref[l]), l
    st8.close()
    plan.close()


def test_stack_share_two_layers_in_one_launch():
    """The TP8 stack share: a global and a sliding-window layer in one launch, bitwise equal to the
    two layers called one by one; the sliding-window layer's output checked against the oracle on
    the device's output of the global layer."""
    w = synth.WORKLOADS["stack_tp8"]
    _log("stack launch: generating")
    run0 = harness.GpuRun(w, layer=0)
    run1 = harness.GpuRun(w, layer=1, plan=run0.plan)
    windows = [w.layer_window(0), w.layer_window(1)]
    x = run0.t["x"].contiguous()
    out0 = run0.run(fused=True)
    out1 = run1.run(fused=True, x=out0["y"])
    rep = {}
    harness.check_against_oracle(run1, out1, report=rep)
    _log(f"stack launch, layer 1 on layer 0's output: {rep}")
    kc, vc = [run0.k0.clone(), run1.k0.clone()], [run0.v0.clone(), run1.v0.clone()]
    st = binding.Stack(run0.plan, [run0.lw, run1.lw], kc, vc, windows)
    y = torch.full_like(x, float("nan"))
    st.decode(x, w.pos, y)
    torch.cuda.synchronize()
    assert run0.plan.status() == binding.MOEL_OK
    assert _same_bytes(y, out1["y"])
    assert _same_bytes(kc[0], out0["k_cache"]) and _same_bytes(vc[0], out0["v_cache"])
    assert _same_bytes(kc[1], out1["k_cache"]) and _same_bytes(vc[1], out1["v_cache"])
    st.close()


def _step(plan, lw, k0, v0, x, pos, window, fused=True):
    kc, vc = k0.clone(), v0.clone()
    y = torch.full_like(x, float("nan"))
    idx = torch.full((x.shape[0], plan.cfg.top_k), -1, dtype=torch.int32, device="cuda")
    plan.layer_decode(lw, kc, vc, x, pos, window, y, dbg={"expert_idx": idx}, fused=fused)
    torch.cuda.synchronize()
    assert plan.status() == binding.MOEL_OK
    return y, kc, vc, idx


@pytest.mark.parametrize("layer", [0, 1], ids=["global_barrier_merge", "swa_set_merge"])
def test_expert_history_and_prefetch_change_nothing(layer):
    """Previous-step expert prefetch (orcarouter.ai English post, "Three bills a kernel this big
    has to pay"): every step writes its tokens per expert to the layer's routing history, and with
    the prefetch on a step first pulls the experts the previous step used most into the
    memory-side cache on the workgroups that have no attention work.  On stack-share layers (one
    kv head, so 7 of 8 barrier groups have no attention work): results bitwise those without
    history or prefetch, two steps in a row with different inputs (the second prefetches what
    the first used), the history equal to the counts of the chosen experts; the one-kernel-per-
    step chain writes the same history."""
    w = synth.WORKLOADS["stack_tp8"]
    plan = binding.Plan(binding.config_from_workload(w))
    _log(f"prefetch layer {layer}: generating")
    t = synth.make_layer(w, layer, "cuda")
    lw = plan.pack_layer(t)
    window = w.layer_window(layer)
    k0, v0 = t["k_cache"].clone(), t["v_cache"].clone()
    xs = [t["x"].contiguous(), (0.5 * t["x"].flip(0)).contiguous()]
    refs = [_step(plan, lw, k0, v0, x, w.pos, window) for x in xs]
    hist = torch.zeros(w.n_experts, dtype=torch.int32, device="cuda")
    lw.set_history(hist)
    plan.set_expert_prefetch(14)
    for i, x in enumerate(xs):
        y, kc, vc, idx = _step(plan, lw, k0, v0, x, w.pos, window)
        assert _same_bytes(y, refs[i][0]) and _same_bytes(kc, refs[i][1]) and _same_bytes(vc, refs[i][2]), i
        assert torch.equal(idx, refs[i][3]), i
        counts = torch.bincount(idx.flatten().long(), minlength=w.n_experts)
        assert torch.equal(hist.long(), counts), i
    _log(f"prefetch layer {layer}: {int((hist > 0).sum())} experts in the history")
    plan.set_expert_prefetch(0)
    hist.zero_()
    _step(plan, lw, k0, v0, xs[1], w.pos, window, fused=False)
    assert torch.equal(hist.long(), torch.bincount(refs[1][3].flatten().long(), minlength=w.n_experts))
    lw.set_history(None)
    plan.close()
