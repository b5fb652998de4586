"""Pins of the layer oracle (CPU only).

The vectorised oracle (oracle/layer.py) is checked against: closed forms
(RMSNorm of a constant vector, RoPE at position 0 and a hand-derived rotation),
library routines (torch rms_norm, scaled_dot_product_attention with an explicit
mask, torch.topk), invariants (norm preservation, relative positions, window
and causal masks, routing), a special case (top-k = E is a dense softmax
mixture computed here with einsum) and the loop-only oracle (oracle/brute.py)
on tiny shapes.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, formats, layer
from moe_layer_persistent_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    H, eps = 64, 1e-6
    gamma = np.linspace(0.5, 1.5, H)
    for c in (-3.0, 0.25, 7.0):
        out = layer.rmsnorm(np.full((1, H), c), gamma, eps)
        np.testing.assert_allclose(out[0], c / math.sqrt(c * c + eps) * gamma, rtol=1e-15)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 96)) * 3
    g = 1 + 0.02 * rng.standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.tensor(x), (96,), torch.tensor(g), eps=1e-6).numpy()
    np.testing.assert_allclose(layer.rmsnorm(x, g, 1e-6), want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity_and_norm_preserved():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((3, 2, 16))
    np.testing.assert_array_equal(layer.rope(v, np.zeros(3, dtype=int), 10000.0), v)
    r = layer.rope(v, np.array([5, 999, 123456]), 10000.0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-13)


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 32))
    k = rng.standard_normal((1, 1, 32))
    def dot(m, n):
        return float(np.sum(layer.rope(q, np.array([m]), 1e4) * layer.rope(k, np.array([n]), 1e4)))
    for (m, n, s) in [(3, 1, 10), (100, 40, 777), (0, 9, 5)]:
        assert abs(dot(m, n) - dot(m + s, n + s)) < 1e-10


def test_rope_hand_example():
    """D = 4, theta = 1e4, position 1: pair (0, 2) turns by 1 rad, pair (1, 3) by 0.01 rad."""
    v = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    got = layer.rope(v, np.array([1]), 10000.0)[0, 0]
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    want = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    np.testing.assert_allclose(got, want, rtol=1e-15)


# ---------------------------------------------------------------- attention
def _sdpa_reference(q, kc, vc, pos, window):
    """torch SDPA with an explicit boolean mask, per (token, head), fp64 on the CPU."""
    T, Hq, D = q.shape
    Hkv, C, _ = kc.shape
    grp = Hq // Hkv
    out = np.zeros_like(q)
    for h in range(Hq):
        g = h // grp
        mask = torch.zeros(T, C, dtype=torch.bool)
        for t in range(T):
            p = pos + t
            for j in range(C):
                mask[t, j] = j <= p and (window == 0 or j > p - window)
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[None, :, h]), torch.tensor(kc[None, g]), torch.tensor(vc[None, g]),
            attn_mask=mask[None])
        out[:, h] = o[0].numpy()
    return out


@pytest.mark.parametrize("window", [0, 1, 5])
def test_attention_matches_sdpa(window):
    rng = np.random.default_rng(4)
    T, Hq, Hkv, D, pos = 4, 6, 2, 8, 9
    C = pos + T + 3
    q = rng.standard_normal((T, Hq, D))
    kc = rng.standard_normal((Hkv, C, D))
    vc = rng.standard_normal((Hkv, C, D))
    np.testing.assert_allclose(layer.attention(q, kc, vc, pos, window),
                               _sdpa_reference(q, kc, vc, pos, window), rtol=1e-12, atol=1e-12)


def test_attention_invisible_keys_do_not_matter():
    rng = np.random.default_rng(5)
    T, Hq, Hkv, D, pos, W = 3, 4, 2, 8, 20, 6
    C = pos + T + 4
    q = rng.standard_normal((T, Hq, D))
    kc = rng.standard_normal((Hkv, C, D))
    vc = rng.standard_normal((Hkv, C, D))
    base = layer.attention(q, kc, vc, pos, W)
    for t in range(T):
        lo, hi = layer.visible_range(pos + t, W)
        assert hi - lo == min(W, pos + t + 1)
    kc2, vc2 = kc.copy(), vc.copy()
    lo0, _ = layer.visible_range(pos, W)
    kc2[:, :lo0] = 99.0                     # before every token's window
    vc2[:, :lo0] = -99.0
    kc2[:, pos + T:] = 55.0                 # future slots
    vc2[:, pos + T:] = 55.0
    np.testing.assert_array_equal(layer.attention(q, kc2, vc2, pos, W), base)
    # the last new key is in the future of token 0 only: changing it must leave token 0 alone
    kc3 = kc.copy()
    kc3[:, pos + T - 1] += 3.0
    np.testing.assert_array_equal(layer.attention(q, kc3, vc, pos, W)[0], base[0])


def test_attention_single_key_and_equal_keys():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 2, 8))
    kc = rng.standard_normal((1, 4, 8))
    vc = rng.standard_normal((1, 4, 8))
    o = layer.attention(q, kc, vc, pos=0, window=0)         # only key 0 is visible
    np.testing.assert_array_equal(o[0, 0], vc[0, 0])
    kc_eq = np.repeat(kc[:, :1], 4, axis=1)
    o = layer.attention(q, kc_eq, vc, pos=3, window=0)
    np.testing.assert_allclose(o[0, 1], vc[0].mean(axis=0), rtol=1e-13)


# ---------------------------------------------------------------- routing
def test_route_golden_ties():
    vals = {}
    for line in open(os.path.join(GOLDEN, "router_ties.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            vals[k] = v
    logits = np.array([[float(v) for v in vals["logits"]]])
    idx, gates, gap = layer.route(logits, int(vals["k"][0]))
    assert idx[0].tolist() == [int(v) for v in vals["idx"]]
    np.testing.assert_allclose(gates[0], 1 / 3, rtol=1e-15)
    assert gap[0] == 2.0          # 3rd selected (5) minus the best unselected (3)


def test_route_invariants_and_topk():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((16, 256))
    idx, gates, gap = layer.route(logits, 8)
    for t in range(16):
        assert len(set(idx[t])) == 8
        sel = logits[t, idx[t]]
        assert np.all(np.diff(sel) < 0)
        assert np.min(sel) >= np.max(np.delete(logits[t], idx[t]))
        vals, ind = torch.topk(torch.tensor(logits[t]), 8)
        assert ind.tolist() == idx[t].tolist()
        assert abs(gap[t] - (sel[-1] - np.sort(logits[t])[-9])) < 1e-15
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(np.diff(gates, axis=1) <= 0)


# ---------------------------------------------------------------- whole layer
def _np_inputs(w: synth.Workload, layer_id=0, routing="iid"):
    t = synth.make_layer(w, layer_id, "cpu", routing=routing)
    f = {k: v.double().numpy() if v.dtype in (torch.float32, torch.bfloat16) else v.numpy()
         for k, v in t.items()}
    return t, f


def _dims(w: synth.Workload):
    return layer.Dims(w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.pooled, w.inter,
                      w.n_experts, w.top_k, w.n_shards, 0, w.rms_eps, w.rope_theta)


def _raw_getter(f, w):
    if w.expert_dtype == synth.NVFP4:
        return lambda e: {m: (f[m + "_codes"][e], f[m + "_scales"][e], float(f[m + "_ts"][e]))
                          for m in ("gate", "up", "down")}
    return lambda e: {m: f[m][e] for m in ("gate", "up", "down")}


def _experts(f, w):
    getter = _raw_getter(f, w)
    return layer.nvfp4_experts(getter) if w.expert_dtype == synth.NVFP4 else layer.bf16_experts(getter)


TINY_SHAPES = [
    dict(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, pooled=32, inter=64, n_experts=8, top_k=3,
         window=5, pos=9, T=3),
    dict(hidden=48, n_q_heads=2, n_kv_heads=1, head_dim=8, pooled=32, inter=32, n_experts=6, top_k=2,
         window=0, pos=4, T=2, expert_dtype=synth.BF16),
    dict(hidden=64, n_q_heads=4, n_kv_heads=1, head_dim=16, pooled=64, inter=64, n_experts=8, top_k=2,
         window=3, pos=6, T=4, n_shards=2),
]


@pytest.mark.parametrize("shape", TINY_SHAPES)
def test_layer_matches_bruteforce(shape):
    w = synth.small_workload(**shape)
    _, f = _np_inputs(w)
    dims = _dims(w)
    got = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w))
    ref = brute.layer_step(f, dims, w.pos, w.window, _raw_getter(f, w),
                           nvfp4=w.expert_dtype == synth.NVFP4)
    assert got["idx"].tolist() == ref["idx"]
    np.testing.assert_allclose(got["logits"], np.array(ref["logits"]), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["k_new"], np.array(ref["k_new"]), rtol=0, atol=0)
    np.testing.assert_allclose(got["v_new"], np.array(ref["v_new"]), rtol=0, atol=0)
    np.testing.assert_allclose(got["h"], np.array(ref["h"]), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["y"], np.array(ref["y"]), rtol=1e-9, atol=1e-10)


def test_tiny_workload_matches_bruteforce():
    w = synth.WORKLOADS["tiny"]
    _, f = _np_inputs(w)
    dims = _dims(w)
    got = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w))
    ref = brute.layer_step(f, dims, w.pos, w.window, _raw_getter(f, w), nvfp4=True)
    assert got["idx"].tolist() == ref["idx"]
    np.testing.assert_allclose(got["y"], np.array(ref["y"]), rtol=1e-9, atol=1e-10)
    assert np.isfinite(got["y"]).all()


def test_full_topk_is_dense_softmax_mixture():
    """With k = E the MoE block is sum_e softmax(logits)_e * expert_e(pl): computed here directly."""
    w = synth.small_workload(hidden=64, n_q_heads=2, n_kv_heads=1, head_dim=16, pooled=32, inter=64,
                             n_experts=5, top_k=5, window=0, pos=3, T=2)
    _, f = _np_inputs(w)
    dims = _dims(w)
    out = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w))
    experts = [_experts(f, w)(e) for e in range(5)]
    Wg = np.stack([e[0] for e in experts])
    Wu = np.stack([e[1] for e in experts])
    Wd = np.stack([e[2] for e in experts])
    lg = out["hn"] @ f["w_router"].T
    prob = np.exp(lg - lg.max(axis=1, keepdims=True))
    prob /= prob.sum(axis=1, keepdims=True)
    g = np.einsum("eik,tk->tei", Wg, out["pl"])
    u = np.einsum("eik,tk->tei", Wu, out["pl"])
    a = g / (1 + np.exp(-g)) * u
    d = np.einsum("epi,tei->tep", Wd, a)
    m = np.einsum("te,tep->tp", prob, d)
    y = out["h"] + m @ f["w_unpool"].T
    np.testing.assert_allclose(out["y"], y, rtol=1e-10, atol=1e-10)


def test_force_idx_reproduces_router_choice():
    w = synth.small_workload(**TINY_SHAPES[0])
    _, f = _np_inputs(w)
    dims = _dims(w)
    a = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w))
    b = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w), force_idx=a["idx"])
    np.testing.assert_array_equal(a["y"], b["y"])


def test_cache_write_set_is_exact():
    w = synth.small_workload(**TINY_SHAPES[0])
    _, f = _np_inputs(w)
    out = layer.layer_step(f, _dims(w), w.pos, w.window, _experts(f, w))
    changed = np.any(out["k_cache"] != f["k_cache"], axis=-1)
    written = np.zeros_like(changed)
    written[:, w.pos:w.pos + w.T] = True
    assert not np.any(changed & ~written)
    np.testing.assert_array_equal(out["k_cache"][:, w.pos:w.pos + w.T].transpose(1, 0, 2), out["k_new"])


# ---------------------------------------------------------------- token-tree verify
# A 16-node tree of candidate tokens (two branches off the root, one of them branching again)
TREE16 = [-1, 0, 1, 2, 0, 4, 5, 1, 7, 3, 9, 4, 11, 12, 2, 14]
TREES = [
    [-1, 0, 0, 1],           # root with two children, one grandchild
    [-1, -1, 0, 1],          # two roots (both attach to the cached prefix)
    [-1, 0, 1, 2],           # the chain
]


def _path(parents, t):
    out = []
    while t != -1:
        out.append(t)
        t = parents[t]
    return out[::-1]


def test_tree_depths_and_rejects_bad_parents():
    np.testing.assert_array_equal(layer.tree_depths(TREE16), [len(_path(TREE16, t)) - 1 for t in range(16)])
    with pytest.raises(ValueError):
        layer.tree_depths([-1, 1])
    with pytest.raises(ValueError):
        layer.tree_depths([0])


@pytest.mark.parametrize("tree", TREES, ids=["fork", "two_roots", "chain"])
def test_tree_matches_bruteforce(tree):
    shape = dict(TINY_SHAPES[0], T=len(tree), window=0)
    w = synth.small_workload(**shape)
    _, f = _np_inputs(w)
    dims = _dims(w)
    got = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w), parents=tree)
    ref = brute.layer_step(f, dims, w.pos, w.window, _raw_getter(f, w), nvfp4=True, parents=tree)
    assert got["idx"].tolist() == ref["idx"]
    np.testing.assert_allclose(got["k_new"], np.array(ref["k_new"]), rtol=0, atol=0)
    np.testing.assert_allclose(got["h"], np.array(ref["h"]), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["y"], np.array(ref["y"]), rtol=1e-9, atol=1e-10)


def test_tree_window_matches_bruteforce():
    """A window shorter than the tree's depth: the window rule applies to node positions."""
    tree = [-1, 0, 1, 2, 1]
    w = synth.small_workload(**dict(TINY_SHAPES[0], T=5, window=3, pos=9))
    _, f = _np_inputs(w)
    dims = _dims(w)
    got = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w), parents=tree)
    ref = brute.layer_step(f, dims, w.pos, w.window, _raw_getter(f, w), nvfp4=True, parents=tree)
    np.testing.assert_allclose(got["h"], np.array(ref["h"]), rtol=1e-10, atol=1e-12)


def test_chain_parents_are_the_chain():
    w = synth.small_workload(**TINY_SHAPES[0])
    _, f = _np_inputs(w)
    a = layer.layer_step(f, _dims(w), w.pos, w.window, _experts(f, w))
    b = layer.layer_step(f, _dims(w), w.pos, w.window, _experts(f, w), parents=list(range(-1, w.T - 1)))
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(b["k_new"], a["k_new"])


def test_tree_node_equals_the_chain_of_its_path():
    """Every node of a tree computes what a chain verify of the root-to-node path computes for
    its last token (attention sees the same keys at the same positions; the rest is per token)."""
    w = synth.small_workload(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, pooled=32, inter=64,
                             n_experts=8, top_k=3, window=0, pos=9, T=16)
    _, f = _np_inputs(w)
    dims = _dims(w)
    tree = layer.layer_step(f, dims, w.pos, 0, _experts(f, w), parents=TREE16)
    for t in (3, 6, 10, 13, 15):
        path = _path(TREE16, t)
        g = dict(f, x=f["x"][path])
        chain = layer.layer_step(g, dims, w.pos, 0, _experts(f, w))
        np.testing.assert_allclose(tree["o"][t], chain["o"][-1], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(tree["k_new"][t], chain["k_new"][-1], rtol=0, atol=0)
        np.testing.assert_allclose(tree["y"][t], chain["y"][-1], rtol=1e-10, atol=1e-11)
        if tree["gap"][t] > 1e-9:
            assert tree["idx"][t].tolist() == chain["idx"][-1].tolist()


def test_tree_nodes_outside_the_path_do_not_matter():
    w = synth.small_workload(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, pooled=32, inter=64,
                             n_experts=8, top_k=3, window=0, pos=9, T=16)
    _, f = _np_inputs(w)
    dims = _dims(w)
    a = layer.layer_step(f, dims, w.pos, 0, _experts(f, w), parents=TREE16)
    g = dict(f, x=f["x"].copy())
    off_path = [i for i in range(16) if i not in _path(TREE16, 13)]
    g["x"][off_path] += 1.0
    b = layer.layer_step(g, dims, w.pos, 0, _experts(f, w), parents=TREE16)
    np.testing.assert_array_equal(a["y"][13], b["y"][13])
    assert not np.array_equal(a["y"][off_path[-1]], b["y"][off_path[-1]])


# ---------------------------------------------------------------- fp4 gather of the SwiGLU output
def test_fp4_gather_row_two_implementations_agree():
    """The vectorised encoder (nearest grid point by distance) and the loop-only one (E4M3 by
    significand rounding, E2M1 by its decision points) give identical rows."""
    rng = np.random.default_rng(17)
    for trial in range(6):
        n = 16 * int(rng.integers(1, 9))
        a = rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 1)
        a[rng.random(n) < 0.1] = 0.0
        ts = float(np.float32(10.0 ** rng.uniform(-6, -1)))
        want = brute._fp4_gather([float(v) for v in a], ts)
        got = layer.down_input_nvfp4(a, ts)
        np.testing.assert_array_equal(got, np.array(want))


def _fp4_gather_shape(**kw):
    base = dict(hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, pooled=32, inter=64, n_experts=8,
                top_k=3, window=5, pos=9, T=3, down_input=synth.DOWN_NVFP4)
    base.update(kw)
    return synth.small_workload(**base)


@pytest.mark.parametrize("shards", [1, 2])
def test_layer_fp4_gather_matches_bruteforce(shards):
    w = _fp4_gather_shape(n_shards=shards)
    _, f = _np_inputs(w)
    dims = layer.Dims(w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.pooled, w.inter,
                      w.n_experts, w.top_k, w.n_shards, shards - 1, w.rms_eps, w.rope_theta)
    got = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w), act_scales=f["act_ts"])
    ref = brute.layer_step(f, dims, w.pos, w.window, _raw_getter(f, w), nvfp4=True,
                           act_scales=f["act_ts"])
    assert got["idx"].tolist() == ref["idx"]
    np.testing.assert_allclose(got["y"], np.array(ref["y"]), rtol=1e-9, atol=1e-10)
    plain = layer.layer_step(f, dims, w.pos, w.window, _experts(f, w))
    dd = np.nanmax(np.abs(plain["d"] - got["d"]))
    assert dd > 1e-2 * np.nanmax(np.abs(plain["d"]))      # the gather is not a no-op here


def test_fp4_gather_changes_only_the_down_input():
    """Everything up to the SwiGLU output is unchanged; the down projection reads the encoded
    a (on the 16-element block grid, with the expert's scale) and d is exactly W_d times it."""
    w = _fp4_gather_shape()
    _, f = _np_inputs(w)
    dims = _dims(w)
    ex = _experts(f, w)
    q = layer.layer_step(f, dims, w.pos, w.window, ex, act_scales=f["act_ts"])
    p = layer.layer_step(f, dims, w.pos, w.window, ex)
    for key in ("h", "logits", "pl", "a"):
        np.testing.assert_array_equal(q[key], p[key])
    np.testing.assert_array_equal(q["idx"], p["idx"])
    np.testing.assert_array_equal(p["a_in"], p["a"])
    for t in range(w.T):
        for kk in range(w.top_k):
            e = int(q["idx"][t, kk])
            ts = float(np.float32(f["act_ts"][e]))
            a_in, a = q["a_in"][t, kk], q["a"][t, kk]
            # every value is a code times the block's scale times ts, and within half a code
            # step (a quarter of the block's top step, 2 scale units) of a
            blk_scale = np.abs(a_in).reshape(-1, 16).max(axis=1) / 6.0
            assert np.all(np.abs(a_in - a) <= np.repeat(blk_scale, 16) * 1.0 + 1e-300)
            _, _, Wd = ex(e)
            np.testing.assert_allclose(q["d"][t, kk], Wd @ a_in, rtol=1e-12, atol=1e-15)
            assert not np.array_equal(a_in, a)
            assert 0 < ts
