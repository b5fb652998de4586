"""ctypes binding of libmoel.so (argument marshalling only; every step runs in the HIP kernels).

Names follow include/moel.h.  Tensors are torch tensors on the GPU; the library only
receives their device pointers and the current HIP stream.
"""
from __future__ import annotations

import ctypes
import os
import sys
from typing import Dict, Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoel.so")

MOEL_OK = 0
MOEL_ERR_ARG = -1
MOEL_ERR_SHAPE = -2
MOEL_ERR_ALIGN = -3
MOEL_ERR_HIP = -4
MOEL_ERR_TIMEOUT = -5
MOEL_ERR_ABORTED = -6
MOEL_ERR_UNSUPPORTED = -7
MOEL_LAUNCH_PLAIN = 0
MOEL_LAUNCH_COOPERATIVE = 1
MOEL_ACQUIRE_AUTO = 0
MOEL_ACQUIRE_L2_INVALIDATE = 1
MOEL_ERR_INTERNAL = -8
MOEL_EXPERT_NVFP4 = 0
MOEL_EXPERT_BF16 = 1
MOEL_DOWN_INPUT_EXACT = 0
MOEL_DOWN_INPUT_NVFP4 = 1
MOEL_N_STAMPS = 32
MOEL_MAX_REQUESTS = 8
MOEL_MAX_TOKENS = 32
STACK_LAYERS_PER_LAUNCH = 4  # MOEL_STACK_LAYERS_PER_LAUNCH


class MoelError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} ({code})")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_q_heads", "n_kv_heads", "head_dim", "pooled", "inter", "n_experts", "top_k",
        "expert_dtype", "n_shards", "shard_rank", "kv_capacity")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("down_input", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "gamma1", "gamma2", "w_qkv", "w_o", "w_router", "w_pool", "w_unpool", "w_gate", "w_up",
        "w_down", "ts_gate", "ts_up", "ts_down", "ts_act", "expert_hist")]


class Request(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "pos", "kv_base", "kv_slots")]


def _requests(reqs):
    """A ctypes array of moel_request from (T, pos, kv_base, kv_slots) tuples."""
    arr = (Request * max(1, len(reqs)))()
    for i, r in enumerate(reqs):
        arr[i] = Request(*[int(v) for v in r])
    return arr


class Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("expert_idx", "gates", "router_logits", "timestamps")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m moe_layer_persistent_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        sigs = {
            "moel_status_string": (ctypes.c_char_p, [i32]),
            "moel_abi_version": (i32, []),
            "moel_validate_config": (i32, [P(Config)]),
            "moel_validate_call": (i32, [P(Config), P(Weights), vp, vp, vp, i32, i32, i32, vp]),
            "moel_packed_dense_bytes": (sz, [i32, i32]),
            "moel_packed_experts_bytes": (sz, [P(Config), i32]),
            "moel_plan_create": (i32, [P(Config), P(vp)]),
            "moel_plan_destroy": (i32, [vp]),
            "moel_plan_workgroups": (i32, [vp]),
            "moel_plan_status": (i32, [vp]),
            "moel_plan_set_abort": (i32, [vp, i32, vp]),
            "moel_plan_poison_scratch": (i32, [vp, vp]),
            "moel_plan_set_launch": (i32, [vp, i32]),
            "moel_plan_set_acquire": (i32, [vp, i32]),
            "moel_plan_set_expert_prefetch": (i32, [vp, i32]),
            "moel_plan_l2_coherent": (i32, [vp]),
            "moel_plan_scratch": (i32, [vp, i32, P(vp), P(sz)]),
            "moel_pack_dense": (i32, [vp, i32, i32, i32, vp, vp]),
            "moel_pack_experts": (i32, [P(Config), i32, vp, vp, vp, vp]),
            "moel_layer_decode": (i32, [vp, P(Weights), vp, vp, vp, i32, i32, i32, vp, P(Debug), vp]),
            "moel_layer_decode_unfused": (i32, [vp, P(Weights), vp, vp, vp, i32, i32, i32, vp, P(Debug), vp]),
            "moel_layer_decode_tree": (i32, [vp, P(Weights), vp, vp, vp, i32, i32, i32, vp, vp, P(Debug), vp]),
            "moel_layer_decode_tree_unfused": (i32, [vp, P(Weights), vp, vp, vp, i32, i32, i32, vp, vp, P(Debug),
                                                     vp]),
            "moel_validate_tree": (i32, [vp, i32]),
            "moel_validate_batch": (i32, [P(Config), i32, vp, i32]),
            "moel_layer_decode_batch": (i32, [vp, P(Weights), vp, vp, vp, i32, vp, i32, vp, P(Debug), vp]),
            "moel_layer_decode_batch_unfused": (i32, [vp, P(Weights), vp, vp, vp, i32, vp, i32, vp, P(Debug),
                                                      vp]),
            "moel_layer_decode_noalloc": (i32, [P(Config), P(Weights), vp, vp, vp, i32, i32, i32, vp, vp, vp]),
            "moel_stack_create": (i32, [vp, i32, P(Weights), vp, vp, vp, P(vp)]),
            "moel_stack_decode": (i32, [vp, vp, i32, i32, vp, vp]),
            "moel_stack_destroy": (i32, [vp]),
            "moel_measure_read_bandwidth": (i32, [vp, sz, i32, P(ctypes.c_float), vp]),
        }
        for name, (res, args) in sigs.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().moel_status_string(code).decode()


def measure_read_bandwidth(buf, reps: int = 10, stream=None) -> float:
    """moel_measure_read_bandwidth over the bytes of the CUDA tensor `buf`: GB/s."""
    g = ctypes.c_float()
    st = torch.cuda.current_stream() if stream is None else stream
    _check(lib().moel_measure_read_bandwidth(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                             int(reps), ctypes.byref(g), ctypes.c_void_p(st.cuda_stream)),
           "moel_measure_read_bandwidth")
    return float(g.value)


def _check(code: int, what: str):
    if code != MOEL_OK:
        raise MoelError(code, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def config_from_workload(w, kv_capacity: Optional[int] = None) -> Config:
    return Config(w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.pooled, w.inter, w.n_experts,
                  w.top_k, w.expert_dtype, w.n_shards, getattr(w, "shard_rank", 0),
                  w.kv_capacity if kv_capacity is None else kv_capacity, w.rms_eps, w.rope_theta,
                  getattr(w, "down_input", MOEL_DOWN_INPUT_EXACT))


class LayerWeights:
    """Packed weights of one layer (device tensors owned here) and their moel_weights struct."""

    def __init__(self, packed: Dict[str, torch.Tensor], ts: Dict[str, Optional[torch.Tensor]]):
        self.packed = packed
        self.ts = ts
        self.struct = Weights(
            _ptr(packed["gamma1"]), _ptr(packed["gamma2"]), _ptr(packed["w_qkv"]), _ptr(packed["w_o"]),
            _ptr(packed["w_router"]), _ptr(packed["w_pool"]), _ptr(packed["w_unpool"]),
            _ptr(packed["w_gate"]), _ptr(packed["w_up"]), _ptr(packed["w_down"]),
            _ptr(ts["gate"]), _ptr(ts["up"]), _ptr(ts["down"]), _ptr(ts.get("act")), None)
        self.history = None

    def set_history(self, hist: Optional[torch.Tensor]):
        """The layer's routing history (int32 or uint32 [E] device tensor, zeroed before the
        layer's first step; None: none): each step writes its tokens per expert there."""
        self.history = hist
        self.struct.expert_hist = _ptr(hist)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.packed.values())


class Plan:
    def __init__(self, cfg: Config):
        self.cfg = cfg
        h = ctypes.c_void_p()
        _check(lib().moel_plan_create(ctypes.byref(cfg), ctypes.byref(h)), "moel_plan_create")
        self.handle = h

    def close(self):
        if self.handle:
            lib().moel_plan_destroy(self.handle)
            self.handle = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # at interpreter shutdown the HIP runtime (and a profiler attached to it) may already
        # be finalised: leave the workspace to the process exit instead of calling hipFree
        # (the check is bound when the class is defined: module globals may be gone by then)
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    @property
    def workgroups(self) -> int:
        return lib().moel_plan_workgroups(self.handle)

    def status(self) -> int:
        return lib().moel_plan_status(self.handle)

    SCRATCH = {"q": 0, "o": 1, "h": 2, "logits": 3, "pl": 4, "a": 5, "d": 6, "m": 7, "aq": 8}

    def scratch(self, name: str) -> torch.Tensor:
        """Copy of an intermediate activation of the last completed step (fp32, flat)."""
        ptr, n = ctypes.c_void_p(), ctypes.c_size_t()
        _check(lib().moel_plan_scratch(self.handle, self.SCRATCH[name], ctypes.byref(ptr), ctypes.byref(n)),
               "moel_plan_scratch")
        out = torch.empty(n.value // 4, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        import ctypes as _c
        hip = _c.CDLL("libamdhip64.so")
        hip.hipMemcpy.argtypes = [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_int]
        rc = hip.hipMemcpy(_c.c_void_p(out.data_ptr()), ptr, n.value, 3)  # device to device
        if rc != 0:
            raise RuntimeError(f"hipMemcpy failed: {rc}")
        return out

    def set_launch(self, mode: int):
        """MOEL_LAUNCH_PLAIN (default) or MOEL_LAUNCH_COOPERATIVE, see include/moel.h."""
        _check(lib().moel_plan_set_launch(self.handle, int(mode)), "moel_plan_set_launch")

    def set_expert_prefetch(self, n_experts: int):
        """Previous-step expert prefetch of the n_experts most-used experts (0 = off), for layers
        whose weights carry a routing history (LayerWeights.set_history), see include/moel.h."""
        _check(lib().moel_plan_set_expert_prefetch(self.handle, int(n_experts)), "moel_plan_set_expert_prefetch")

    def set_acquire(self, mode: int):
        """MOEL_ACQUIRE_AUTO (default) or MOEL_ACQUIRE_L2_INVALIDATE, see include/moel.h."""
        _check(lib().moel_plan_set_acquire(self.handle, int(mode)), "moel_plan_set_acquire")

    @property
    def l2_coherent(self) -> bool:
        """Whether the device passed the L2 coherence check when the plan was created."""
        return lib().moel_plan_l2_coherent(self.handle) == 1

    def set_abort(self, flag: bool, stream=None):
        _check(lib().moel_plan_set_abort(self.handle, int(flag), _stream(stream)), "moel_plan_set_abort")

    def poison_scratch(self, stream=None):
        """All-ones words (NaN) into the plan's activation scratch, see include/moel.h."""
        _check(lib().moel_plan_poison_scratch(self.handle, _stream(stream)), "moel_plan_poison_scratch")

    # ---- packing -------------------------------------------------------------------------
    def pack_dense(self, src: torch.Tensor, rope_head_dim: int = 0, stream=None) -> torch.Tensor:
        assert src.dtype == torch.bfloat16 and src.is_contiguous() and src.dim() == 2
        N, K = src.shape
        dst = torch.empty(lib().moel_packed_dense_bytes(N, K), dtype=torch.uint8, device=src.device)
        _check(lib().moel_pack_dense(_ptr(src), N, K, rope_head_dim, _ptr(dst), _stream(stream)),
               "moel_pack_dense")
        return dst

    def pack_experts(self, which: int, src: torch.Tensor, scales: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
        assert src.is_contiguous() and (scales is None or scales.is_contiguous())
        n = lib().moel_packed_experts_bytes(ctypes.byref(self.cfg), which)
        dst = torch.empty(n, dtype=torch.uint8, device=src.device)
        _check(lib().moel_pack_experts(ctypes.byref(self.cfg), which, _ptr(src), _ptr(scales), _ptr(dst),
                                       _stream(stream)), "moel_pack_experts")
        return dst

    def pack_layer(self, t: Dict[str, torch.Tensor], stream=None) -> LayerWeights:
        """Packs the canonical tensors of synth.make_layer into the kernels' layouts."""
        c = self.cfg
        packed = {
            "gamma1": t["gamma1"].contiguous(), "gamma2": t["gamma2"].contiguous(),
            "w_qkv": self.pack_dense(t["w_qkv"], rope_head_dim=c.head_dim, stream=stream),
            "w_o": self.pack_dense(t["w_o"], stream=stream),
            "w_router": self.pack_dense(t["w_router"], stream=stream),
            "w_pool": self.pack_dense(t["w_pool"], stream=stream),
            "w_unpool": self.pack_dense(t["w_unpool"], stream=stream),
        }
        ts = {"gate": None, "up": None, "down": None}
        for which, m in enumerate(("gate", "up", "down")):
            if c.expert_dtype == MOEL_EXPERT_BF16:
                packed["w_" + m] = self.pack_experts(which, t[m], None, stream=stream)
            else:
                packed["w_" + m] = self.pack_experts(which, t[m + "_codes"], t[m + "_scales"], stream=stream)
                ts[m] = t[m + "_ts"].contiguous()
        if c.down_input == MOEL_DOWN_INPUT_NVFP4:
            ts["act"] = t["act_ts"].contiguous()
        return LayerWeights(packed, ts)

    # ---- the step ------------------------------------------------------------------------
    def layer_decode(self, lw: LayerWeights, k_cache: torch.Tensor, v_cache: torch.Tensor, x: torch.Tensor,
                     pos: int, window: int, y: torch.Tensor, dbg: Optional[Dict[str, torch.Tensor]] = None,
                     fused: bool = True, stream=None, T: Optional[int] = None, parents=None) -> None:
        """One verify step; `parents` (T ints, -1 for a root) makes it a token-tree verify."""
        T = x.shape[0] if T is None else T
        d = None
        if dbg is not None:
            d = Debug(_ptr(dbg.get("expert_idx")), _ptr(dbg.get("gates")), _ptr(dbg.get("router_logits")),
                      _ptr(dbg.get("timestamps")))
        dp = None if d is None else ctypes.byref(d)
        if parents is None:
            name = "moel_layer_decode" if fused else "moel_layer_decode_unfused"
            rc = getattr(lib(), name)(self.handle, ctypes.byref(lw.struct), _ptr(k_cache), _ptr(v_cache), _ptr(x),
                                      T, pos, window, _ptr(y), dp, _stream(stream))
        else:
            par = (ctypes.c_int32 * len(parents))(*[int(v) for v in parents])
            name = "moel_layer_decode_tree" if fused else "moel_layer_decode_tree_unfused"
            rc = getattr(lib(), name)(self.handle, ctypes.byref(lw.struct), _ptr(k_cache), _ptr(v_cache), _ptr(x),
                                      T, pos, window, ctypes.cast(par, ctypes.c_void_p), _ptr(y), dp,
                                      _stream(stream))
        _check(rc, name)

    def layer_decode_batch(self, lw: LayerWeights, k_pool: torch.Tensor, v_pool: torch.Tensor, x: torch.Tensor,
                           requests, window: int, y: torch.Tensor, dbg: Optional[Dict[str, torch.Tensor]] = None,
                           fused: bool = True, stream=None) -> None:
        """One verify step over several requests: `requests` holds (T, pos, kv_base, kv_slots)
        tuples, whose tokens are consecutive rows of x and y in order."""
        d = None
        if dbg is not None:
            d = Debug(_ptr(dbg.get("expert_idx")), _ptr(dbg.get("gates")), _ptr(dbg.get("router_logits")),
                      _ptr(dbg.get("timestamps")))
        arr = _requests(requests)
        name = "moel_layer_decode_batch" if fused else "moel_layer_decode_batch_unfused"
        rc = getattr(lib(), name)(self.handle, ctypes.byref(lw.struct), _ptr(k_pool), _ptr(v_pool), _ptr(x),
                                  len(requests), ctypes.cast(arr, ctypes.c_void_p), window, _ptr(y),
                                  None if d is None else ctypes.byref(d), _stream(stream))
        _check(rc, name)


def validate_batch(cfg: Config, reqs, workgroups: int = 0) -> int:
    """moel_validate_batch over (T, pos, kv_base, kv_slots) tuples; returns the status."""
    arr = _requests(reqs)
    return lib().moel_validate_batch(ctypes.byref(cfg), len(reqs), ctypes.cast(arr, ctypes.c_void_p), workgroups)


def layer_decode_noalloc(cfg: Config, lw: LayerWeights, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         x: torch.Tensor, pos: int, window: int, y: torch.Tensor,
                         status: Optional[torch.Tensor] = None, stream=None, T: Optional[int] = None) -> None:
    """moel_layer_decode_noalloc: one verify step without a plan (the library's static scratch);
    `status` is an optional int32 device tensor of one element that receives the device status."""
    T = x.shape[0] if T is None else T
    rc = lib().moel_layer_decode_noalloc(ctypes.byref(cfg), ctypes.byref(lw.struct), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(x), T, pos, window, _ptr(y), _ptr(status), _stream(stream))
    _check(rc, "moel_layer_decode_noalloc")


class Stack:
    """A stack of layers of one plan's shape run as one persistent launch per step
    (moel_stack_create / moel_stack_decode, include/moel.h)."""

    def __init__(self, plan: Plan, layers, k_caches, v_caches, windows):
        n = len(layers)
        self.plan, self.layers, self.k, self.v = plan, list(layers), list(k_caches), list(v_caches)
        warr = (Weights * n)(*[lw.struct for lw in layers])
        karr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_caches])
        varr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_caches])
        wins = (ctypes.c_int32 * n)(*[int(x) for x in windows])
        h = ctypes.c_void_p()
        _check(lib().moel_stack_create(plan.handle, n, warr, karr, varr, wins, ctypes.byref(h)), "moel_stack_create")
        self.handle = h

    def decode(self, x: torch.Tensor, pos: int, y: torch.Tensor, stream=None, T: Optional[int] = None) -> None:
        T = x.shape[0] if T is None else T
        _check(lib().moel_stack_decode(self.handle, _ptr(x), T, pos, _ptr(y), _stream(stream)), "moel_stack_decode")

    def close(self):
        if self.handle:
            lib().moel_stack_destroy(self.handle)
            self.handle = None

    def __del__(self, _finalizing=sys.is_finalizing):
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass
