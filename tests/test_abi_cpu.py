"""The C-ABI library on a machine without a GPU: it loads, exports every entry point the
header declares, and its host-side validation returns the documented error codes."""
import ctypes
import os
import re

import pytest

from moe_layer_persistent_amd import binding, synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moel.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moel_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    names = _declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert L.moel_abi_version() == 7


def test_plan_options_reject_a_missing_plan():
    L = binding.lib()
    assert L.moel_plan_set_launch(None, binding.MOEL_LAUNCH_PLAIN) == binding.MOEL_ERR_ARG
    assert L.moel_plan_set_launch(None, 5) == binding.MOEL_ERR_ARG
    assert L.moel_plan_set_acquire(None, binding.MOEL_ACQUIRE_AUTO) == binding.MOEL_ERR_ARG
    assert L.moel_plan_set_expert_prefetch(None, 14) == binding.MOEL_ERR_ARG
    assert L.moel_plan_poison_scratch(None, None) == binding.MOEL_ERR_ARG
    assert L.moel_plan_l2_coherent(None) == -1


def test_tree_validation():
    L = binding.lib()
    arr = lambda v: (ctypes.c_int32 * len(v))(*v)
    assert L.moel_validate_tree(None, 16) == binding.MOEL_OK
    assert L.moel_validate_tree(arr([-1, 0, 0, 1]), 4) == binding.MOEL_OK
    assert L.moel_validate_tree(arr([-1, -1, 1]), 3) == binding.MOEL_OK
    assert L.moel_validate_tree(arr([-1, 1]), 2) == binding.MOEL_ERR_ARG      # not before its child
    assert L.moel_validate_tree(arr([0]), 1) == binding.MOEL_ERR_ARG
    assert L.moel_validate_tree(arr([-2, 0]), 2) == binding.MOEL_ERR_ARG
    assert L.moel_validate_tree(arr([-1] * 32), 32) == binding.MOEL_OK
    assert L.moel_validate_tree(arr([-1] * 33), 33) == binding.MOEL_ERR_ARG    # T > 32


def test_shapes_beyond_the_32_bit_work_split_are_rejected():
    L = binding.lib()
    for field, value in (("hidden", 1 << 17), ("pooled", 1 << 17), ("inter", 1 << 18)):
        c = _cfg(**{field: value})
        assert L.moel_validate_config(ctypes.byref(c)) == binding.MOEL_ERR_SHAPE, field


def _cfg(**kw):
    w = synth.WORKLOADS["swa_fp4"]
    c = binding.config_from_workload(w)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,code", [
    ("hidden", 100, binding.MOEL_ERR_SHAPE),
    ("head_dim", 96, binding.MOEL_ERR_SHAPE),
    ("n_q_heads", 60, binding.MOEL_ERR_SHAPE),
    ("top_k", 9, binding.MOEL_ERR_SHAPE),
    ("n_experts", 8, binding.MOEL_ERR_SHAPE),
    ("inter", 4000, binding.MOEL_ERR_SHAPE),
    ("shard_rank", 1, binding.MOEL_ERR_ARG),
    ("expert_dtype", 7, binding.MOEL_ERR_ARG),
    ("kv_capacity", 0, binding.MOEL_ERR_ARG),
    ("rms_eps", 0.0, binding.MOEL_ERR_ARG),
    ("down_input", 2, binding.MOEL_ERR_ARG),
])
def test_validate_config_rejects(field, value, code):
    assert binding.lib().moel_validate_config(ctypes.byref(_cfg(**{field: value}))) == code


def test_validate_config_accepts_workloads():
    for w in synth.WORKLOADS.values():
        c = binding.config_from_workload(w)
        assert binding.lib().moel_validate_config(ctypes.byref(c)) == binding.MOEL_OK, w.name


def test_fp4_gather_needs_nvfp4_experts_and_scales():
    L = binding.lib()
    c = _cfg(down_input=binding.MOEL_DOWN_INPUT_NVFP4)
    assert L.moel_validate_config(ctypes.byref(c)) == binding.MOEL_OK
    cb = _cfg(down_input=binding.MOEL_DOWN_INPUT_NVFP4, expert_dtype=binding.MOEL_EXPERT_BF16)
    assert L.moel_validate_config(ctypes.byref(cb)) == binding.MOEL_ERR_SHAPE
    w = _fake_weights()
    vp = ctypes.c_void_p
    args = (vp(0x100000), vp(0x200000), vp(0x300000), 16, 0, 0, vp(0x400000))
    assert L.moel_validate_call(ctypes.byref(c), ctypes.byref(w), *args) == binding.MOEL_OK
    w.ts_act = None
    assert L.moel_validate_call(ctypes.byref(c), ctypes.byref(w), *args) == binding.MOEL_ERR_ARG
    c0 = _cfg()
    assert L.moel_validate_call(ctypes.byref(c0), ctypes.byref(w), *args) == binding.MOEL_OK


def _fake_weights(base=0x10000):
    vals = [base + 0x1000 * i for i in range(14)]
    return binding.Weights(*[ctypes.c_void_p(v) for v in vals])


@pytest.mark.parametrize("T,pos,window,code", [
    (0, 10, 0, binding.MOEL_ERR_ARG),
    (33, 10, 0, binding.MOEL_ERR_ARG),
    (32, 10, 0, binding.MOEL_OK),
    (16, -1, 0, binding.MOEL_ERR_ARG),
    (16, 10, -1, binding.MOEL_ERR_ARG),
    (16, 8192 + 1, 0, binding.MOEL_ERR_ARG),     # pos + T > kv_capacity (8208)
    (16, 8192, 2048, binding.MOEL_OK),
    (1, 0, 0, binding.MOEL_OK),
])
def test_validate_call_ranges(T, pos, window, code):
    c = _cfg()
    w = _fake_weights()
    vp = ctypes.c_void_p
    got = binding.lib().moel_validate_call(ctypes.byref(c), ctypes.byref(w), vp(0x100000), vp(0x200000),
                                          vp(0x300000), T, pos, window, vp(0x400000))
    assert got == code


def test_validate_call_alignment_and_alias():
    c = _cfg()
    w = _fake_weights()
    vp = ctypes.c_void_p
    L = binding.lib()
    assert L.moel_validate_call(ctypes.byref(c), ctypes.byref(w), vp(0x100008), vp(0x200000), vp(0x300000),
                                16, 0, 0, vp(0x400000)) == binding.MOEL_ERR_ALIGN
    assert L.moel_validate_call(ctypes.byref(c), ctypes.byref(w), vp(0x100000), vp(0x200000), vp(0x300000),
                                16, 0, 0, vp(0x300000 + 4096)) == binding.MOEL_ERR_ARG   # y overlaps x
    assert L.moel_validate_call(ctypes.byref(c), ctypes.byref(w), None, vp(0x200000), vp(0x300000),
                                16, 0, 0, vp(0x400000)) == binding.MOEL_ERR_ARG
    w.expert_hist = 0x500002  # the routing history takes 4-byte words
    assert L.moel_validate_call(ctypes.byref(c), ctypes.byref(w), vp(0x100000), vp(0x200000), vp(0x300000),
                                16, 0, 0, vp(0x400000)) == binding.MOEL_ERR_ALIGN
    w.expert_hist = 0x500004
    assert L.moel_validate_call(ctypes.byref(c), ctypes.byref(w), vp(0x100000), vp(0x200000), vp(0x300000),
                                16, 0, 0, vp(0x400000)) == binding.MOEL_OK
    w.ts_up = None
    assert L.moel_validate_call(ctypes.byref(c), ctypes.byref(w), vp(0x100000), vp(0x200000), vp(0x300000),
                                16, 0, 0, vp(0x400000)) == binding.MOEL_ERR_ARG


def test_packed_sizes_equal_canonical_bytes():
    L = binding.lib()
    w = synth.WORKLOADS["swa_fp4"]
    c = binding.config_from_workload(w)
    assert L.moel_packed_dense_bytes(10240, 8192) == 10240 * 8192 * 2
    per = 4096 * 4096 // 2 + 4096 * 4096 // 16
    for which in range(3):
        assert L.moel_packed_experts_bytes(ctypes.byref(c), which) == 256 * per
    s = synth.WORKLOADS["stack_tp8"]
    c4 = binding.config_from_workload(s)
    assert L.moel_packed_experts_bytes(ctypes.byref(c4), 0) == 256 * 512 * (4096 // 2 + 4096 // 16)
    assert L.moel_packed_experts_bytes(ctypes.byref(c4), 2) == 256 * 512 * (4096 // 2 + 4096 // 16)


def test_status_strings():
    for code in range(0, -8, -1):
        assert binding.status_string(code) != "unknown status"


def test_nvfp4_tile_numbers_must_fit_the_hand_out_words():
    """The NVFP4 expert phases hand tiles out as (sequence << 16) | tile: shapes whose tile
    numbers (64-row tiles per expert x active experts) would not fit 15 bits are rejected."""
    L = binding.lib()
    # 65536 intermediate rows = 1024 tiles per expert, 64 experts active: 65536 tiles
    c = _cfg(inter=65536, n_experts=64, top_k=4)
    assert L.moel_validate_config(ctypes.byref(c)) == binding.MOEL_ERR_SHAPE
    # the same shape split over 8 GPUs fits (128 tiles per expert)
    c = _cfg(inter=65536, n_experts=64, top_k=4, n_shards=8)
    assert L.moel_validate_config(ctypes.byref(c)) == binding.MOEL_OK
    # bf16 experts hand out plain tile numbers
    c = _cfg(inter=65536, n_experts=64, top_k=4, expert_dtype=binding.MOEL_EXPERT_BF16)
    assert L.moel_validate_config(ctypes.byref(c)) == binding.MOEL_OK
    # the full-width layer: 64 tiles per expert, at most 256 active entries
    assert L.moel_validate_config(ctypes.byref(_cfg())) == binding.MOEL_OK


def test_stack_calls_reject_missing_arguments():
    L = binding.lib()
    out = ctypes.c_void_p()
    assert L.moel_stack_create(None, 2, None, None, None, None, ctypes.byref(out)) == binding.MOEL_ERR_ARG
    assert L.moel_stack_decode(None, None, 16, 0, None, None) == binding.MOEL_ERR_ARG
    assert L.moel_stack_destroy(None) == binding.MOEL_ERR_ARG


def test_read_bandwidth_reference_rejects_bad_arguments():
    """moel_measure_read_bandwidth checks its host arguments before any HIP call."""
    L = binding.lib()
    g = ctypes.c_float()
    assert L.moel_measure_read_bandwidth(None, 1 << 20, 10, ctypes.byref(g), None) == binding.MOEL_ERR_ARG
    assert L.moel_measure_read_bandwidth(ctypes.c_void_p(4096), 1 << 20, 10, None, None) == binding.MOEL_ERR_ARG
    assert L.moel_measure_read_bandwidth(ctypes.c_void_p(4096), 1 << 20, 0, ctypes.byref(g), None) == binding.MOEL_ERR_ARG
    assert L.moel_measure_read_bandwidth(ctypes.c_void_p(4096), 1 << 20, 1001, ctypes.byref(g), None) == binding.MOEL_ERR_ARG
    assert L.moel_measure_read_bandwidth(ctypes.c_void_p(4100), 1 << 20, 10, ctypes.byref(g), None) == binding.MOEL_ERR_ALIGN


def test_validate_batch():
    c = _cfg()  # kv_capacity 8208, 8 kv heads
    ok = binding.MOEL_OK
    v = lambda reqs, wg=0: binding.validate_batch(c, reqs, wg)
    assert v([(5, 100, 0, 1000), (7, 0, 1000, 1000), (4, 990, 2000, 1000)]) == ok
    assert v([(16, 8192, 0, 8208)]) == ok                          # one request over the whole pool
    assert v([(1, 0, 8 * i, 8) for i in range(8)]) == ok           # eight requests
    assert v([]) == binding.MOEL_ERR_ARG                           # no request
    assert v([(1, 0, 8 * i, 8) for i in range(9)]) == binding.MOEL_ERR_ARG   # more than 8
    assert v([(0, 10, 0, 100)]) == binding.MOEL_ERR_ARG            # T = 0
    assert v([(2, -1, 0, 100)]) == binding.MOEL_ERR_ARG            # pos < 0
    assert v([(2, 0, -1, 100)]) == binding.MOEL_ERR_ARG            # kv_base < 0
    assert v([(2, 0, 0, 0)]) == binding.MOEL_ERR_ARG               # no slots
    assert v([(2, 99, 0, 100)]) == binding.MOEL_ERR_ARG            # pos + T > kv_slots
    assert v([(2, 98, 0, 100)]) == ok
    assert v([(2, 0, 8200, 9)]) == binding.MOEL_ERR_ARG            # past kv_capacity
    assert v([(2, 0, 8199, 9)]) == ok
    assert v([(2, 0, 0, 100), (2, 0, 99, 100)]) == binding.MOEL_ERR_ARG   # slot ranges overlap
    assert v([(2, 0, 100, 100), (2, 0, 0, 101)]) == binding.MOEL_ERR_ARG  # overlap, other order
    assert v([(2, 0, 0, 100), (2, 0, 100, 100)]) == ok                    # adjacent
    assert v([(17, 0, 0, 100), (16, 0, 100, 100)]) == binding.MOEL_ERR_ARG  # 33 tokens
    assert v([(16, 0, 0, 100), (16, 0, 100, 100)]) == ok
    reqs = [(1, 0, 8 * i, 8) for i in range(3)]
    assert v(reqs, 24) == ok                                       # 3 x 8 attention items
    assert v(reqs, 23) == binding.MOEL_ERR_SHAPE
    reqs = [(9, 0, 0, 100), (8, 0, 100, 100)]                      # two 16-token tiles
    assert v(reqs, 32) == ok                                       # 2 x 8 x 2 attention items
    assert v(reqs, 31) == binding.MOEL_ERR_SHAPE


def test_batch_calls_reject_bad_requests_before_any_launch():
    # no plan: rejected before anything else; a NULL request array: rejected by validation
    L = binding.lib()
    w = _fake_weights()
    vp = ctypes.c_void_p
    reqs = binding._requests([(4, 0, 0, 100)])
    for name in ("moel_layer_decode_batch", "moel_layer_decode_batch_unfused"):
        f = getattr(L, name)
        assert f(None, ctypes.byref(w), vp(0x100000), vp(0x200000), vp(0x300000), 1,
                 ctypes.cast(reqs, vp), 0, vp(0x400000), None, None) == binding.MOEL_ERR_ARG
