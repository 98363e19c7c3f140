"""CPU tests of the native library: it loads, exports every entry point the header
declares, and its slot manager (the same code prepare() runs) matches the oracle
bit for bit on the workload traces.  No GPU call is made."""
import os
import re

import numpy as np
import pytest

from expert_slot_cache_amd import binding, synth
from oracle.lru import LayerLRU

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_pool.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = binding.lib()
    declared = _header_functions()
    assert len(declared) >= 20
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(binding.exported_symbols()) == declared


def test_expert_bytes_match_generator_layout():
    for wtype, H, I in [("f32", 64, 32), ("bf16", 2048, 1024), ("int4", 2560, 640),
                        ("bf16", 4096, 1536), ("int4", 128, 256)]:
        assert binding.expert_bytes(wtype, H, I) == synth.expert_bytes(wtype, H, I)
    assert binding.expert_bytes("int4", 2560, 640) == 2534400
    assert binding.expert_bytes("int4", 100, 128) == 0
    assert binding.expert_bytes("bf16", 2044, 1024) == 0


def _compare(E, N, trace, rule="distinct"):
    ref = LayerLRU(E, N, rule)
    lib = binding.SlotLRU(E, N, rule)
    for ids in trace:
        r = ref.step(ids)
        slot_ids, path, misses = lib.step(ids)
        assert path == r.path
        assert (slot_ids == r.slot_ids).all()
        assert misses == r.misses
    m, o, l = lib.state()
    assert m.tolist() == ref.map
    assert o.tolist() == ref.owner
    order = ref.lru_order()
    assert l.tolist() == order + [-1] * (N - len(order))
    st = lib.stats()
    assert (st["steps"], st["hits"], st["misses"], st["fallbacks"]) == \
        (ref.steps, ref.hits, ref.misses, ref.fallbacks)
    return st


@pytest.mark.parametrize("name,slots", [("tiny_f32_e8", 4), ("tiny_f32_e8", 1),
                                        ("olmoe_bf16_e64", 16), ("olmoe_bf16_e64", 64),
                                        ("fanout_int4_e512", 16), ("fanout_int4_e512", 64)])
def test_native_lru_matches_oracle_on_traces(name, slots):
    wl = synth.WORKLOADS[name]
    steps = wl.steps if wl.experts <= 64 else 128
    trace = synth.make_trace(wl.with_(layers=min(wl.layers, 3)), steps=steps)
    for layer in range(trace.shape[1]):
        _compare(wl.experts, slots, [trace[s, layer] for s in range(trace.shape[0])])


@pytest.mark.parametrize("rule", ["distinct", "static"])
def test_native_lru_multi_token_and_fallback(rule):
    wl = synth.WORKLOADS["batched_bf16_e128"].with_(layers=1, tokens=4)
    trace = synth.make_trace(wl, steps=300)
    st = _compare(128, 32, [trace[s, 0] for s in range(300)], rule)
    if rule == "static":
        assert st["fallbacks"] == 0          # 4 tokens x top-8 = 32 <= 32
    wl = wl.with_(tokens=8)
    trace = synth.make_trace(wl, steps=100)
    st = _compare(128, 32, [trace[s, 0] for s in range(100)], rule)
    assert st["fallbacks"] > 0


def test_native_lru_random_small():
    rng = np.random.default_rng(4)
    for _ in range(400):
        E = int(rng.integers(1, 9))
        K = int(rng.integers(1, E + 1))
        N = int(rng.integers(0, E + 2))
        trace = [np.stack([rng.permutation(E)[:K] for _ in range(int(rng.integers(1, 4)))])
                 for _ in range(int(rng.integers(1, 12)))]
        _compare(E, N, trace, "distinct" if rng.random() < 0.5 else "static")


def test_native_lru_errors_leave_state():
    lib = binding.SlotLRU(8, 2)
    lib.step(np.array([[1, 2]]))
    before = [a.copy() for a in lib.state()], lib.stats()
    with pytest.raises(binding.ExpertRangeError):
        lib.step(np.array([[1, 8]]))
    with pytest.raises(binding.ExpertRangeError):
        lib.step(np.array([[-3, 1]]))
    after = lib.state(), lib.stats()
    assert all((a == b).all() for a, b in zip(before[0], after[0])) and before[1] == after[1]
    with pytest.raises(binding.MoeError):
        binding.SlotLRU(0, 2)


def test_native_lru_empty_step():
    lib = binding.SlotLRU(8, 2)
    out, path, misses = lib.step(np.zeros((0, 2), np.int32))
    assert path == binding.PATH_POOL and misses == [] and out.shape == (0, 2)
    assert lib.stats()["steps"] == 1


def test_read_calibration_rejects_bad_arguments_without_a_gpu():
    """The calibration entry point validates its arguments before touching the GPU."""
    import ctypes as C
    us = C.c_double(0)
    L = binding.lib()
    assert L.moe_read_calibration(None, 1 << 20, 1 << 16, 4, None, C.byref(us)) == binding.EINVAL
    assert L.moe_read_calibration(C.c_void_p(16), 1 << 20, 1 << 21, 4, None, C.byref(us)) == binding.EINVAL
    assert L.moe_read_calibration(C.c_void_p(16), 1 << 20, 100, 4, None, C.byref(us)) == binding.EINVAL
    assert L.moe_read_calibration(C.c_void_p(16), 1 << 20, 1 << 16, 0, None, C.byref(us)) == binding.EINVAL
    assert L.moe_link_calibration(100, 4, binding.COPY_KERNEL, 1, None, C.byref(us)) == binding.EINVAL
    assert L.moe_link_calibration(1 << 20, 0, binding.COPY_DMA, 1, None, C.byref(us)) == binding.EINVAL
    assert L.moe_link_calibration(1 << 20, 4, 7, 1, None, C.byref(us)) == binding.EINVAL
    assert L.moe_link_calibration(1 << 20, 4, binding.COPY_DMA, 0, None, C.byref(us)) == binding.EINVAL
    assert L.moe_link_calibration(1 << 20, 4, binding.COPY_DMA, 9, None, C.byref(us)) == binding.EINVAL


def test_create_rejects_bad_eviction_and_prefetch_settings():
    """Config validation of the eviction policy and the prefetch buffer, before any
    GPU call: a policy outside the five, a non-LRU policy with the host slot manager,
    decayed-count placement with read-through steps, prefetch entries out of range,
    with the host slot manager or all-resident."""
    import ctypes as C

    def cfg(policy, evict, pf, resident=0, rt=0):
        return binding.Config(1, 8, 2, 64, 32, 4, binding.WTYPES["f32"], binding.ATYPES["f32"],
                              binding.RULES["distinct"], resident, 1, 1, 0, 0, 0, binding.COPY_KERNEL, policy, rt,
                              evict, pf)
    for c in (cfg(binding.POLICY_DEVICE, 5, 0), cfg(binding.POLICY_DEVICE, -1, 0),
              cfg(binding.POLICY_HOST, binding.EVICT_LFU, 0), cfg(binding.POLICY_HOST, binding.EVICT_DECAY, 0),
              cfg(binding.POLICY_DEVICE, binding.EVICT_DECAY, 0, rt=1), cfg(binding.POLICY_DEVICE, 0, 65),
              cfg(binding.POLICY_DEVICE, 0, -1), cfg(binding.POLICY_HOST, 0, 4),
              cfg(binding.POLICY_DEVICE, 0, 4, resident=1)):
        h = C.c_void_p()
        assert binding.lib().moe_pool_create(C.byref(c), None, C.byref(h)) == binding.EINVAL
        assert not h.value


def test_create_rejects_read_through_without_the_device_policy():
    """Config validation happens before any GPU call."""
    import ctypes as C
    for policy, rt in ((binding.POLICY_HOST, 1), (binding.POLICY_DEVICE, 2)):
        cfg = binding.Config(1, 8, 2, 64, 32, 4, binding.WTYPES["f32"], binding.ATYPES["f32"],
                             binding.RULES["distinct"], 0, 1, 1, 0, 0, 0, binding.COPY_KERNEL, policy, rt)
        h = C.c_void_p()
        assert binding.lib().moe_pool_create(C.byref(cfg), None, C.byref(h)) == binding.EINVAL
        assert not h.value
