"""GPU tests of prepare(): slot maps, miss lists, counters, LRU order and slot bytes,
bit-exact against the oracle.  Re-creates the unit list of the vLLM PR "Run MoE
models exceeding VRAM via expert CPU offloading with GPU cache" (test results) and
the llama.cpp discussion's checks (bypass control, stale map table)."""
import time

import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, check_close, from_dev_act, to_dev_act
from expert_slot_cache_amd import binding, synth
from oracle.lru import FALLBACK, POOL, LayerLRU

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.Workload("small_bf16_e32", 2, 32, 4, 256, 128, 8, 1, 64, "bf16", "bf16",
                            1.0, 0.5, 0, 99)
SMALL_INT4 = synth.Workload("small_int4_e32", 2, 32, 4, 256, 128, 8, 1, 64, "int4", "bf16",
                            1.0, 0.5, 0, 98)


def _run_trace_prepare(rig, trace, lrus):
    for s in range(trace.shape[0]):
        for l in range(trace.shape[1]):
            ids = trace[s, l]
            ids_d = torch.from_numpy(ids).to(DEV)
            slot_d = torch.empty_like(ids_d)
            path, misses = rig.pool.prepare(l, ids_d, ids.shape[0], slot_d)
            r = lrus[l].step(ids)
            assert path == r.path, (s, l)
            assert misses == r.misses, (s, l)
            assert (slot_d.cpu().numpy() == r.slot_ids).all(), (s, l)


def _check_state(rig, lrus):
    for l, ref in enumerate(lrus):
        m, o, order = rig.pool.state(l)
        assert m.tolist() == ref.map
        assert o.tolist() == ref.owner
        lo = ref.lru_order()
        assert order.tolist() == lo + [-1] * (len(o) - len(lo))
        st = rig.pool.stats(l)
        assert (st["steps"], st["hits"], st["misses"], st["fallbacks"]) == \
            (ref.steps, ref.hits, ref.misses, ref.fallbacks)


@pytest.mark.parametrize("name,slots,steps,layers", [
    ("tiny_f32_e8", 4, 256, 1),
    ("tiny_f32_e8", 1, 64, 1),
    ("olmoe_bf16_e64", 16, 96, 2),
    ("fanout_int4_e512", 32, 48, 2),
])
def test_prepare_matches_oracle(name, slots, steps, layers):
    wl = synth.WORKLOADS[name].with_(layers=layers)
    trace = synth.make_trace(wl, steps=steps)
    # prepare never reads slot bytes: a store of zeros keeps set-up cheap
    eb = synth.expert_bytes(wl.wtype, wl.hidden, wl.inter)
    zero = np.zeros(eb, np.uint8)
    rig = Rig(wl, slots=slots, experts=[[zero] * wl.experts] * layers)
    lrus = [LayerLRU(wl.experts, slots) for _ in range(layers)]
    _run_trace_prepare(rig, trace, lrus)
    _check_state(rig, lrus)
    rig.close()


def test_evict_then_reinsert_in_same_step():
    """Ascending processing can evict an expert of the step before its own turn:
    with LRU order [5, 7], step [1, 5] evicts 5 for 1's miss, then re-inserts 5 by
    evicting 7.  The map table must end with the step's final entries (here the
    update list holds expert 5 twice)."""
    wl = SMALL_BF16.with_(layers=1, experts=8, top_k=2)
    rig = Rig(wl, slots=2)
    ref = LayerLRU(8, 2)
    for ids in ([[5, 7]], [[1, 5]], [[5, 1]], [[7, 5]], [[1, 7]]):
        ids = np.array(ids, np.int32)
        ids_d = torch.from_numpy(ids).to(DEV)
        slot_d = torch.empty_like(ids_d)
        path, misses = rig.pool.prepare(0, ids_d, 1, slot_d)
        r = ref.step(ids)
        assert misses == r.misses and (slot_d.cpu().numpy() == r.slot_ids).all(), (ids, misses)
    assert ref.misses == 2 + 2 + 0 + 1 + 1   # [7,5]: 5 hits, 7 evicts 1; [1,7]: 1 evicts 5
    rig.close()


@pytest.mark.parametrize("engine", ["dma", "kernel"])
def test_slot_bytes_equal_store_after_eviction(engine):
    """test_gpu_buffer_matches_source_weights / _correct_after_eviction and the
    scale tests: every occupied slot holds exactly its owner's bytes (codes and
    scales for INT4), after heavy churn, with either copy engine."""
    for wl in (SMALL_BF16, SMALL_INT4):
        rig = Rig(wl, slots=5, fast=True, copy_chunk_bytes=4096, copy_streams=3, copy_engine=engine)
        trace = synth.make_trace(wl, steps=40)
        lrus = [LayerLRU(wl.experts, 5) for _ in range(wl.layers)]
        _run_trace_prepare(rig, trace, lrus)
        assert sum(l.misses for l in lrus) > 40
        for l in range(wl.layers):
            _, owner, _ = rig.pool.state(l)
            for s, e in enumerate(owner):
                if e >= 0:
                    got = rig.pool.read_slot(l, s)
                    assert (got == rig.experts[l][e]).all(), (wl.name, l, s, e)
                    assert (rig.pool.store_view(l, e) == rig.experts[l][e]).all()
        st = rig.pool.stats()
        assert st["bytes_h2d"] == st["misses"] * rig.pool.expert_nbytes
        rig.close()


def test_store_is_pinned_and_slots_fixed():
    wl = SMALL_BF16
    rig = Rig(wl, slots=4)
    assert binding.is_pinned_host(rig.pool.store_ptr(0, 3))
    assert not binding.is_pinned_host(np.zeros(16, np.uint8).ctypes.data)
    before = [rig.pool.slot_ptr(l, s) for l in range(wl.layers) for s in range(4)]
    trace = synth.make_trace(wl, steps=30)
    _run_trace_prepare(rig, trace, [LayerLRU(wl.experts, 4) for _ in range(wl.layers)])
    after = [rig.pool.slot_ptr(l, s) for l in range(wl.layers) for s in range(4)]
    assert before == after
    eb = rig.pool.expert_nbytes
    assert after[1] - after[0] == eb
    rig.close()


def test_capacity_equal_experts_and_capacity_one():
    wl = SMALL_BF16.with_(layers=1)
    trace = synth.make_trace(wl, steps=60)
    rig = Rig(wl, slots=wl.experts)
    lrus = [LayerLRU(wl.experts, wl.experts)]
    _run_trace_prepare(rig, trace, lrus)
    seen = len(set(trace.ravel().tolist()))
    assert rig.pool.stats()["misses"] == seen
    _run_trace_prepare(rig, trace, lrus)          # warm: no new misses
    assert rig.pool.stats()["misses"] == seen
    rig.close()
    wl1 = wl.with_(top_k=1)
    trace = synth.make_trace(wl1, steps=80)
    rig = Rig(wl1, slots=1)
    _run_trace_prepare(rig, trace, [LayerLRU(wl.experts, 1)])
    changes = 1 + int((trace[1:, 0, 0, 0] != trace[:-1, 0, 0, 0]).sum())
    assert rig.pool.stats()["misses"] == changes
    rig.close()


def test_overflow_falls_back_exactly_above_capacity():
    """test_overflow_raises / test_no_overflow_at_capacity, with the fallback in
    place of the raise: D == N pools, D == N + 1 falls back and leaves the pool
    untouched; staging holds the step's experts in ascending id order."""
    wl = SMALL_BF16.with_(layers=1, top_k=4)
    rig = Rig(wl, slots=8, max_tokens=4)
    ids = np.array([[0, 1, 2, 3], [4, 5, 6, 7]], np.int32)          # D = 8 = N
    ids_d = torch.from_numpy(ids).to(DEV)
    slot_d = torch.empty_like(ids_d)
    path, misses = rig.pool.prepare(0, ids_d, 2, slot_d)
    assert path == binding.PATH_POOL and len(misses) == 8
    snap = [a.copy() for a in rig.pool.state(0)], rig.pool.stats(0)
    ids9 = np.array([[0, 1, 2, 3], [4, 5, 6, 7], [30, 1, 2, 3]], np.int32)   # D = 9 > N
    ids_d = torch.from_numpy(ids9).to(DEV)
    slot_d = torch.empty_like(ids_d)
    path, misses = rig.pool.prepare(0, ids_d, 3, slot_d)
    assert path == binding.PATH_FALLBACK and misses == []
    assert slot_d.cpu().numpy().tolist() == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 1, 2, 3]]
    now = rig.pool.state(0), rig.pool.stats(0)
    assert all((a == b).all() for a, b in zip(snap[0], now[0]))
    assert {k: v for k, v in now[1].items() if k not in ("steps", "fallbacks", "bytes_h2d", "staged")} == \
        {k: v for k, v in snap[1].items() if k not in ("steps", "fallbacks", "bytes_h2d", "staged")}
    assert now[1]["fallbacks"] == 1 and now[1]["staged"] == 9
    for r, e in enumerate(sorted(set(ids9.ravel().tolist()))):
        assert (rig.pool.read_staging(r) == rig.experts[0][e]).all()
    rig.close()


def test_out_of_range_id_rejected_state_untouched():
    wl = SMALL_BF16.with_(layers=1)
    rig = Rig(wl, slots=4)
    ok = torch.tensor([[1, 2, 3, 4]], dtype=torch.int32, device=DEV)
    slot_d = torch.empty_like(ok)
    rig.pool.prepare(0, ok, 1, slot_d)
    snap = [a.copy() for a in rig.pool.state(0)], rig.pool.stats(0)
    for bad in ([[1, 2, 3, 32]], [[-1, 2, 3, 4]]):
        with pytest.raises(binding.ExpertRangeError):
            rig.pool.prepare(0, torch.tensor(bad, dtype=torch.int32, device=DEV), 1, slot_d)
    now = rig.pool.state(0), rig.pool.stats(0)
    assert all((a == b).all() for a, b in zip(snap[0], now[0])) and snap[1] == now[1]
    rig.close()


def test_step_out_of_range_id_rejected_then_resumes():
    """A bad id in a one-call step is reported, leaves the slot state untouched and
    prepares nothing; the next step runs at once and is correct."""
    wl = SMALL_BF16.with_(layers=1)
    rig = Rig(wl, slots=4, one_call=True)
    rng = synth.streams(wl)[2]
    x = synth.draw_activations(rng, (1, wl.hidden), "bf16")
    w = synth.draw_gate_weights(rng, (1, wl.top_k))
    xd, wd = to_dev_act(x, "bf16"), torch.from_numpy(w).to(DEV)
    ok = np.array([[1, 2, 3, 4]], np.int32)
    rig.step(0, ok, xd, wd)
    snap = [a.copy() for a in rig.pool.state(0)], rig.pool.stats(0)
    out = torch.empty((1, wl.hidden), dtype=torch.bfloat16, device=DEV)
    s = torch.empty((1, wl.top_k), dtype=torch.int32, device=DEV)
    for bad in ([[1, 2, 3, 32]], [[-1, 2, 3, 4]]):
        with pytest.raises(binding.ExpertRangeError):
            rig.pool.step(0, torch.tensor(bad, dtype=torch.int32, device=DEV), 1, s, xd, wd, out)
    now = rig.pool.state(0), rig.pool.stats(0)
    assert all((a == b).all() for a, b in zip(snap[0], now[0])) and snap[1] == now[1]
    with pytest.raises(binding.StateError):          # the failed step prepared nothing
        rig.pool.forward(0, xd, s, wd, out, 1)
    t0 = time.perf_counter()
    ids = np.array([[4, 5, 6, 1]], np.int32)
    _, misses, _, got = rig.step(0, ids, xd, wd)
    torch.cuda.synchronize()
    assert time.perf_counter() - t0 < 2.0
    assert sorted(m[0] for m in misses) == [5, 6]
    check_close(from_dev_act(got), rig.reference(0, x, ids, w), "bf16", "bf16", "after a rejected step")
    rig.close()


def test_mixed_call_styles_share_staging():
    """Layers driven by one-call steps and by prepare + forward, interleaved, with
    small pools so that several layers fall back into the shared staging area:
    bit-identical to the all-resident layers, and the miss/fallback counts match
    the oracle LRU."""
    wl = synth.Workload("mixed", 3, 24, 4, 256, 128, 5, 2, 0, "bf16", "bf16", 1.1, 0.4, 0, 21)
    trace = synth.make_trace(wl, steps=16)
    rng = synth.streams(wl)[2]
    xs = [synth.draw_activations(rng, (2, wl.hidden), "bf16") for _ in range(16)]
    ws = [synth.draw_gate_weights(rng, (2, wl.top_k)) for _ in range(16)]
    mixed = Rig(wl, slots=5)
    res = Rig(wl, slots=5, resident=True, experts=mixed.experts)
    refs = [LayerLRU(wl.experts, 5) for _ in range(wl.layers)]
    for s_ in range(16):
        xd, wd = to_dev_act(xs[s_], "bf16"), torch.from_numpy(ws[s_]).to(DEV)
        for l in range(wl.layers):
            mixed.one_call = (s_ + l) % 2 == 0
            path, misses, _, got = mixed.step(l, trace[s_, l], xd, wd)
            _, _, _, want = res.step(l, trace[s_, l], xd, wd)
            r = refs[l].step(trace[s_, l])
            assert path == r.path and misses == r.misses, (s_, l)
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (s_, l)
    st = mixed.pool.stats()
    assert st["fallbacks"] == sum(r.fallbacks for r in refs) > 0
    mixed.close()
    res.close()


def test_forward_without_prepare_is_state_error():
    wl = SMALL_BF16.with_(layers=2)
    rig = Rig(wl, slots=4)
    x = torch.zeros((1, wl.hidden), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((1, wl.top_k), dtype=torch.float32, device=DEV)
    s = torch.zeros((1, wl.top_k), dtype=torch.int32, device=DEV)
    out = torch.empty_like(x)
    with pytest.raises(binding.StateError):
        rig.pool.forward(0, x, s, w, out, 1)
    rig.pool.prepare(0, torch.tensor([[0, 1, 2, 3]], dtype=torch.int32, device=DEV), 1, s)
    with pytest.raises(binding.StateError):
        rig.pool.forward(0, x, s, w, out, 2)         # n_tokens differs from prepare
    with pytest.raises(binding.StateError):
        rig.pool.forward(1, x, s, w, out, 1)         # other layer never prepared
    rig.pool.forward(0, x, s, w, out, 1)
    rig.pool.reset()
    with pytest.raises(binding.StateError):
        rig.pool.forward(0, x, s, w, out, 1)
    assert rig.pool.stats()["steps"] == 0
    rig.close()


def test_zero_tokens_and_zero_slots():
    wl = SMALL_BF16.with_(layers=1)
    rig = Rig(wl, slots=0, max_tokens=2)
    ids = torch.tensor([[3, 1, 2, 0]], dtype=torch.int32, device=DEV)
    s = torch.empty_like(ids)
    path, misses = rig.pool.prepare(0, ids, 1, s)
    assert path == binding.PATH_FALLBACK and s.cpu().tolist() == [[3, 1, 2, 0]]
    path, misses = rig.pool.prepare(0, ids, 0, s)
    assert path == binding.PATH_POOL and misses == []
    st = rig.pool.stats(0)
    assert st["steps"] == 2 and st["fallbacks"] == 1 and st["hits"] == st["misses"] == 0
    rig.close()


def test_read_calibration_times_a_plain_read():
    """The streaming-read calibration returns a positive duration, and a larger read
    takes longer than a small one."""
    buf = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
    buf.fill_(3)
    small = binding.read_calibration(buf, 1 << 20, reps=8)
    big = binding.read_calibration(buf, 32 << 20, reps=8)
    assert 0 < small < big


@pytest.mark.parametrize("one_call", [False, True])
def test_copy_kernel_many_misses_and_staging(one_call):
    """More misses in one step than a copy-kernel launch carries (batches of 16),
    and a fallback that stages every expert of the step: every slot and every
    staging entry equals its expert's bytes, and the step's outputs equal those of
    the DMA engine bit for bit."""
    wl = synth.Workload("manymiss", 1, 48, 8, 256, 128, 24, 4, 0, "bf16", "bf16", 1.0, 0.0, 0, 31)
    rng = np.random.default_rng(5)

    def rows(lo, hi):        # 4 tokens x 8 distinct ids that together cover [lo, hi)
        span = np.arange(lo, hi)
        out = [np.resize(np.roll(span, -8 * t), 8) for t in range(4)]
        return np.stack([rng.permutation(r) for r in out]).astype(np.int32)

    steps = [rows(0, 20),      # 20 misses: two copy batches
             rows(10, 40),     # 30 distinct > 24 slots: fallback, 30 experts staged
             rows(20, 40)]     # 20 misses, 16 of them evicting
    steps += [np.stack([rng.permutation(48)[:8] for _ in range(4)]).astype(np.int32) for _ in range(4)]
    a = Rig(wl, slots=24, copy_engine="kernel", copy_streams=2, one_call=one_call, max_tokens=4)
    b = Rig(wl, slots=24, copy_engine="dma", experts=a.experts, one_call=one_call, max_tokens=4)
    _, _, rx, rw = synth.streams(wl)
    for ids in steps:
        x = to_dev_act(synth.draw_activations(rx, (4, wl.hidden), "bf16"), "bf16")
        w = torch.from_numpy(synth.draw_gate_weights(rw, (4, wl.top_k))).to(DEV)
        pa, ma, sa, oa = a.step(0, ids, x, w)
        pb, mb, sb, ob = b.step(0, ids, x, w)
        assert (pa, ma) == (pb, mb) and (sa == sb).all()
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
        if pa == binding.PATH_FALLBACK:
            for r, e in enumerate(sorted(set(ids.ravel().tolist()))):
                assert (a.pool.read_staging(r) == a.experts[0][e]).all(), (r, e)
    assert a.pool.stats()["fallbacks"] > 0 and a.pool.stats()["misses"] > 16
    _, owner, _ = a.pool.state(0)
    for s_, e in enumerate(owner):
        if e >= 0:
            assert (a.pool.read_slot(0, s_) == a.experts[0][e]).all()
    a.close()
    b.close()


def test_link_calibration_both_engines():
    """Both copy engines move a 4 MiB expert-sized copy in a positive, finite time."""
    for engine in ("kernel", "dma"):
        us = binding.link_calibration(4 << 20, engine=engine, reps=4)
        assert 0 < us < 1e6, (engine, us)
