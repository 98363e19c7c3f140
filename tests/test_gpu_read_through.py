"""GPU tests of the read-through decode step (device policy, one token per step):
the forward's kernels read each missed or staged expert from the pinned store and
write a missed one through to its slot, instead of a copy before the forward.  The
cache is the one of vLLM PR "Run MoE models exceeding VRAM via expert CPU offloading
with GPU cache" (section "How it works": a miss lands in its slot and later steps hit
it there); reading a miss straight from pinned host memory is the zero-copy path of
"Running 125B MoE on Two 32 GB Cards" (section 4.3).  A read-through step must give
what the copying step gives: the same slot ids, misses, counters and output bits,
and afterwards every occupied slot holds its owner's bytes."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, check_close, from_dev_act, to_dev_act
from expert_slot_cache_amd import binding, synth
from oracle.lru import LayerLRU

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("wl,slots,steps", [
    (synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=2), 16, 12),
    (synth.WORKLOADS["fanout_int4_e512"].with_(layers=2), 16, 8),
    (synth.WORKLOADS["tiny_f32_e8"], 4, 64),
    (synth.WORKLOADS["tiny_f32_e8"], 1, 32),                     # N < K: every step stages
    (synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=1), 4, 6),  # N < K: every step stages
    (synth.WORKLOADS["fanout_int4_e512"].with_(layers=1), 0, 4),  # no pool
    # churn: 48 experts, top-8, 12 slots, weak locality (many evictions, INT4 scales)
    (synth.Workload("rtchurn", 1, 48, 8, 512, 256, 12, 1, 0, "int4", "bf16", 0.6, 0.2, 0, 51), 12, 40),
], ids=["olmoe", "int4", "f32", "f32-stage", "olmoe-stage", "int4-n0", "int4-churn"])
def test_read_through_equals_copying_step(wl, slots, steps):
    trace = synth.make_trace(wl, steps=steps)
    _, _, rx, rw = synth.streams(wl)
    xs = [synth.draw_activations(rx, (1, wl.hidden), wl.atype) for _ in range(steps)]
    ws = [synth.draw_gate_weights(rw, (1, wl.top_k)) for _ in range(steps)]
    copy = Rig(wl, slots=slots, one_call=True, policy="device")
    rt = Rig(wl, slots=slots, one_call=True, policy="device", read_through=True, experts=copy.experts)
    lrus = [LayerLRU(wl.experts, slots) for _ in range(wl.layers)]
    for s in range(steps):
        xd = to_dev_act(xs[s], wl.atype)
        wd = torch.from_numpy(ws[s]).to(DEV)
        for l in range(wl.layers):
            _, _, sc, oc = copy.step(l, trace[s, l], xd, wd)
            _, _, sr, orr = rt.step(l, trace[s, l], xd, wd)
            r = lrus[l].step(trace[s, l])
            assert rt.pool.last_step(l) == (r.path, r.misses), (s, l)
            assert (sr == sc).all() and (sr == r.slot_ids).all(), (s, l)
            assert torch.equal(_bits(orr), _bits(oc)), (s, l)
            if s % 4 == 0:
                ref = rt.reference(l, xs[s], trace[s, l], ws[s])
                check_close(from_dev_act(orr), ref, wl.atype, wl.wtype, f"step {s} layer {l}")
    assert rt.pool.stats() == copy.pool.stats()
    for l in range(wl.layers):
        m, owner, order = rt.pool.state(l)
        assert owner.tolist() == lrus[l].owner
        for s_, e in enumerate(owner):
            if e >= 0:
                assert (rt.pool.read_slot(l, s_) == rt.experts[l][e]).all(), (l, s_, e)
    copy.close()
    rt.close()


def test_read_through_pool_still_copies_for_prepare_and_forward():
    """prepare + forward on a read-through pool copy as before (a prepare alone must
    leave its misses in their slots); a step's table belongs to its own forward."""
    wl = synth.Workload("rtsplit", 1, 24, 4, 256, 128, 6, 1, 0, "bf16", "bf16", 0.8, 0.3, 0, 52)
    trace = synth.make_trace(wl, steps=24)
    _, _, rx, rw = synth.streams(wl)
    rig = Rig(wl, slots=6, policy="device", read_through=True)
    ref = LayerLRU(24, 6)
    for s in range(24):
        x = synth.draw_activations(rx, (1, wl.hidden), wl.atype)
        w = synth.draw_gate_weights(rw, (1, wl.top_k))
        rig.one_call = s % 2 == 0
        _, _, sd, od = rig.step(0, trace[s, 0], to_dev_act(x, wl.atype), torch.from_numpy(w).to(DEV))
        r = ref.step(trace[s, 0])
        assert (sd == r.slot_ids).all()
        check_close(from_dev_act(od), rig.reference(0, x, trace[s, 0], w), wl.atype, wl.wtype, f"step {s}")
    for s_, e in enumerate(rig.pool.state(0)[1]):
        if e >= 0:
            assert (rig.pool.read_slot(0, s_) == rig.experts[0][e]).all()
    # after a read-through step its forward has run: another forward needs a prepare
    ids_d = torch.tensor([[1, 2, 3, 4]], dtype=torch.int32, device=DEV)
    slot_d = torch.empty_like(ids_d)
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device=DEV)
    w = torch.full((1, 4), 0.25, dtype=torch.float32, device=DEV)
    out = torch.empty_like(x)
    rig.pool.step(0, ids_d, 1, slot_d, x, w, out)
    with pytest.raises(binding.StateError):
        rig.pool.forward(0, x, slot_d, w, out, 1)
    rig.close()


def test_read_through_timing_splits_link_and_hbm_launches():
    """With timing on, forwards that read experts over the link count as copy time
    (bytes = experts read through x expert bytes); hit-only forwards count as kernel
    time."""
    wl = synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=3)
    trace = synth.make_trace(wl, steps=30)
    rig = Rig(wl, slots=16, one_call=True, policy="device", read_through=True, timing=1)
    xd = torch.zeros((1, wl.hidden), dtype=torch.bfloat16, device=DEV)
    wd = torch.full((1, wl.top_k), 1.0 / wl.top_k, dtype=torch.float32, device=DEV)
    for s in range(30):
        for l in range(3):
            rig.step(l, trace[s, l], xd, wd)
    rig.pool.sync()
    tm = rig.pool.timing()
    st = rig.pool.stats()
    assert tm["copy_calls"] > 0 and tm["kernel_calls"] > 0
    assert tm["copy_bytes"] % rig.pool.expert_nbytes == 0
    assert tm["copy_bytes"] <= st["bytes_h2d"]
    gbps = tm["copy_bytes"] / (tm["copy_ms"] * 1e-3) / 1e9
    assert 5.0 < gbps < 80.0, gbps
    rig.close()


@pytest.mark.parametrize("wl", [
    synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=2),
    # top-10 (two rounds of ids), INT4 weights
    synth.Workload("rtres10", 1, 40, 10, 256, 128, 40, 1, 0, "int4", "bf16", 0.8, 0.2, 0, 53),
], ids=["olmoe", "int4-top10"])
def test_read_through_all_resident_equals_copying_step(wl):
    """In the all-resident mode every id hits at slot = id: the fused step's lookup
    (which still reads the state's map, and drops it) gives the copying step's slot
    ids, counters and output bits."""
    steps = 6
    trace = synth.make_trace(wl, steps=steps)
    _, _, rx, rw = synth.streams(wl)
    copy = Rig(wl, slots=wl.experts, one_call=True, policy="device", resident=True)
    rt = Rig(wl, slots=wl.experts, one_call=True, policy="device", resident=True, read_through=True,
             experts=copy.experts)
    for s in range(steps):
        x = synth.draw_activations(rx, (1, wl.hidden), wl.atype)
        w = synth.draw_gate_weights(rw, (1, wl.top_k))
        xd, wd = to_dev_act(x, wl.atype), torch.from_numpy(w).to(DEV)
        for l in range(wl.layers):
            _, _, sc, oc = copy.step(l, trace[s, l], xd, wd)
            _, _, sr, orr = rt.step(l, trace[s, l], xd, wd)
            assert (sr == trace[s, l]).all() and (sc == sr).all(), (s, l)
            assert torch.equal(_bits(orr), _bits(oc)), (s, l)
            if s == 0:
                check_close(from_dev_act(orr), rt.reference(l, x, trace[s, l], w), wl.atype, wl.wtype,
                            f"step {s} layer {l}")
    assert rt.pool.stats() == copy.pool.stats()
    copy.close()
    rt.close()
