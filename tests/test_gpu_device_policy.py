"""GPU tests of the slot manager on the GPU (policy "device"): the same LRU as the
prepare() of the vLLM PR "Run MoE models exceeding VRAM via expert CPU offloading
with GPU cache" (section "How it works" and the review thread's OrderedDict form)
and the same route rule (llama.cpp "Persistent expert slot pool" prefill rule), run
by a kernel on device-resident state.  Every step's path, miss list and slot ids,
and the final map / owners / LRU order / counters, are bit-exact against the
oracle; the outputs equal the host policy's bit for bit."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, check_close, from_dev_act, to_dev_act
from expert_slot_cache_amd import binding, synth
from oracle.lru import LayerLRU

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("name,slots,steps,layers,rule,tokens", [
    ("tiny_f32_e8", 4, 256, 1, "distinct", 1),
    ("tiny_f32_e8", 1, 64, 1, "distinct", 1),
    ("tiny_f32_e8", 16, 64, 1, "distinct", 1),        # more slots than experts
    ("tiny_f32_e8", 80, 64, 1, "distinct", 1),        # ... and more than one wave's lanes
    ("olmoe_bf16_e64", 16, 96, 2, "distinct", 1),
    ("fanout_int4_e512", 32, 48, 2, "distinct", 1),
    ("olmoe_bf16_e64", 16, 40, 1, "distinct", 4),     # 32 pairs, often > 16 distinct: fallbacks
    ("olmoe_bf16_e64", 24, 40, 1, "static", 3),       # 24 pairs: pooled; 4 tokens would fall back
    ("olmoe_bf16_e64", 0, 8, 1, "distinct", 1),       # no pool: every step stages
    # 2048 experts, the device policy's limit (its state lives in LDS): state loads and
    # write-back past the first 512 experts, more than 256 slots, the LDS walk
    pytest.param(synth.Workload("dev2048", 1, 2048, 8, 64, 32, 300, 1, 64, "f32", "f32", 1.1, 0.0, 0, 47),
                 300, 64, 1, "distinct", 1, id="e2048-n300"),
    pytest.param(synth.Workload("dev2048t", 1, 2048, 8, 64, 32, 100, 8, 24, "f32", "f32", 1.1, 0.0, 0, 48),
                 100, 24, 1, "distinct", 8, id="e2048-n100-t8"),
])
def test_device_policy_matches_oracle(name, slots, steps, layers, rule, tokens):
    base = synth.WORKLOADS[name] if isinstance(name, str) else name
    wl = base.with_(layers=layers, tokens=tokens)
    trace = synth.make_trace(wl, steps=steps)
    eb = synth.expert_bytes(wl.wtype, wl.hidden, wl.inter)
    zero = np.zeros(eb, np.uint8)          # the policy never reads expert bytes
    rig = Rig(wl, slots=slots, rule=rule, policy="device", experts=[[zero] * wl.experts] * layers,
              max_tokens=max(tokens, 4))
    lrus = [LayerLRU(wl.experts, slots, rule) for _ in range(layers)]
    for s in range(steps):
        for l in range(layers):
            ids = trace[s, l]
            ids_d = torch.from_numpy(ids).to(DEV)
            slot_d = torch.empty_like(ids_d)
            path, misses = rig.pool.prepare(l, ids_d, ids.shape[0], slot_d)
            assert path == -1 and misses == []          # known on the GPU only
            r = lrus[l].step(ids)
            got_path, got_misses = rig.pool.last_step(l)
            assert (got_path, got_misses) == (r.path, r.misses), (s, l)
            assert (slot_d.cpu().numpy() == r.slot_ids).all(), (s, l)
    _check_state(rig, lrus)
    assert sum(x.fallbacks for x in lrus) == rig.pool.stats()["fallbacks"]
    rig.close()


@pytest.mark.parametrize("wl_name,slots,layers,steps", [
    ("olmoe_bf16_e64", 16, 2, 10),
    ("fanout_int4_e512", 16, 1, 6),
    ("tiny_f32_e8", 4, 1, 64),
])
def test_device_policy_outputs_equal_host_policy(wl_name, slots, layers, steps):
    """Same trace, same experts: the device and host policies give the same slot
    ids, misses, counters and output bits; sampled steps are checked against the
    oracle's float64 layer."""
    wl = synth.WORKLOADS[wl_name].with_(layers=layers)
    trace = synth.make_trace(wl, steps=steps)
    _, _, rx, rw = synth.streams(wl)
    xs = [synth.draw_activations(rx, (1, wl.hidden), wl.atype) for _ in range(steps)]
    ws = [synth.draw_gate_weights(rw, (1, wl.top_k)) for _ in range(steps)]
    host = Rig(wl, slots=slots, one_call=True)
    dev = Rig(wl, slots=slots, one_call=True, policy="device", experts=host.experts)
    for s in range(steps):
        xd = to_dev_act(xs[s], wl.atype)
        wd = torch.from_numpy(ws[s]).to(DEV)
        for l in range(layers):
            ph, mh, sh, oh = host.step(l, trace[s, l], xd, wd)
            _, _, sd, od = dev.step(l, trace[s, l], xd, wd)
            assert dev.pool.last_step(l) == (ph, mh), (s, l)
            assert (sd == sh).all(), (s, l)
            assert torch.equal(od.view(torch.int16) if od.dtype == torch.bfloat16 else od.view(torch.int32),
                               oh.view(torch.int16) if oh.dtype == torch.bfloat16 else oh.view(torch.int32)), (s, l)
            if s % 5 == 0:
                ref = dev.reference(l, xs[s], trace[s, l], ws[s])
                check_close(from_dev_act(od), ref, wl.atype, wl.wtype, f"step {s} layer {l}")
    assert dev.pool.stats() == host.pool.stats()
    host.close()
    dev.close()


def test_device_policy_slot_and_staging_bytes():
    """After churn and fallbacks under the device policy, every occupied slot holds
    its owner's bytes and the last fallback's staging entries hold its experts."""
    wl = synth.Workload("devbytes", 1, 32, 4, 256, 128, 6, 2, 0, "int4", "bf16", 1.0, 0.3, 0, 41)
    trace = synth.make_trace(wl, steps=40)
    rig = Rig(wl, slots=6, policy="device", max_tokens=2)
    ref = LayerLRU(32, 6)
    last_fb = None
    for s in range(40):
        ids_d = torch.from_numpy(trace[s, 0]).to(DEV)
        slot_d = torch.empty_like(ids_d)
        rig.pool.prepare(0, ids_d, 2, slot_d)
        r = ref.step(trace[s, 0])
        if r.path == binding.PATH_FALLBACK:
            last_fb = sorted(set(trace[s, 0].ravel().tolist()))
    assert ref.misses > 20 and ref.fallbacks > 0
    _, owner, _ = rig.pool.state(0)
    assert owner.tolist() == ref.owner
    for s_, e in enumerate(owner):
        if e >= 0:
            assert (rig.pool.read_slot(0, s_) == rig.experts[0][e]).all(), (s_, e)
    for r_, e in enumerate(last_fb):            # only fallbacks write staging
        assert (rig.pool.read_staging(r_) == rig.experts[0][e]).all(), (r_, e)
    st = rig.pool.stats()
    assert st["bytes_h2d"] == (st["misses"] + st["staged"]) * rig.pool.expert_nbytes
    rig.close()


def test_device_policy_out_of_range_id_changes_nothing():
    wl = synth.Workload("devrange", 1, 16, 2, 256, 128, 4, 1, 0, "bf16", "bf16", 1.0, 0.0, 0, 42)
    rig = Rig(wl, slots=4, policy="device")
    ref = LayerLRU(16, 4)

    def prep(ids):
        ids = np.array([ids], np.int32)
        ids_d = torch.from_numpy(ids).to(DEV)
        slot_d = torch.empty_like(ids_d)
        rig.pool.prepare(0, ids_d, 1, slot_d)
        return slot_d

    prep([3, 5])
    ref.step(np.array([[3, 5]]))
    before = [a.copy() for a in rig.pool.state(0)], rig.pool.stats(0)
    slot_d = prep([3, 16])                      # 16 is outside [0, 16)
    assert (slot_d.cpu().numpy() == -1).all()
    with pytest.raises(binding.ExpertRangeError):
        rig.pool.last_step(0)
    after = rig.pool.state(0), rig.pool.stats(0)
    assert all((a == b).all() for a, b in zip(before[0], after[0])) and before[1] == after[1]
    prep([-1, 2])
    with pytest.raises(binding.ExpertRangeError):   # sync reports it once the GPU has run the step
        rig.pool.sync()
    prep([2, 3])                                # resumes
    r = ref.step(np.array([[2, 3]]))
    assert rig.pool.last_step(0) == (binding.PATH_POOL, r.misses)
    assert rig.pool.state(0)[1].tolist() == ref.owner
    rig.close()


def test_device_policy_prepare_order_and_empty_steps():
    """A forward must follow its own prepare with no other layer's prepare in
    between (staging is shared and the host does not know which steps fell back);
    a step with no tokens counts as a step with nothing to do."""
    wl = synth.Workload("devorder", 2, 16, 2, 256, 128, 4, 1, 0, "bf16", "bf16", 1.0, 0.0, 0, 43)
    rig = Rig(wl, slots=4, policy="device")
    ids_d = torch.tensor([[1, 2]], dtype=torch.int32, device=DEV)
    slot_d = torch.empty_like(ids_d)
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device=DEV)
    w = torch.ones((1, 2), dtype=torch.float32, device=DEV)
    out = torch.empty_like(x)
    rig.pool.prepare(0, ids_d, 1, slot_d)
    rig.pool.prepare(1, ids_d, 1, slot_d)
    with pytest.raises(binding.StateError):
        rig.pool.forward(0, x, slot_d, w, out, 1)
    rig.pool.forward(1, x, slot_d, w, out, 1)
    rig.pool.prepare(0, ids_d, 1, slot_d)
    rig.pool.forward(0, x, slot_d, w, out, 1)
    empty = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    rig.pool.prepare(1, empty, 0, empty)
    assert rig.pool.last_step(1) == (binding.PATH_POOL, [])
    st = rig.pool.stats(1)
    assert (st["steps"], st["hits"], st["misses"]) == (2, 0, 2)
    st = rig.pool.stats(0)
    assert (st["steps"], st["hits"], st["misses"]) == (2, 2, 2)
    rig.close()
