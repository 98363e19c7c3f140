"""GPU tests of the eviction policies of the device slot manager: LRU (the policy
the vLLM PR "Run MoE models exceeding VRAM via expert CPU offloading with GPU
cache" ships) and the three its review thread lists besides it (FIFO, LFU, SLRU
with a 20 % / 80 % split).  Every step's path, miss list and slot ids, and the
final map, owners, eviction order and counters, are bit-exact against the oracle
(oracle/lru.py) on traces with heavy churn; the fused one-token step gives the
same bits as prepare + forward, and sampled outputs match the float64 layer."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, check_close, from_dev_act, to_dev_act
from expert_slot_cache_amd import binding, synth
from oracle.lru import POLICIES, LayerLRU

pytestmark = pytest.mark.gpu


def _check_state(rig, lrus):
    for l, ref in enumerate(lrus):
        m, o, order = rig.pool.state(l)
        assert m.tolist() == ref.map, l
        assert o.tolist() == ref.owner, l
        lo = ref.eviction_order()
        assert order.tolist() == lo + [-1] * (len(o) - len(lo)), l
        st = rig.pool.stats(l)
        assert (st["steps"], st["hits"], st["misses"], st["fallbacks"]) == \
            (ref.steps, ref.hits, ref.misses, ref.fallbacks), l


CASES = [
    # name, experts, slots, top_k, tokens, steps, zipf s, repeat p, rule
    ("e24-n6", 24, 6, 4, 1, 120, 0.7, 0.3, "distinct"),
    ("e64-n16", 64, 16, 8, 1, 96, 1.0, 0.5, "distinct"),
    ("e512-n64", 512, 64, 10, 1, 64, 1.2, 0.2, "distinct"),
    ("e512-n16-t4", 512, 16, 4, 4, 48, 1.6, 0.0, "distinct"),   # fallbacks and churn
    ("e100-n90", 100, 90, 8, 8, 24, 0.8, 0.0, "distinct"),      # N > 64: several slots per lane
    ("e48-n12-static", 48, 12, 4, 2, 60, 0.9, 0.2, "static"),
    ("e2048-n300", 2048, 300, 8, 1, 48, 1.1, 0.0, "distinct"),
]


@pytest.mark.parametrize("evict", POLICIES)
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_policy_prepare_matches_oracle(case, evict):
    name, E, N, K, T, steps, zs, rp, rule = case
    wl = synth.Workload(f"pol-{name}", 2, E, K, 64, 32, N, T, steps, "f32", "f32", zs, rp, 0, 60 + E)
    trace = synth.make_trace(wl, steps=steps)
    eb = synth.expert_bytes("f32", 64, 32)
    zero = np.zeros(eb, np.uint8)          # the decision never reads expert bytes
    rig = Rig(wl, slots=N, rule=rule, policy="device", evict=evict, experts=[[zero] * E] * 2,
              max_tokens=T)
    lrus = [LayerLRU(E, N, rule, evict) for _ in range(2)]
    for s in range(steps):
        for l in range(2):
            ids = trace[s, l]
            ids_d = torch.from_numpy(ids).to(DEV)
            slot_d = torch.empty_like(ids_d)
            rig.pool.prepare(l, ids_d, T, slot_d)
            r = lrus[l].step(ids)
            assert rig.pool.last_step(l) == (r.path, r.misses), (s, l)
            assert (slot_d.cpu().numpy() == r.slot_ids).all(), (s, l)
        if s % 16 == 15:
            _check_state(rig, lrus)
    _check_state(rig, lrus)
    assert sum(x.misses for x in lrus) > 0
    rig.close()


@pytest.mark.parametrize("evict", POLICIES)
@pytest.mark.parametrize("wl,slots,steps", [
    (synth.Workload("polstep", 2, 32, 8, 256, 128, 12, 1, 0, "bf16", "bf16", 0.8, 0.3, 0, 70), 12, 40),
    (synth.Workload("polstep4", 1, 64, 10, 256, 128, 16, 1, 0, "int4", "bf16", 0.9, 0.2, 0, 71), 16, 30),
    (synth.Workload("polstage", 1, 16, 4, 64, 32, 3, 1, 0, "f32", "f32", 0.5, 0.0, 0, 72), 3, 20),
], ids=["bf16", "int4", "f32-stage"])
def test_policy_fused_step_equals_prepare_forward(wl, slots, steps, evict):
    """The fused one-token step and prepare + forward give the same slot ids, misses,
    counters, output bits, slot bytes and eviction order, and the oracle's."""
    trace = synth.make_trace(wl, steps=steps)
    _, _, rx, rw = synth.streams(wl)
    a = Rig(wl, slots=slots, policy="device", evict=evict)
    b = Rig(wl, slots=slots, policy="device", evict=evict, one_call=True, read_through=True, experts=a.experts)
    lrus = [LayerLRU(wl.experts, slots, "distinct", evict) for _ in range(wl.layers)]
    for s in range(steps):
        x = synth.draw_activations(rx, (1, wl.hidden), wl.atype)
        w = synth.draw_gate_weights(rw, (1, wl.top_k))
        xd, wd = to_dev_act(x, wl.atype), torch.from_numpy(w).to(DEV)
        for l in range(wl.layers):
            _, _, sa, oa = a.step(l, trace[s, l], xd, wd)
            _, _, sb, ob = b.step(l, trace[s, l], xd, wd)
            r = lrus[l].step(trace[s, l])
            assert b.pool.last_step(l) == (r.path, r.misses), (s, l)
            assert (sa == r.slot_ids).all() and (sb == r.slot_ids).all(), (s, l)
            ab = oa.view(torch.int16) if oa.dtype == torch.bfloat16 else oa.view(torch.int32)
            bb = ob.view(torch.int16) if ob.dtype == torch.bfloat16 else ob.view(torch.int32)
            assert torch.equal(ab, bb), (s, l)
            if s % 7 == 0:
                check_close(from_dev_act(ob), b.reference(l, x, trace[s, l], w), wl.atype, wl.wtype, f"{s} {l}")
    assert a.pool.stats() == b.pool.stats()
    _check_state(b, lrus)
    for l in range(wl.layers):
        _, owner, _ = b.pool.state(l)
        for s_, e in enumerate(owner):
            if e >= 0:
                assert (b.pool.read_slot(l, s_) == b.experts[l][e]).all(), (l, s_, e)
    a.close()
    b.close()


def test_host_policy_rejects_other_evictions():
    wl = synth.Workload("polhost", 1, 8, 2, 64, 32, 4, 1, 0, "f32", "f32", 1.0, 0.0, 0, 73)
    with pytest.raises(binding.MoeError):
        Rig(wl, slots=4, policy="host", evict="lfu")


def test_set_eviction_switches_policy_from_cold():
    """moe_pool_set_eviction returns the pool to cold under the new policy: the steps
    after it match a fresh oracle of that policy, and the slot bytes their owners'."""
    from oracle.decay import LayerDecay
    wl = synth.Workload("polswitch", 1, 24, 4, 64, 32, 6, 1, 0, "f32", "f32", 0.7, 0.3, 12, 74)
    trace = synth.make_trace(wl, steps=120)
    rig = Rig(wl, slots=6, policy="device")
    for evict, s0 in (("lfu", 0), ("decay", 40), ("slru", 80), ("lru", 0)):
        rig.pool.set_eviction(evict)
        ref = LayerDecay(24, 6) if evict == "decay" else LayerLRU(24, 6, "distinct", evict)
        for s in range(s0, s0 + 40):
            ids_d = torch.from_numpy(trace[s, 0]).to(DEV)
            slot_d = torch.empty_like(ids_d)
            rig.pool.prepare(0, ids_d, 1, slot_d)
            r = ref.step(trace[s, 0])
            assert rig.pool.last_step(0) == (r.path, r.misses), (evict, s)
            assert (slot_d.cpu().numpy() == r.slot_ids).all(), (evict, s)
        m, o, _ = rig.pool.state(0)
        assert m.tolist() == ref.map and o.tolist() == ref.owner, evict
        for s_, e in enumerate(o):
            if e >= 0:
                assert (rig.pool.read_slot(0, s_) == rig.experts[0][e]).all(), (evict, s_, e)
    rig.close()
    rt = Rig(wl, slots=6, policy="device", read_through=True)
    with pytest.raises(binding.MoeError):
        rt.pool.set_eviction("decay")
    rt.close()


@pytest.mark.parametrize("evict", POLICIES)
@pytest.mark.parametrize("T,K,N,rule", [(8, 4, 12, "distinct"), (4, 4, 16, "static"), (16, 4, 14, "distinct")])
def test_prepare_all_hit_steps_with_repeated_ids(T, K, N, rule, evict):
    """Decode batches of several tokens (up to 64 ids, experts repeated across tokens) on a
    small, hot expert set: most steps hit every id, and such a step's keys are updated in
    place by the launch's lead.  Every step's path, misses and slot ids, and the state and
    counters, match the oracle; steps with repeated ids that all hit do occur."""
    E = 16
    wl = synth.Workload(f"allhit-{T}", 1, E, K, 64, 32, N, T, 0, "f32", "f32", 1.4, 0.6, 0, 97 + T)
    steps = 48
    trace = synth.make_trace(wl, steps=steps)
    zero = np.zeros(synth.expert_bytes("f32", 64, 32), np.uint8)
    rig = Rig(wl, slots=N, rule=rule, policy="device", evict=evict, experts=[[zero] * E], max_tokens=T)
    ref = LayerLRU(E, N, rule, evict)
    repeated_all_hit = 0
    for s in range(steps):
        ids = trace[s, 0]
        ids_d = torch.from_numpy(ids).to(DEV)
        slot_d = torch.empty_like(ids_d)
        rig.pool.prepare(0, ids_d, T, slot_d)
        r = ref.step(ids)
        assert rig.pool.last_step(0) == (r.path, r.misses), s
        assert (slot_d.cpu().numpy() == r.slot_ids).all(), s
        if r.path == 0 and not r.misses and len(np.unique(ids)) < ids.size:
            repeated_all_hit += 1
    _check_state(rig, [ref])
    assert repeated_all_hit > 0
    rig.close()
