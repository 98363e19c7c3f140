"""GPU tests of placement by decayed use counts ("Running 125B MoE on Two 32 GB
Cards", sections 4.3 and 4.4) in the device slot manager: every step's path, move /
insertion list and slot ids (a host-read expert's slot id is n_slots + its staging
entry), and the final map, owners, count order and counters, are bit-exact against
oracle/decay.py on traces with drifting popularity; outputs of steps that read
experts from the host through staging (decode GEMVs and the grouped MFMA path) match
the float64 layer and the slots hold their experts' bytes."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, check_close, from_dev_act, to_dev_act
from expert_slot_cache_amd import binding, synth
from oracle.decay import LayerDecay

pytestmark = pytest.mark.gpu


def _check_state(rig, refs):
    for l, ref in enumerate(refs):
        m, o, order = rig.pool.state(l)
        assert m.tolist() == ref.map, l
        assert o.tolist() == ref.owner, l
        lo = ref.eviction_order()
        assert order.tolist() == lo + [-1] * (len(o) - len(lo)), l
        st = rig.pool.stats(l)
        got = (st["steps"], st["hits"], st["misses"], st["fallbacks"], st["staged"], st["moves"])
        assert got == (ref.steps, ref.hits, ref.misses, ref.fallbacks, ref.staged, ref.moves), (l, got)


CASES = [
    # name, experts, slots, top_k, tokens, steps, zipf s, repeat p, rule, reshuffle
    ("e24-n6", 24, 6, 4, 1, 240, 0.7, 0.3, "distinct", 0),
    ("e64-n16-drift", 64, 16, 8, 1, 200, 1.0, 0.5, "distinct", 40),
    ("e512-n64-drift", 512, 64, 10, 1, 160, 1.2, 0.2, "distinct", 48),
    ("e512-n12-t4", 512, 12, 4, 4, 96, 1.6, 0.0, "distinct", 0),       # fallbacks too
    ("e100-n90-t8", 100, 90, 8, 8, 64, 0.8, 0.0, "distinct", 0),       # N > 64
    ("e48-n12-static", 48, 12, 4, 2, 160, 0.9, 0.2, "static", 24),
    ("e2048-n300", 2048, 300, 8, 1, 200, 1.1, 0.0, "distinct", 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decay_prepare_matches_oracle(case):
    name, E, N, K, T, steps, zs, rp, rule, rs = case
    wl = synth.Workload(f"dec-{name}", 2, E, K, 64, 32, N, T, steps, "f32", "f32", zs, rp, rs, 90 + E)
    trace = synth.make_trace(wl, steps=steps)
    eb = synth.expert_bytes("f32", 64, 32)
    zero = np.zeros(eb, np.uint8)          # the decision never reads expert bytes
    rig = Rig(wl, slots=N, rule=rule, policy="device", evict="decay", experts=[[zero] * E] * 2,
              max_tokens=T)
    refs = [LayerDecay(E, N, rule) for _ in range(2)]
    for s in range(steps):
        for l in range(2):
            ids = trace[s, l]
            ids_d = torch.from_numpy(ids).to(DEV)
            slot_d = torch.empty_like(ids_d)
            rig.pool.prepare(l, ids_d, T, slot_d)
            r = refs[l].step(ids)
            assert rig.pool.last_step(l) == (r.path, r.misses), (s, l)
            assert (slot_d.cpu().numpy() == r.slot_ids).all(), (s, l)
        if s % 32 == 31:
            _check_state(rig, refs)
    _check_state(rig, refs)
    assert sum(x.staged for x in refs) > 0
    if name != "e100-n90-t8":
        assert sum(x.moves for x in refs) > 0
    rig.close()


@pytest.mark.parametrize("wl,slots,steps", [
    (synth.Workload("decf32", 2, 24, 4, 64, 32, 6, 1, 0, "f32", "f32", 0.7, 0.3, 16, 81), 6, 64),
    (synth.Workload("decbf16", 1, 32, 8, 256, 128, 12, 1, 0, "bf16", "bf16", 0.9, 0.3, 16, 82), 12, 48),
    (synth.Workload("decint4", 1, 64, 10, 256, 128, 16, 1, 0, "int4", "bf16", 0.9, 0.2, 16, 83), 16, 40),
    (synth.Workload("decgrp", 1, 32, 4, 128, 128, 16, 12, 0, "bf16", "bf16", 1.0, 0.0, 8, 84), 16, 24),
], ids=["f32", "bf16", "int4", "bf16-grouped-t12"])
def test_decay_outputs_and_slot_bytes(wl, slots, steps):
    """Steps whose experts are partly read from the host (slot ids past the pool) give
    the float64 layer's outputs; slots hold their owners' bytes; one-call steps give
    the same bits as prepare + forward."""
    trace = synth.make_trace(wl, steps=steps)
    _, _, rx, rw = synth.streams(wl)
    T = wl.tokens
    a = Rig(wl, slots=slots, policy="device", evict="decay")
    b = Rig(wl, slots=slots, policy="device", evict="decay", one_call=True, experts=a.experts)
    refs = [LayerDecay(wl.experts, slots) for _ in range(wl.layers)]
    mixed = 0
    for s in range(steps):
        x = synth.draw_activations(rx, (T, wl.hidden), wl.atype)
        w = synth.draw_gate_weights(rw, (T, wl.top_k))
        xd, wd = to_dev_act(x, wl.atype), torch.from_numpy(w).to(DEV)
        for l in range(wl.layers):
            _, _, sa, oa = a.step(l, trace[s, l], xd, wd)
            _, _, sb, ob = b.step(l, trace[s, l], xd, wd)
            r = refs[l].step(trace[s, l])
            assert (sa == r.slot_ids).all() and (sb == r.slot_ids).all(), (s, l)
            host = bool((r.slot_ids >= slots).any())
            mixed += host
            ab = oa.view(torch.int16) if oa.dtype == torch.bfloat16 else oa.view(torch.int32)
            bb = ob.view(torch.int16) if ob.dtype == torch.bfloat16 else ob.view(torch.int32)
            assert torch.equal(ab, bb), (s, l)
            if host or s % 5 == 0:
                check_close(from_dev_act(oa), a.reference(l, x, trace[s, l], w), wl.atype, wl.wtype, f"{s} {l}")
    assert mixed > 0
    assert a.pool.stats() == b.pool.stats()
    _check_state(a, refs)
    for l in range(wl.layers):
        _, owner, _ = a.pool.state(l)
        for s_, e in enumerate(owner):
            if e >= 0:
                assert (a.pool.read_slot(l, s_) == a.experts[l][e]).all(), (l, s_, e)
    a.close()
    b.close()


def test_decay_rejects_read_through_and_host_policy():
    wl = synth.Workload("dechost", 1, 8, 2, 64, 32, 4, 1, 0, "f32", "f32", 1.0, 0.0, 0, 85)
    with pytest.raises(binding.MoeError):
        Rig(wl, slots=4, policy="host", evict="decay")
    with pytest.raises(binding.MoeError):
        Rig(wl, slots=4, policy="device", evict="decay", read_through=True)
