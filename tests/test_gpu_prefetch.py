"""GPU tests of the cross-layer prefetch (moe_pool_prefetch): predicted experts of a
layer's next step are copied on a copy stream into the layer's prefetch buffer and
the step joins that copy through an event (vLLM PR "Run MoE models exceeding VRAM
via expert CPU offloading with GPU cache", "Planned follow-ups": async H2D with
cross-layer prediction; the article on vLLM PR #51710: prefetch started after one
layer, waited for before a later one).  A prefetch only changes where a missed or
staged expert's bytes come from: slot ids, misses, evictions, outputs and slot
bytes equal those of the same steps without prefetching, whatever the prediction."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, check_close, from_dev_act, to_dev_act
from expert_slot_cache_amd import binding, synth
from oracle.lru import LayerLRU

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _predict(trace, q, rng, E):
    """The next step's ids with probability q per (step, layer), else a fresh draw."""
    pred = trace.copy()
    S, L, T, K = trace.shape
    for s in range(S):
        for l in range(L):
            if rng.random() >= q:
                pred[s, l] = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    return pred


@pytest.mark.parametrize("mode", ["fused", "prepare", "fused-early"])
@pytest.mark.parametrize("q", [1.0, 0.5, 0.0])
@pytest.mark.parametrize("wl,slots,pf,steps", [
    (synth.Workload("pfbf16", 3, 32, 8, 256, 128, 12, 1, 0, "bf16", "bf16", 0.8, 0.3, 0, 80), 12, 8, 30),
    (synth.Workload("pfint4", 2, 48, 10, 256, 128, 16, 1, 0, "int4", "bf16", 0.7, 0.2, 0, 81), 16, 12, 24),
    (synth.Workload("pfstage", 2, 16, 4, 64, 32, 3, 1, 0, "f32", "f32", 0.5, 0.0, 0, 82), 3, 4, 20),
], ids=["bf16", "int4", "f32-stage"])
def test_prefetch_changes_nothing_but_the_source(wl, slots, pf, steps, q, mode):
    trace = synth.make_trace(wl, steps=steps)
    pred = _predict(trace, q, np.random.default_rng(7), wl.experts)
    _, _, rx, rw = synth.streams(wl)
    fused = mode.startswith("fused")
    early = mode == "fused-early"          # start each copy as soon as the layer's last step is done
    a = Rig(wl, slots=slots, policy="device", one_call=fused, read_through=fused)
    b = Rig(wl, slots=slots, policy="device", one_call=fused, read_through=fused, prefetch_slots=pf,
            experts=a.experts)
    lrus = [LayerLRU(wl.experts, slots) for _ in range(wl.layers)]
    nmiss_pred = 0
    # the predictions stay in device memory: a prefetch reads them on a copy stream
    pred_d = torch.from_numpy(pred).to(DEV)
    for s in range(steps):
        x = synth.draw_activations(rx, (1, wl.hidden), wl.atype)
        w = synth.draw_gate_weights(rw, (1, wl.top_k))
        xd, wd = to_dev_act(x, wl.atype), torch.from_numpy(w).to(DEV)
        b.pool.prefetch(0, pred_d[s, 0], 1, after="layer" if early else "queued")
        for l in range(wl.layers):
            if l + 1 < wl.layers:        # the next layer's copy overlaps this layer's step
                b.pool.prefetch(l + 1, pred_d[s, l + 1], 1, after="layer" if early else "queued")
            _, _, sa, oa = a.step(l, trace[s, l], xd, wd)
            _, _, sb, ob = b.step(l, trace[s, l], xd, wd)
            held = {e for e in range(wl.experts) if lrus[l].map[e] >= 0}
            r = lrus[l].step(trace[s, l])
            assert b.pool.last_step(l) == (r.path, r.misses), (s, l)
            assert (sb == sa).all() and (sb == r.slot_ids).all(), (s, l)
            assert torch.equal(_bits(oa), _bits(ob)), (s, l)
            if (pred[s, l] == trace[s, l]).all():
                # what the prediction made the layer fetch ahead: the step's experts it did
                # not hold when the step began (an expert evicted and reloaded within the
                # step is a miss too, and may or may not still sit in the buffer)
                moved = [m[0] for m in r.misses] if r.path == binding.PATH_POOL else r.distinct
                nmiss_pred += sum(1 for e in moved if e not in held)
            if s % 9 == 0:
                check_close(from_dev_act(ob), b.reference(l, x, trace[s, l], w), wl.atype, wl.wtype, f"{s} {l}")
    sa_, sb_ = a.pool.stats(), b.pool.stats()
    for k in ("steps", "hits", "misses", "fallbacks", "staged"):
        assert sa_[k] == sb_[k], k
    eb = b.pool.expert_nbytes
    assert sb_["bytes_h2d"] + sb_["prefetched"] * eb == sa_["bytes_h2d"]
    assert sb_["prefetch_bytes"] % eb == 0
    if q == 1.0:
        assert sb_["prefetched"] >= nmiss_pred > 0
    if q == 0.0:
        assert sb_["prefetched"] <= sb_["prefetch_bytes"] // eb
    for l in range(wl.layers):
        _, owner, _ = b.pool.state(l)
        for s_, e in enumerate(owner):
            if e >= 0:
                assert (b.pool.read_slot(l, s_) == b.experts[l][e]).all(), (l, s_, e)
    a.close()
    b.close()


def test_prefetch_after_reload_uses_the_new_bytes():
    """load_expert replaces an expert's bytes: a copy prefetched before must not be
    used afterwards."""
    wl = synth.Workload("pfreload", 1, 8, 2, 64, 32, 2, 1, 0, "f32", "f32", 1.0, 0.0, 0, 83)
    rig = Rig(wl, slots=2, policy="device", prefetch_slots=2, one_call=True, read_through=True)
    ids = torch.tensor([[5, 6]], dtype=torch.int32, device=DEV)
    rig.pool.prefetch(0, ids, 1)
    rig.pool.sync()
    assert rig.pool.stats()["prefetch_bytes"] == 2 * rig.pool.expert_nbytes
    new = synth.draw_expert(np.random.default_rng(9), "f32", 64, 32)
    rig.experts[0][5] = new
    rig.pool.load_expert(0, 5, new)
    x = np.random.default_rng(1).standard_normal((1, 64)).astype(np.float32)
    w = np.array([[0.75, 0.25]], np.float32)
    _, _, _, out = rig.step(0, np.array([[5, 6]], np.int32), to_dev_act(x, "f32"), torch.from_numpy(w).to(DEV))
    check_close(from_dev_act(out), rig.reference(0, x, np.array([[5, 6]]), w), "f32", "f32", "reloaded")
    assert (rig.pool.read_slot(0, rig.pool.state(0)[0][5]) == new).all()
    rig.close()


def test_prefetch_argument_errors():
    wl = synth.Workload("pferr", 1, 8, 2, 64, 32, 2, 1, 0, "f32", "f32", 1.0, 0.0, 0, 84)
    rig = Rig(wl, slots=2, policy="device")
    ids = torch.tensor([[1, 2]], dtype=torch.int32, device=DEV)
    with pytest.raises(binding.MoeError):          # no prefetch buffer
        rig.pool.prefetch(0, ids, 1)
    rig.close()
    rig = Rig(wl, slots=2, policy="device", prefetch_slots=2)
    with pytest.raises(binding.MoeError):
        rig.pool.prefetch(0, ids, 0)
    with pytest.raises(binding.MoeError):
        rig.pool.prefetch(1, ids, 1)                 # no such layer
    bad = torch.tensor([[-3, 99]], dtype=torch.int32, device=DEV)
    rig.pool.prefetch(0, bad, 1)                     # ignored
    rig.pool.sync()
    assert rig.pool.stats()["prefetch_bytes"] == 0
    rig.close()
    with pytest.raises(binding.MoeError):          # host policy: no prefetch
        Rig(wl, slots=2, policy="host", prefetch_slots=2)
