"""GPU test: a decode step under the device slot manager is captured in a HIP graph
(torch.cuda.CUDAGraph on the pool's own stream) and replayed token after token.
Nothing in such a step waits for the host -- the decision, the miss copies, the
remap and the two GEMVs are kernels on the pool's stream, and the fixed-address
slots and tables are what makes that possible (vLLM PR "Run MoE models exceeding
VRAM via expert CPU offloading with GPU cache", section "torch.compile
compatibility": fixed addresses and in-place tables).  Every replay's slot ids and
output bits must equal those of the same steps run eagerly on a second pool, with
eager work and synchronisations between the replays, and the final cache state and
counters must equal the oracle's."""
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
    (synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=3), 16, 24),
    (synth.WORKLOADS["fanout_int4_e512"].with_(layers=2), 16, 16),
    (synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=2), 4, 8),     # every step stages
], ids=["olmoe", "int4", "olmoe-stage"])
def test_graph_replay_of_device_policy_decode_steps(wl, slots, steps):
    L, K, H = wl.layers, wl.top_k, wl.hidden
    trace = synth.make_trace(wl, steps=steps)
    _, _, rx, rw = synth.streams(wl)
    xs = [synth.draw_activations(rx, (1, H), wl.atype) for _ in range(steps)]
    ws = [synth.draw_gate_weights(rw, (1, K)) for _ in range(steps)]
    eager = Rig(wl, slots=slots, one_call=True, policy="device")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        rig = Rig(wl, slots=slots, one_call=True, policy="device", experts=eager.experts)
    dt = torch.float32 if wl.atype == "f32" else torch.bfloat16
    ids_buf = torch.zeros((L, 1, K), dtype=torch.int32, device=DEV)
    slot_buf = torch.zeros((L, 1, K), dtype=torch.int32, device=DEV)
    w_buf = torch.zeros((L, 1, K), dtype=torch.float32, device=DEV)
    x_buf = torch.zeros((1, H), dtype=dt, device=DEV)
    outs = torch.zeros((L, 1, H), dtype=dt, device=DEV)

    def load(s):
        ids_buf.copy_(torch.from_numpy(np.ascontiguousarray(trace[s])).to(DEV))
        w_buf.copy_(torch.from_numpy(ws[s]).to(DEV).expand(L, 1, K))
        x_buf.copy_(to_dev_act(xs[s], wl.atype))

    def record():
        for l in range(L):
            inp = x_buf if l == 0 else outs[l - 1]
            rig.pool.step(l, ids_buf[l], 1, slot_buf[l], inp, w_buf[l], outs[l])

    lrus = [LayerLRU(wl.experts, slots) for _ in range(L)]

    def check(s):
        # the same token, eagerly, on the other pool
        x = to_dev_act(xs[s], wl.atype)
        wd = torch.from_numpy(ws[s]).to(DEV)
        for l in range(L):
            _, _, se, oe = eager.step(l, trace[s, l], x, wd)
            r = lrus[l].step(trace[s, l])
            assert (slot_buf[l].cpu().numpy() == se).all() and (se == r.slot_ids).all(), (s, l)
            assert torch.equal(_bits(outs[l]), _bits(oe)), (s, l)
            x = oe
        if s % 6 == 0:
            ref = eager.reference(0, xs[s], trace[s, 0], ws[s])
            check_close(from_dev_act(outs[0]), ref, wl.atype, wl.wtype, f"step {s}")

    # token 0 eagerly on the capture stream, then capture token 1's step and replay it
    with torch.cuda.stream(side):
        load(0)
        record()
    side.synchronize()
    check(0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        load(1)
    side.synchronize()
    with torch.cuda.graph(g, stream=side):
        record()
    for s in range(1, steps):
        with torch.cuda.stream(side):
            load(s)
            g.replay()
        side.synchronize()
        check(s)
        torch.cuda.synchronize()
    assert rig.pool.stats() == eager.pool.stats()
    for l in range(L):
        m, owner, order = rig.pool.state(l)
        assert owner.tolist() == lrus[l].owner and m.tolist() == lrus[l].map
        st = rig.pool.stats(l)
        assert (st["steps"], st["hits"], st["misses"], st["fallbacks"]) == \
            (lrus[l].steps, lrus[l].hits, lrus[l].misses, lrus[l].fallbacks)
        for s_, e in enumerate(owner):
            if e >= 0:
                assert (rig.pool.read_slot(l, s_) == rig.experts[l][e]).all(), (l, s_, e)
    g.reset()
    rig.close()
    eager.close()
