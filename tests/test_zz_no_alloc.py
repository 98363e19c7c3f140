"""GPU test of moe_forward_slots, the forward that allocates nothing (its scratch is a
static device array): called through the C ABI on a pool's own slots, it gives the
same bits as moe_pool_forward on the same slot ids, on two calls in a row (the
second with fewer tokens), on the decode and the grouped paths; a call that needs
more scratch than the array holds is refused."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, to_dev_act
from expert_slot_cache_amd import binding, synth

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("wl,tokens", [
    (synth.Workload("na-bf16", 1, 16, 4, 256, 128, 16, 8, 0, "bf16", "bf16", 1.0, 0.0, 0, 90), [8, 3]),
    (synth.Workload("na-int4", 1, 12, 4, 256, 128, 12, 4, 0, "int4", "bf16", 1.0, 0.0, 0, 91), [4, 1]),
    (synth.Workload("na-f32", 1, 8, 2, 64, 32, 8, 2, 0, "f32", "f32", 1.0, 0.0, 0, 92), [2, 1]),
    (synth.Workload("na-grp", 1, 16, 4, 256, 128, 16, 40, 0, "bf16", "bf16", 1.0, 0.0, 0, 93), [40, 12]),
], ids=["bf16", "int4", "f32", "grouped"])
def test_no_alloc_forward_equals_pool_forward(wl, tokens):
    rig = Rig(wl, slots=wl.experts, resident=True, policy="device", max_tokens=max(tokens))
    import ctypes as C
    base = C.c_void_p()
    binding._check(binding.lib().moe_pool_slot_ptr(rig.pool._h, 0, 0, C.byref(base)))
    rng = np.random.default_rng(5)
    dt = torch.float32 if wl.atype == "f32" else torch.bfloat16
    for T in tokens:
        ids = np.stack([rng.permutation(wl.experts)[:wl.top_k] for _ in range(T)]).astype(np.int32)
        x = to_dev_act(synth.draw_activations(rng, (T, wl.hidden), wl.atype), wl.atype)
        w = torch.from_numpy(synth.draw_gate_weights(rng, (T, wl.top_k))).to(DEV)
        ids_d = torch.from_numpy(ids).to(DEV)
        slot_d = torch.empty_like(ids_d)
        ref = torch.empty((T, wl.hidden), dtype=dt, device=DEV)
        rig.pool.prepare(0, ids_d, T, slot_d)            # resident: slot = id
        rig.pool.forward(0, x, slot_d, w, ref, T, resid=x)
        got = torch.full((T, wl.hidden), 7.0, dtype=dt, device=DEV)
        binding.forward_slots(wtype=wl.wtype, atype=wl.atype, hidden=wl.hidden, inter=wl.inter, top_k=wl.top_k,
                              slots=base.value, n_slots=wl.experts, slot_ids=slot_d, x=x, topk_w=w, out=got,
                              n_tokens=T, resid=x)
        torch.cuda.synchronize()
        assert (slot_d.cpu().numpy() == ids).all()
        assert torch.equal(_bits(got), _bits(ref)), (wl.name, T)
    rig.close()


def test_no_alloc_forward_refuses_more_than_its_scratch():
    wl = synth.Workload("na-big", 1, 8, 8, 2048, 1024, 8, 1, 0, "bf16", "bf16", 1.0, 0.0, 0, 94)
    x = torch.zeros((4096, 2048), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((4096, 8), dtype=torch.int32, device=DEV)
    w = torch.zeros((4096, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(binding.MoeError) as e:
        binding.forward_slots(wtype="bf16", atype="bf16", hidden=2048, inter=1024, top_k=8, slots=x,
                              n_slots=8, slot_ids=ids, x=x, topk_w=w, out=x, n_tokens=4096)
    assert e.value.status == binding.EINVAL and "scratch" in str(e.value)
