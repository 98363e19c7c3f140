"""GPU test: the event-timing period of a pool created with timing events can be
switched at run time.  Switched off, the pool's steps take no samples, which is what a
HIP-graph capture of those steps needs; a pool created without events refuses to
switch sampling on, and a negative period is refused."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, to_dev_act
from expert_slot_cache_amd import binding, synth

pytestmark = pytest.mark.gpu


def test_set_timing_switches_sampling():
    wl = synth.Workload("timing", 1, 16, 2, 256, 128, 4, 1, 0, "bf16", "bf16", 1.0, 0.0, 0, 44)
    rig = Rig(wl, slots=4, one_call=True, policy="device", timing=1)
    rng = synth.streams(wl)[2]
    x = to_dev_act(synth.draw_activations(rng, (1, wl.hidden), "bf16"), "bf16")
    w = torch.from_numpy(synth.draw_gate_weights(rng, (1, wl.top_k))).to(DEV)
    ids = np.array([[1, 2]], np.int32)

    def steps(n):
        for _ in range(n):
            rig.step(0, ids, x, w)
        rig.pool.sync()

    steps(3)
    n0 = rig.pool.timing()["kernel_calls"]
    assert n0 >= 1
    rig.pool.set_timing(0)
    steps(3)
    assert rig.pool.timing()["kernel_calls"] == n0
    rig.pool.set_timing(1)
    steps(3)
    assert rig.pool.timing()["kernel_calls"] > n0
    with pytest.raises(binding.MoeError) as e:
        rig.pool.set_timing(-1)
    assert e.value.status == binding.EINVAL
    rig.close()

    plain = Rig(wl, slots=4, policy="device")
    with pytest.raises(binding.MoeError) as e:
        plain.pool.set_timing(1)
    assert e.value.status == binding.EINVAL
    plain.pool.set_timing(0)
    plain.close()
