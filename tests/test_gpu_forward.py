"""GPU parity of the slot-indexed fused MoE against the float64 oracle, and
bit-identity of the pooled layer with the all-resident layer (the pooled GPU path
must match the all-resident GPU path exactly; the vLLM PR's FullGPUProvider is the
all-resident path; the llama.cpp discussion's backend matrix compares pooled and
host-copy paths bit for bit over dtype x ubatch {1, 3} x cold / full eviction /
hit + reload / rebuild)."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, check_close, from_dev_act, to_dev_act
from expert_slot_cache_amd import binding, synth
from oracle.lru import LayerLRU

pytestmark = pytest.mark.gpu


def _inputs(wl, steps, T):
    _, _, rx, rw = synth.streams(wl)
    xs = [synth.draw_activations(rx, (T, wl.hidden), wl.atype) for _ in range(steps)]
    ws = [synth.draw_gate_weights(rw, (T, wl.top_k)) for _ in range(steps)]
    return xs, ws


def _run(rig, trace, xs, ws, layer_major=False, check_every=1, resid=None):
    """Runs the trace through the rig; returns outputs [step][layer] (host fp32) and
    checks a sample against the oracle."""
    outs = []
    S, L = trace.shape[:2]
    for s in range(S):
        row = []
        xd = to_dev_act(xs[s], rig.wl.atype)
        wd = torch.from_numpy(ws[s]).to(DEV)
        rd = None if resid is None else to_dev_act(resid[s], rig.wl.atype)
        for l in range(L):
            path, misses, slots, out = rig.step(l, trace[s, l], xd, wd, rd)
            got = from_dev_act(out)
            row.append(got)
            if s % check_every == 0:
                ref = rig.reference(l, xs[s], trace[s, l], ws[s],
                                    resid=None if resid is None else resid[s])
                check_close(got, ref, rig.wl.atype, rig.wl.wtype, f"step {s} layer {l}")
        outs.append(row)
    return outs


def _assert_bitwise(a, b, what):
    for s, (ra, rb) in enumerate(zip(a, b)):
        for l, (x, y) in enumerate(zip(ra, rb)):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"{what}: step {s} layer {l}"


# one_call: one moe_pool_step per layer instead of prepare + forward
ONE_CALL = pytest.mark.parametrize("one_call", [False, True], ids=["two_call", "step"])


@ONE_CALL
def test_tiny_f32_full_trace_and_resident_identity(one_call):
    wl = synth.WORKLOADS["tiny_f32_e8"]
    trace = synth.make_trace(wl)
    xs, ws = _inputs(wl, wl.steps, 1)
    pooled = Rig(wl, slots=4, fast=False, one_call=one_call)
    out_p = _run(pooled, trace, xs, ws)
    st = pooled.pool.stats()
    assert st["misses"] > 0 and st["hits"] > st["misses"]
    resident = Rig(wl, slots=4, resident=True, experts=pooled.experts)
    out_r = _run(resident, trace, xs, ws, check_every=64)
    _assert_bitwise(out_p, out_r, "pooled vs resident")
    pooled.close()
    resident.close()


@ONE_CALL
@pytest.mark.parametrize("engine", ["dma", "kernel"])
def test_olmoe_bf16_and_resident_identity(one_call, engine):
    wl = synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=2)
    steps = 12
    trace = synth.make_trace(wl, steps=steps)
    xs, ws = _inputs(wl, steps, 1)
    pooled = Rig(wl, slots=16, one_call=one_call, copy_engine=engine)
    out_p = _run(pooled, trace, xs, ws)
    resident = Rig(wl, slots=16, resident=True, experts=pooled.experts)
    out_r = _run(resident, trace, xs, ws, check_every=steps)
    _assert_bitwise(out_p, out_r, "pooled vs resident")
    pooled.close()
    resident.close()


@ONE_CALL
@pytest.mark.parametrize("engine", ["dma", "kernel"])
def test_fanout_int4_and_resident_identity(one_call, engine):
    wl = synth.WORKLOADS["fanout_int4_e512"].with_(layers=1)
    steps = 6
    trace = synth.make_trace(wl, steps=steps)
    xs, ws = _inputs(wl, steps, 1)
    pooled = Rig(wl, slots=16, one_call=one_call, copy_engine=engine)
    out_p = _run(pooled, trace, xs, ws)
    resident = Rig(wl, slots=16, resident=True, experts=pooled.experts)
    out_r = _run(resident, trace, xs, ws, check_every=steps)
    _assert_bitwise(out_p, out_r, "pooled vs resident")
    pooled.close()
    resident.close()


@pytest.mark.parametrize("wtype,atype", [("f32", "f32"), ("bf16", "bf16"), ("int4", "bf16"),
                                         ("bf16", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("T", [1, 3])
@ONE_CALL
def test_backend_matrix(wtype, atype, T, one_call):
    """dtype x ubatch x {cold, full eviction, hit + reload, reset}: pooled equals
    all-resident bit for bit, and both are within tolerance of the oracle."""
    wl = synth.Workload("matrix", 1, 24, 3, 256, 128, 6, T, 0, wtype, atype, 1.0, 0.0, 0, 7)
    rng = np.random.default_rng(17)
    cold = [np.stack([rng.permutation(6)[:3] for _ in range(T)])]              # experts 0..5
    evict = [np.stack([rng.permutation(6)[:3] + 6 for _ in range(T)]),         # 6..11: evicts
             np.stack([rng.permutation(6)[:3] + 12 for _ in range(T)])]
    hit_reload = [cold[0], np.stack([rng.permutation(24)[:3] for _ in range(T)]), cold[0]]
    seq = cold + evict + hit_reload
    trace = np.stack(seq)[:, None].astype(np.int32)                           # [S, 1, T, K]
    xs, ws = _inputs(wl, len(seq), T)
    pooled = Rig(wl, slots=6, fast=False, std=0.05, one_call=one_call)
    resident = Rig(wl, slots=6, resident=True, experts=pooled.experts, one_call=one_call)
    out_p = _run(pooled, trace, xs, ws)
    out_r = _run(resident, trace, xs, ws)
    _assert_bitwise(out_p, out_r, "pooled vs resident")
    pooled.pool.reset()
    out_p2 = _run(pooled, trace, xs, ws, check_every=100)
    _assert_bitwise(out_p, out_p2, "after reset")
    pooled.close()
    resident.close()


@pytest.mark.parametrize("wtype,atype,H,I", [("bf16", "bf16", 256, 128), ("bf16", "bf16", 2048, 256),
                                             ("f32", "f32", 256, 128), ("bf16", "f32", 512, 128),
                                             ("int4", "bf16", 256, 128)])
@pytest.mark.parametrize("T", [2, 5, 8])
def test_decode_tokens_sharing_experts(wtype, atype, H, I, T):
    """Decode ubatches whose tokens share experts (the w13 GEMV reads a shared expert's
    rows once for all of its pairs): every token's row has the bits of the same token
    run alone, pooled equals all-resident bit for bit, and the step is within tolerance
    of the oracle."""
    E, K = 12, 4
    wl = synth.Workload("shared", 1, E, K, H, I, E, T, 0, wtype, atype, 1.0, 0.0, 0, 23)
    rng = np.random.default_rng(29 + T)
    rows = [rng.permutation(5)[:K] for _ in range(T - 1)] + [np.array([8, 9, 10, 11])]
    ids = np.stack(rows).astype(np.int32)                      # most pairs on experts 0..4
    xs, ws = _inputs(wl, 1, T)
    res = Rig(wl, slots=E, resident=True, std=0.05, max_tokens=T)
    pooled = Rig(wl, slots=E, experts=res.experts, max_tokens=T)
    xd, wd = to_dev_act(xs[0], atype), torch.from_numpy(ws[0]).to(DEV)
    got_r = from_dev_act(res.step(0, ids, xd, wd)[3])
    got_p = from_dev_act(pooled.step(0, ids, xd, wd)[3])
    assert np.array_equal(got_p.view(np.uint32), got_r.view(np.uint32)), "pooled vs resident"
    check_close(got_r, res.reference(0, xs[0], ids, ws[0]), atype, wtype, f"T={T}")
    for t in range(T):
        one = from_dev_act(res.step(0, ids[t:t + 1], to_dev_act(xs[0][t:t + 1], atype),
                                    torch.from_numpy(np.ascontiguousarray(ws[0][t:t + 1])).to(DEV))[3])
        assert np.array_equal(one[0].view(np.uint32), got_r[t].view(np.uint32)), f"token {t} alone"
    res.close()
    pooled.close()


@ONE_CALL
def test_fallback_bitwise_equal_to_no_pool(one_call):
    """Bypass control: with a pool allocated, steps that overflow it take the
    selective-copy path and produce exactly what a pool of size 0 produces."""
    wl = synth.Workload("bypass", 1, 32, 4, 256, 128, 6, 2, 0, "bf16", "bf16", 1.0, 0.0, 0, 8)
    trace = synth.make_trace(wl, steps=30)
    xs, ws = _inputs(wl, 30, 2)
    pooled = Rig(wl, slots=6, one_call=one_call)
    nopool = Rig(wl, slots=0, experts=pooled.experts, one_call=one_call)
    ref_lru = LayerLRU(32, 6)
    out_p = _run(pooled, trace, xs, ws)
    out_n = _run(nopool, trace, xs, ws, check_every=100)
    fb = 0
    for s in range(30):
        r = ref_lru.step(trace[s, 0])
        if r.path == 1:
            fb += 1
            assert np.array_equal(out_p[s][0].view(np.uint32), out_n[s][0].view(np.uint32)), s
    assert fb > 0 and pooled.pool.stats()["fallbacks"] == fb
    assert nopool.pool.stats()["fallbacks"] == 30
    pooled.close()
    nopool.close()


@ONE_CALL
def test_evict_and_use_in_same_step_reads_fresh_table(one_call):
    """The llama.cpp stale-table failure: a miss evicts a slot and the same step
    reads it; the output must use the new expert's weights."""
    wl = synth.Workload("stale", 1, 8, 2, 256, 128, 2, 1, 0, "bf16", "bf16", 1.0, 0.0, 0, 9)
    trace = np.array([[[[0, 1]]], [[[1, 5]]], [[[5, 0]]], [[[2, 3]]]], np.int32)
    xs, ws = _inputs(wl, 4, 1)
    rig = Rig(wl, slots=2, fast=False, std=0.05, one_call=one_call)
    _run(rig, trace, xs, ws)
    assert rig.pool.stats()["misses"] == 2 + 1 + 1 + 2
    rig.close()


def test_residual_and_multi_token():
    wl = synth.Workload("resid", 2, 16, 4, 512, 256, 8, 3, 0, "bf16", "bf16", 1.0, 0.5, 0, 10)
    trace = synth.make_trace(wl, steps=10)
    xs, ws = _inputs(wl, 10, 3)
    _, _, rx, _ = synth.streams(wl.with_(seed=11))
    resid = [synth.draw_activations(rx, (3, wl.hidden), "bf16") for _ in range(10)]
    rig = Rig(wl, slots=8, one_call=True)
    _run(rig, trace, xs, ws, resid=resid)
    rig.close()


def test_prefill_ubatch_leaves_pool_untouched():
    """Prefill ubatches on the OLMoE shapes: 512 tokens touch all 64 experts, so with
    16 slots (distinct rule) and with 64 slots (static rule, 8 * 512 > 64) the step
    takes the selective-copy path; the pool state is bit-identical afterwards and
    decode resumes on it.  Outputs checked on sampled tokens."""
    base = synth.WORKLOADS["prefill_bf16_e64"].with_(layers=1)
    trace_dec = synth.make_trace(synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=1), steps=6)
    trace_pf = synth.make_trace(base, steps=1)
    rng = synth.streams(base)[2]
    x_pf = synth.draw_activations(rng, (512, base.hidden), "bf16")
    w_pf = synth.draw_gate_weights(rng, (512, base.top_k))
    xs, ws = _inputs(base.with_(tokens=1), 6, 1)
    experts = None
    for slots, rule in ((16, "distinct"), (64, "static")):
        rig = Rig(base, slots=slots, rule=rule, max_tokens=512, experts=experts)
        experts = rig.experts
        for s in range(3):
            rig.step(0, trace_dec[s, 0], to_dev_act(xs[s], "bf16"), torch.from_numpy(ws[s]).to(DEV))
        snap = [a.copy() for a in rig.pool.state(0)], rig.pool.stats(0)
        path, misses, slots_h, out = rig.step(0, trace_pf[0, 0], to_dev_act(x_pf, "bf16"),
                                              torch.from_numpy(w_pf).to(DEV))
        assert path == binding.PATH_FALLBACK and misses == []
        now = rig.pool.state(0), rig.pool.stats(0)
        assert all((a == b).all() for a, b in zip(snap[0], now[0]))
        assert now[1]["hits"] == snap[1]["hits"] and now[1]["misses"] == snap[1]["misses"]
        sample = [0, 1, 255, 511]
        ref = rig.reference(0, x_pf, trace_pf[0, 0], w_pf, tokens=sample)
        check_close(from_dev_act(out)[sample], ref[sample], "bf16", "bf16", f"prefill N={slots}")
        for s in range(3, 6):     # decode resumes on the untouched pool
            path, _, _, out = rig.step(0, trace_dec[s, 0], to_dev_act(xs[s], "bf16"),
                                       torch.from_numpy(ws[s]).to(DEV))
            assert path == binding.PATH_POOL
            ref = rig.reference(0, xs[s], trace_dec[s, 0], ws[s])
            check_close(from_dev_act(out), ref, "bf16", "bf16", "decode after prefill")
        rig.close()


def test_step_equals_prepare_then_forward():
    """moe_pool_step is prepare + forward in one call: same misses, slot ids and
    bit-identical outputs on the same trace."""
    wl = synth.Workload("stepcall", 2, 32, 4, 512, 256, 6, 2, 0, "bf16", "bf16", 1.0, 0.3, 0, 12)
    trace = synth.make_trace(wl, steps=20)
    xs, ws = _inputs(wl, 20, 2)
    a = Rig(wl, slots=6)
    b = Rig(wl, slots=6, experts=a.experts)
    for s in range(20):
        xd = to_dev_act(xs[s], "bf16")
        wd = torch.from_numpy(ws[s]).to(DEV)
        for l in range(2):
            pa, ma, sa, oa = a.step(l, trace[s, l], xd, wd, xd)
            ids_d = torch.from_numpy(trace[s, l]).to(DEV)
            sb = torch.empty_like(ids_d)
            ob = torch.empty_like(oa)
            pb, mb = b.pool.step(l, ids_d, 2, sb, xd, wd, ob, resid=xd)
            assert (pa, ma) == (pb, mb)
            assert (sb.cpu().numpy() == sa).all()
            assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), (s, l)
    assert a.pool.stats() == b.pool.stats()
    a.close()
    b.close()


@pytest.mark.parametrize("T", [9, 33, 64, 128, 256, 1024, 2048])
@pytest.mark.parametrize("atype", ["bf16", "f32"])
@pytest.mark.parametrize("inter", [128, 256])
def test_grouped_path_oracle_and_bitwise_across_paths(T, atype, inter):
    """n_tokens above the decode limit run the slot-grouped MFMA GEMMs.  With skewed
    routing some slot groups span several tiles (T = 128 and 256 give ~21 and ~43
    pairs per expert: tiles of 64 and 128 rows, i.e. 2 and 4 row blocks per wave,
    with ragged last blocks).  All experts resident, a pool large enough for every
    step, and a pool small enough that every step falls back to staging must give the
    same bits; all within tolerance of the oracle.  With intermediate 256 (hidden and
    intermediate multiples of 256) the 128-row tiles run the GEMMs that stage both
    operands through LDS (T = 1024 and 2048: ~170 and ~340 pairs per expert, groups
    over several tiles)."""
    wl = synth.Workload("grouped", 1, 24, 4, 256, inter, 24, T, 0, "bf16", atype, 1.3, 0.0, 0, 13)
    trace = synth.make_trace(wl, steps=4)
    xs, ws = _inputs(wl, 4, T)
    big = Rig(wl, slots=24, std=0.05)
    small = Rig(wl, slots=6, experts=big.experts)
    res = Rig(wl, slots=24, resident=True, experts=big.experts)
    counts = np.bincount(trace[0, 0].ravel(), minlength=24)
    out_b = _run(big, trace, xs, ws)
    out_s = _run(small, trace, xs, ws, check_every=100)
    out_r = _run(res, trace, xs, ws, check_every=100)
    _assert_bitwise(out_b, out_r, "pooled vs resident")
    _assert_bitwise(out_s, out_r, "fallback vs resident")
    assert small.pool.stats()["fallbacks"] == 4
    if T == 64:
        assert counts.max() > 32          # a group spans two tiles
    if T == 256:
        assert counts.max() > 128 and counts.max() % 32  # several 128-row tiles, ragged last block
    for r in (big, small, res):
        r.close()


@pytest.mark.parametrize("atype", ["bf16", "f32"])
@pytest.mark.parametrize("inter,tokens", [(128, 256), (256, 256), (256, 1024), (256, 2048)])
def test_grouped_rows_do_not_depend_on_the_batch(atype, inter, tokens):
    """A token's output depends only on its own inputs: computed in a 256-, 1024- or
    2048-token step (128-row tiles; with intermediate 256 the kernels that stage both
    operands through LDS) and again in a 12-token step (32-row tiles, the
    staged-activation kernels) it has the same bits."""
    wl = synth.Workload("grouped", 1, 24, 4, 256, inter, 24, tokens, 0, "bf16", atype, 1.3, 0.0, 0, 14)
    trace = synth.make_trace(wl, steps=1)
    xs, ws = _inputs(wl, 1, tokens)
    rig = Rig(wl, slots=24, resident=True, std=0.05)
    _, _, _, out_all = rig.step(0, trace[0, 0], to_dev_act(xs[0], atype), torch.from_numpy(ws[0]).to(DEV))
    got_all = from_dev_act(out_all)
    pick = np.array([0, 3, 17, 64, 100, 129, 130, 200, 201, 240, 254, 255])
    _, _, _, out_few = rig.step(0, np.ascontiguousarray(trace[0, 0][pick]), to_dev_act(xs[0][pick], atype),
                                torch.from_numpy(np.ascontiguousarray(ws[0][pick])).to(DEV))
    got_few = from_dev_act(out_few)
    assert np.array_equal(got_all[pick].view(np.uint32), got_few.view(np.uint32))
    ref = rig.reference(0, xs[0], trace[0, 0], ws[0], tokens=list(pick[:4]))
    check_close(got_all[pick[:4]], ref[pick[:4]], atype, "bf16", "256-token step")
    rig.close()


def test_grouped_full_batched_shape_sampled():
    """The batched-decode shapes (128 experts, H 4096, I 1536, top-8, 64 sequences),
    all resident: sampled tokens against the oracle."""
    wl = synth.WORKLOADS["batched_bf16_e128"].with_(layers=1)
    trace = synth.make_trace(wl, steps=1)
    gen = synth.WindowedExperts(wl)
    experts = [[gen.expert(0, e) for e in range(wl.experts)]]
    rig = Rig(wl, slots=wl.experts, resident=True, experts=experts)
    xs, ws = _inputs(wl, 1, wl.tokens)
    _, _, _, out = rig.step(0, trace[0, 0], to_dev_act(xs[0], "bf16"), torch.from_numpy(ws[0]).to(DEV))
    got = from_dev_act(out)
    sample = [0, 31, 63]
    ref = rig.reference(0, xs[0], trace[0, 0], ws[0], tokens=sample)
    check_close(got[sample], ref[sample], "bf16", "bf16", "batched shape")
    rig.close()


@pytest.mark.parametrize("wtype,atype,T", [("f32", "f32", 1), ("bf16", "bf16", 1), ("int4", "bf16", 1),
                                           ("bf16", "f32", 3), ("int4", "bf16", 3), ("bf16", "bf16", 24)])
def test_slot_ids_outside_the_range_contribute_nothing(wtype, atype, T):
    """A slot id outside the prepared range (-1, or past the pool) contributes nothing
    and is never used as an address (the flash-2x32 page, section 3.4: an id of -1 must
    not reach a kernel).  Since the k sum is fma(w_k, y_k, acc) in k order, the output
    equals, bit for bit, the forward with those pairs' slots intact and gate weights 0,
    and the oracle on the remaining pairs.  T = 24 takes the grouped GEMM path."""
    K, N = 4, 8
    wl = synth.Workload("badslot", 1, 16, K, 256, 128, N, T, 0, wtype, atype, 1.0, 0.0, 0, 23)
    rig = Rig(wl, slots=N, fast=False, std=0.05)
    rng = np.random.default_rng(5)
    ids = np.stack([rng.permutation(N)[:K] for _ in range(T)]).astype(np.int32)   # fits the pool
    xs, ws = _inputs(wl, 1, T)
    x, w = xs[0], ws[0]
    ids_d = torch.from_numpy(ids).to(DEV)
    slot_d = torch.empty_like(ids_d)
    path, _ = rig.pool.prepare(0, ids_d, T, slot_d)
    assert path == binding.PATH_POOL
    bad = np.zeros((T, K), bool)
    bad[0, 1] = bad[T - 1, K - 1] = True
    if T > 1:
        bad[1, 0] = True
    slots = slot_d.cpu().numpy()
    slots_bad = slots.copy()
    slots_bad[bad] = np.where(np.arange(bad.sum()) % 2 == 0, -1, N + 3)
    w0 = w.copy()
    w0[bad] = 0.0
    dt = torch.float32 if atype == "f32" else torch.bfloat16
    xd = to_dev_act(x, atype)
    out_bad = torch.empty((T, wl.hidden), dtype=dt, device=DEV)
    out_w0 = torch.empty_like(out_bad)
    rig.pool.forward(0, xd, torch.from_numpy(slots_bad).to(DEV), torch.from_numpy(w).to(DEV), out_bad, T)
    rig.pool.forward(0, xd, slot_d, torch.from_numpy(w0).to(DEV), out_w0, T)
    got, want = from_dev_act(out_bad), from_dev_act(out_w0)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    check_close(got, rig.reference(0, x, ids, w0), atype, wtype, "outside slots skipped")
    rig.close()


@pytest.mark.parametrize("wtype,atype", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("T", [1, 3])
def test_gemv_ragged_row_blocks(wtype, atype, T):
    """H = 80, I = 48: the w13 GEMV's row block (128 rows for bf16 weights, 64 for fp32)
    is larger than I, and for bf16 weights the w2 kernel's last workgroup holds 16 of its
    32 rows; the rows past the end are computed from clamped reads and dropped.  Oracle
    within tolerance and pooled = all-resident bit for bit, through evictions."""
    wl = synth.Workload("ragged", 1, 12, 3, 80, 48, 6, T, 0, wtype, atype, 1.0, 0.0, 0, 19)
    rng = np.random.default_rng(29)
    seq = [np.stack([rng.permutation(12)[:3] for _ in range(T)]) for _ in range(6)]
    trace = np.stack(seq)[:, None].astype(np.int32)
    xs, ws = _inputs(wl, len(seq), T)
    pooled = Rig(wl, slots=6, fast=False, std=0.05)
    resident = Rig(wl, slots=6, resident=True, experts=pooled.experts)
    out_p = _run(pooled, trace, xs, ws)
    out_r = _run(resident, trace, xs, ws)
    _assert_bitwise(out_p, out_r, "pooled vs resident")
    assert pooled.pool.stats()["misses"] > 0
    pooled.close()
    resident.close()


@pytest.mark.parametrize("wtype,K,T", [("bf16", 20, 1), ("bf16", 64, 1), ("int4", 20, 1), ("f32", 24, 3),
                                       ("bf16", 20, 12)])
def test_large_top_k(wtype, K, T):
    """top_k above 16 gives the w2 kernel more (expert, part) tasks than waves, so it
    takes its looping form; at T = 12 (bf16) the grouped path's combine sums the k terms
    over several chunks of 8, the last one partial; 64 is the largest top_k accepted.
    Oracle within tolerance and pooled = all-resident bit for bit."""
    atype = "f32" if wtype == "f32" else "bf16"
    wl = synth.Workload("bigk", 1, 64, K, 256, 128, 64, T, 0, wtype, atype, 1.0, 0.0, 0, 31)
    rng = np.random.default_rng(37)
    seq = [np.stack([rng.permutation(64)[:K] for _ in range(T)]) for _ in range(3)]
    trace = np.stack(seq)[:, None].astype(np.int32)
    xs, ws = _inputs(wl, len(seq), T)
    pooled = Rig(wl, slots=64, fast=False, std=0.05)
    resident = Rig(wl, slots=64, resident=True, experts=pooled.experts)
    out_p = _run(pooled, trace, xs, ws)
    out_r = _run(resident, trace, xs, ws)
    _assert_bitwise(out_p, out_r, "pooled vs resident")
    pooled.close()
    resident.close()
