"""GPU parity at the full shapes of the prefill and batched workloads, as written.

* Prefill fallback on the OLMoE shapes (64 experts, hidden 2048, intermediate 1024,
  top-8) with 2048-token ubatches: at 16 slots the distinct rule fires (every ubatch
  touches all 64 experts), at 64 slots the static rule does (8 x 2048 > 64).  The
  llama.cpp discussion "Persistent expert slot pool" ("Why not the other approaches
  on the table": prefill takes the selective-copy path and never touches the pool).
  The pool state is bit-identical before and after, the output equals the
  all-resident layer's bit for bit, sampled rows spread over the tiles match the
  oracle, and the same tokens run as decode steps match the prefill rows.
* Batched decode (128 experts, hidden 4096, intermediate 1536, top-8, 64 sequences)
  with 32 slots: every step touches more than 32 experts and falls back; same checks.
* The grouped path fed by the DMA copy engine while staging and slots are refilled
  between steps (host slot manager), bit for bit against the all-resident layer.
"""
import numpy as np
import pytest
import torch

from _gpu_helpers import DEV, Rig, check_close, from_dev_act, to_dev_act
from expert_slot_cache_amd import binding, synth
from oracle import moe as omoe

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


class Big:
    """A pooled and an all-resident pool over the same windowed experts (large
    stores fill in seconds; see synth.WindowedExperts)."""

    def __init__(self, wl, slots, rule, max_tokens, policy="device"):
        self.wl = wl
        self.gen = synth.WindowedExperts(wl)
        kw = dict(layers=wl.layers, experts=wl.experts, top_k=wl.top_k, hidden=wl.hidden, inter=wl.inter,
                  wtype=wl.wtype, atype=wl.atype, max_tokens=max_tokens, policy=policy)
        self.pool = binding.MoePool(slots=slots, rule=rule, **kw)
        self.res = binding.MoePool(slots=wl.experts, resident=True, **kw)
        buf = np.empty(self.pool.expert_nbytes, np.uint8)
        for l in range(wl.layers):
            for e in range(wl.experts):
                self.gen.expert(l, e, self.pool.store_view(l, e))
                self.res.load_expert(l, e, self.gen.expert(l, e, buf))

    def ref_rows(self, layer, x, ids, w, rows):
        """The oracle on the given rows, one row at a time (a row's 8 experts are
        widened to float64 for that row only)."""
        out = np.zeros((len(rows), self.wl.hidden))
        for i, r in enumerate(rows):
            out[i] = omoe.moe_layer(x[r:r + 1], ids[r:r + 1], w[r:r + 1], lambda e: self.gen.expert(layer, e),
                                    self.wl.wtype, self.wl.hidden, self.wl.inter, atype=self.wl.atype)[0]
        return out

    def close(self):
        self.pool.close()
        self.res.close()


def _step(pool, layer, ids, x_d, w_d, T, H):
    ids_d = torch.from_numpy(np.ascontiguousarray(ids)).to(DEV)
    slot_d = torch.empty_like(ids_d)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    pool.step(layer, ids_d, T, slot_d, x_d, w_d, out)
    return out


@pytest.mark.timeout(600)
@pytest.mark.parametrize("slots,rule", [(16, "distinct"), (64, "static")])
def test_prefill_2048_falls_back_and_leaves_the_pool_untouched(slots, rule):
    base = synth.WORKLOADS["prefill_bf16_e64"].with_(layers=1, tokens=2048)
    dec = synth.WORKLOADS["olmoe_bf16_e64"].with_(layers=1)
    T, H = 2048, base.hidden
    big = Big(base, slots, rule, max_tokens=T)
    trace_dec = synth.make_trace(dec, steps=4)
    trace_pf = synth.make_trace(base, steps=1)[0, 0]
    rng = np.random.default_rng(2048 + slots)
    x = synth.draw_activations(rng, (T, H), "bf16")
    w = synth.draw_gate_weights(rng, (T, base.top_k))
    x_d, w_d = to_dev_act(x, "bf16"), torch.from_numpy(w).to(DEV)
    # decode first, so that the pool holds experts when the prefill comes
    for s in range(4):
        xs = synth.draw_activations(rng, (1, H), "bf16")
        ws = synth.draw_gate_weights(rng, (1, base.top_k))
        _step(big.pool, 0, trace_dec[s, 0], to_dev_act(xs, "bf16"), torch.from_numpy(ws).to(DEV), 1, H)
    before = [a.copy() for a in big.pool.state(0)], big.pool.stats(0)
    out = _step(big.pool, 0, trace_pf, x_d, w_d, T, H)
    assert big.pool.last_step(0) == (binding.PATH_FALLBACK, [])
    after = big.pool.state(0), big.pool.stats(0)
    assert all((a == b).all() for a, b in zip(before[0], after[0]))
    for k in ("hits", "misses"):
        assert after[1][k] == before[1][k]
    assert after[1]["fallbacks"] == before[1]["fallbacks"] + 1
    # bit for bit the all-resident layer
    out_r = _step(big.res, 0, trace_pf, x_d, w_d, T, H)
    assert torch.equal(_bits(out), _bits(out_r))
    # 16 rows over the ubatch (different tiles of different slot groups) against the oracle
    rows = list(range(0, T, T // 16))
    got = from_dev_act(out)[rows]
    check_close(got, big.ref_rows(0, x, trace_pf, w, rows), "bf16", "bf16", f"prefill 2048, N={slots}")
    # the same tokens run as decode steps (one token per step, on the resident layer)
    for r in rows[:6]:
        o1 = _step(big.res, 0, trace_pf[r:r + 1], to_dev_act(x[r:r + 1], "bf16"),
                   torch.from_numpy(w[r:r + 1]).to(DEV), 1, H)
        check_close(from_dev_act(o1)[0], got[rows.index(r)], "bf16", "bf16", f"decode row {r} vs prefill")
    big.close()


@pytest.mark.timeout(600)
def test_batched_decode_as_written_every_step_falls_back():
    wl = synth.WORKLOADS["batched_bf16_e128"].with_(layers=2)
    T, H = wl.tokens, wl.hidden
    big = Big(wl, 32, "distinct", max_tokens=T)
    trace = synth.make_trace(wl, steps=2)
    rng = np.random.default_rng(64)
    cold = [a.copy() for a in big.pool.state(0)]
    for s in range(2):
        x = synth.draw_activations(rng, (T, H), "bf16")
        w = synth.draw_gate_weights(rng, (T, wl.top_k))
        x_d, w_d = to_dev_act(x, "bf16"), torch.from_numpy(w).to(DEV)
        for l in range(2):
            D = len(np.unique(trace[s, l]))
            assert D > 32
            out = _step(big.pool, l, trace[s, l], x_d, w_d, T, H)
            assert big.pool.last_step(l) == (binding.PATH_FALLBACK, [])
            out_r = _step(big.res, l, trace[s, l], x_d, w_d, T, H)
            assert torch.equal(_bits(out), _bits(out_r)), (s, l)
            if s == 0 and l == 0:
                rows = list(range(0, T, 4))          # 16 rows
                check_close(from_dev_act(out)[rows], big.ref_rows(l, x, trace[s, l], w, rows), "bf16", "bf16",
                            f"batched step {s} layer {l}")
    for l in range(2):
        assert all((a == b).all() for a, b in zip(cold, big.pool.state(l)))
    st = big.pool.stats()
    assert (st["hits"], st["misses"], st["fallbacks"]) == (0, 0, 4)
    big.close()


@pytest.mark.parametrize("T", [9, 24, 64])
def test_grouped_path_with_dma_copies_under_churn(T):
    """Host slot manager, DMA engine (hipMemcpyAsync into slots and staging), a small
    pool: slots are refilled and staging is rewritten between steps, and each step's
    grouped GEMMs must read the fresh bytes."""
    wl = synth.Workload("dmagrp", 1, 32, 4, 256, 128, 10, T, 0, "bf16", "bf16", 0.6, 0.1, 0, 95)
    trace = synth.make_trace(wl, steps=12)
    _, _, rx, rw = synth.streams(wl)
    pooled = Rig(wl, slots=10, copy_engine="dma", copy_chunk_bytes=64 << 10, copy_streams=3, policy="host")
    res = Rig(wl, slots=10, resident=True, experts=pooled.experts)
    fb = 0
    for s in range(12):
        x = synth.draw_activations(rx, (T, wl.hidden), "bf16")
        w = synth.draw_gate_weights(rw, (T, wl.top_k))
        x_d, w_d = to_dev_act(x, "bf16"), torch.from_numpy(w).to(DEV)
        path, _, _, out = pooled.step(0, trace[s, 0], x_d, w_d)
        fb += path == binding.PATH_FALLBACK
        _, _, _, out_r = res.step(0, trace[s, 0], x_d, w_d)
        assert torch.equal(_bits(out), _bits(out_r)), s
        if s % 4 == 0:
            check_close(from_dev_act(out), pooled.reference(0, x, trace[s, 0], w), "bf16", "bf16", f"step {s}")
    st = pooled.pool.stats()
    assert st["misses"] > 10 or fb > 2
    pooled.close()
    res.close()
