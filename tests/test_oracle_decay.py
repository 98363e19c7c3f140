"""Pins for the decayed-count placement oracle (oracle/decay.py; "Running 125B MoE on
Two 32 GB Cards", sections 4.3-4.4): the decay constant against its half-life,
hand-derived cases (a move, the threshold, the tie rule), an independently
written formulation on every short trace, and invariants."""
import itertools
import json
import os

import numpy as np
import pytest

from expert_slot_cache_amd import synth
from oracle.decay import DECAY, DECIDE_EVERY, LayerDecay
from oracle.lru import FALLBACK, POOL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_half_life_is_512_steps():
    """64 decisions 8 steps apart halve a count (to float32 rounding)."""
    c = np.float32(1024.0)
    for _ in range(512 // DECIDE_EVERY):
        c = np.float32(c * DECAY)
    assert abs(float(c) - 512.0) < 512.0 * 2e-5
    assert DECAY == np.float32(0.5 ** (1 / 64))


def test_hand_cases_golden():
    g = json.load(open(os.path.join(GOLDEN, "decay_hand_cases.json")))
    for c in g["cases"]:
        lay = LayerDecay(c["n_experts"], c["n_slots"])
        for ids, exp_m, exp_s in zip(c["steps"], c["copied"], c["slot_ids"]):
            r = lay.step(np.array(ids))
            assert [list(m) for m in r.misses] == exp_m, (c["name"], ids)
            assert r.slot_ids.tolist() == exp_s, (c["name"], ids)
        f = c["final"]
        assert lay.map == f["map"] and lay.owner == f["owner"], c["name"]
        assert (lay.hits, lay.misses, lay.moves, lay.staged) == (f["hits"], f["misses"], f["moves"], f["staged"])


class Plain:
    """The same placement written step by step with plain lists and a counter array."""

    def __init__(self, E, N):
        self.E, self.N = E, N
        self.where = {}                # expert -> slot
        self.free = list(range(N))
        self.cnt = [np.float32(0.0)] * E
        self.t = 0

    def step(self, ids):
        ids = np.asarray(ids)
        u = sorted(set(int(v) for v in ids.ravel()))
        if len(u) > self.N:
            return None
        self.t += 1
        out = []
        if self.t % 8 == 0:
            self.cnt = [np.float32(c * DECAY) for c in self.cnt]
            outside = [e for e in range(self.E) if e not in self.where]
            inside = [e for e in range(self.E) if e in self.where]
            if outside and inside and not self.free:
                best = outside[0]
                for e in outside[1:]:
                    if self.cnt[e] > self.cnt[best]:
                        best = e
                worst = inside[0]
                for e in inside[1:]:
                    if self.cnt[e] < self.cnt[worst]:
                        worst = e
                if np.float32(self.cnt[best] - self.cnt[worst]) > 2:
                    s = self.where.pop(worst)
                    self.where[best] = s
                    out.append((best, s, worst))
        reads = [e for e in u if e not in self.where and not self.free]
        for e in u:
            if e not in self.where and self.free:
                s = self.free.pop()
                self.where[e] = s
                out.append((e, s, -1))
        reads = [e for e in u if e not in self.where]
        for v in ids.ravel():
            self.cnt[int(v)] = np.float32(self.cnt[int(v)] + np.float32(1.0))
        slot = [[self.where[int(v)] if int(v) in self.where else self.N + reads.index(int(v)) for v in row]
                for row in ids]
        return out, slot


def test_against_plain_formulation_on_short_traces():
    rng = np.random.default_rng(5)
    for _ in range(300):
        E = int(rng.integers(2, 6))
        N = int(rng.integers(1, E + 1))
        K = int(rng.integers(1, min(E, 2) + 1))
        a, b = LayerDecay(E, N), Plain(E, N)
        pop = rng.dirichlet(np.ones(E) * 0.5)
        for s in range(int(rng.integers(8, 60))):
            ids = np.stack([rng.choice(E, K, replace=False, p=pop)]).astype(np.int32)
            r = a.step(ids)
            q = b.step(ids)
            if q is None:
                assert r.path == FALLBACK
                continue
            assert r.path == POOL
            assert r.misses == q[0], (s, ids)
            assert r.slot_ids.tolist() == q[1]
        assert a.map == [b.where.get(e, -1) for e in range(E)]


@pytest.mark.parametrize("name", ["olmoe_bf16_e64", "fanout_int4_e512"])
def test_invariants_on_workload_traces(name):
    wl = synth.WORKLOADS[name]
    trace = synth.make_trace(wl, steps=200)
    lay = LayerDecay(wl.experts, wl.slots)
    for s in range(200):
        before = np.array(lay.count)
        r = lay.step(trace[s, 0])
        res = [e for e in range(wl.experts) if lay.map[e] >= 0]
        assert len(res) <= wl.slots
        for e in res:
            assert lay.owner[lay.map[e]] == e
        flat = trace[s, 0].ravel()
        for e, v in zip(flat, r.slot_ids.ravel()):
            if v < wl.slots:
                assert lay.owner[v] == e
            else:
                assert lay.map[e] < 0
        assert sum(1 for m in r.misses if m[2] >= 0) <= 1          # one move per decision at most
    assert lay.moves > 0 and lay.hits > 0


def test_fallback_changes_nothing_but_the_counter():
    lay = LayerDecay(16, 3)
    lay.step(np.array([[1, 2]]))
    snap = (list(lay.map), list(lay.owner), lay.count.copy(), lay.pooled_steps)
    r = lay.step(np.array([[1, 2], [3, 4]]))              # 4 distinct > 3 slots
    assert r.path == FALLBACK and r.slot_ids.tolist() == [[0, 1], [2, 3]]
    assert (lay.map, lay.owner, lay.pooled_steps) == snap[:2] + (snap[3],)
    assert (lay.count == snap[2]).all() and lay.fallbacks == 1
