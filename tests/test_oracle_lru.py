"""Pins for the slot-manager oracle (CPU only).

The oracle states the step of vLLM PR "Run MoE models exceeding VRAM via expert
CPU offloading with GPU cache" ("How it works"; the review thread's LRU and its
list of eviction policies) as "each resident expert carries its policy's key; the
victim is the smallest".  It is checked here against things other than itself:
hand-derived cases (one per policy), an independently written queue formulation
on every short trace, and invariants that hold for any correct slot manager.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.lru import FALLBACK, POLICIES, POOL, ExpertIdError, LayerLRU, simulate
from expert_slot_cache_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# An independent formulation: every policy kept as explicit queues (Python lists,
# front = first to go), moved element by element -- no keys, no clock.
# ---------------------------------------------------------------------------
class ListCache:
    def __init__(self, E, N, rule="distinct", policy="lru"):
        self.E, self.N, self.rule, self.policy = E, N, rule, policy
        self.slot_of = {}           # expert -> slot
        self.q = []                 # lru: recency (front = least recent); fifo: insertion order
        self.cnt = {}               # lfu: touches since insertion
        self.prob, self.prot = [], []   # slru segments, front = oldest placement
        self.cap = (4 * N) // 5
        self.hits = self.misses = self.fallbacks = 0

    def _hit(self, e):
        if self.policy == "lru" or self.policy == "lfu":
            self.q.remove(e)
            self.q.append(e)
            self.cnt[e] = self.cnt.get(e, 0) + 1
        elif self.policy == "slru":
            if e in self.prob:
                self.prob.remove(e)
                self.prot.append(e)
                if len(self.prot) > self.cap:
                    self.prob.append(self.prot.pop(0))
            else:
                self.prot.remove(e)
                self.prot.append(e)

    def _victim(self, done):
        if self.policy in ("lru", "fifo"):
            return next(e for e in self.q if e not in done)
        if self.policy == "lfu":
            c = [e for e in self.q if e not in done]
            lo = min(self.cnt[e] for e in c)
            return next(e for e in c if self.cnt[e] == lo)
        c = [e for e in self.prob if e not in done]
        return c[0] if c else next(e for e in self.prot if e not in done)

    def _drop(self, e):
        for lst in (self.q, self.prob, self.prot):
            if e in lst:
                lst.remove(e)
        self.cnt.pop(e, None)

    def step(self, ids):
        ids = np.asarray(ids)
        T, K = ids.shape
        u = sorted(set(int(v) for v in ids.ravel()))
        big = len(u) > self.N if self.rule == "distinct" else (K * T > self.N)
        if big:
            self.fallbacks += 1
            return [[u.index(int(v)) for v in row] for row in ids], FALLBACK, []
        misses, done = [], set()
        for e in u:
            if e in self.slot_of:
                self.hits += 1
                self._hit(e)
            else:
                used = set(self.slot_of.values())
                free = [s for s in range(self.N) if s not in used]
                if free:
                    slot, ev = max(free), -1
                else:
                    ev = self._victim(done)
                    slot = self.slot_of.pop(ev)
                    self._drop(ev)
                self.slot_of[e] = slot
                if self.policy == "slru":
                    self.prob.append(e)
                else:
                    self.q.append(e)
                    self.cnt[e] = 1
                self.misses += 1
                misses.append((e, slot, ev))
            done.add(e)
        return [[self.slot_of[int(v)] for v in row] for row in ids], POOL, misses

    def order(self):
        if self.policy == "slru":
            return self.prob + self.prot
        if self.policy == "lfu":
            return sorted(self.q, key=lambda e: (self.cnt[e], self.q.index(e)))
        return list(self.q)


def _run_both(E, N, trace, rule="distinct", policy="lru"):
    a, b = LayerLRU(E, N, rule, policy), ListCache(E, N, rule, policy)
    for ids in trace:
        ra = a.step(ids)
        sb, pb, mb = b.step(ids)
        assert ra.path == pb
        assert ra.slot_ids.tolist() == sb
        assert ra.misses == mb
        assert a.lru_order() == b.order()
    assert (a.hits, a.misses, a.fallbacks) == (b.hits, b.misses, b.fallbacks)
    return a


def test_hand_case_golden():
    g = json.load(open(os.path.join(GOLDEN, "lru_hand_case.json")))
    lru = LayerLRU(g["n_experts"], g["n_slots"])
    for ids, exp in zip(g["steps"], g["expect"]):
        r = lru.step(np.array(ids))
        assert r.slot_ids.tolist() == exp["slot_ids"]
        assert [list(m) for m in r.misses] == exp["misses"]
        assert r.path == exp["path"]
    f = g["final"]
    assert (lru.hits, lru.misses) == (f["hits"], f["misses"])
    assert lru.lru_order() == f["lru_front_to_back"]
    assert lru.map == f["map"] and lru.owner == f["owner"]


def test_policy_hand_cases_golden():
    g = json.load(open(os.path.join(GOLDEN, "policy_hand_cases.json")))
    for c in g["cases"]:
        lru = LayerLRU(c["n_experts"], c["n_slots"], policy=c["policy"])
        for ids, exp in zip(c["steps"], c["misses"]):
            r = lru.step(np.array(ids))
            assert [list(m) for m in r.misses] == exp, (c["policy"], ids)
            assert r.path == POOL
        f = c["final"]
        assert (lru.hits, lru.misses) == (f["hits"], f["misses"]), c["policy"]
        assert lru.eviction_order() == f["order"], c["policy"]
        assert lru.map == f["map"] and lru.owner == f["owner"], c["policy"]


def test_policies_agree_until_the_first_eviction():
    """The policy only decides victims: with as many slots as experts every policy
    gives the same slot ids, misses and counters (free slots from the top down)."""
    wl = synth.WORKLOADS["tiny_f32_e8"]
    trace = synth.make_trace(wl, steps=64)
    runs = []
    for pol in POLICIES:
        lru = LayerLRU(wl.experts, wl.experts, policy=pol)
        runs.append(([lru.step(trace[s, 0]).slot_ids.tolist() for s in range(64)], lru.hits, lru.misses))
    assert all(r == runs[0] for r in runs[1:])


def _rows(E, K):
    return [list(p) for p in itertools.permutations(range(E), K)]


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("E,K,N,length", [(4, 1, 1, 5), (4, 1, 2, 5), (4, 1, 3, 5),
                                          (4, 2, 2, 4), (4, 2, 3, 4), (3, 2, 1, 4)])
def test_brute_force_against_list_queues(E, K, N, length, policy):
    rows = _rows(E, K)
    for L in range(1, length + 1):
        for tr in itertools.product(rows, repeat=L):
            _run_both(E, N, [np.array([r]) for r in tr], policy=policy)


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("rule", ["distinct", "static"])
def test_random_multi_token_against_list_queues(rule, policy):
    rng = np.random.default_rng(11 + POLICIES.index(policy))
    for _ in range(1500):
        E = int(rng.integers(2, 7))
        K = int(rng.integers(1, min(E, 3) + 1))
        N = int(rng.integers(0, E + 1))
        trace = []
        for _ in range(int(rng.integers(1, 7))):
            T = int(rng.integers(1, 4))
            trace.append(np.stack([rng.permutation(E)[:K] for _ in range(T)]))
        _run_both(E, N, trace, rule, policy)


def _invariants(lru: LayerLRU, ids, r):
    res = [e for e in range(lru.E) if lru.map[e] >= 0]
    # map and owner are inverse bijections on the resident experts
    for e in res:
        assert lru.owner[lru.map[e]] == e
    for s, e in enumerate(lru.owner):
        if e >= 0:
            assert lru.map[e] == s
    assert sorted(res) == sorted(lru.lru_order())
    assert len(res) <= lru.N
    if r.path == POOL:
        flat = np.asarray(ids).ravel()
        assert all(lru.map[e] >= 0 for e in flat)
        assert (np.asarray([lru.map[e] for e in flat]) == r.slot_ids.ravel()).all()
        assert (np.asarray([lru.owner[s] for s in r.slot_ids.ravel()]) == flat).all()


@pytest.mark.parametrize("name", ["tiny_f32_e8", "olmoe_bf16_e64"])
def test_invariants_on_workload_traces(name):
    wl = synth.WORKLOADS[name]
    trace = synth.make_trace(wl, steps=min(wl.steps, 128))
    for layer in range(min(wl.layers, 2)):
        lru = LayerLRU(wl.experts, wl.slots)
        last_use = {}
        sum_d = 0
        for s in range(trace.shape[0]):
            ids = trace[s, layer]
            before = dict(hits=lru.hits, misses=lru.misses)
            r = lru.step(ids)
            _invariants(lru, ids, r)
            D = len(set(ids.ravel().tolist()))
            if r.path == POOL:
                sum_d += D
                assert lru.hits - before["hits"] + lru.misses - before["misses"] == D
                for e in sorted(set(ids.ravel().tolist())):
                    last_use[e] = (s, e)
            # LRU order = residents sorted by (last step used, id within step)
            order = lru.lru_order()
            assert order == sorted(order, key=lambda e: last_use[e])
        assert lru.hits + lru.misses == sum_d


def test_capacity_equal_to_experts_no_misses_after_warmup():
    wl = synth.WORKLOADS["olmoe_bf16_e64"]
    trace = synth.make_trace(wl, steps=200)
    lru = LayerLRU(wl.experts, wl.experts)
    seen = set()
    for s in range(trace.shape[0]):
        before = lru.misses
        lru.step(trace[s, 0])
        new = set(trace[s, 0].ravel().tolist()) - seen
        seen |= new
        assert lru.misses - before == len(new)
    assert lru.misses == len(seen)
    # warm: replaying the trace misses nothing
    m = lru.misses
    for s in range(trace.shape[0]):
        lru.step(trace[s, 0])
    assert lru.misses == m


def test_repeated_step_has_no_misses():
    lru = LayerLRU(16, 4)
    ids = np.array([[3, 9], [9, 12]])
    lru.step(ids)
    m = lru.misses
    for _ in range(5):
        r = lru.step(ids)
        assert r.misses == [] and r.path == POOL
    assert lru.misses == m


def test_capacity_one_top1_every_change_misses():
    rng = np.random.default_rng(3)
    seq = rng.integers(0, 5, 300)
    lru = LayerLRU(5, 1)
    changes = 1 + int((seq[1:] != seq[:-1]).sum())
    for e in seq:
        lru.step(np.array([[e]]))
    assert lru.misses == changes
    assert lru.hits == len(seq) - changes


def test_overflow_exactly_above_capacity():
    # N distinct ids fit; N + 1 fall back, with the pool untouched
    lru = LayerLRU(10, 3)
    r = lru.step(np.array([[1, 4, 7]]))
    assert r.path == POOL
    snap = (lru.state(), lru.hits, lru.misses)
    r = lru.step(np.array([[1, 4], [7, 9]]))
    assert r.path == FALLBACK and r.misses == []
    assert r.slot_ids.tolist() == [[0, 1], [2, 3]]
    assert (lru.state(), lru.hits, lru.misses) == snap
    assert lru.fallbacks == 1
    # static rule: K*T > N falls back even though D <= N
    s = LayerLRU(10, 3, rule="static")
    r = s.step(np.array([[1, 4], [4, 1]]))
    assert r.path == FALLBACK and r.slot_ids.tolist() == [[0, 1], [1, 0]]
    assert s.state() == LayerLRU(10, 3).state()


def test_zero_slots_always_falls_back():
    lru = LayerLRU(6, 0)
    for ids in ([[0]], [[5, 2]], [[1, 2], [3, 4]]):
        r = lru.step(np.array(ids))
        assert r.path == FALLBACK
    assert lru.fallbacks == 3 and lru.hits == lru.misses == 0


def test_out_of_range_rejected_state_untouched():
    lru = LayerLRU(8, 2)
    lru.step(np.array([[1, 2]]))
    snap = (lru.state(), lru.counters())
    for bad in ([[1, 8]], [[-1, 2]]):
        with pytest.raises(ExpertIdError):
            lru.step(np.array(bad))
        assert (lru.state(), lru.counters()) == snap


def test_eviction_reuse_in_same_step():
    """A step that evicts a slot and uses the newly loaded expert in that same step
    must see the new mapping (the stale-table failure of the llama.cpp discussion,
    'Validation' items 4-5)."""
    lru = LayerLRU(8, 2)
    lru.step(np.array([[0, 1]]))
    r = lru.step(np.array([[1, 5]]))       # 5 evicts 0 and must read the slot 0 had
    assert r.misses == [(5, lru.map[5], 0)]
    assert r.slot_ids.tolist() == [[lru.map[1], lru.map[5]]]
    assert lru.owner[r.slot_ids[0, 1]] == 5


def test_simulate_counts_match_layers():
    wl = synth.WORKLOADS["tiny_f32_e8"]
    trace = synth.make_trace(wl)
    stack, miss_count, paths = simulate(trace, wl.experts, wl.slots)
    assert miss_count.sum() == stack.layers[0].misses
    assert (paths == POOL).all()      # top-2 of 8 always fits 4 slots
    # 0.8 repeat probability and Zipf(1.2) give a high hit rate
    lay = stack.layers[0]
    assert lay.hits / (lay.hits + lay.misses) > 0.8
