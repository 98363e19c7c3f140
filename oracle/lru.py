"""Per-layer expert slot manager with LRU eviction -- the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources (the pages):

* vLLM PR "Run MoE models exceeding VRAM via expert CPU offloading with GPU cache
  (--moe-expert-cache-size)", section "How it works": prepare() takes the unique
  expert ids of the batch, treats each as a hit (move to the most recently used
  end) or a miss (evict the least recently used, copy host -> GPU slot, update
  the mapping), then remaps topk_ids to slot ids through the persistent mapping.
* Same page, review thread: the OrderedDict form -- ``move_to_end`` on a hit,
  ``popitem(last=False)`` to evict, free slots ``list(range(capacity))`` taken
  with ``pop()`` (so from the end), counters ``hits``/``misses`` per unique id;
  the persistent int32 GPU mapping updated in place at each miss.
* Same page, test list: an overflow check exactly when the unique ids exceed the
  capacity, and none at capacity.
* llama.cpp discussion "Persistent expert slot pool for MoE CPU offload", section
  "Why not the other approaches on the table" and "Design" item 2: a ubatch that
  can select more distinct experts than slots (n_expert_used * n_tokens >
  n_slots) takes the selective-copy path and never touches the pool.

Readings where the pages leave a step open:

* unique ids are processed in ascending order (``Tensor.unique`` sorts), one at
  a time, so a hit moves to the MRU end before a later miss of the same step
  evicts;
* a non-resident expert maps to -1, and an evicted expert's entry is reset to -1;
* fallback rule "distinct" (default): D > N distinct ids; rule "static": K*T > N;
  N = 0 always falls back when the step has any id.  A fallback changes nothing
  in the pool except the ``fallbacks`` counter, and its slot ids are the ranks of
  the ids in the ascending distinct list (the staging order);
* an id outside [0, E) rejects the whole step with the state untouched;
* ``steps`` counts every accepted step, pooled or not.
"""
from __future__ import annotations

from collections import OrderedDict
from dataclasses import dataclass, field

import numpy as np

POOL = 0
FALLBACK = 1


class ExpertIdError(ValueError):
    pass


@dataclass
class StepResult:
    slot_ids: np.ndarray            # int32, same shape as ids
    path: int                       # POOL or FALLBACK
    misses: list = field(default_factory=list)   # [(expert, slot, evicted or -1)]
    distinct: list = field(default_factory=list)  # ascending distinct ids


class LayerLRU:
    """One layer's slot pool bookkeeping, exactly as the page-1 prepare() does it."""

    def __init__(self, n_experts: int, n_slots: int, rule: str = "distinct"):
        if rule not in ("distinct", "static"):
            raise ValueError(rule)
        self.E = int(n_experts)
        self.N = int(n_slots)
        self.rule = rule
        self.reset()

    def reset(self):
        self.map = [-1] * self.E                # expert -> slot, -1 when not resident
        self.owner = [-1] * self.N              # slot -> expert, -1 when free
        self.free = list(range(self.N))         # taken with pop(): slot N-1 first
        self.order: OrderedDict[int, None] = OrderedDict()   # front = least recently used
        self.hits = 0
        self.misses = 0
        self.fallbacks = 0
        self.steps = 0

    # -- the step ----------------------------------------------------------
    def step(self, ids) -> StepResult:
        ids = np.asarray(ids, dtype=np.int64)
        if ids.ndim != 2:
            raise ValueError("ids must be [tokens, top_k]")
        T, K = ids.shape
        flat = ids.ravel().tolist()
        for e in flat:
            if e < 0 or e >= self.E:
                raise ExpertIdError(f"expert id {e} outside [0, {self.E})")
        unique_ids = sorted(set(flat))
        D = len(unique_ids)
        self.steps += 1

        if self.rule == "distinct":
            overflow = D > self.N
        else:
            overflow = K * T > self.N and D > 0
        if overflow:
            self.fallbacks += 1
            rank = {e: r for r, e in enumerate(unique_ids)}
            slot_ids = np.array([rank[e] for e in flat], dtype=np.int32).reshape(T, K)
            return StepResult(slot_ids, FALLBACK, [], unique_ids)

        misses = []
        for e in unique_ids:
            if self.map[e] >= 0:
                self.order.move_to_end(e)
                self.hits += 1
            else:
                if self.free:
                    slot = self.free.pop()
                    evicted = -1
                else:
                    evicted, _ = self.order.popitem(last=False)
                    slot = self.map[evicted]
                    self.map[evicted] = -1
                self.map[e] = slot
                self.owner[slot] = e
                self.order[e] = None
                self.misses += 1
                misses.append((e, slot, evicted))
        slot_ids = np.array([self.map[e] for e in flat], dtype=np.int32).reshape(T, K)
        return StepResult(slot_ids, POOL, misses, unique_ids)

    # -- views ---------------------------------------------------------------
    def lru_order(self) -> list:
        """Resident experts, least recently used first."""
        return list(self.order.keys())

    def state(self):
        return list(self.map), list(self.owner), self.lru_order()

    def counters(self) -> dict:
        return dict(steps=self.steps, hits=self.hits, misses=self.misses,
                    fallbacks=self.fallbacks)


class StackLRU:
    """Independent pools, one per layer."""

    def __init__(self, n_layers: int, n_experts: int, n_slots: int, rule: str = "distinct"):
        self.layers = [LayerLRU(n_experts, n_slots, rule) for _ in range(n_layers)]

    def step(self, layer: int, ids) -> StepResult:
        return self.layers[layer].step(ids)


def simulate(trace: np.ndarray, n_experts: int, n_slots: int, rule: str = "distinct"):
    """Run a whole trace ids[step, layer, token, k]; returns per-layer counters and the
    per-step miss counts miss_count[step, layer]."""
    S, L = trace.shape[:2]
    stack = StackLRU(L, n_experts, n_slots, rule)
    miss_count = np.zeros((S, L), dtype=np.int64)
    paths = np.zeros((S, L), dtype=np.int8)
    for s in range(S):
        for l in range(L):
            r = stack.step(l, trace[s, l])
            miss_count[s, l] = len(r.misses)
            paths[s, l] = r.path
    return stack, miss_count, paths
