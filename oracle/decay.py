"""Per-layer expert placement by decayed use counts -- the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

"Running 125B MoE on Two 32 GB Cards", sections 4.3 and 4.4 (moving experts at run
time): the router counts every selected (token, expert) row; every 8 steps the use
counts are decayed with a half-life of 512 steps, and the most used expert held in
host memory changes places with the least used expert held on the GPU when its
count exceeds the other's by more than 2 -- one pair per layer per decision.  An
expert selected while in host memory is read from there (no eviction on a miss);
prefill does not count.

How that maps onto a layer's slot pool (the readings, listed in the design notes):

* the pool starts empty; while it has a free slot, a selected non-resident expert
  takes the highest free slot (as the LRU cache does), so the pool fills from the
  first steps; once it is full, a selected non-resident expert is read from the host
  for that step only (it goes to staging and the pool is left as it is);
* the step counter counts pooled steps; a step whose count is a multiple of 8 makes
  the decision first, from the counts of the steps before it: every count is
  multiplied by 2**(-8/512) (float32); then, if the pool is full (with a free slot a
  host expert simply takes it when next selected), among non-resident experts the
  largest count (lowest id on ties) and among resident experts the smallest count
  (lowest id on ties) are compared, and if the difference exceeds 2 the first takes
  the second's slot (a move: copied in like a miss, recorded as (expert, slot,
  evicted));
* then the step's distinct ids are processed in ascending order: resident -> hit,
  free slot -> inserted (a miss), else -> read from the host (staged, at the rank
  among the step's host-read experts, in ascending order);
* finally each expert's count grows by the number of (token, k) rows that selected
  it in the step (added once per step in float32);
* a step that bypasses the pool (the route rule, prefill) changes nothing but the
  fallback counter: it does not count.

Slot ids: a pool slot in [0, N), or N + staging rank for an expert read from the
host.  The float32 arithmetic (products, sums, the comparison) is the device's.
"""
from __future__ import annotations

import numpy as np

from oracle.lru import FALLBACK, POOL, ExpertIdError, StepResult

DECIDE_EVERY = 8
HALF_LIFE = 512
THRESHOLD = 2.0
DECAY = np.float32(2.0 ** (-DECIDE_EVERY / HALF_LIFE))   # float32 of 2**(-1/64)


class LayerDecay:
    """One layer's pool under decayed-count placement."""

    def __init__(self, n_experts: int, n_slots: int, rule: str = "distinct"):
        if rule not in ("distinct", "static"):
            raise ValueError(rule)
        self.E = int(n_experts)
        self.N = int(n_slots)
        self.rule = rule
        self.reset()

    def reset(self):
        self.map = [-1] * self.E
        self.owner = [-1] * self.N
        self.free_slots = list(range(self.N))
        self.count = np.zeros(self.E, dtype=np.float32)
        self.pooled_steps = 0
        self.hits = 0
        self.misses = 0          # experts copied into a slot (insertions and moves)
        self.moves = 0
        self.staged = 0          # experts read from the host by pooled or bypassing steps
        self.fallbacks = 0
        self.steps = 0

    def _decide(self):
        """Decay, then one move if the gap is large enough; returns the move or None."""
        self.count = (self.count * DECAY).astype(np.float32)
        if self.free_slots:
            return None
        host = [e for e in range(self.E) if self.map[e] < 0]
        gpu = [e for e in range(self.E) if self.map[e] >= 0]
        if not host or not gpu:
            return None
        h = max(host, key=lambda e: (self.count[e], -e))      # largest count, lowest id
        g = min(gpu, key=lambda e: (self.count[e], e))        # smallest count, lowest id
        gap = np.float32(self.count[h] - self.count[g])
        if not gap > np.float32(THRESHOLD):
            return None
        slot = self.map[g]
        self.map[g] = -1
        self.map[h] = slot
        self.owner[slot] = h
        self.moves += 1
        self.misses += 1
        return (h, slot, g)

    def step(self, ids) -> StepResult:
        ids = np.asarray(ids, dtype=np.int64)
        if ids.ndim != 2:
            raise ValueError("ids must be [tokens, top_k]")
        T, K = ids.shape
        flat = ids.ravel().tolist()
        bad = [e for e in flat if not 0 <= e < self.E]
        if bad:
            raise ExpertIdError(f"expert id {bad[0]} outside [0, {self.E})")
        distinct = sorted(set(flat))
        D = len(distinct)
        self.steps += 1
        bypass = D > self.N if self.rule == "distinct" else (D > 0 and K * T > self.N)
        if bypass:
            self.fallbacks += 1
            self.staged += D
            rank = {e: r for r, e in enumerate(distinct)}
            return StepResult(np.array([rank[e] for e in flat], np.int32).reshape(T, K), FALLBACK, [], distinct)

        self.pooled_steps += 1
        copied = []
        if self.pooled_steps % DECIDE_EVERY == 0:
            mv = self._decide()
            if mv is not None:
                copied.append(mv)
        host_rank = {}
        for e in distinct:
            if self.map[e] >= 0:
                self.hits += 1
            elif self.free_slots:
                slot = self.free_slots.pop()
                self.map[e] = slot
                self.owner[slot] = e
                self.misses += 1
                copied.append((e, slot, -1))
            else:
                host_rank[e] = len(host_rank)
        self.staged += len(host_rank)
        occ = np.bincount(np.asarray(flat, dtype=np.int64), minlength=self.E).astype(np.float32)
        self.count = (self.count + occ).astype(np.float32)
        slot_ids = np.array([self.map[e] if e not in host_rank else self.N + host_rank[e] for e in flat],
                            np.int32).reshape(T, K)
        return StepResult(slot_ids, POOL, copied, distinct)

    def eviction_order(self) -> list:
        """Resident experts by use count, the next to leave first (lowest id on ties)."""
        return sorted((e for e in range(self.E) if self.map[e] >= 0), key=lambda e: (self.count[e], e))

    def lru_order(self) -> list:
        return self.eviction_order()

    def state(self):
        return list(self.map), list(self.owner), self.eviction_order()
