"""Per-layer expert slot manager -- the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What a step computes (vLLM PR "Run MoE models exceeding VRAM via expert CPU
offloading with GPU cache (--moe-expert-cache-size)", section "How it works" and
the review thread; llama.cpp discussion "Persistent expert slot pool for MoE CPU
offload", "Design" item 2 and the prefill rule under "Why not the other approaches
on the table"):

1. every id must lie in [0, E), else the whole step is rejected and nothing
   changes;
2. the step's distinct expert ids are taken in ascending order (``unique`` sorts);
3. route: a step that touches more distinct experts than there are slots (rule
   "distinct", the default), or whose top_k * n_tokens exceeds the slot count
   (rule "static"), bypasses the pool: its slot ids are the ranks of its ids in the
   ascending distinct list (the staging order) and only ``fallbacks`` changes;
4. otherwise each distinct id in turn is a hit (already holds a slot: the eviction
   policy records the use) or a miss (takes a free slot -- free slots are handed
   out from the highest index down -- or the slot of the resident expert the
   policy picks as victim, whose map entry goes back to -1);
5. slot ids are ``map[id]`` after the step.

This module states that rule directly: every resident expert carries the numbers
its policy orders by, and a victim is the smallest of them.  Each event (a touch,
an insertion, a demotion) draws the next value of one per-layer counter ``tick``.

Eviction policies (the review thread of the vLLM PR lists four, selected by name;
LRU is the one the PR ships):

* ``lru``  -- key = tick of the last touch;
* ``fifo`` -- key = tick of the insertion (a hit changes nothing);
* ``lfu``  -- key = (touches since insertion, tick of the last touch);
* ``slru`` -- two segments with the 20 % / 80 % split the thread gives:
  ``prot_cap = (4 * N) // 5`` experts may sit in the protected segment.  A miss
  enters the probationary segment; a hit there moves the expert to the protected
  segment, and when that segment then holds more than ``prot_cap`` experts its
  smallest key is demoted to the probationary segment; a hit in the protected
  segment refreshes the key.  The key is the tick at which the expert took its
  place in its segment.  A victim comes from the probationary segment while it
  has a candidate, else from the protected one.

Readings where the pages leave a step open (each listed in the design notes):

* an expert the step has already processed is never a victim of the same step,
  whatever its key: the step's later ids could otherwise evict an expert the
  step itself needs.  For LRU this is what the printed algorithm does anyway (a
  processed expert is the most recent), and a pooled step always has a candidate
  (it processed fewer than D <= N ids, and a full pool holds N);
* a non-resident expert maps to -1, and an evicted expert's entry is reset to -1;
* ``steps`` counts every accepted step, pooled or not; N = 0 always falls back.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

POOL = 0
FALLBACK = 1
POLICIES = ("lru", "fifo", "lfu", "slru")


class ExpertIdError(ValueError):
    pass


@dataclass
class StepResult:
    slot_ids: np.ndarray            # int32, same shape as ids
    path: int                       # POOL or FALLBACK
    misses: list = field(default_factory=list)   # [(expert, slot, evicted or -1)]
    distinct: list = field(default_factory=list)  # ascending distinct ids


@dataclass
class _Entry:
    """What the policies know about one resident expert."""
    inserted: int        # tick of the insertion
    last: int            # tick of the last touch (the insertion counts as one)
    uses: int            # touches since the insertion
    place: int           # tick at which it took its place in its segment (SLRU)
    protected: bool = False


class LayerLRU:
    """One layer's slot pool bookkeeping (``policy`` picks the eviction rule)."""

    def __init__(self, n_experts: int, n_slots: int, rule: str = "distinct", policy: str = "lru"):
        if rule not in ("distinct", "static"):
            raise ValueError(rule)
        if policy not in POLICIES:
            raise ValueError(policy)
        self.E = int(n_experts)
        self.N = int(n_slots)
        self.rule = rule
        self.policy = policy
        self.prot_cap = (4 * self.N) // 5
        self.reset()

    def reset(self):
        self.map = [-1] * self.E                # expert -> slot, -1 when not resident
        self.owner = [-1] * self.N              # slot -> expert, -1 when free
        self.free_slots = list(range(self.N))   # the last entry is handed out first
        self.entries: dict[int, _Entry] = {}    # resident expert -> its policy numbers
        self.tick = 0
        self.hits = 0
        self.misses = 0
        self.fallbacks = 0
        self.steps = 0

    # -- policy numbers -------------------------------------------------------
    def _next_tick(self) -> int:
        t = self.tick
        self.tick += 1
        return t

    def _key(self, e: int):
        d = self.entries[e]
        if self.policy == "lru":
            return d.last
        if self.policy == "fifo":
            return d.inserted
        if self.policy == "lfu":
            return (d.uses, d.last)
        return d.place                           # slru, within a segment

    def _victim(self, processed: set) -> int:
        cands = [e for e in self.entries if e not in processed]
        if self.policy == "slru":
            prob = [e for e in cands if not self.entries[e].protected]
            cands = prob if prob else cands
        return min(cands, key=self._key)

    def _touch(self, e: int):
        d = self.entries[e]
        t = self._next_tick()
        d.last = t
        d.uses += 1
        if self.policy != "slru":
            return
        d.place = t
        if not d.protected:
            d.protected = True
            prot = [x for x in self.entries if self.entries[x].protected]
            if len(prot) > self.prot_cap:
                dem = min(prot, key=lambda x: self.entries[x].place)
                self.entries[dem].protected = False
                self.entries[dem].place = self._next_tick()

    def _insert(self, e: int):
        t = self._next_tick()
        self.entries[e] = _Entry(inserted=t, last=t, uses=1, place=t)

    # -- the step ----------------------------------------------------------
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

        if self.rule == "distinct":
            bypass = D > self.N
        else:
            bypass = D > 0 and K * T > self.N
        if bypass:
            self.fallbacks += 1
            rank = {e: r for r, e in enumerate(distinct)}
            staged = np.array([rank[e] for e in flat], dtype=np.int32).reshape(T, K)
            return StepResult(staged, FALLBACK, [], distinct)

        misses = []
        processed: set[int] = set()
        for e in distinct:
            if e in self.entries:
                self.hits += 1
                self._touch(e)
            else:
                if self.free_slots:
                    slot, victim = self.free_slots.pop(), -1
                else:
                    victim = self._victim(processed)
                    slot = self.map[victim]
                    self.map[victim] = -1
                    del self.entries[victim]
                self.map[e] = slot
                self.owner[slot] = e
                self._insert(e)
                self.misses += 1
                misses.append((e, slot, victim))
            processed.add(e)
        slot_ids = np.array([self.map[e] for e in flat], dtype=np.int32).reshape(T, K)
        return StepResult(slot_ids, POOL, misses, distinct)

    # -- views ---------------------------------------------------------------
    def eviction_order(self) -> list:
        """Resident experts in the order the policy would evict them (with nothing
        processed): the least recently used first for LRU; for SLRU the probationary
        segment, then the protected one."""
        if self.policy == "slru":
            prob = sorted((e for e in self.entries if not self.entries[e].protected), key=self._key)
            prot = sorted((e for e in self.entries if self.entries[e].protected), key=self._key)
            return prob + prot
        return sorted(self.entries, key=self._key)

    def lru_order(self) -> list:
        return self.eviction_order()

    def state(self):
        return list(self.map), list(self.owner), self.eviction_order()

    def counters(self) -> dict:
        return dict(steps=self.steps, hits=self.hits, misses=self.misses,
                    fallbacks=self.fallbacks)


class StackLRU:
    """Independent pools, one per layer."""

    def __init__(self, n_layers: int, n_experts: int, n_slots: int, rule: str = "distinct",
                 policy: str = "lru"):
        self.layers = [LayerLRU(n_experts, n_slots, rule, policy) for _ in range(n_layers)]

    def step(self, layer: int, ids) -> StepResult:
        return self.layers[layer].step(ids)


def simulate(trace: np.ndarray, n_experts: int, n_slots: int, rule: str = "distinct",
             policy: str = "lru"):
    """Run a whole trace ids[step, layer, token, k]; returns the stack, the per-step
    miss counts miss_count[step, layer] and the paths."""
    S, L = trace.shape[:2]
    stack = StackLRU(L, n_experts, n_slots, rule, policy)
    miss_count = np.zeros((S, L), dtype=np.int64)
    paths = np.zeros((S, L), dtype=np.int8)
    for s in range(S):
        for l in range(L):
            r = stack.step(l, trace[s, l])
            miss_count[s, l] = len(r.misses)
            paths[s, l] = r.path
    return stack, miss_count, paths
