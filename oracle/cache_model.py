"""Reference model of the per-layer expert cache (test infrastructure only:
imported by tests/ and nothing on the product path).

The pages keep each layer's routed experts in an LRU cache with an optional
pinned store of the hot ones, and choose what to pin from the usage they
record while running, re-choosable in session (colibrì README, "Idea";
labhub post, "让它变得可以忍受的那些装置": the usage profile and --repin;
CSDN feature, "冷启动与热缓存的辩证法").  They do not fix slot-level
details, so this model states the replacement the library documents, plainly
and sequentially, one miss at a time:

* a call needs a set R of experts (the batch's routed pairs, -1 skipped);
  the clock advances; each pair adds one to its expert's use count;
* every expert of R already resident is a hit: its slot's last use becomes
  the clock;
* the missing experts of R, in increasing expert order, each take the
  unpinned slot not used by this call with the smallest (last use, slot
  index), evicting what it held; an empty slot has last use 0;
* repin(n): unpin everything; the n experts with the largest use counts
  (ties: lower index) are served like a call (hits, usage and counters not
  counted), then their slots are pinned.
"""
from __future__ import annotations


class ExpertCacheModel:
    def __init__(self, n_experts: int, n_slots: int):
        if not 1 <= n_slots <= n_experts:
            raise ValueError("need 1 <= n_slots <= n_experts")
        self.E, self.S = n_experts, n_slots
        self.clock = 0
        self.slot_of = [-1] * n_experts
        self.expert_of = [-1] * n_slots
        self.last_use = [0] * n_slots
        self.pinned = [0] * n_slots
        self.use_count = [0] * n_experts
        self.hits = 0
        self.misses = 0
        self.error = 0
        self.copies: list[tuple[int, int]] = []

    def _serve(self, need: list[int], count: bool) -> None:
        for e in need:
            if self.slot_of[e] >= 0:
                self.last_use[self.slot_of[e]] = self.clock
        missing = [e for e in need if self.slot_of[e] < 0]
        if count:
            self.hits += len(need) - len(missing)
            self.misses += len(missing)
        self.copies = []
        for e in missing:
            free = [s for s in range(self.S)
                    if not self.pinned[s] and self.last_use[s] < self.clock]
            if not free:
                self.error |= 1
                break
            v = min(free, key=lambda s: (self.last_use[s], s))
            old = self.expert_of[v]
            if old >= 0:
                self.slot_of[old] = -1
            self.slot_of[e] = v
            self.expert_of[v] = e
            self.last_use[v] = self.clock
            self.copies.append((e, v))

    def step(self, experts) -> None:
        """One call whose routed pairs select ``experts`` (any iterable of
        expert indices; -1 entries are dropped slots)."""
        self.clock += 1
        need = {}
        for e in experts:
            e = int(e)
            if e >= 0:
                need[e] = need.get(e, 0) + 1
        for e, n in need.items():
            self.use_count[e] += n
        self._serve(sorted(need), count=True)

    def repin(self, n_pin: int) -> None:
        self.clock += 1
        self.pinned = [0] * self.S
        top = sorted(range(self.E), key=lambda e: (-self.use_count[e], e))[:n_pin]
        self._serve(sorted(top), count=False)
        for e in top:
            if self.slot_of[e] >= 0:
                self.pinned[self.slot_of[e]] = 1

    def resident(self) -> set[int]:
        return {e for e in self.expert_of if e >= 0}
