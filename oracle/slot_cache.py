"""Slot-cache simulator for the GPU-resident expert slot cache (oracle; test infrastructure only).

ExactMoE (page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
Inference", Abstract) keeps all quantised experts in pinned host memory and
runs every selected expert from a configurable number of GPU slots.  The page
gives no replacement policy or rule for more needed experts than slots; the
reading taken:

* a step needs a set R of experts; it runs in rounds until R is covered;
* a round takes the needed experts already resident (hits), then missing ones
  until the slots are full;
* each miss goes into a victim slot chosen among the slots not holding an
  expert of the round, empty slots first;
* every slot used in the round gets the round's timestamp (a counter that
  increases by one per round);
* later rounds of the same step may evict experts of earlier rounds (their
  work is finished).

Two policies fix the remaining choices.

LRU: misses enter in ascending expert id; victims are the least recently used
slots, ties to the lower slot index.

Cost-aware (page "MoE-APEX: An Efficient MoE Inference System with Adaptive
Precision Expert Offloading", sections "This paper's idea" and "Why it works":
a sequence-level caching policy keeps resident the experts whose reload would
cost most, weighing reload cost against the memory they occupy).  The page
gives no formula; the reading taken: every expert carries a usage estimate u_e,
an exponential average over the steps of the sequence of "e is needed in this
step" (u <- decay * u + (1 - decay) * [e needed], updated once per step before
its rounds, u = 0 at the start); the expected cost of evicting e is u_e times
the bytes its reload copies (one slot's worth for every expert of a four-bit
cache, so the slot size divides out).  Victims: empty slots first, then the
lowest expected cost, then least recently used, then the lower slot.  Misses
enter a round in increasing expected cost (ties: ascending id), so the experts
most likely needed again are loaded in the step's last round and stay resident.

Prefetch (experts expected in a later round or step copied ahead of it), the
reading taken: the predicted experts not resident go into victim slots chosen
among the slots not holding a predicted expert, by the policy's victim order, at
most max_copies of them: in ascending id (LRU) or in decreasing usage, ties
ascending id (cost-aware); the prefetched slots get a new timestamp, like a
round.
"""

POLICY_LRU, POLICY_COST = 0, 1


class SlotCacheSim:
    def __init__(self, num_experts, num_slots, policy=POLICY_LRU, decay=0.9):
        self.E, self.S = num_experts, num_slots
        self.policy, self.decay = policy, float(decay)
        self.slot_expert = [-1] * num_slots
        self.slot_stamp = [-1] * num_slots
        self.usage = [0.0] * num_experts
        self.clock = 0

    def resident(self):
        return {e: s for s, e in enumerate(self.slot_expert) if e >= 0}

    def begin_step(self, needed):
        """Usage update of the cost-aware policy (the step's needed set)."""
        needed = set(needed)
        self.usage = [self.decay * u + (1.0 - self.decay) * (1.0 if e in needed else 0.0)
                      for e, u in enumerate(self.usage)]

    def _victim_key(self, s):
        e = self.slot_expert[s]
        if self.policy == POLICY_COST:
            return (0 if e < 0 else 1, -1.0 if e < 0 else self.usage[e], self.slot_stamp[s], s)
        return (self.slot_stamp[s], s)

    def _miss_order(self, experts):
        if self.policy == POLICY_COST:
            return sorted(experts, key=lambda e: (self.usage[e], e))
        return sorted(experts)

    def load_round(self, pending):
        """One round for the pending experts -> (subset, hits, copies[(expert, slot)])."""
        res = self.resident()
        pending = sorted(set(pending))
        hits = [e for e in pending if e in res]
        misses = self._miss_order([e for e in pending if e not in res])[: self.S - len(hits)]
        hit_slots = {res[e] for e in hits}
        victims = sorted((s for s in range(self.S) if s not in hit_slots), key=self._victim_key)
        copies = []
        for e, s in zip(misses, victims):
            self.slot_expert[s] = e
            copies.append((e, s))
        self.clock += 1
        for s, e in enumerate(self.slot_expert):
            if e in hits or e in misses:
                self.slot_stamp[s] = self.clock
        return sorted(hits + misses), hits, copies

    def step(self, needed):
        """begin_step, then all rounds of one step -> list of (subset, hits, copies)."""
        self.begin_step(needed)
        pending = set(needed)
        rounds = []
        while pending:
            subset, hits, copies = self.load_round(pending)
            rounds.append((subset, hits, copies))
            pending -= set(subset)
        return rounds

    def prefetch(self, predicted, max_copies):
        """Prefetch -> copies[(expert, slot)]."""
        res = self.resident()
        predicted = sorted(set(predicted))
        want = [e for e in predicted if e not in res]
        if self.policy == POLICY_COST:
            want.sort(key=lambda e: (-self.usage[e], e))
        keep = {res[e] for e in predicted if e in res}
        victims = sorted((s for s in range(self.S) if s not in keep), key=self._victim_key)
        copies = list(zip(want[:max(0, max_copies)], victims))
        self.clock += 1
        for e, s in copies:
            self.slot_expert[s] = e
            self.slot_stamp[s] = self.clock
        return copies


class LRUSlotCache(SlotCacheSim):
    """The LRU policy (the default of the GPU cache)."""

    def __init__(self, num_experts, num_slots):
        super().__init__(num_experts, num_slots, POLICY_LRU)
