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

Precision-aware loads (page "MoE-APEX: An Efficient MoE Inference System with
Adaptive Precision Expert Offloading", "This paper's idea": a cache-miss expert
that is less critical for the current tokens is loaded as its low-precision
variant), the reading taken: the experts' blobs start with their two-bit part
(a prefix of prefix_bytes; nested two/four-bit layout), every needed expert
comes with its precision for the step (four bits or two), and a slot holds an
expert's whole blob or only its prefix.  A resident expert is a hit and keeps
its slot; if it holds only the prefix and is needed at four bits, its low planes
(the rest of the blob) are copied into the slot ("lo").  A miss copies the prefix
("hi", two bits) or the whole blob ("all", four bits).  The cost-aware policy
weighs usage by the bytes a slot's reload would copy: usage times the prefix or
the whole blob, as the slot holds.

Prefetch (experts expected in a later round or step copied ahead of it), the
reading taken: the predicted experts not resident go into victim slots chosen
among the slots not holding a predicted expert, by the policy's victim order, at
most max_copies of them: in ascending id (LRU) or in decreasing usage, ties
ascending id (cost-aware); the prefetched slots get a new timestamp, like a
round.
"""

POLICY_LRU, POLICY_COST = 0, 1


class SlotCacheSim:
    def __init__(self, num_experts, num_slots, policy=POLICY_LRU, decay=0.9, prefix_bytes=None, blob_bytes=None):
        self.E, self.S = num_experts, num_slots
        self.policy, self.decay = policy, float(decay)
        self.slot_expert = [-1] * num_slots
        self.slot_stamp = [-1] * num_slots
        self.slot_full = [False] * num_slots
        self.usage = [0.0] * num_experts
        self.clock = 0
        # precision-aware mode: blob bytes and its two-bit prefix
        self.prefix_bytes, self.blob_bytes = prefix_bytes, blob_bytes

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
            cost = -1.0 if e < 0 else self.usage[e]
            if e >= 0 and self.prefix_bytes is not None:
                cost = self.usage[e] * float(self.blob_bytes if self.slot_full[s] else self.prefix_bytes)
            return (0 if e < 0 else 1, cost, self.slot_stamp[s], s)
        return (self.slot_stamp[s], s)

    def _miss_order(self, experts):
        if self.policy == POLICY_COST:
            return sorted(experts, key=lambda e: (self.usage[e], e))
        return sorted(experts)

    def load_round(self, pending, full=None):
        """One round for the pending experts -> (subset, hits, copies).  Whole-blob mode:
        copies are (expert, slot).  Precision-aware mode: `full` is the set of experts
        needed at four bits (the others at two) and copies are (expert, slot, part),
        part "all", "hi" (the two-bit prefix) or "lo" (the rest, for a resident
        two-bit expert needed at four bits)."""
        res = self.resident()
        pending = sorted(set(pending))
        mixed = self.prefix_bytes is not None
        full = set(pending) if (full is None or not mixed) else set(full)
        hits = [e for e in pending if e in res]
        misses = self._miss_order([e for e in pending if e not in res])[: self.S - len(hits)]
        hit_slots = {res[e] for e in hits}
        victims = sorted((s for s in range(self.S) if s not in hit_slots), key=self._victim_key)
        copies = []
        if mixed:
            for e in hits:
                if e in full and not self.slot_full[res[e]]:
                    copies.append((e, res[e], "lo"))
                    self.slot_full[res[e]] = True
        for e, s in zip(misses, victims):
            self.slot_expert[s] = e
            if mixed:
                self.slot_full[s] = e in full
                copies.append((e, s, "all" if e in full else "hi"))
            else:
                self.slot_full[s] = True
                copies.append((e, s))
        self.clock += 1
        for s, e in enumerate(self.slot_expert):
            if e in hits or e in misses:
                self.slot_stamp[s] = self.clock
        return sorted(hits + misses), hits, copies

    def copy_bytes(self, copies):
        """Bytes moved by a list of precision-aware copies."""
        size = {"all": self.blob_bytes, "hi": self.prefix_bytes, "lo": self.blob_bytes - self.prefix_bytes}
        return sum(size[c[2]] for c in copies)

    def step(self, needed, full=None):
        """begin_step, then all rounds of one step -> list of (subset, hits, copies)."""
        self.begin_step(needed)
        pending = set(needed)
        rounds = []
        while pending:
            subset, hits, copies = self.load_round(pending, full)
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
            self.slot_full[s] = True
        return copies


class LRUSlotCache(SlotCacheSim):
    """The LRU policy (the default of the GPU cache)."""

    def __init__(self, num_experts, num_slots):
        super().__init__(num_experts, num_slots, POLICY_LRU)
