"""LRU simulator for the GPU-resident expert slot cache (oracle; test infrastructure only).

ExactMoE (page "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
Inference", Abstract) keeps all quantised experts in pinned host memory and
runs every selected expert from a configurable number of GPU slots.  The page
gives no replacement policy or rule for more needed experts than slots; the
reading taken:

* a step needs a set R of experts; it runs in rounds until R is covered;
* a round takes the needed experts already resident (hits), then the missing
  ones in ascending id until the slots are full;
* each miss goes into a victim slot chosen among the slots not holding a hit,
  empty slots first, then least recently used, ties to the lower slot index;
* every slot used in the round gets the round's timestamp (a counter that
  increases by one per round);
* later rounds of the same step may evict experts of earlier rounds (their
  work is finished).

Prefetch (the next-layer overlap: experts a layer is expected to need are copied
while an earlier layer computes), the reading taken: the predicted experts not
resident, in ascending id and at most max_copies of them, go into victim slots
chosen among the slots not holding a predicted expert, by the same order (empty,
then least recently used, ties to the lower slot); the prefetched slots get a new
timestamp, like a round.
"""


class LRUSlotCache:
    def __init__(self, num_experts, num_slots):
        self.E, self.S = num_experts, num_slots
        self.slot_expert = [-1] * num_slots
        self.slot_stamp = [-1] * num_slots
        self.clock = 0

    def resident(self):
        return {e: s for s, e in enumerate(self.slot_expert) if e >= 0}

    def load_round(self, pending):
        """One round for the pending experts -> (subset, hits, copies[(expert, slot)])."""
        res = self.resident()
        pending = sorted(set(pending))
        hits = [e for e in pending if e in res]
        misses = [e for e in pending if e not in res][: self.S - len(hits)]
        hit_slots = {res[e] for e in hits}
        victims = sorted((s for s in range(self.S) if s not in hit_slots),
                         key=lambda s: (self.slot_stamp[s], s))
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
        """All rounds of one step -> list of (subset, hits, copies)."""
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
        keep = {res[e] for e in predicted if e in res}
        victims = sorted((s for s in range(self.S) if s not in keep), key=lambda s: (self.slot_stamp[s], s))
        copies = list(zip(want[:max(0, max_copies)], victims))
        self.clock += 1
        for e, s in copies:
            self.slot_expert[s] = e
            self.slot_stamp[s] = self.clock
        return copies
