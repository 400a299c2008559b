"""Expert-sorted permutation of (token, slot) pairs (oracle; test infrastructure only).

The fused grouped kernels of ExactMoE (page "Every Expert Counts: ExactMoE for
Memory-Efficient W4A16 Inference", Abstract) run all selected experts in one
grouped pass, which needs the pairs grouped by expert.  The page does not say
how; the reading taken is a stable counting sort:

* pair p = t * k + j carries expert ids[t, j];
* counts[e] = number of pairs routed to e; offsets = exclusive prefix sum
  (offsets[E] = T * k);
* sorted_pairs lists the pairs of expert 0, then expert 1, ..., each group in
  increasing p (stable);
* pair_pos[p] is the position of p in sorted_pairs (inverse permutation);
* active lists the experts with at least one pair, ascending;
* tile_offsets (for a tile height block_m > 0) is the exclusive prefix sum of
  ceil(counts[e] / block_m).
"""
import numpy as np


def align(ids, E, block_m=0):
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    P = ids.size
    counts = np.zeros(E, dtype=np.int64)
    for e in ids:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = np.empty(P, dtype=np.int64)
    fill = offsets[:-1].copy()
    for p in range(P):                      # visiting p in increasing order keeps it stable
        e = ids[p]
        sorted_pairs[fill[e]] = p
        fill[e] += 1
    pair_pos = np.empty(P, dtype=np.int64)
    pair_pos[sorted_pairs] = np.arange(P)
    active = np.nonzero(counts)[0]
    out = {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "sorted_pairs": sorted_pairs.astype(np.int32),
        "pair_pos": pair_pos.astype(np.int32),
        "active": active.astype(np.int32),
    }
    if block_m > 0:
        tiles = (counts + block_m - 1) // block_m
        to = np.zeros(E + 1, dtype=np.int64)
        to[1:] = np.cumsum(tiles)
        out["tile_offsets"] = to.astype(np.int32)
    return out
