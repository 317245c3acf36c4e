"""Token-by-expert permutation of the T*k (token, slot) pairs.

Pairs q = t*k + j are ordered by the key (expert, t, j) ascending: a stable
counting sort by expert.  ``expert_off`` is the exclusive prefix sum of the
per-expert pair counts, so the pairs of expert e are
pair_perm[expert_off[e] : expert_off[e+1]].
"""

import numpy as np


def permutation(topk_idx: np.ndarray, E: int):
    idx = np.asarray(topk_idx, dtype=np.int64).ravel()
    counts = [0] * E
    for e in idx:
        counts[int(e)] += 1
    off = [0] * (E + 1)
    for e in range(E):
        off[e + 1] = off[e] + counts[e]
    cursor = list(off[:E])
    perm = [0] * idx.size
    for q, e in enumerate(idx):          # ascending q -> stable within an expert
        perm[cursor[int(e)]] = q
        cursor[int(e)] += 1
    return np.array(perm, dtype=np.int32), np.array(off, dtype=np.int32)
