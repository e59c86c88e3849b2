"""Top-k expert routing and the grouped (expert-sorted) permutation.

The int8 card's model table ("Weights") describes routed experts chosen by a
bf16 router; the cards give neither the top-k rule nor the permutation, so
the readings are:
  * each token t takes the k experts of largest logit, ties going to the
    lower expert index; slot j of token t is the j-th in that order;
  * a NaN logit ranks after every number (-inf included), NaNs among
    themselves by index like any tie, so the ids are always valid experts;
    a token whose chosen logits hold a NaN gets NaN weights;
  * its weights are the softmax over those k logits only (no further
    renormalisation);
  * pair p = t * k + j; experts own contiguous runs of an expert-sorted list
    given by an exclusive scan of the per-expert pair counts, with pairs in
    increasing p inside each run (a stable scatter); pos is the inverse map.
"""

import numpy as np


def topk(logits, k):
    """logits [T, E] float32 -> (ids int32 [T, k], weights fp64 [T, k])."""
    lg = np.asarray(logits, dtype=np.float64)
    t_count, e_count = lg.shape
    ids = np.zeros((t_count, k), dtype=np.int32)
    w = np.zeros((t_count, k), dtype=np.float64)
    experts = np.arange(e_count)
    for t in range(t_count):
        # primary key: larger logit first (NaN last); secondary: lower
        # expert index. NumPy's sorts place NaN after every number.
        order = np.lexsort((experts, -lg[t]))
        sel = order[:k]
        ids[t] = sel
        z = np.exp(lg[t, sel] - lg[t, sel[0]])
        w[t] = z / z.sum()
    return ids, w


def permute(ids, num_experts):
    """ids [T, k] -> (expert_off int32 [E+1], sorted_pairs int32 [P],
    pair_pos int32 [P])."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    p_count = flat.size
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    off = np.zeros(num_experts + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    fill = off[:-1].copy()
    sorted_pairs = np.zeros(p_count, dtype=np.int64)
    for p in range(p_count):                 # increasing p: stable
        e = flat[p]
        sorted_pairs[fill[e]] = p
        fill[e] += 1
    pos = np.zeros(p_count, dtype=np.int64)
    pos[sorted_pairs] = np.arange(p_count)
    return off.astype(np.int32), sorted_pairs.astype(np.int32), pos.astype(np.int32)


def route(logits, k):
    """Everything the routing step produces, as a dict."""
    ids, w = topk(logits, k)
    off, sorted_pairs, pos = permute(ids, np.asarray(logits).shape[1])
    return {"ids": ids, "weights": w, "expert_off": off,
            "sorted_pairs": sorted_pairs, "pair_pos": pos}
