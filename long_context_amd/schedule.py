"""Anchor-layer selection for a layer stack (Kascade abstract on the
opentrain.ai page, "Abstract": anchors chosen by a dynamic-programming
objective that maximises cross-layer similarity over a development set;
summary, "Methodology" step 4: the schedule that maximises the overlap of
top-k sets across layers).

Reading of the pages, made concrete here:
- similarity(a, l), for an anchor layer a <= l, is the mean over units
  (b, KV head[, tile]) of |S_a & S_l| / |S_l|: the share of layer l's own exact
  top-k set that the anchor's set covers (1 when l == a);
- a schedule's score is the sum over layers of the similarity of each layer to
  the nearest preceding anchor; layers before the first anchor attend densely
  and count 1 (exact);
- with M anchors, the best schedule maximises the score.
The top-k sets come from the library's anchor calls on each layer (on the
GPU); this module only compares index sets and runs the dynamic program.
"""
import itertools

import numpy as np


def topk_overlap(idx_anchor, idx_layer):
    """Mean over units of |S_a & S_l| / |S_l| for index arrays [..., k] with -1
    padding (units with an empty S_l are skipped)."""
    a = np.asarray(idx_anchor).reshape(-1, np.asarray(idx_anchor).shape[-1])
    l = np.asarray(idx_layer).reshape(-1, np.asarray(idx_layer).shape[-1])
    if a.shape[0] != l.shape[0]:
        raise ValueError("index arrays must have the same units")
    shares = []
    for ra, rl in zip(a, l):
        sl = rl[rl >= 0]
        if sl.size == 0:
            continue
        shares.append(np.isin(sl, ra[ra >= 0]).sum() / sl.size)
    return float(np.mean(shares)) if shares else 0.0


def similarity_matrix(idx_per_layer):
    """sim[a, l] = topk_overlap(S_a, S_l) for a <= l (1 on the diagonal), 0 below it."""
    n = len(idx_per_layer)
    sim = np.zeros((n, n))
    for a in range(n):
        sim[a, a] = 1.0
        for l in range(a + 1, n):
            sim[a, l] = topk_overlap(idx_per_layer[a], idx_per_layer[l])
    return sim


def schedule_score(sim, anchors):
    """Sum over layers of the similarity to the nearest preceding anchor (1 for
    the dense layers before the first anchor)."""
    sim = np.asarray(sim)
    n = sim.shape[0]
    anchors = sorted(set(anchors))
    score, last = 0.0, None
    for l in range(n):
        if l in anchors:
            last = l
        score += 1.0 if last is None else sim[last, l]
    return score


def dp_anchor_schedule(sim, n_anchors, first=0):
    """Anchor list of n_anchors layers maximising schedule_score.

    Layers 0..first-1 attend densely (a fixed choice of the caller: dense
    layers always score 1, so they are not something to optimise) and the
    first anchor is layer `first`; the other anchors are placed by dynamic
    programming: best[i][m] is the best score of layers i..n-1 when layer i is
    an anchor and m more anchors follow it, layers i..j-1 taking sim[i, l]
    until the next anchor j. O(n^2 * M)."""
    sim = np.asarray(sim, dtype=np.float64)
    n = sim.shape[0]
    if not 0 <= first < n:
        raise ValueError(f"the first anchor must lie in [0, {n})")
    if not 1 <= n_anchors <= n - first:
        raise ValueError(f"need 1 <= n_anchors <= {n - first}")
    # run[i, j] = sum_{l=i}^{j-1} sim[i, l]
    run = np.zeros((n, n + 1))
    for i in range(n):
        run[i, i + 1:] = np.cumsum(sim[i, i:])
    neg = -np.inf
    best = np.full((n, n_anchors), neg)
    nxt = np.full((n, n_anchors), -1, dtype=np.int64)
    for i in range(n - 1, first - 1, -1):
        best[i, 0] = run[i, n]
        for m in range(1, n_anchors):
            for j in range(i + 1, n):
                if best[j, m - 1] == neg:
                    continue
                v = run[i, j] + best[j, m - 1]
                if v > best[i, m]:
                    best[i, m] = v
                    nxt[i, m] = j
    anchors, i, m = [first], first, n_anchors - 1
    while m > 0:
        i = int(nxt[i, m])
        anchors.append(i)
        m -= 1
    return anchors, float(first + best[first, n_anchors - 1])


def brute_force_schedule(sim, n_anchors, first=0):
    """Exhaustive search over anchor sets (small stacks); for checking the DP."""
    n = np.asarray(sim).shape[0]
    best, arg = -np.inf, None
    for combo in itertools.combinations(range(first + 1, n), n_anchors - 1):
        v = schedule_score(sim, (first,) + combo)
        if v > best:
            best, arg = v, [first, *combo]
    return arg, float(best)


def layer_topk_sets(qs, ks, top_k, q_tile=128):
    """Each layer's own exact top-k index sets (an anchor call per layer on the
    GPU, through the library), returned on the host."""
    import torch

    from . import kascade as K
    sets = []
    for q, k in zip(qs, ks):
        if q.shape[2] == 1:
            idx = K.anchor_decode(q, k, None, min(top_k, k.shape[2]))
        else:
            idx = K.anchor_prefill(q, k, None, top_k, q_tile)
        sets.append(idx)
    torch.cuda.synchronize()
    return [s.cpu().numpy() for s in sets]


def select_anchors(qs, ks, top_k, n_anchors, first=0, q_tile=128):
    """Anchor layers for a stack from development inputs: per-layer top-k sets,
    their cross-layer overlaps, and the dynamic program. Returns (anchors,
    score, similarity matrix)."""
    sim = similarity_matrix(layer_topk_sets(qs, ks, top_k, q_tile))
    anchors, score = dp_anchor_schedule(sim, n_anchors, first)
    return anchors, score, sim
