"""Oracle of the offline layer-map search: per-layer sensitivity on synthetic
inputs, intra-layer Pareto pruning of (bK, bV) pairs, and the budgeted choice
of one pair per layer.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only the tests import
it. It shares no code with the library's search (``layer_wise_mixed_amd/
search.py``), which runs the HIP kernels.

What it follows (KVTuner summary page, "Method"; abstract page): keys and
values of each layer get their own precision, chosen offline as a static
per-layer map; the search space is shrunk by intra-layer precision-pair
pruning (a pair that costs more bits and loses more accuracy than another
pair of the same layer is dropped). Readings taken where the pages are
silent (the pages calibrate on model accuracy, which needs models and
datasets): a layer's sensitivity to a pair is the relative L2 error of its
decode-attention output on seeded synthetic q, K, V against attention on the
unquantized fp16 K, V; a pair costs bK + bV bits per element pair (the map's
equivalent precision is the mean of (bK + bV) / 2); the map minimises the sum
of the layer errors with the mean of (bK + bV) / 2 at most the budget.

Functions:
  layer_error  -- relative L2 error of one layer, every (request, KV head)
                  stream quantized and attended by the oracle (fp64)
  pareto_front -- the non-dominated pairs of one layer, by the pairwise
                  definition of dominance
  best_map     -- one option per layer, minimum total error under a total
                  bit budget, by the plain recursion over layers and budget
  frontier     -- the least total error at every total bit count where it
                  drops (best_map at every budget)
  cluster_layers, best_clustered_map -- inter-layer clustering by complete
                  linkage on log errors, and one pair per cluster
"""
from __future__ import annotations

import math

import numpy as np

from . import attention, decode_stream


def layer_error(q_fp16, k_fp16, v_fp16, kb: int, vb: int, k_token: bool, scale: float) -> float:
    """q: fp16 [batch, Hq, 128]; k, v: fp16 [batch, Hkv, L, 128]. Returns
    sqrt(sum |o_pair - o_fp16|^2) / sqrt(sum |o_fp16|^2) over all rows."""
    q = np.asarray(q_fp16)
    k = np.asarray(k_fp16)
    v = np.asarray(v_fp16)
    batch, hq = q.shape[0], q.shape[1]
    hkv = k.shape[1]
    g = hq // hkv
    num = 0.0
    den = 0.0
    for r in range(batch):
        for h in range(hkv):
            rows = q[r, h * g:(h + 1) * g]
            o_pair, _ = decode_stream(rows, k[r, h], v[r, h], kb, vb, k_token, scale)
            o_ref, _ = attention(rows, k[r, h].astype(np.float64), v[r, h].astype(np.float64), scale)
            num += float(np.sum((o_pair - o_ref) ** 2))
            den += float(np.sum(o_ref ** 2))
    return math.sqrt(num) / math.sqrt(den)


def dominates(a, b) -> bool:
    """Point a = (bits, err) dominates b: no more bits, no more error, and
    strictly less of one of them."""
    return a[0] <= b[0] and a[1] <= b[1] and (a[0] < b[0] or a[1] < b[1])


def pareto_front(points) -> list[int]:
    """Indices (ascending) of the points no other point dominates."""
    return [i for i, p in enumerate(points)
            if not any(dominates(o, p) for j, o in enumerate(points) if j != i)]


def best_map(options, budget: int):
    """options[l]: list of (bits, err) of layer l, bits a non-negative int;
    budget: the most total bits. Returns (choice list, total error), choice[l]
    an index into options[l], minimising the total error; among equal totals
    the smaller bit sum, then the earlier options. None if no choice fits."""
    n = len(options)
    memo = {}

    def solve(l, left):
        # best (error, bits, choices) for layers l.. with `left` bits to spend
        if l == n:
            return (0.0, 0, ())
        key = (l, left)
        if key in memo:
            return memo[key]
        best = None
        for i, (bits, err) in enumerate(options[l]):
            if bits > left:
                continue
            rest = solve(l + 1, left - bits)
            if rest is None:
                continue
            cand = (err + rest[0], bits + rest[1], (i,) + rest[2])
            if best is None or cand[:2] < best[:2] or (cand[:2] == best[:2] and cand[2] < best[2]):
                best = cand
        memo[key] = best
        return best

    res = solve(0, budget)
    if res is None:
        return None
    return list(res[2]), res[0]


# ---------------------------------------------------------------------------
# Maps for every budget, and inter-layer clustering (KVTuner summary page,
# "Method": a multi-objective search over per-layer pairs, with inter-layer
# clustering shrinking its space). Readings: the two objectives are the total
# bits and the total error, and the frontier is every total bit count whose
# least error is below that of every smaller count; two layers' distance is
# the largest difference of their log errors over the pairs; clusters are
# formed by complete-linkage agglomeration while the closest two clusters are
# at most tau apart (the distance of two clusters: the largest distance
# between their members); a cluster takes one pair for all its layers.

def frontier(options):
    """[(total bits, least total error, choice)] for every total bit count
    at which the least error (at most that many bits) drops, ascending."""
    lo = sum(min(b for b, _ in o) for o in options)
    hi = sum(max(b for b, _ in o) for o in options)
    out = []
    for b in range(lo, hi + 1):
        res = best_map(options, b)
        if res is None:
            continue
        bits = sum(options[l][c][0] for l, c in enumerate(res[0]))
        if bits != b:
            continue  # the least error at this budget was already reached with fewer bits
        if not out or res[1] < out[-1][1]:
            out.append((b, res[1], res[0]))
    return out


def layer_distance(e1, e2) -> float:
    return max(abs(math.log(max(a, 1e-300)) - math.log(max(b, 1e-300))) for a, b in zip(e1, e2))


def cluster_layers(errors, tau: float):
    """errors[l][p]: layer l's error under pair p. Returns clusters as sorted
    lists of layer indices, ordered by their first layer."""
    clusters = [[l] for l in range(len(errors))]

    def diameter(c):
        return max((layer_distance(errors[i], errors[j]) for i in c for j in c), default=0.0)

    while len(clusters) > 1:
        best = None
        for a in range(len(clusters)):
            for b in range(a + 1, len(clusters)):
                d = diameter(clusters[a] + clusters[b])
                if best is None or d < best[0]:
                    best = (d, a, b)
        if best[0] > tau:
            break
        _, a, b = best
        merged = sorted(clusters[a] + clusters[b])
        clusters = [c for k, c in enumerate(clusters) if k not in (a, b)] + [merged]
        clusters.sort(key=lambda c: c[0])
    return clusters


def best_clustered_map(errors, bits, clusters, budget: int):
    """One pair per cluster (every layer of a cluster takes it): the least
    total error with at most `budget` total bits. Returns (pair index per
    layer, total error) or None."""
    options = [[(len(c) * bits[p], sum(errors[l][p] for l in c)) for p in range(len(bits))] for c in clusters]
    res = best_map(options, budget)
    if res is None:
        return None
    per_layer = [0] * len(errors)
    for c, p in zip(clusters, res[0]):
        for l in c:
            per_layer[l] = p
    return per_layer, res[1]
