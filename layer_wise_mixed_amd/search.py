"""Offline layer-map search on the library's own kernels.

The static per-layer (bK, bV) map that ``kvq_plan_layers`` takes is searched
offline (KVTuner summary page, "Method": per-layer key and value precisions,
searched offline with intra-layer precision-pair pruning; the result is
applied with no online decision). Here, with no model or dataset:

  profile()   -- each layer's sensitivity to each pair: the relative L2
                 error of its decode-attention output on seeded synthetic
                 q, K, V (the model's head shape, keys with seeded outlier
                 channels), against the same attention on the unquantized
                 fp16 K, V. Every candidate pair and the fp16 reference is a
                 layer of one plan; the cache is filled by
                 ``kvq_quantize_append`` and attended by
                 ``kvq_decode_attention``.
  prune()     -- the pairs of a layer that no other pair of that layer beats
                 on both bits and error (intra-layer Pareto pruning).
  choose()    -- one surviving pair per layer with the least total error
                 whose mean (bK + bV) / 2 is within a bit budget (an exact
                 dynamic program over the integer total of bK + bV).
  frontier()  -- the least total error at every total bit count where it
                 drops: the maps of every budget from one table (the search's
                 two objectives, bits and error).
  cluster_layers(), choose_clustered() -- inter-layer clustering: layers with
                 close error profiles share one pair, which shrinks the
                 search to one choice per cluster.
  search()    -- profile, prune and choose (optionally by clusters); returns
                 the map, its figures and the frontier.

Run as ``python -m layer_wise_mixed_amd.search --hq 32 --hkv 8 --layers 32
--budget 3.25`` to print a map as JSON (``--tau T`` clusters first).
"""
from __future__ import annotations

import argparse
import json
import math
import sys
import time

import numpy as np

from . import decode_attention, load, make_shape, plan_layers, quantize_append, workspace_bytes

PAIRS = [(2, 2), (2, 4), (2, 8), (4, 2), (4, 4), (4, 8), (8, 2), (8, 4), (8, 8)]


def profile(hq: int, hkv: int, layers, pairs=PAIRS, *, k_axis: int = 0, batch: int = 4, seq_len: int = 512,
            seed: int = 0, outliers=(4, 10.0), device="cuda") -> np.ndarray:
    """errors[i][j]: relative L2 error of layer layers[i] under pairs[j]."""
    import torch

    import synthetic as syn

    load()
    cfgs = [(16, 16, 0, 1)] + [(kb, vb, k_axis, 1) for kb, vb in pairs]
    plan = plan_layers(make_shape(hq, hkv, batch, max_tokens=seq_len), cfgs)
    cache = torch.empty(plan.total_bytes, dtype=torch.uint8, device=device)
    lens0 = torch.zeros(batch, dtype=torch.int32, device=device)
    lens = torch.full((batch,), seq_len, dtype=torch.int32, device=device)
    ws = torch.empty(workspace_bytes(plan, batch, seq_len) // 4 + 1, dtype=torch.float32, device=device)
    outs = torch.empty(len(cfgs), batch, hq, 128, dtype=torch.float32, device=device)
    scale = 1.0 / math.sqrt(128.0)
    errors = np.zeros((len(layers), len(pairs)))
    for i, li in enumerate(layers):
        k = syn.keys_fp16(seed, li, range(batch), range(hkv), 0, seq_len, outlier_count=outliers[0],
                          outlier_factor=outliers[1], num_kv_heads=hkv).to(device)
        v = syn.values_fp16(seed, li, range(batch), range(hkv), 0, seq_len).to(device)
        q = syn.queries_fp16(seed, li, 0, batch, hq).to(device)
        for j in range(len(cfgs)):
            quantize_append(plan, j, cache, k, v, lens0)
            decode_attention(plan, j, cache, q, lens, seq_len, scale, outs[j], None, ws)
        o = outs.cpu().numpy().astype(np.float64)
        ref = o[0]
        den = np.sqrt(np.sum(ref * ref))
        for j in range(len(pairs)):
            d = o[j + 1] - ref
            errors[i, j] = np.sqrt(np.sum(d * d)) / den
    return errors


def prune(bits, errs) -> list[int]:
    """Indices (ascending) of the pairs no other pair beats: a pair is dropped
    when another has no more bits and no more error, and strictly less of one.
    One sweep over the pairs sorted by (bits, error)."""
    order = sorted(range(len(bits)), key=lambda i: (bits[i], errs[i]))
    keep = []
    best = math.inf  # least error among strictly fewer bits
    pos = 0
    while pos < len(order):
        end = pos
        while end < len(order) and bits[order[end]] == bits[order[pos]]:
            end += 1
        least = errs[order[pos]]
        if least < best:
            keep += [i for i in order[pos:end] if errs[i] == least]
            best = least
        pos = end
    return sorted(keep)


def _table(options, B: int):
    """cost[b]: the least error of all layers spending exactly b bits (inf if
    none), with per-layer back pointers."""
    n = len(options)
    inf = math.inf
    # cost[b]: least error of layers 0..l-1 spending exactly b bits
    cost = np.full(B + 1, inf)
    cost[0] = 0.0
    back = []
    for l in range(n):
        new = np.full(B + 1, inf)
        pick = np.full(B + 1, -1, dtype=np.int64)
        for i, (bits, err) in enumerate(options[l]):
            if bits > B:
                continue
            cand = np.full(B + 1, inf)
            cand[bits:] = cost[:B + 1 - bits] + err
            better = cand < new
            new[better] = cand[better]
            pick[better] = i
        cost = new
        back.append(pick)
    return cost, back


def _walk_back(options, back, b: int):
    choices = [0] * len(options)
    for l in range(len(options) - 1, -1, -1):
        i = int(back[l][b])
        choices[l] = i
        b -= options[l][i][0]
    return choices


def choose(options, budget_total: int):
    """options[l]: list of (bits, err), bits = bK + bV. Returns (choices, total
    error) with sum of bits <= budget_total and the least total error (ties:
    fewer bits, then earlier options), or None if nothing fits."""
    cost, back = _table(options, budget_total)
    if not np.isfinite(cost).any():
        return None
    b = int(np.argmin(cost))  # the least error; np.argmin takes the fewest bits among equal ones
    return _walk_back(options, back, b), float(cost[b])


def frontier(options):
    """Maps for every budget at once (the two objectives of the search: total
    bits and total error): [(total bits, least total error, choices)] at every
    total bit count where the least error drops below that of all smaller
    counts, ascending. One table serves every budget."""
    B = sum(max(b for b, _ in o) for o in options)
    cost, back = _table(options, B)
    out = []
    best = math.inf
    for b in range(B + 1):
        if cost[b] < best:
            best = float(cost[b])
            out.append((b, best, _walk_back(options, back, b)))
    return out


def cluster_layers(errors, tau: float):
    """Inter-layer clustering (KVTuner summary page, "Method"): layers whose
    error profiles over the pairs are close share one pair. Distance of two
    layers: the largest difference of their log errors; clusters: complete
    linkage, merged while the closest two are at most tau apart. Returns
    sorted lists of layer indices, ordered by their first layer."""
    from scipy.cluster.hierarchy import fcluster, linkage

    e = np.log(np.maximum(np.asarray(errors, dtype=np.float64), 1e-300))
    if len(e) == 1:
        return [[0]]
    labels = fcluster(linkage(e, method="complete", metric="chebyshev"), t=tau, criterion="distance")
    groups = {}
    for l, lab in enumerate(labels):
        groups.setdefault(int(lab), []).append(l)
    return sorted(groups.values(), key=lambda c: c[0])


def choose_clustered(errors, bits, clusters, budget_total: int):
    """One pair per cluster, every layer of a cluster taking it: the least
    total error within budget_total bits (the clusters' pairs pruned first).
    Returns (pair index per layer, total error) or None."""
    errors = np.asarray(errors, dtype=np.float64)
    kept, options = [], []
    for c in clusters:
        cb = [len(c) * b for b in bits]
        ce = [float(errors[c, p].sum()) for p in range(len(bits))]
        k = prune(cb, ce)
        kept.append(k)
        options.append([(cb[p], ce[p]) for p in k])
    res = choose(options, budget_total)
    if res is None:
        return None
    per_layer = [0] * len(errors)
    for c, k, i in zip(clusters, kept, res[0]):
        for l in c:
            per_layer[l] = k[i]
    return per_layer, res[1]


def search(hq: int, hkv: int, num_layers: int, budget: float, pairs=PAIRS, tau=None, **profile_kw):
    """Profile every layer, prune each layer's pairs, and choose the map
    (with tau: one pair per cluster of layers within tau of each other).
    Returns a dict: map (one (bK, bV) per layer), equiv_bits, total_error,
    the per-layer kept pair indices, the clusters, the error table and the
    per-layer frontier [(equiv bits, total error)]."""
    layers = list(range(num_layers))
    errs = profile(hq, hkv, layers, pairs, **profile_kw)
    bits = [kb + vb for kb, vb in pairs]
    kept = [prune(bits, list(errs[i])) for i in range(num_layers)]
    options = [[(bits[j], float(errs[i, j])) for j in kept[i]] for i in range(num_layers)]
    budget_total = int(math.floor(2 * num_layers * budget + 1e-9))
    clusters = None
    if tau is None:
        res = choose(options, budget_total)
        if res is not None:
            res = ([kept[i][c] for i, c in enumerate(res[0])], res[1])
    else:
        clusters = cluster_layers(errs, tau)
        res = choose_clustered(errs, bits, clusters, budget_total)
    if res is None:
        raise ValueError(f"budget {budget} bits is below every map of these pairs")
    chosen = [pairs[p] for p in res[0]]
    front = [(b / (2 * num_layers), e) for b, e, _ in frontier(options)]
    return {"map": [list(p) for p in chosen], "equiv_bits": sum(kb + vb for kb, vb in chosen) / (2 * num_layers),
            "total_error": res[1], "kept": kept, "clusters": clusters, "errors": errs.tolist(),
            "pairs": [list(p) for p in pairs], "frontier": front}


def main(argv=None):
    ap = argparse.ArgumentParser(description="search a per-layer (bK, bV) map on synthetic inputs")
    ap.add_argument("--hq", type=int, default=32)
    ap.add_argument("--hkv", type=int, default=8)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--budget", type=float, default=3.25, help="mean of (bK + bV) / 2 over layers, at most")
    ap.add_argument("--batch", type=int, default=4)
    ap.add_argument("--seq-len", type=int, default=512)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--outliers", type=float, nargs=2, default=(4, 10.0), metavar=("COUNT", "FACTOR"))
    ap.add_argument("--per-token-keys", action="store_true")
    ap.add_argument("--tau", type=float, default=None, help="cluster layers within this log-error distance")
    args = ap.parse_args(argv)
    t0 = time.perf_counter()
    res = search(args.hq, args.hkv, args.layers, args.budget, tau=args.tau, batch=args.batch, seq_len=args.seq_len,
                 seed=args.seed, outliers=(int(args.outliers[0]), args.outliers[1]),
                 k_axis=1 if args.per_token_keys else 0)
    res["seconds"] = time.perf_counter() - t0
    print(json.dumps(res))


if __name__ == "__main__":
    sys.exit(main())
