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
  search()    -- the three in a row; returns the map and its figures.

Run as ``python -m layer_wise_mixed_amd.search --hq 32 --hkv 8 --layers 32
--budget 3.25`` to print a map as JSON.
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


def choose(options, budget_total: int):
    """options[l]: list of (bits, err), bits = bK + bV. Returns (choices, total
    error) with sum of bits <= budget_total and the least total error (ties:
    fewer bits, then earlier options), or None if nothing fits."""
    n = len(options)
    B = budget_total
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
    if not np.isfinite(cost).any():
        return None
    b = int(np.argmin(cost))  # the least error; np.argmin takes the fewest bits among equal ones
    total = float(cost[b])
    choices = [0] * n
    for l in range(n - 1, -1, -1):
        i = int(back[l][b])
        choices[l] = i
        b -= options[l][i][0]
    return choices, total


def search(hq: int, hkv: int, num_layers: int, budget: float, pairs=PAIRS, **profile_kw):
    """Profile every layer, prune each layer's pairs, and choose the map.
    Returns a dict: map (one (bK, bV) per layer), equiv_bits, total_error,
    the per-layer kept pair indices and the error table."""
    layers = list(range(num_layers))
    errs = profile(hq, hkv, layers, pairs, **profile_kw)
    bits = [kb + vb for kb, vb in pairs]
    kept = [prune(bits, list(errs[i])) for i in range(num_layers)]
    options = [[(bits[j], float(errs[i, j])) for j in kept[i]] for i in range(num_layers)]
    budget_total = int(math.floor(2 * num_layers * budget + 1e-9))
    res = choose(options, budget_total)
    if res is None:
        raise ValueError(f"budget {budget} bits is below every map of these pairs")
    choices, total = res
    chosen = [pairs[kept[i][c]] for i, c in enumerate(choices)]
    return {"map": [list(p) for p in chosen], "equiv_bits": sum(kb + vb for kb, vb in chosen) / (2 * num_layers),
            "total_error": total, "kept": kept, "errors": errs.tolist(), "pairs": [list(p) for p in pairs]}


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
    args = ap.parse_args(argv)
    t0 = time.perf_counter()
    res = search(args.hq, args.hkv, args.layers, args.budget, batch=args.batch, seq_len=args.seq_len,
                 seed=args.seed, outliers=(int(args.outliers[0]), args.outliers[1]),
                 k_axis=1 if args.per_token_keys else 0)
    res["seconds"] = time.perf_counter() - t0
    print(json.dumps(res))


if __name__ == "__main__":
    sys.exit(main())
