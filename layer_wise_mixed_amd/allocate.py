"""INT2/INT4 allocation per token tag under an average-bit budget.

TriAxialKV page, "Facts": tokens carry tags (temporal, modal and semantic
roles); each tag k has a distortion D_k(b) at b = 2 and 4 bits; the allocator
gives every tag INT2 or INT4 under an average-bit budget, exhaustively for up
to 22 tags and by a greedy per-bit-gain rule beyond. Its result says which
tokens the paged pool stores as INT2 (whole 32-token runs of INT2 tags) and
which as INT4.

Conventions (the page leaves them open): the budget bounds the
token-weighted mean, sum_k n_k b_k <= budget * sum_k n_k, with n_k the
tag's token count; the objective is the total distortion sum_k D_k(b_k);
exact ties go to fewer bits, then to the assignment that is smaller as a
tuple of bits in tag order. Greedy: INT2 everywhere, then tags in decreasing
order of gain per added bit (D_k(2) - D_k(4)) / (2 n_k) (ties: lower tag
first), each raised to INT4 when the budget still allows and its gain is
positive.
"""
from __future__ import annotations

import numpy as np

EXHAUSTIVE_MAX_TAGS = 22
_CHUNK = 1 << 16


def _exhaustive(n, d2, d4, budget):
    K = len(n)
    limit = budget * n.sum()
    base_bits = 2.0 * n.sum()
    base_dist = d2.sum()
    step_bits = 2.0 * n          # INT4 instead of INT2
    step_dist = d4 - d2
    best = None                  # (dist, bits, masks with that pair)
    weights = 1 << np.arange(K, dtype=np.int64)
    for start in range(0, 1 << K, _CHUNK):
        masks = np.arange(start, min(start + _CHUNK, 1 << K), dtype=np.int64)
        sel = ((masks[:, None] & weights[None, :]) != 0).astype(np.float64)
        bits = base_bits + sel @ step_bits
        ok = bits <= limit
        if not ok.any():
            continue
        dist = base_dist + sel @ step_dist
        dist_ok = np.where(ok, dist, np.inf)
        dmin = dist_ok.min()
        cand = ok & (dist_ok == dmin)
        bmin = bits[cand].min()
        cand &= bits == bmin
        key = (dmin, bmin)
        if best is None or key < best[:2]:
            best = (dmin, bmin, list(masks[cand]))
        elif key == best[:2]:
            best[2].extend(masks[cand])
    if best is None:
        return None
    # the smallest tuple of bits in tag order: compare tag 0's bit first
    mask = min(best[2], key=lambda m: [(int(m) >> k) & 1 for k in range(K)])
    return [4 if (int(mask) >> k) & 1 else 2 for k in range(K)]


def _greedy(n, d2, d4, budget):
    K = len(n)
    limit = budget * n.sum()
    used = 2.0 * n.sum()
    if used > limit:
        return None
    gain = np.where(n > 0, (d2 - d4) / np.where(n > 0, 2.0 * n, 1.0), 0.0)
    order = np.lexsort((np.arange(K), -gain))  # decreasing gain, then lower tag
    bits = [2] * K
    for k in order:
        if gain[k] <= 0:
            break
        if used + 2.0 * n[k] <= limit:
            bits[int(k)] = 4
            used += 2.0 * n[k]
    return bits


def allocate(counts, d2, d4, budget: float):
    """counts: tokens per tag; d2, d4: each tag's distortion at INT2 and INT4;
    budget: the largest token-weighted mean bits. Returns a list of 2 or 4 per
    tag, or None when even INT2 everywhere exceeds the budget."""
    n = np.asarray(counts, dtype=np.float64)
    a = np.asarray(d2, dtype=np.float64)
    b = np.asarray(d4, dtype=np.float64)
    if len(n) <= EXHAUSTIVE_MAX_TAGS:
        return _exhaustive(n, a, b, budget)
    return _greedy(n, a, b, budget)


def int2_tokens(tags, bits_per_tag):
    """Which tokens of one request the paged pool stores as INT2, given each
    token's tag (arrival order) and the allocation: the tokens of INT2 tags,
    taken in arrival order in runs of 32 (a key group spans 32 tokens); the
    last len % 32 of them go through the INT4 per-token path with every
    other token (TriAxialKV page, "Facts": leftover INT2 tokens take the INT4
    path). Returns (int2 token indices, a multiple of 32 long; INT4 token
    indices), both in arrival order."""
    tags = np.asarray(tags)
    is2 = np.asarray(bits_per_tag)[tags] == 2
    cand = np.flatnonzero(is2)
    n2 = len(cand) - len(cand) % 32
    int2 = cand[:n2]
    rest = np.ones(len(tags), dtype=bool)
    rest[int2] = False
    return int2.tolist(), np.flatnonzero(rest).tolist()
