"""Oracle of the per-tag INT2/INT4 allocator.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

What it follows (TriAxialKV page, "Facts"): tokens carry tags; each tag k has
a distortion D_k(b) at b = 2 and b = 4 bits; the allocator gives every tag
INT2 or INT4 under an average-bit budget, by exhaustive search when there are
22 tags or fewer and by a greedy per-bit-gain rule otherwise. Readings taken
where the page is silent: the budget bounds the token-weighted mean bits,
sum_k n_k b_k <= budget * sum_k n_k (n_k = the tag's token count); the
objective is the total distortion sum_k D_k(b_k); exact ties go to fewer
bits, then to the assignment that is smaller as a tuple of bits in tag order.
The greedy rule starts from INT2 everywhere and takes tags in decreasing
order of gain per added bit, (D_k(2) - D_k(4)) / (2 n_k) (ties: lower tag
first), raising each to INT4 if the budget still allows and its gain is
positive.

Functions:
  allocate_exhaustive -- every one of the 2^K assignments
  allocate_greedy     -- the greedy rule above
  allocate            -- exhaustive for K <= 22, greedy above
"""
from __future__ import annotations

import itertools


def _fits(counts, bits, budget) -> bool:
    return sum(n * b for n, b in zip(counts, bits)) <= budget * sum(counts)


def allocate_exhaustive(counts, d2, d4, budget):
    """Returns the list of bits (2 or 4) per tag, or None if even INT2
    everywhere exceeds the budget."""
    best = None
    for bits in itertools.product((2, 4), repeat=len(counts)):
        if not _fits(counts, bits, budget):
            continue
        total = sum(d2[k] if b == 2 else d4[k] for k, b in enumerate(bits))
        key = (total, sum(n * b for n, b in zip(counts, bits)), bits)
        if best is None or key < best:
            best = key
    return None if best is None else list(best[2])


def allocate_greedy(counts, d2, d4, budget):
    K = len(counts)
    bits = [2] * K
    if not _fits(counts, bits, budget):
        return None
    gains = []
    for k in range(K):
        gains.append(((d2[k] - d4[k]) / (2 * counts[k]) if counts[k] > 0 else 0.0, k))
    # decreasing gain, lower tag first among equal gains
    gains.sort(key=lambda g: (-g[0], g[1]))
    for gain, k in gains:
        if gain <= 0:
            break
        trial = list(bits)
        trial[k] = 4
        if _fits(counts, trial, budget):
            bits = trial
    return bits


def allocate(counts, d2, d4, budget):
    if len(counts) <= 22:
        return allocate_exhaustive(counts, d2, d4, budget)
    return allocate_greedy(counts, d2, d4, budget)
