"""The per-tag INT2/INT4 allocator: oracle pins, and the library's allocator against the oracle.

Pins of the oracle: with equal token counts the budget admits a number of INT4 tags and the
optimum takes the tags whose INT2 -> INT4 saving is largest (the objective is separable and the
constraint a cardinality bound), which also makes the greedy rule optimal there; hand cases fix
the budget's edges and a knapsack case where the greedy rule, as stated, is not optimal.
Distortions lie on a 1/1024 grid so every sum is exact and ties are decided alike."""
import numpy as np
import pytest

from layer_wise_mixed_amd import allocate as lib_alloc
from oracle import allocate as oalloc


def test_budget_edges():
    counts, d2, d4 = [10, 10, 10], [0.5, 0.25, 0.75], [0.125, 0.125, 0.125]
    assert oalloc.allocate_exhaustive(counts, d2, d4, 1.99) is None
    assert oalloc.allocate_exhaustive(counts, d2, d4, 2.0) == [2, 2, 2]
    assert oalloc.allocate_exhaustive(counts, d2, d4, 4.0) == [4, 4, 4]
    # room for one INT4 tag (mean 2 + 2/3): the one that saves most, tag 2
    assert oalloc.allocate_exhaustive(counts, d2, d4, 2.0 + 2 / 3) == [2, 2, 4]
    # a tag that INT4 does not help stays INT2 (fewer bits at the same distortion)
    assert oalloc.allocate_exhaustive([5, 5], [0.25, 0.5], [0.25, 0.25], 4.0) == [2, 4]


@pytest.mark.parametrize("seed", range(15))
def test_equal_counts_take_the_largest_savings(seed):
    rng = np.random.default_rng(seed)
    K = int(rng.integers(1, 9))
    d4 = rng.integers(0, 256, K) / 1024
    d2 = d4 + rng.permutation(np.arange(1, K + 1)) / 64  # distinct savings
    m = int(rng.integers(0, K + 1))
    budget = 2 + 2 * m / K
    want = [4 if k in set(np.argsort(-(d2 - d4))[:m]) else 2 for k in range(K)]
    counts = [7] * K
    assert oalloc.allocate_exhaustive(counts, list(d2), list(d4), budget) == want
    assert oalloc.allocate_greedy(counts, list(d2), list(d4), budget) == want


def test_greedy_follows_its_rule_where_it_is_not_optimal():
    # gain per added bit: tag 0 0.625 / 20, tag 1 0.5 / 20, tag 2 0.4375 / 20; room for 20
    # extra token-bits over the 60 of INT2 everywhere: tag 0 only
    counts, d2, d4 = [10, 10, 10], [0.625, 0.5, 0.4375], [0.0, 0.0, 0.0]
    assert oalloc.allocate_greedy(counts, d2, d4, 2 + 20 / 30) == [4, 2, 2]
    # a knapsack where the best single tag beats the greedy pick: 20 token-bits to add; greedy
    # takes tag 1 (gain 0.5/8 per bit, +8), then neither tag 0 (+20) nor tag 2 (+14) fits;
    # the optimum spends all 20 on tag 0
    counts, d2, d4 = [10, 4, 7], [1.0, 0.5, 0.125], [0.0, 0.0, 0.0]
    budget = 2 + 2 * 10 / 21
    assert oalloc.allocate_greedy(counts, d2, d4, budget) == [2, 4, 2]
    assert oalloc.allocate_exhaustive(counts, d2, d4, budget) == [4, 2, 2]


def _instance(rng, K):
    counts = [int(c) for c in rng.integers(1, 200, K)]
    d4 = rng.integers(0, 512, K) / 1024
    d2 = d4 + rng.integers(0, 512, K) / 1024
    budget = float(rng.choice([2.0, 2.5, 3.0, 3.25, 3.5, 4.0])) - float(rng.integers(0, 2)) * 0.125
    return counts, list(d2), list(d4), budget


@pytest.mark.parametrize("seed", range(25))
def test_library_exhaustive_equals_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    counts, d2, d4, budget = _instance(rng, int(rng.integers(1, 11)))
    assert lib_alloc.allocate(counts, d2, d4, budget) == oalloc.allocate_exhaustive(counts, d2, d4, budget)


@pytest.mark.parametrize("seed", range(10))
def test_library_greedy_equals_oracle(seed):
    rng = np.random.default_rng(2000 + seed)
    counts, d2, d4, budget = _instance(rng, int(rng.integers(23, 57)))  # 56 = 4 x 2 x 7 tag values
    assert lib_alloc.allocate(counts, d2, d4, budget) == oalloc.allocate_greedy(counts, d2, d4, budget)


def test_library_exhaustive_at_22_tags():
    rng = np.random.default_rng(7)
    counts, d2, d4, budget = _instance(rng, 22)
    bits = lib_alloc.allocate(counts, d2, d4, 3.0)
    assert bits is not None and sum(n * b for n, b in zip(counts, bits)) <= 3.0 * sum(counts)
    # no single change of one tag improves it within the budget
    def total(bs):
        return sum(d2[k] if b == 2 else d4[k] for k, b in enumerate(bs))
    for k in range(22):
        alt = list(bits)
        alt[k] = 6 - alt[k]
        if sum(n * b for n, b in zip(counts, alt)) <= 3.0 * sum(counts):
            assert total(alt) >= total(bits)


def test_int2_tokens_whole_runs_and_leftovers():
    tags = [0] * 40 + [1] * 10 + [0] * 30 + [2] * 5
    int2, int4 = lib_alloc.int2_tokens(tags, [2, 4, 2])
    # tag 0 and 2 tokens in arrival order: 0..39, 50..79, 80..84 -> 75 of them, 64 in two runs
    cand = list(range(40)) + list(range(50, 85))
    assert int2 == cand[:64]
    assert int4 == sorted(set(range(85)) - set(cand[:64]))
    assert len(int2) % 32 == 0
    int2, int4 = lib_alloc.int2_tokens([1] * 20, [2, 4])
    assert int2 == [] and int4 == list(range(20))
