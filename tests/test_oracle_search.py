"""Pins of the search oracle (oracle/search.py) and the library's host-side search logic.

The oracle's pruning is the pairwise definition of dominance, pinned by hand cases and by the
two properties that define a Pareto front; its budgeted choice is checked against exhaustive
enumeration of every map on small instances (errors are multiples of 1/1024, so every sum is
exact and ties are decided the same way); its layer error reduces to zero where the pages fix
the result (fp16 pairs, and streams shorter than one group, which stay fp16), does not depend
on the key pair when q = 0, and for q = 0 over one group equals the mean of the values
dequantized by the group quantizer alone. The library's prune() and choose() are then checked
against the oracle on random instances."""
import itertools
import math

import numpy as np
import pytest

import synthetic as syn
from layer_wise_mixed_amd import search as lib_search
from oracle import search as osearch

SCALE = 1 / math.sqrt(128)


def test_pareto_hand_case():
    pts = [(4, 0.5), (6, 0.2), (6, 0.3), (8, 0.2), (3, 0.9), (4, 0.5)]
    # (6, 0.3) and (8, 0.2) are beaten by (6, 0.2); the two (4, 0.5) tie and both stay
    assert osearch.pareto_front(pts) == [0, 1, 4, 5]
    assert osearch.pareto_front([(4, 0.1)]) == [0]
    assert osearch.pareto_front([(4, 0.1), (4, 0.1)]) == [0, 1]
    assert osearch.pareto_front([(2, 0.3), (4, 0.3)]) == [0]  # same error, more bits: dropped


def _random_points(rng, n):
    return [(int(rng.integers(1, 9)) * 2, float(rng.integers(0, 6)) / 8) for _ in range(n)]


@pytest.mark.parametrize("seed", range(20))
def test_pareto_front_properties(seed):
    rng = np.random.default_rng(seed)
    pts = _random_points(rng, int(rng.integers(1, 12)))
    front = osearch.pareto_front(pts)
    assert front, "a non-empty set has a front"
    for i in front:
        assert not any(osearch.dominates(p, pts[i]) for p in pts)
    for i in set(range(len(pts))) - set(front):
        assert any(osearch.dominates(pts[j], pts[i]) for j in front)


def _exhaustive(options, budget):
    best = None
    for choice in itertools.product(*[range(len(o)) for o in options]):
        bits = sum(options[l][c][0] for l, c in enumerate(choice))
        if bits > budget:
            continue
        err = sum(options[l][c][1] for l, c in enumerate(choice))
        key = (err, bits, choice)
        if best is None or key < best:
            best = key
    return best


@pytest.mark.parametrize("seed", range(30))
def test_best_map_matches_exhaustive(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 5))
    options = [[(int(rng.choice([4, 6, 8, 10, 12, 16])), int(rng.integers(0, 64)) / 1024)
                for _ in range(int(rng.integers(1, 6)))] for _ in range(L)]
    budget = int(rng.integers(4 * L - 2, 16 * L + 2))
    want = _exhaustive(options, budget)
    got = osearch.best_map(options, budget)
    if want is None:
        assert got is None
        return
    choice, total = got
    assert tuple(choice) == want[2] and total == want[0]


def test_best_map_infeasible_and_exact_budget():
    options = [[(8, 0.5), (16, 0.0)], [(8, 0.25), (16, 0.0)]]
    assert osearch.best_map(options, 15) is None
    assert osearch.best_map(options, 16) == ([0, 0], 0.75)
    assert osearch.best_map(options, 24) == ([1, 0], 0.25)  # the larger saving goes first
    assert osearch.best_map(options, 32) == ([1, 1], 0.0)


def _inputs(seed, batch, hq, hkv, L, layer=0):
    k = syn.keys_fp16(seed, layer, range(batch), range(hkv), 0, L, num_kv_heads=hkv).numpy()
    v = syn.values_fp16(seed, layer, range(batch), range(hkv), 0, L).numpy()
    q = syn.queries_fp16(seed, layer, 0, batch, hq).numpy()
    return q, k, v


def test_layer_error_fp16_pair_and_short_streams_are_exact(oq):
    q, k, v = _inputs(1, 2, 4, 2, 80)
    assert osearch.layer_error(q, k, v, 16, 16, False, SCALE) == 0.0
    q, k, v = _inputs(1, 2, 4, 2, 31)  # fewer than a group: every token stays fp16
    for kb, vb in [(2, 2), (4, 8), (8, 4)]:
        assert osearch.layer_error(q, k, v, kb, vb, False, SCALE) == 0.0


def test_layer_error_ignores_keys_when_q_is_zero(oq):
    q, k, v = _inputs(2, 2, 4, 2, 96)
    q0 = np.zeros_like(q)
    e = [osearch.layer_error(q0, k, v, kb, 4, False, SCALE) for kb in (2, 4, 8)]
    assert e[0] == e[1] == e[2] > 0.0


def test_layer_error_one_group_q_zero_is_mean_of_dequantized_values(oq):
    """q = 0 over exactly 32 tokens: attention is the mean of the dequantized values, and the
    values are quantized per token and 32-channel group by the group quantizer alone."""
    batch, hq, hkv, L, vb = 1, 2, 1, 32, 2
    q, k, v = _inputs(3, batch, hq, hkv, L)
    q0 = np.zeros_like(q)
    got = osearch.layer_error(q0, k, v, 8, vb, False, SCALE)
    deq = np.zeros((L, 128))
    for j in range(L):
        for n in range(4):
            s, z, codes = oq.quantize_group(v[0, 0, j, 32 * n:32 * n + 32], vb)
            deq[j, 32 * n:32 * n + 32] = [float(oq.dequant(int(c), s, z)) for c in codes]
    mean_q = deq.mean(axis=0)
    mean_ref = v[0, 0].astype(np.float64).mean(axis=0)
    want = np.linalg.norm(np.tile(mean_q - mean_ref, hq)) / np.linalg.norm(np.tile(mean_ref, hq))
    assert got == pytest.approx(want, rel=1e-12)


def test_layer_error_wide_pairs_beat_narrow(oq):
    """Directional: on keys with outlier channels, K8V8 loses less than K2V2."""
    q, k, v = _inputs(4, 2, 4, 2, 128)
    assert osearch.layer_error(q, k, v, 8, 8, False, SCALE) < osearch.layer_error(q, k, v, 2, 2, False, SCALE)


# ------------------------------------------------ the library's host-side search logic


@pytest.mark.parametrize("seed", range(20))
def test_library_prune_equals_oracle(seed):
    rng = np.random.default_rng(500 + seed)
    pts = _random_points(rng, int(rng.integers(1, 14)))
    bits, errs = [p[0] for p in pts], [p[1] for p in pts]
    assert lib_search.prune(bits, errs) == osearch.pareto_front(pts)


@pytest.mark.parametrize("seed", range(20))
def test_library_choose_equals_oracle(seed):
    rng = np.random.default_rng(900 + seed)
    L = int(rng.integers(1, 9))
    options = [[(int(rng.choice([4, 6, 8, 10, 12, 16])), int(rng.integers(0, 64)) / 1024)
                for _ in range(int(rng.integers(1, 6)))] for _ in range(L)]
    budget = int(rng.integers(4 * L - 2, 16 * L + 2))
    want = osearch.best_map(options, budget)
    got = lib_search.choose(options, budget)
    if want is None:
        assert got is None
        return
    # the same least error and, among maps with it, the same least bit total
    assert got[1] == want[1]
    bits = lambda ch: sum(options[l][c][0] for l, c in enumerate(ch))
    assert bits(got[0]) == bits(want[0]) <= budget
    assert sum(options[l][c][1] for l, c in enumerate(got[0])) == got[1]


# ------------------------------------------------ frontier and inter-layer clustering


def _brute_frontier(options):
    pts = {}
    for choice in itertools.product(*[range(len(o)) for o in options]):
        b = sum(options[l][c][0] for l, c in enumerate(choice))
        e = sum(options[l][c][1] for l, c in enumerate(choice))
        pts[b] = min(pts.get(b, math.inf), e)
    out, best = [], math.inf
    for b in sorted(pts):
        if pts[b] < best:
            best = pts[b]
            out.append((b, best))
    return out


@pytest.mark.parametrize("seed", range(15))
def test_frontier_matches_brute_force(seed):
    rng = np.random.default_rng(3000 + seed)
    L = int(rng.integers(1, 5))
    options = [[(int(rng.choice([4, 6, 8, 10, 12, 16])), int(rng.integers(0, 64)) / 1024)
                for _ in range(int(rng.integers(1, 5)))] for _ in range(L)]
    want = _brute_frontier(options)
    got = osearch.frontier(options)
    assert [(b, e) for b, e, _ in got] == want
    for b, e, ch in got:
        assert sum(options[l][c][0] for l, c in enumerate(ch)) == b
        assert sum(options[l][c][1] for l, c in enumerate(ch)) == e
    lib = lib_search.frontier(options)
    assert [(b, e) for b, e, _ in lib] == want


def _profiles(rng, L, P=9):
    return np.exp(rng.normal(-3.0, 1.0, (L, P)))


def test_clustering_hand_cases():
    base = np.array([0.01, 0.02, 0.05, 0.1])
    errs = np.stack([base, base, base * 1.05, base * 3.0, base * 3.1])
    # log distances: layers 0, 1 identical; 2 is log(1.05) = 0.049 away; 3, 4 are log(3.1/3) = 0.033 apart
    assert osearch.cluster_layers(errs, 0.0) == [[0, 1], [2], [3], [4]]
    assert osearch.cluster_layers(errs, 0.04) == [[0, 1], [2], [3, 4]]
    assert osearch.cluster_layers(errs, 0.1) == [[0, 1, 2], [3, 4]]
    assert osearch.cluster_layers(errs, 10.0) == [[0, 1, 2, 3, 4]]
    for tau in (0.0, 0.04, 0.1, 10.0):
        assert lib_search.cluster_layers(errs, tau) == osearch.cluster_layers(errs, tau)


@pytest.mark.parametrize("seed", range(12))
def test_clusters_are_tight_and_separated(seed):
    rng = np.random.default_rng(4000 + seed)
    errs = _profiles(rng, int(rng.integers(2, 9)))
    tau = float(rng.uniform(0.5, 3.0))
    cl = osearch.cluster_layers(errs, tau)
    assert sorted(l for c in cl for l in c) == list(range(len(errs)))
    diam = lambda c: max((osearch.layer_distance(errs[i], errs[j]) for i in c for j in c), default=0.0)
    for c in cl:
        assert diam(c) <= tau
    for a in range(len(cl)):
        for b in range(a + 1, len(cl)):
            assert diam(cl[a] + cl[b]) > tau  # the agglomeration stopped: no two clusters fit together
    assert lib_search.cluster_layers(errs, tau) == cl


@pytest.mark.parametrize("seed", range(12))
def test_clustered_map_matches_brute_force(seed):
    rng = np.random.default_rng(5000 + seed)
    L = int(rng.integers(2, 6))
    errs = np.round(_profiles(rng, L, 4) * 1024) / 1024 + 1 / 1024
    bits = [4, 6, 8, 12]
    clusters = osearch.cluster_layers(errs, float(rng.uniform(0.2, 2.0)))
    budget = int(rng.integers(4 * L, 12 * L + 1))
    best = None
    for choice in itertools.product(range(len(bits)), repeat=len(clusters)):
        per = [0] * L
        for c, p in zip(clusters, choice):
            for l in c:
                per[l] = p
        b = sum(bits[p] for p in per)
        if b > budget:
            continue
        e = sum(errs[l][p] for l, p in enumerate(per))
        if best is None or (e, b) < best[:2]:
            best = (e, b, per)
    got = osearch.best_clustered_map(errs, bits, clusters, budget)
    lib = lib_search.choose_clustered(errs, bits, clusters, budget)
    if best is None:
        assert got is None and lib is None
        return
    for res in (got, lib):
        per, e = res
        assert e == best[0] and sum(bits[p] for p in per) == best[1]
        for c in clusters:
            assert len({per[l] for l in c}) == 1  # one pair per cluster


def test_singleton_clusters_equal_the_per_layer_choice():
    rng = np.random.default_rng(6)
    errs = np.round(_profiles(rng, 5, 4) * 1024) / 1024 + 1 / 1024
    bits = [4, 6, 8, 12]
    options = [[(bits[p], errs[l][p]) for p in range(4)] for l in range(5)]
    want = osearch.best_map(options, 35)
    got = osearch.best_clustered_map(errs, bits, [[l] for l in range(5)], 35)
    assert got[1] == want[1] and got[0] == want[0]
