"""GPU parity of the offline layer-map search (layer_wise_mixed_amd/search.py): the layer
errors the library measures with its own append and decode kernels against the oracle's
(oracle/search.py, fp64 attention on its own quantization of the same seeded inputs), and the
map it chooses against the oracle's pruning and budgeted choice on the oracle's errors."""
import math

import numpy as np
import pytest

import synthetic as syn
from oracle import search as osearch

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(128)
HQ, HKV, BATCH, SEQ = 8, 2, 2, 200  # six full groups and an 8-token fp16 tail per stream
LAYERS = [0, 1, 2, 3]


@pytest.fixture(scope="module")
def profiled(gpu):
    from layer_wise_mixed_amd import search

    errs = search.profile(HQ, HKV, LAYERS, search.PAIRS, batch=BATCH, seq_len=SEQ, seed=7)
    return search, errs


def _oracle_errors(pairs):
    out = np.zeros((len(LAYERS), len(pairs)))
    for i, li in enumerate(LAYERS):
        k = syn.keys_fp16(7, li, range(BATCH), range(HKV), 0, SEQ, num_kv_heads=HKV).numpy()
        v = syn.values_fp16(7, li, range(BATCH), range(HKV), 0, SEQ).numpy()
        q = syn.queries_fp16(7, li, 0, BATCH, HQ).numpy()
        for j, (kb, vb) in enumerate(pairs):
            out[i, j] = osearch.layer_error(q, k, v, kb, vb, False, SCALE)
    return out


@pytest.fixture(scope="module")
def oracle_errs(profiled, oq):
    search, _ = profiled
    return _oracle_errors(search.PAIRS)


def test_layer_errors_match_oracle(profiled, oracle_errs):
    _, got = profiled
    want = oracle_errs
    assert np.all(want > 0)
    # both attend to the same quantized cache; the kernel's outputs sit ~1e-6 (relative) from
    # the oracle's, so the error figures agree to well below their own size
    diff = np.abs(got - want)
    assert np.all(diff <= 2e-5 + 1e-3 * want), f"max diff {diff.max():.3g}"


@pytest.mark.parametrize("budget", [3.0, 3.25, 4.0, 5.0])
def test_map_matches_oracle_choice(profiled, oracle_errs, budget):
    search, errs = profiled
    bits = [kb + vb for kb, vb in search.PAIRS]
    pts = [[(bits[j], float(oracle_errs[i, j])) for j in range(len(bits))] for i in range(len(LAYERS))]
    kept = [osearch.pareto_front(p) for p in pts]
    total_budget = int(math.floor(2 * len(LAYERS) * budget + 1e-9))
    want = osearch.best_map([[pts[i][j] for j in kept[i]] for i in range(len(LAYERS))], total_budget)
    assert want is not None
    want_pairs = [search.PAIRS[kept[i][c]] for i, c in enumerate(want[0])]

    kept_lib = [search.prune(bits, list(errs[i])) for i in range(len(LAYERS))]
    assert kept_lib == kept, "the same pairs survive pruning"
    options = [[(bits[j], float(errs[i, j])) for j in kept_lib[i]] for i in range(len(LAYERS))]
    got = search.choose(options, total_budget)
    got_pairs = [search.PAIRS[kept_lib[i][c]] for i, c in enumerate(got[0])]
    assert sum(kb + vb for kb, vb in got_pairs) <= total_budget
    assert got_pairs == want_pairs
    assert got[1] == pytest.approx(want[1], rel=1e-3)


def test_frontier_matches_oracle(profiled, oracle_errs):
    search, errs = profiled
    bits = [kb + vb for kb, vb in search.PAIRS]
    o_opts, l_opts = [], []
    for i in range(len(LAYERS)):
        ko = osearch.pareto_front([(bits[j], float(oracle_errs[i, j])) for j in range(len(bits))])
        o_opts.append([(bits[j], float(oracle_errs[i, j])) for j in ko])
        kl = search.prune(bits, list(errs[i]))
        l_opts.append([(bits[j], float(errs[i, j])) for j in kl])
    want = osearch.frontier(o_opts)
    got = search.frontier(l_opts)
    assert [b for b, _, _ in got] == [b for b, _, _ in want]
    for (_, eg, _), (_, ew, _) in zip(got, want):
        assert eg == pytest.approx(ew, rel=1e-3)


@pytest.mark.parametrize("tau", [0.05, 0.3, 1.0])
def test_clustered_map_matches_oracle(profiled, oracle_errs, tau):
    search, errs = profiled
    bits = [kb + vb for kb, vb in search.PAIRS]
    want_cl = osearch.cluster_layers(oracle_errs, tau)
    got_cl = search.cluster_layers(errs, tau)
    assert got_cl == want_cl
    budget = int(math.floor(2 * len(LAYERS) * 3.5 + 1e-9))
    want = osearch.best_clustered_map(oracle_errs, bits, want_cl, budget)
    got = search.choose_clustered(errs, bits, got_cl, budget)
    assert got[0] == want[0]
    assert got[1] == pytest.approx(want[1], rel=1e-3)
