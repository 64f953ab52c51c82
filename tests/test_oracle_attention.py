"""Pins of the oracle's fp64 decode attention and log-sum-exp merge: closed forms,
special cases, a library routine (torch SDPA in float64 on the CPU) for the b = 16
passthrough, and the invariances the split design relies on (TriAxialKV page,
"Facts": flash-decoding splits merged by online log-sum-exp; any token order)."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn

D = 128


def _stream(seed, L, outliers=4, factor=10.0):
    k = syn.keys_fp16(seed, 0, [0], [0], 0, L, outlier_count=outliers, outlier_factor=factor,
                      num_kv_heads=1)[0, 0].numpy()
    v = syn.values_fp16(seed, 0, [0], [0], 0, L)[0, 0].numpy()
    return k, v


def test_two_token_closed_form(oq):
    """q = e_0, k_0 = 0, k_1 = x e_0, scale 1: out = (v_0 + e^x v_1) / (1 + e^x),
    lse = log(1 + e^x)."""
    x = 1.25
    q = np.zeros((1, D), np.float16)
    q[0, 0] = 1.0
    kd = np.zeros((2, D), np.float32)
    kd[1, 0] = x
    rng = np.random.default_rng(0)
    vd = rng.standard_normal((2, D)).astype(np.float32)
    out, lse = oq.attention(q, kd, vd, 1.0)
    w = math.exp(x)
    ref = (vd[0].astype(np.float64) + w * vd[1].astype(np.float64)) / (1 + w)
    assert np.allclose(out[0], ref, rtol=1e-14, atol=1e-15)
    assert abs(lse[0] - math.log1p(w)) < 1e-14


def test_single_token_returns_its_value(oq):
    k, v = _stream(1, 1)
    q = syn.queries_fp16(1, 0, 0, 1, 3)[0].numpy()
    for kb, vb in ((8, 4), (16, 16)):
        sq = oq.quantize_stream(k, v, kb, vb)
        kd, vd = oq.dequant_stream(sq)
        out, lse = oq.attention(q, kd, vd, 1 / math.sqrt(D))
        for g in range(3):
            assert np.array_equal(out[g], vd[0].astype(np.float64))


def test_zero_query_is_mean_of_values(oq):
    k, v = _stream(2, 77)
    sq = oq.quantize_stream(k, v, 4, 2)
    kd, vd = oq.dequant_stream(sq)
    q = np.zeros((2, D), np.float16)
    out, lse = oq.attention(q, kd, vd, 0.3)
    ref = vd.astype(np.float64).mean(axis=0)
    assert np.allclose(out[0], ref, rtol=1e-13, atol=1e-14)
    assert abs(lse[0] - math.log(77)) < 1e-13


def test_empty_cache(oq):
    q = syn.queries_fp16(0, 0, 0, 1, 1)[0].numpy()
    out, lse = oq.attention(q, np.zeros((0, D), np.float32), np.zeros((0, D), np.float32), 1.0)
    assert np.all(out == 0) and lse[0] == -math.inf


@pytest.mark.parametrize("L", [1, 31, 32, 95, 300])
def test_passthrough_equals_sdpa_float64(oq, L):
    """K16V16 is plain attention: compare with torch's scaled_dot_product_attention in float64."""
    k, v = _stream(3, L)
    q = syn.queries_fp16(3, 0, 0, 1, 4)[0].numpy()
    out, lse = oq.decode_stream(q, k, v, 16, 16, False, 1 / math.sqrt(D))
    qt = torch.from_numpy(q.astype(np.float64)).view(1, 4, 1, D)
    kt = torch.from_numpy(k.astype(np.float64)).view(1, 1, L, D).expand(1, 4, L, D)
    vt = torch.from_numpy(v.astype(np.float64)).view(1, 1, L, D).expand(1, 4, L, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1 / math.sqrt(D))
    assert np.allclose(out, ref.view(4, D).numpy(), rtol=1e-12, atol=1e-13)
    s = (qt @ kt.transpose(-1, -2)).view(4, L) / math.sqrt(D)
    assert np.allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("parts", [1, 2, 3, 7])
def test_lse_merge_of_any_partition_is_single_pass(oq, parts):
    L = 200
    k, v = _stream(4, L)
    q = syn.queries_fp16(4, 0, 0, 1, 2)[0].numpy()
    sq = oq.quantize_stream(k, v, 8, 4)
    kd, vd = oq.dequant_stream(sq)
    full, full_lse = oq.attention(q, kd, vd, 0.088)
    rng = np.random.default_rng(parts)
    cuts = sorted(rng.choice(np.arange(1, L), size=parts - 1, replace=False).tolist())
    bounds = [0] + cuts + [L]
    # an extra empty split must carry zero weight
    bounds_e = bounds + [L]
    for g in range(2):
        o_parts, l_parts = [], []
        for a, b in zip(bounds_e[:-1], bounds_e[1:]):
            o, l = oq.attention(q[g:g + 1], kd[a:b], vd[a:b], 0.088)
            o_parts.append(o[0])
            l_parts.append(l[0])
        out, lse = oq.lse_merge(np.array(o_parts), np.array(l_parts))
        assert np.allclose(out, full[g], rtol=1e-12, atol=1e-14)
        assert abs(lse - full_lse[g]) < 1e-12


def test_permutation_invariance(oq):
    k, v = _stream(5, 150)
    q = syn.queries_fp16(5, 0, 0, 1, 4)[0].numpy()
    sq = oq.quantize_stream(k, v, 4, 4)
    kd, vd = oq.dequant_stream(sq)
    out, lse = oq.attention(q, kd, vd, 0.1)
    perm = np.random.default_rng(5).permutation(150)
    out2, lse2 = oq.attention(q, kd[perm], vd[perm], 0.1)
    assert np.allclose(out, out2, rtol=1e-12, atol=1e-14) and np.allclose(lse, lse2, rtol=1e-13)


def test_duplicate_query_rows(oq):
    k, v = _stream(6, 90)
    q = syn.queries_fp16(6, 0, 0, 1, 2)[0].numpy()
    q2 = np.stack([q[0], q[1], q[0]])
    sq = oq.quantize_stream(k, v, 2, 2)
    kd, vd = oq.dequant_stream(sq)
    out, lse = oq.attention(q2, kd, vd, 0.1)
    assert np.array_equal(out[0], out[2]) and lse[0] == lse[2]
