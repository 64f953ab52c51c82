"""Pins of the oracle's per-tag distortion D_k(b) (TriAxialKV page, "Facts": attention-output
MSE, max over heads, mean over requests, sum over layers): a tag with no tokens and a tag the
quantizer stores without loss give zero; a small case against a brute-force computation written
out here with numpy (per-token 4-bit quantization, softmax); the INT2-groups-then-INT4 storage
against the stream quantizer and the per-token quantizer; and each aggregation step."""
import math

import numpy as np
import pytest

import synthetic as syn
from oracle import dequant, dequant_stream, quantize_stream, quantize_tokens
from oracle.distortion import tag_dequantized, tag_distortion

SCALE = 1 / math.sqrt(128)


def _data(seed, B, hkv, G, L, layer=0):
    k = syn.keys_fp16(seed, layer, range(B), range(hkv), 0, L, num_kv_heads=hkv).numpy()
    v = syn.values_fp16(seed, layer, range(B), range(hkv), 0, L).numpy()
    q = syn.queries_fp16(seed, layer, 0, B, hkv * G).numpy()
    return q, k, v


def test_absent_tag_has_zero_distortion():
    q, k, v = _data(1, 2, 1, 2, 40)
    tags = [np.zeros(40, int), np.zeros(40, int)]
    D = tag_distortion([(q, k, v)], tags, 3, SCALE)
    assert np.all(D[1:] == 0.0) and np.all(D[0] > 0)


def test_lossless_tag_has_zero_distortion():
    """Tag-1 tokens all equal one vector that is constant on each 32-channel group: every
    INT2 key group (one channel over 32 tokens), value group and INT4 token group has scale
    0 and dequantizes to its zero point exactly, at either width."""
    q, k, v = _data(2, 1, 1, 3, 70)
    tags = np.zeros(70, int)
    tags[3:70:2] = 1  # 34 tokens: one INT2 group + 2 INT4 leftovers at 2 bits
    row = np.repeat(np.array([0.5, -1.25, 2.0, 0.0], np.float16), 32)
    k[0, 0, tags == 1] = row
    v[0, 0, tags == 1] = row[::-1]
    D = tag_distortion([(q, k, v)], [tags], 2, SCALE)
    assert D[1, 0] == 0.0 and D[1, 1] == 0.0
    assert D[0, 0] > 0 and D[0, 1] > 0


def _int4_token_numpy(x):
    """Per-token 4-bit quantization of one fp16 token, written out: per 32-channel group,
    fp32 scale = (max - min) / 15, code = clamp(round-half-even((x - min) / scale)), value =
    code * scale + min rounded once to fp32."""
    out = np.zeros(128, np.float32)
    for n in range(4):
        g = x[32 * n:32 * n + 32].astype(np.float32)
        mn, mx = g.min(), g.max()
        s = np.float32(np.float32(mx - mn) / np.float32(15.0))
        if s == 0:
            out[32 * n:32 * n + 32] = mn
            continue
        c = np.clip(np.rint(np.float32(g - mn) / s), 0, 15)
        out[32 * n:32 * n + 32] = (c.astype(np.float64) * np.float64(s) + np.float64(mn)).astype(np.float32)
    return out


def test_brute_force_small_case():
    """One request, one KV head, two query heads, six tokens, tag 0 on tokens 1 and 4 (fewer
    than 32, so INT4 per token at either width): D by hand with numpy."""
    q, k, v = _data(3, 1, 1, 2, 6)
    tags = np.array([1, 0, 1, 1, 0, 1])
    D = tag_distortion([(q, k, v)], [tags], 2, SCALE)
    kf = k[0, 0].astype(np.float64)
    vf = v[0, 0].astype(np.float64)
    kq, vq = kf.copy(), vf.copy()
    for j in (1, 4):
        kq[j] = _int4_token_numpy(k[0, 0, j])
        vq[j] = _int4_token_numpy(v[0, 0, j])

    def attend(qrow, kk, vv):
        s = (kk @ qrow.astype(np.float64)) * SCALE
        p = np.exp(s - s.max())
        return (p[:, None] * vv).sum(axis=0) / p.sum()

    mse = [np.mean((attend(q[0, g], kq, vq) - attend(q[0, g], kf, vf)) ** 2) for g in range(2)]
    want = max(mse)
    assert abs(D[0, 0] - want) <= 1e-12 * max(want, 1e-30) + 1e-18
    assert abs(D[0, 1] - want) <= 1e-12 * max(want, 1e-30) + 1e-18


def test_int2_groups_then_int4_leftovers():
    """40 tag tokens at 2 bits: the first 32 as one INT2 group (keys per-channel, values
    per-token, 2 bits), the last 8 per-token at 4 bits; at 4 bits all 40 per-token."""
    _, k, v = _data(4, 1, 1, 1, 40)
    k, v = k[0, 0], v[0, 0]
    kd, vd = tag_dequantized(k, v, 2)
    k2, v2 = dequant_stream(quantize_stream(k[:32], v[:32], 2, 2, False))
    assert np.array_equal(kd[:32], k2) and np.array_equal(vd[:32], v2)

    def int4(x):
        codes, sc, zr = quantize_tokens(x, 4)
        return np.array([[dequant(codes[j, c], sc[j, c // 32], zr[j, c // 32]) for c in range(128)]
                         for j in range(x.shape[0])], np.float32)

    assert np.array_equal(kd[32:], int4(k[32:])) and np.array_equal(vd[32:], int4(v[32:]))
    kd4, vd4 = tag_dequantized(k, v, 4)
    assert np.array_equal(kd4, int4(k)) and np.array_equal(vd4, int4(v))


def test_aggregation_max_mean_sum():
    q, k, v = _data(5, 2, 2, 2, 50)
    tags = [np.array(syn.seeded_tags(5, r, 50, 3)) for r in range(2)]
    D = tag_distortion([(q, k, v)], tags, 3, SCALE)
    # sum over layers: the same layer twice doubles it
    assert np.allclose(tag_distortion([(q, k, v), (q, k, v)], tags, 3, SCALE), 2 * D, rtol=1e-14, atol=0)
    # mean over requests: each request alone, averaged
    per = [tag_distortion([(q[r:r + 1], k[r:r + 1], v[r:r + 1])], [tags[r]], 3, SCALE) for r in range(2)]
    assert np.allclose((per[0] + per[1]) / 2, D, rtol=1e-14, atol=0)
    # max over heads: with one query head per KV head, each head alone, the larger one
    q1 = q[:, ::2].copy()
    D1 = tag_distortion([(q1, k, v)], tags, 3, SCALE)
    one = [[tag_distortion([(q1[r:r + 1, h:h + 1], k[r:r + 1, h:h + 1], v[r:r + 1, h:h + 1])], [tags[r]], 3, SCALE)
            for h in range(2)] for r in range(2)]
    want = (np.maximum(one[0][0], one[0][1]) + np.maximum(one[1][0], one[1][1])) / 2
    assert np.allclose(D1, want, rtol=1e-14, atol=0)
