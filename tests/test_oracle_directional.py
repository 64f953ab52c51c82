"""Directional checks on synthetic data (signs, never the pages' values), plus the
equivalent-precision arithmetic the pages print.

- KVTuner summary page, "Measured effects" table: per-channel-asym keys have lower
  relative key error than per-token-asym (0.012280 -> 0.004869 on a real model);
  first page, "Facts": keys have channel-wise outliers.
- KVTuner summary page, "Measured effects" table: at matched memory K4V2 gives lower
  relative attention-output error than K2V4 (0.453 vs 0.892 on a real model).
- First page, "Facts": a K8V2 pair is "5-bit", a K4V8 pair "6-bit"; the 3.25-bit
  Llama map; KVSplit thread: K8V4 and K4V8 use the same number of bits.
"""
import math

import numpy as np

import synthetic as syn


def _kv(seed, L, heads=4, outliers=4, factor=10.0):
    k = syn.keys_fp16(seed, 0, [0], range(heads), 0, L, outlier_count=outliers,
                      outlier_factor=factor, num_kv_heads=heads)[0].numpy()
    v = syn.values_fp16(seed, 0, [0], range(heads), 0, L)[0].numpy()
    return k, v


def test_per_channel_keys_beat_per_token_with_outliers(oq):
    k, v = _kv(21, 256)
    e_ch, e_tok, ref = 0.0, 0.0, 0.0
    for h in range(k.shape[0]):
        kf = k[h].astype(np.float64)
        kd_c, _ = oq.dequant_stream(oq.quantize_stream(k[h], v[h], 4, 16, k_token=False))
        kd_t, _ = oq.dequant_stream(oq.quantize_stream(k[h], v[h], 4, 16, k_token=True))
        e_ch += np.sum((kd_c - kf) ** 2)
        e_tok += np.sum((kd_t - kf) ** 2)
        ref += np.sum(kf ** 2)
    assert math.sqrt(e_ch / ref) < math.sqrt(e_tok / ref)


def test_key_priority_k4v2_beats_k2v4(oq):
    k, v = _kv(22, 512)
    q = syn.queries_fp16(22, 0, 0, 1, 4 * 4)[0].numpy().reshape(4, 4, 128)
    num = {"K4V2": 0.0, "K2V4": 0.0}
    den = 0.0
    for h in range(4):
        exact, _ = oq.decode_stream(q[h], k[h], v[h], 16, 16, False, 1 / math.sqrt(128))
        den += np.sum(exact ** 2)
        for name, kb, vb in (("K4V2", 4, 2), ("K2V4", 2, 4)):
            out, _ = oq.decode_stream(q[h], k[h], v[h], kb, vb, False, 1 / math.sqrt(128))
            num[name] += np.sum((out - exact) ** 2)
    assert num["K4V2"] < num["K2V4"]


def test_equivalent_precision_pins(oq):
    assert oq.equiv_bits([(8, 2)]) == 5.0
    assert oq.equiv_bits([(4, 8)]) == 6.0
    assert oq.equiv_bits([(8, 4)]) == oq.equiv_bits([(4, 8)])
    assert oq.equiv_bits([(4, 2)] * 24 + [(4, 4)] * 8) == 3.25
    # 28 layers of K8V4 and K4V2 cannot average exactly 4.0; 9 + 19 gives 111/28
    assert abs(oq.equiv_bits([(8, 4)] * 9 + [(4, 2)] * 19) - 111 / 28) < 1e-15
    assert all(abs(oq.equiv_bits([(8, 4)] * a + [(4, 2)] * (28 - a)) - 4.0) > 1e-9 for a in range(29))
