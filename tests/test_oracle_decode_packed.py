"""Pins of the oracle's batch decode over its own packed layer (`decode_packed`, the function
the CPU baseline times): every row must be the fp64 attention of its query rows over the
stream it names, dequantized from the stream's own quantization (TriAxialKV page, "Facts":
asymmetric groupwise codes with group 32; flash decoding attends over every cached token).
Streams sit at arbitrary ids in a buffer whose stride is larger than one stream, the lengths
are ragged (0, 1, 31, 32, 33, 95) and the thread count varies, so a wrong stride, id, length
or per-thread buffer shows up as a row that differs."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn

D = 128
CAP_GROUPS = 3  # 96 tokens of capacity: 3 group records + the tail record


def _stream(seed, L):
    k = syn.keys_fp16(seed, 1, [0], [0], 0, L, outlier_count=4, outlier_factor=10.0,
                      num_kv_heads=1)[0, 0].numpy()
    v = syn.values_fp16(seed, 1, [0], [0], 0, L)[0, 0].numpy()
    return k, v


@pytest.mark.parametrize("kb,vb,kt", [(8, 4, False), (4, 2, False), (2, 8, False), (4, 4, True),
                                      (8, 2, True), (16, 16, False), (16, 4, False)])
@pytest.mark.parametrize("nthreads", [1, 3])
def test_decode_packed_is_attention_over_each_named_stream(oq, kb, vb, kt, nthreads):
    lens = [33, 0, 95, 1, 31, 32]
    ids = [5, 0, 2, 7, 3, 6]  # not in order, with unused slots 1 and 4
    G = 3
    stride = oq.stream_bytes(kb, vb, CAP_GROUPS) + 4096  # a gap after each stream
    buf = np.full(8 * stride, 0xA5, np.uint8)  # garbage everywhere no stream is packed
    qs = np.zeros((len(ids), G, D), np.float16)
    want = []
    for s, (sid, L) in enumerate(zip(ids, lens)):
        k, v = _stream(40 + s, L)
        sq = oq.quantize_stream(k, v, kb, vb, kt)
        packed, _ = oq.pack_stream(sq, CAP_GROUPS)
        buf[sid * stride: sid * stride + len(packed)] = packed
        q = syn.queries_fp16(7, 1, s, 1, G)[0].numpy()
        qs[s] = q
        kd, vd = oq.dequant_stream(sq)
        want.append(oq.attention(q, kd, vd, 1 / math.sqrt(D)))
    out, lse, used = oq.decode_packed(buf, stride, ids, lens, kb, vb, kt, CAP_GROUPS, qs, G, 1 / math.sqrt(D),
                                      nthreads)
    assert used >= 1
    for s, L in enumerate(lens):
        wo, wl = want[s]
        if L == 0:
            assert np.all(out[s] == 0) and np.all(np.isneginf(lse[s]))
            continue
        assert np.allclose(out[s], wo, rtol=0, atol=1e-12), (s, L)
        assert np.allclose(lse[s], wl, rtol=0, atol=1e-12), (s, L)


def test_decode_packed_passthrough_equals_sdpa_float64(oq):
    """K16V16 streams hold the fp16 values as given, so the batch decode must equal torch's
    scaled_dot_product_attention in float64 on those values (a library routine, not the oracle)."""
    lens, ids, G = [70, 5], [1, 0], 2
    stride = oq.stream_bytes(16, 16, CAP_GROUPS)
    buf = np.zeros(2 * stride, np.uint8)
    qs = np.zeros((2, G, D), np.float16)
    refs = []
    for s, (sid, L) in enumerate(zip(ids, lens)):
        k, v = _stream(90 + s, L)
        packed, _ = oq.pack_stream(oq.quantize_stream(k, v, 16, 16), CAP_GROUPS)
        buf[sid * stride: sid * stride + len(packed)] = packed
        qs[s] = syn.queries_fp16(9, 1, s, 1, G)[0].numpy()
        qt = torch.from_numpy(qs[s].astype(np.float64))[None, None]
        kt = torch.from_numpy(k.astype(np.float64))[None, None]
        vt = torch.from_numpy(v.astype(np.float64))[None, None]
        refs.append(torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.1)[0, 0].numpy())
    out, _, _ = oq.decode_packed(buf, stride, ids, lens, 16, 16, False, CAP_GROUPS, qs, G, 0.1, 2)
    for s in range(2):
        assert np.allclose(out[s], refs[s], rtol=1e-12, atol=1e-13)
