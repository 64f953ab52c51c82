"""Pins of the oracle's chunked-prefill attention (oracle.chunk_prefill): a chunk's query
rows attend to the quantized prefix as stored and, causally, to the chunk's own fp16 tokens.

- With no prefix it is causal attention over the chunk, checked against torch's
  scaled_dot_product_attention in float64 (a mask in the wrong direction or one token off
  fails), and its first row has the closed form out = v_0, lse = scale * q . k_0.
- With a prefix that the quantizer stores without loss (every group's values on
  {0, (2^b - 1) / 2^(b - 1)}, so scale = 2^-(b - 1), zero = 0 and code * scale is exact), it
  is attention over the prefix (unmasked) and the causal chunk, checked against
  scaled_dot_product_attention with that explicit mask (a dropped or masked prefix fails).
- On a lossy prefix it equals the log-sum-exp merge of decode attention over the quantized
  prefix with the chunk's own causal attention: the way the library's prefix attention is
  meant to be combined (a wrong merge weight fails)."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn

SCALE = 1 / math.sqrt(128)


def _sdpa(q, k, v, mask):
    """q [C, G, D], k/v [N, D] float64, mask [C, N] bool (True = attend) -> out [C, G, D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [G, C, D]
    G = qt.shape[0]
    kt = torch.from_numpy(k)[None].expand(G, -1, -1)
    vt = torch.from_numpy(v)[None].expand(G, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask)[None],
                                                         scale=SCALE)
    return o.permute(1, 0, 2).numpy()


def _chunk(seed, C, G, L0):
    q = syn.normal_fp16(seed, syn.T_Q, 0, [0], range(G), L0, C)[0].permute(1, 0, 2).contiguous().numpy()
    k = syn.keys_fp16(seed, 0, [0], [0], L0, C, num_kv_heads=1)[0, 0].numpy()
    v = syn.values_fp16(seed, 0, [0], [0], L0, C)[0, 0].numpy()
    return q, k, v


@pytest.mark.parametrize("C,G", [(1, 4), (7, 4), (33, 2), (20, 1)])
def test_no_prefix_is_causal_attention(oq, C, G):
    q, k, v = _chunk(3, C, G, 0)
    empty = np.zeros((0, 128), np.float16)
    out, lse = oq.chunk_prefill(q, empty, empty, k, v, 4, 2, False, SCALE)
    mask = np.tril(np.ones((C, C), bool))
    want = _sdpa(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), mask)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)
    # first row: one key, weight 1
    np.testing.assert_allclose(out[0], np.broadcast_to(v[0].astype(np.float64), (G, 128)), rtol=0, atol=1e-15)
    s0 = q[0].astype(np.float64) @ k[0].astype(np.float64) * SCALE
    np.testing.assert_allclose(lse[0], s0, rtol=1e-14, atol=1e-14)


def _lossless(seed, n, bits_k, bits_v, k_token):
    """fp16 K, V [n, 128] on {0, M_b}, M_b = (2^b - 1) / 2^(b - 1): exact under the quantizer."""
    rng = np.random.default_rng(seed)
    mk = (2 ** bits_k - 1) / 2 ** (bits_k - 1) if bits_k < 16 else 1.5
    mv = (2 ** bits_v - 1) / 2 ** (bits_v - 1) if bits_v < 16 else 1.5
    k = (rng.integers(0, 2, (n, 128)) * mk).astype(np.float16)
    v = (rng.integers(0, 2, (n, 128)) * mv).astype(np.float16)
    return k, v


@pytest.mark.parametrize("kb,vb,k_token,L", [(2, 2, False, 64), (4, 8, False, 77), (8, 4, True, 45), (2, 4, True, 32)])
def test_lossless_prefix_is_unmasked(oq, kb, vb, k_token, L):
    C, G = 9, 4
    kp, vp = _lossless(L, L, kb, vb, k_token)
    sq = oq.quantize_stream(kp, vp, kb, vb, k_token)
    kd, vd = oq.dequant_stream(sq)
    assert np.array_equal(kd, kp.astype(np.float32)) and np.array_equal(vd, vp.astype(np.float32))
    q, kc, vc = _chunk(5, C, G, L)
    out, lse = oq.chunk_prefill(q, kp, vp, kc, vc, kb, vb, k_token, SCALE)
    keys = np.concatenate([kp, kc]).astype(np.float64)
    vals = np.concatenate([vp, vc]).astype(np.float64)
    mask = np.concatenate([np.ones((C, L), bool), np.tril(np.ones((C, C), bool))], axis=1)
    want = _sdpa(q.astype(np.float64), keys, vals, mask)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kb,vb,k_token,L", [(2, 2, False, 70), (4, 4, True, 33), (8, 2, False, 96), (16, 4, False, 5)])
def test_merge_of_prefix_and_chunk_parts(oq, kb, vb, k_token, L):
    C, G = 6, 4
    kp = syn.keys_fp16(9, 1, [0], [0], 0, L, num_kv_heads=1)[0, 0].numpy()
    vp = syn.values_fp16(9, 1, [0], [0], 0, L)[0, 0].numpy()
    q, kc, vc = _chunk(9, C, G, L)
    out, lse = oq.chunk_prefill(q, kp, vp, kc, vc, kb, vb, k_token, SCALE)
    op, lp = oq.decode_stream(q.reshape(C * G, 128), kp, vp, kb, vb, k_token, SCALE)
    op, lp = op.reshape(C, G, 128), lp.reshape(C, G)
    for i in range(C):
        oc, lc = oq.attention(q[i], kc[:i + 1].astype(np.float32), vc[:i + 1].astype(np.float32), SCALE)
        for g in range(G):
            m, ml = oq.lse_merge(np.stack([op[i, g], oc[g]]), np.array([lp[i, g], lc[g]]))
            np.testing.assert_allclose(out[i, g], m, rtol=0, atol=1e-12)
            assert lse[i, g] == pytest.approx(ml, abs=1e-12)
