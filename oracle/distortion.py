"""Oracle of the per-tag distortion D_k(b).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

What it follows (TriAxialKV page, "Facts"): each token tag k has a distortion
D_k(b) at b = 2 and b = 4 bits, the attention-output MSE aggregated as the max
over heads, the mean over requests and the sum over layers. Readings taken
where the page is silent (the same as the library's): tag k's tokens alone are
quantized, the way the paged pool stores them -- b = 2: INT2 groups of 32 of
the tag's tokens in arrival order (keys per-channel, values per-token, 2
bits), the last n mod 32 tokens per-token at 4 bits; b = 4: every tag-k token
per-token at 4 bits, keys and values -- every other token stays fp16; the
MSE is the mean over a query head's 128 output channels of the squared
difference from attention over the fp16 cache; heads are query heads.

The steps in the definition's order, with the oracle's own quantizer and its
fp64 attention: dequantize the tag's tokens, attend per (layer, request, KV
head) with every query head of the group, square the differences, average the
channels, take the max over query heads, the mean over requests, the sum over
layers.
"""
from __future__ import annotations

import numpy as np

from . import attention, pack_paged, paged_pool_bytes, unpack_paged

GROUP = 32
PAGE = 16


def tag_dequantized(k_fp16, v_fp16, bits):
    """fp32 (k, v) [n, 128] of one tag's tokens (arrival order) as the pool stores them at
    `bits`: INT2 groups of 32 then INT4 leftovers (bits = 2), or all INT4 (bits = 4). The oracle's
    own paged pool does the storing: the tokens are packed through a page table of their own and
    unpacked again."""
    k = np.asarray(k_fp16, dtype=np.float16).reshape(-1, 128)
    v = np.asarray(v_fp16, dtype=np.float16).reshape(-1, 128)
    n = k.shape[0]
    if n == 0:
        return np.zeros((0, 128), np.float32), np.zeros((0, 128), np.float32)
    n2 = (n // GROUP) * GROUP if bits == 2 else 0
    int2_pages = 2 * (n2 // GROUP)
    int4_pages = max(1, -(-(n - n2) // PAGE))
    table = np.arange(int2_pages + int4_pages, dtype=np.int32)
    pool = np.zeros(paged_pool_bytes(1, int2_pages, int4_pages), np.uint8)
    pack_paged(pool, k, v, n2, table, int2_pages, 1, 0)
    return unpack_paged(pool, n2, n - n2, table, int2_pages, 1, 0)


def tag_distortion(layers, tags, num_tags, scale):
    """D [num_tags, 2] (columns: 2 and 4 bits). layers: list of (q [B, Hq, 128], k [B, Hkv, L,
    128], v [B, Hkv, L, 128]) fp16 numpy arrays; tags: int [B][L]."""
    D = np.zeros((num_tags, 2))
    for q, k, v in layers:
        q = np.asarray(q, dtype=np.float16)
        B, Hkv = k.shape[0], k.shape[1]
        G = q.shape[1] // Hkv
        for t in range(num_tags):
            for i, bits in enumerate((2, 4)):
                per_request = []
                for r in range(B):
                    tg = np.asarray(tags[r])
                    sel = np.flatnonzero(tg == t)
                    heads = []
                    for h in range(Hkv):
                        kf = k[r, h].astype(np.float32)
                        vf = v[r, h].astype(np.float32)
                        qq = q[r, h * G:(h + 1) * G]
                        ref, _ = attention(qq, kf, vf, scale)
                        kq, vq = kf.copy(), vf.copy()
                        if len(sel):
                            kq[sel], vq[sel] = tag_dequantized(k[r, h, sel], v[r, h, sel], bits)
                        got, _ = attention(qq, kq, vq, scale)
                        heads.extend(((got - ref) ** 2).mean(axis=1))  # one MSE per query head
                    per_request.append(max(heads))
                D[t, i] += float(np.mean(per_request))
    return D
