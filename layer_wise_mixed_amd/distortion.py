"""Per-tag distortion D_k(b) measured on the library's own kernels.

TriAxialKV page, "Facts": every token carries a tag (its temporal, modal and
semantic role); each tag k has a distortion D_k(b) at b = 2 and b = 4 bits,
the attention-output MSE aggregated as the max over heads, the mean over
requests and the sum over layers; the allocator then gives each tag INT2 or
INT4 under an average-bit budget (``allocate.allocate``), and the paged pool
stores the INT2 tags' tokens as 32-token groups, leftovers through the INT4
per-token path (``allocate.int2_tokens``).

Readings, where the page leaves the definition open:
  - D_k(b) quantizes the tokens of tag k alone, at b bits and the way the
    pool stores them (b = 2: INT2 groups of 32 tag-k tokens in arrival
    order, keys per-channel and values per-token, the last n mod 32 tokens
    through the INT4 path; b = 4: every tag-k token INT4, keys and values
    per-token), keeps every other token at fp16, and compares each query
    head's decode-attention output with attention over the fp16 cache;
  - its MSE is the mean over the 128 output channels of the squared
    difference; "heads" are query heads; a request's decode query is one
    token per query head.

Measurement: the tag-k tokens go into a paged INT2/INT4 pool
(``kvq_quantize_append`` with pages), the other tokens into an fp16
(K16V16) cache, and the reference, every token, into another fp16 cache;
each is attended by ``kvq_decode_attention`` with its log-sum-exp. The
attention over the union is the log-sum-exp merge of the two parts (the same
merge that joins flash-decoding splits); it, the MSE and the aggregation are
plain float64 arithmetic on the host.
"""
from __future__ import annotations

import math

import numpy as np

from . import (decode_attention, load, make_pages, make_shape, plan_layers, quantize_append, workspace_bytes)

PAGE = 16


def _merge(o1, l1, o2, l2):
    """Attention over the union of two disjoint token sets from each set's (out, lse)."""
    m = np.maximum(l1, l2)
    m = np.where(np.isfinite(m), m, 0.0)
    w1 = np.where(np.isfinite(l1), np.exp(l1 - m), 0.0)
    w2 = np.where(np.isfinite(l2), np.exp(l2 - m), 0.0)
    den = w1 + w2
    den = np.where(den > 0, den, 1.0)
    return (w1[..., None] * o1 + w2[..., None] * o2) / den[..., None]


def _decode_fp16(torch, hq, hkv, k_parts, v_parts, q, scale, device):
    """Attention of q over per-request fp16 token lists in a K16V16 cache: (out, lse) float64."""
    B = len(k_parts)
    lens = [int(x.shape[1]) for x in k_parts]
    cap = max(32, -(-max(lens + [1]) // 32) * 32)
    plan = plan_layers(make_shape(hq, hkv, B, max_tokens=cap), [(16, 16)])
    cache = torch.zeros(plan.total_bytes, dtype=torch.uint8, device=device)
    z = torch.zeros(1, dtype=torch.int32, device=device)
    lp = plan.layers[0]
    for r in range(B):
        if lens[r] == 0:
            continue
        off = r * hkv * lp.stream_bytes
        quantize_append(plan, 0, cache[off:], k_parts[r][None].contiguous(), v_parts[r][None].contiguous(), z)
    seq = torch.tensor(lens, dtype=torch.int32, device=device)
    ml = max(lens + [0])
    out = torch.empty(B, hq, 128, dtype=torch.float32, device=device)
    lse = torch.empty(B, hq, dtype=torch.float32, device=device)
    ws = torch.empty(workspace_bytes(plan, B, ml) // 4 + 1, dtype=torch.float32, device=device)
    decode_attention(plan, 0, cache, q, seq, ml, scale, out, lse, ws)
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def _decode_pool(torch, hq, hkv, k_parts, v_parts, n2s, q, scale, device):
    """Attention of q over per-request tokens stored in a paged INT2/INT4 pool: the first n2s[r]
    tokens of request r (a multiple of 32) as INT2 groups, the rest as INT4 tokens."""
    B = len(k_parts)
    lens = [int(x.shape[1]) for x in k_parts]
    pairs = [n2 // 32 for n2 in n2s]
    quads = [-(-(L - n2) // PAGE) for L, n2 in zip(lens, n2s)]
    int2_pages = 2 * sum(pairs)
    int4_pages = max(sum(quads), 1)
    max_pages = max(1, max(2 * p + qd for p, qd in zip(pairs, quads)))
    plan = plan_layers(make_shape(hq, hkv, B, page_tokens=PAGE, int2_pages=int2_pages, int4_pages=int4_pages),
                       [(2, 2, 0, 1)])
    pool = torch.zeros(plan.total_bytes, dtype=torch.uint8, device=device)
    table = torch.zeros(B, max_pages, dtype=torch.int32)
    p2, p4 = 0, int2_pages
    for r in range(B):
        row = []
        for _ in range(pairs[r]):
            row += [p2, p2 + 1]
            p2 += 2
        for _ in range(quads[r]):
            row.append(p4)
            p4 += 1
        table[r, :len(row)] = torch.tensor(row, dtype=torch.int32)
    table = table.to(device)
    zero = torch.zeros(B, dtype=torch.int32, device=device)
    for r in range(B):
        if lens[r] == 0:
            continue
        add2 = torch.tensor([n2s[r]], dtype=torch.int32, device=device)
        pages = make_pages(table[r], max_pages, zero[r:], zero[r:], add2)
        quantize_append(plan, 0, pool, k_parts[r][None].contiguous(), v_parts[r][None].contiguous(), None, pages)
    n2 = torch.tensor(n2s, dtype=torch.int32, device=device)
    n4 = torch.tensor([L - a for L, a in zip(lens, n2s)], dtype=torch.int32, device=device)
    ml = max(lens + [0])
    out = torch.empty(B, hq, 128, dtype=torch.float32, device=device)
    lse = torch.empty(B, hq, dtype=torch.float32, device=device)
    ws = torch.empty(workspace_bytes(plan, B, ml) // 4 + 1, dtype=torch.float32, device=device)
    decode_attention(plan, 0, pool, q, None, ml, scale, out, lse, ws, pages=make_pages(table, max_pages, n2, n4))
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def tag_distortion(layers, tags, num_tags: int, scale: float, device="cuda"):
    """D[k, i]: the distortion of tag k at bits (2, 4)[i], summed over `layers`.

    layers: a list of (q, k, v) per layer: q fp16 [B, Hq, 128], k and v fp16 [B, Hkv, L, 128]
    (torch tensors, any device); tags: int [B][L], each token's tag in 0..num_tags-1."""
    import torch

    load()
    tags = [np.asarray(t) for t in tags]
    D = np.zeros((num_tags, 2))
    for q, k, v in layers:
        q = q.to(device).contiguous()
        k = k.to(device)
        v = v.to(device)
        B, hkv = k.shape[0], k.shape[1]
        hq = q.shape[1]
        ref, _ = _decode_fp16(torch, hq, hkv, [k[r] for r in range(B)], [v[r] for r in range(B)], q, scale, device)
        for t in range(num_tags):
            sel = [torch.as_tensor(np.flatnonzero(tags[r] == t), device=device) for r in range(B)]
            rest = [torch.as_tensor(np.flatnonzero(tags[r] != t), device=device) for r in range(B)]
            if all(len(s) == 0 for s in sel):
                continue
            ko = [k[r].index_select(1, rest[r]) for r in range(B)]
            vo = [v[r].index_select(1, rest[r]) for r in range(B)]
            o_rest, l_rest = _decode_fp16(torch, hq, hkv, ko, vo, q, scale, device)
            kt = [k[r].index_select(1, sel[r]) for r in range(B)]
            vt = [v[r].index_select(1, sel[r]) for r in range(B)]
            for i, b in enumerate((2, 4)):
                n2s = [(len(s) // 32) * 32 if b == 2 else 0 for s in sel]
                o_t, l_t = _decode_pool(torch, hq, hkv, kt, vt, n2s, q, scale, device)
                o = _merge(o_t, l_t, o_rest, l_rest)
                mse = ((o - ref) ** 2).mean(axis=2)       # [B, Hq]
                D[t, i] += mse.max(axis=1).mean()          # max over heads, mean over requests
    return D


def calibrate(hq: int, hkv: int, num_tags: int, budget: float, *, layers=(0,), batch: int = 4, seq_len: int = 1024,
              seed: int = 0, outliers=(4, 10.0), device="cuda"):
    """D_k(b) on seeded synthetic (q, K, V) and tags, and the allocation it gives at `budget`
    mean bits: (D [num_tags, 2], bits per tag, token counts per tag)."""
    import synthetic as syn

    from .allocate import allocate

    tags = [np.asarray(syn.seeded_tags(seed, r, seq_len, num_tags)) for r in range(batch)]
    data = []
    for li in layers:
        k = syn.keys_fp16(seed, li, range(batch), range(hkv), 0, seq_len, outlier_count=outliers[0],
                          outlier_factor=outliers[1], num_kv_heads=hkv)
        v = syn.values_fp16(seed, li, range(batch), range(hkv), 0, seq_len)
        q = syn.queries_fp16(seed, li, 0, batch, hq)
        data.append((q, k, v))
    D = tag_distortion(data, tags, num_tags, 1.0 / math.sqrt(128.0), device)
    counts = np.bincount(np.concatenate(tags), minlength=num_tags)
    bits = allocate(counts, D[:, 0], D[:, 1], budget)
    return D, bits, counts
