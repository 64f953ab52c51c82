"""Seeded synthetic inputs for the KV-cache quantization path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds no quantization or attention arithmetic: only a
counter-based integer hash (the MurmurHash3 32-bit finalizer, applied to a
counter built from seed, tensor id, layer, request, head, token and channel)
and an Irwin-Hall approximation of N(0, 1): the sum of twelve 16-bit uniform
integers, centred and divided by 2^16. Every step before the final fp32
multiply by an outlier factor and the fp16 rounding is exact integer
arithmetic, so the same call gives the same fp16 bits on the CPU and on the
GPU, and the oracle can regenerate any one (layer, request, head) stream of a
large cache on its own.

The pages describe keys with channel-wise outliers (KVTuner summary page,
"Facts": per-channel quantization wins because keys have channel outliers);
`outlier_channels` picks such channels per (layer, KV head), the same for every
request and token, and `normal_fp16` multiplies them by a factor.
"""
from __future__ import annotations

import torch

MASK32 = 0xFFFFFFFF
GOLDEN = 0x9E3779B9

# tensor ids of the counter
T_K = 1
T_V = 2
T_Q = 3
T_TAG = 4
T_MAP = 5
T_PAGE = 6


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 tensors holding values in [0, 2^32)."""
    lo = c & 0xFFFF
    hi = c >> 16
    return ((x * lo) + (((x * hi) & 0xFFFF) << 16)) & MASK32


def fmix32(x: torch.Tensor) -> torch.Tensor:
    """MurmurHash3 32-bit finalizer on int64 tensors holding uint32 values."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x85EBCA6B)
    x = x ^ (x >> 13)
    x = _mul32(x, 0xC2B2AE35)
    x = x ^ (x >> 16)
    return x


def fmix32_int(x: int) -> int:
    """Scalar form of :func:`fmix32` (Python ints)."""
    x &= MASK32
    x ^= x >> 16
    x = (x * 0x85EBCA6B) & MASK32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & MASK32
    x ^= x >> 16
    return x


def stream_key(seed: int, tensor: int, layer: int, request: int, head: int) -> int:
    h = fmix32_int(seed)
    for i, f in enumerate((tensor, layer, request, head)):
        h = fmix32_int(h ^ fmix32_int((f + (i + 1) * GOLDEN) & MASK32))
    return h


def _stream_keys(seed, tensor, layer, requests, heads, device) -> torch.Tensor:
    keys = [[stream_key(seed, tensor, layer, int(r), int(h)) for h in heads] for r in requests]
    return torch.tensor(keys, dtype=torch.int64, device=device)


def _irwin_hall(keys: torch.Tensor, elem: torch.Tensor) -> torch.Tensor:
    """Sum of 12 uniform 16-bit integers per element, as an exact fp32 N(0,1)-like value."""
    base = fmix32(keys ^ fmix32((elem + GOLDEN) & MASK32))
    s = torch.zeros_like(base)
    for k in range(6):
        w = fmix32((base + (k + 1) * GOLDEN) & MASK32)
        s = s + (w & 0xFFFF) + (w >> 16)
    # 2*s - 12*65535 is an integer in [-786420, 786420]: exact in fp32;
    # dividing by 2^17 is exact too.
    return (2 * s - 12 * 65535).to(torch.float32) / 131072.0


def outlier_channels(seed: int, layer: int, head: int, count: int, head_dim: int = 128) -> list[int]:
    """`count` distinct channels of one (layer, KV head), chosen by hashing."""
    if count <= 0:
        return []
    key = stream_key(seed, T_K + 100, layer, 0, head)
    order = sorted(range(head_dim), key=lambda c: (fmix32_int(key ^ fmix32_int(c + GOLDEN)), c))
    return sorted(order[:count])


def normal_fp16(seed: int, tensor: int, layer: int, requests, heads, tok_start: int, n_tok: int,
                head_dim: int = 128, device="cpu", outliers: dict | None = None) -> torch.Tensor:
    """fp16 tensor [len(requests), len(heads), n_tok, head_dim] of seeded N(0,1)-like values.

    Element (r, h, t, c) depends only on (seed, tensor, layer, r, h, tok_start + t, c).
    `outliers` maps a head index to (list of channels, factor): those channels
    are multiplied by the factor (fp32) before the fp16 rounding.
    """
    requests = list(requests)
    heads = list(heads)
    keys = _stream_keys(seed, tensor, layer, requests, heads, device).view(len(requests), len(heads), 1, 1)
    tok = torch.arange(tok_start, tok_start + n_tok, dtype=torch.int64, device=device).view(1, 1, -1, 1)
    ch = torch.arange(head_dim, dtype=torch.int64, device=device).view(1, 1, 1, -1)
    elem = tok * head_dim + ch
    x = _irwin_hall(keys, elem)
    if outliers:
        mult = torch.ones(len(heads), head_dim, dtype=torch.float32)
        for hi, h in enumerate(heads):
            if h in outliers:
                chans, factor = outliers[h]
                mult[hi, list(chans)] = float(factor)
        x = x * mult.to(device).view(1, len(heads), 1, head_dim)
    return x.to(torch.float16)


def kv_outliers(seed: int, layer: int, num_kv_heads: int, count: int, factor: float, head_dim: int = 128) -> dict:
    return {h: (outlier_channels(seed, layer, h, count, head_dim), factor) for h in range(num_kv_heads)}


def keys_fp16(seed, layer, requests, heads, tok_start, n_tok, *, outlier_count=4, outlier_factor=10.0,
              num_kv_heads=None, head_dim=128, device="cpu") -> torch.Tensor:
    heads = list(heads)
    nk = num_kv_heads if num_kv_heads is not None else (max(heads) + 1 if heads else 0)
    out = kv_outliers(seed, layer, nk, outlier_count, outlier_factor, head_dim)
    return normal_fp16(seed, T_K, layer, requests, heads, tok_start, n_tok, head_dim, device, out)


def values_fp16(seed, layer, requests, heads, tok_start, n_tok, *, head_dim=128, device="cpu") -> torch.Tensor:
    return normal_fp16(seed, T_V, layer, requests, heads, tok_start, n_tok, head_dim, device, None)


def queries_fp16(seed, layer, step, batch, num_q_heads, *, head_dim=128, device="cpu") -> torch.Tensor:
    """q [batch, num_q_heads, head_dim] of one decode step of one layer."""
    x = normal_fp16(seed, T_Q, layer, range(batch), range(num_q_heads), step, 1, head_dim, device)
    return x[:, :, 0, :].contiguous()


def queries_steps_fp16(seed, layer, batch, num_q_heads, step_start, n_steps, *, head_dim=128,
                       device="cpu") -> torch.Tensor:
    """q [batch, num_q_heads, n_steps, head_dim] of consecutive decode steps of one layer
    (step s equals queries_fp16(seed, layer, s, ...))."""
    return normal_fp16(seed, T_Q, layer, range(batch), range(num_q_heads), step_start, n_steps, head_dim, device)


def seeded_choice(seed: int, tensor: int, n: int, k: int, salt: int = 0) -> list[int]:
    """k distinct indices of range(n), chosen by hashing (used for layer maps)."""
    key = stream_key(seed, tensor, salt, 0, 0)
    order = sorted(range(n), key=lambda i: (fmix32_int(key ^ fmix32_int(i + GOLDEN)), i))
    return sorted(order[:k])


def seeded_bits(seed: int, tensor: int, request: int, n: int, device="cpu") -> torch.Tensor:
    """n seeded fair coin flips (int64 0/1) for one request."""
    key = torch.tensor([stream_key(seed, tensor, 0, request, 0)], dtype=torch.int64, device=device)
    idx = torch.arange(n, dtype=torch.int64, device=device)
    return (fmix32(key ^ fmix32((idx + GOLDEN) & MASK32)) >> 7) & 1


def seeded_permutation(seed: int, tensor: int, n: int, salt: int = 0) -> list[int]:
    key = stream_key(seed, tensor, salt, 1, 0)
    return sorted(range(n), key=lambda i: (fmix32_int(key ^ fmix32_int(i + GOLDEN)), i))


def seeded_tags(seed: int, request: int, length: int, num_tags: int, mean_run: int = 48) -> list[int]:
    """A seeded tag per token of one request (arrival order): runs of one tag, each run's length
    uniform in [1, 2 mean_run - 1] and its tag uniform in [0, num_tags). Stands in for the role
    tags of a chat's spans (system prompt, tool output, user turn, ...); no dataset is used."""
    key = stream_key(seed, T_TAG, 0, request, 1)
    out, i = [], 0
    while len(out) < length:
        h = fmix32_int(key ^ fmix32_int((i + GOLDEN) & MASK32))
        run = 1 + h % (2 * mean_run - 1)
        tag = (h >> 16) % num_tags
        out.extend([tag] * run)
        i += 1
    return out[:length]
