"""GPU: the packed bytes stay bit-exact with the oracle on groups built to land on and next to
rounding ties of (x - zero) / scale, where a quotient that is off by one ulp, or a rounding
that is not half-to-even, changes a code: every 32-token channel group and every 32-channel
token group holds 0 and levels * 2^-k, so scale = 2^-k exactly, and the other values are
(m + 1/2) 2^-k or their fp16 neighbours. Through the prefill append, the decode append (one
token at a time, so groups flush from the tail) and the fused append-and-decode pass. Groups
that hold their own midpoint put (mid - min) / scale within a rounding or two of
(2^b - 1) / 2, where any quotient other than the correctly rounded one can round the other
way."""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

CFGS = [(2, 2, 0, 1), (4, 4, 0, 1), (8, 8, 0, 1), (4, 2, 1, 1), (8, 4, 1, 1), (2, 8, 0, 1)]


def _tie_values(bits, L, k, seed):
    """fp16 [L, 128] for one layer's K or V at this code width."""
    levels = 2 ** bits - 1
    step = 2.0 ** -k
    ties = np.array([(m + 0.5) * step for m in range(levels)], np.float64).astype(np.float16)
    up, down = np.nextafter(ties, np.float16(np.inf)), np.nextafter(ties, np.float16(-np.inf))
    pool = np.concatenate([ties, up, down])
    pool = pool[(pool > 0) & (pool < levels * step)]
    rng = np.random.default_rng(seed)
    x = pool[rng.integers(0, len(pool), (L, 128))]
    j, c = np.meshgrid(np.arange(L), np.arange(128), indexing="ij")
    x = np.where((j + c) % 7 == 0, np.float16(0.0), x)
    x = np.where((j + c) % 7 == 1, np.float16(levels * step), x)
    return x.astype(np.float16)


def _midpoint_values(L, seed, per_token):
    """fp16 [L, 128] whose every group (32 tokens of a channel, or 32 channels of a token when
    per_token) holds its min, its max and their midpoint, so that (mid - min) / scale lies
    within a rounding of the half-integer (2^b - 1) / 2 for every width b."""
    rng = np.random.default_rng(seed)
    x = np.zeros((L, 128), np.float32)
    for g0 in range(0, L if not per_token else 128, 32):
        n = L if per_token else 128
        for k in range(n):
            mn = np.float32(rng.uniform(-20, 20))
            mx = np.float32(np.float16(mn + np.float32(rng.uniform(1e-2, 50))))
            mn = np.float32(np.float16(mn))
            vals = rng.uniform(mn, mx, 32).astype(np.float32)
            vals[rng.permutation(32)[:3]] = [mn, mx, np.float16(mn + (mx - mn) / 2)]
            if per_token:
                x[k, g0:g0 + 32] = vals
            else:
                x[g0:g0 + 32, k] = vals[:min(32, L - g0)]
    return x.astype(np.float16)


def _streams(L, hkv, seed):
    ks, vs = [], []
    for l, (kb, vb, _, _) in enumerate(CFGS):
        ks.append(np.stack([_tie_values(kb, L, 3 + (l + h) % 6, seed + 10 * l + h) for h in range(hkv)]))
        vs.append(np.stack([_tie_values(vb, L, 2 + (l + 2 * h) % 7, seed + 10 * l + h + 5) for h in range(hkv)]))
    return ks, vs


def _check(gpu, oq, plan, cache, ks, vs, L, hkv):
    for l, (kb, vb, ka, _) in enumerate(CFGS):
        lp = plan.layers[l]
        for h in range(hkv):
            sq = oq.quantize_stream(ks[l][h], vs[l][h], kb, vb, ka == 1)
            want, mask = oq.pack_stream(sq, lp.groups_cap)
            a = lp.offset + h * lp.stream_bytes
            got = cache[a:a + lp.stream_bytes].cpu().numpy()
            bad = np.nonzero((want != got) & mask)[0]
            assert bad.size == 0, f"layer {l} K{kb}V{vb} head {h}: {bad.size} bytes differ"


def test_prefill_append_ties(gpu, oq):
    L, hkv = 160, 2
    plan = gpu.plan_layers(gpu.make_shape(hkv * 2, hkv, 1, max_tokens=L), CFGS)
    cache = torch.zeros(plan.total_bytes, dtype=torch.uint8, device="cuda")
    ks, vs = _streams(L, hkv, 1)
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    for l in range(len(CFGS)):
        gpu.quantize_append(plan, l, cache, torch.from_numpy(ks[l][None]).cuda(), torch.from_numpy(vs[l][None]).cuda(),
                            z)
    torch.cuda.synchronize()
    _check(gpu, oq, plan, cache, ks, vs, L, hkv)


def test_prefill_append_midpoints(gpu, oq):
    L, hkv = 96, 2
    plan = gpu.plan_layers(gpu.make_shape(hkv * 2, hkv, 1, max_tokens=L), CFGS)
    cache = torch.zeros(plan.total_bytes, dtype=torch.uint8, device="cuda")
    ks = [np.stack([_midpoint_values(L, 100 * l + h, CFGS[l][2] == 1) for h in range(hkv)]) for l in range(len(CFGS))]
    vs = [np.stack([_midpoint_values(L, 100 * l + h + 50, True) for h in range(hkv)]) for l in range(len(CFGS))]
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    for l in range(len(CFGS)):
        gpu.quantize_append(plan, l, cache, torch.from_numpy(ks[l][None]).cuda(), torch.from_numpy(vs[l][None]).cuda(),
                            z)
    torch.cuda.synchronize()
    _check(gpu, oq, plan, cache, ks, vs, L, hkv)


@pytest.mark.parametrize("fused", [False, True])
def test_token_appends_ties(gpu, oq, fused):
    # 70 tokens one at a time: groups 0 and 1 are flushed by single-token appends
    L, hkv, hq = 70, 2, 4
    plan = gpu.plan_layers(gpu.make_shape(hq, hkv, 1, max_tokens=96), CFGS)
    cache = torch.zeros(plan.total_bytes, dtype=torch.uint8, device="cuda")
    ks, vs = _streams(L, hkv, 2)
    seq = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty(1, hq, 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu.workspace_bytes(plan, 1, 96) // 4 + 1, dtype=torch.float32, device="cuda")
    q = torch.zeros(1, hq, 128, dtype=torch.float16, device="cuda")
    for i in range(L):
        for l in range(len(CFGS)):
            kn = torch.from_numpy(np.ascontiguousarray(ks[l][None, :, i:i + 1])).cuda()
            vn = torch.from_numpy(np.ascontiguousarray(vs[l][None, :, i:i + 1])).cuda()
            if fused:
                gpu.append_decode_attention(plan, l, cache, kn, vn, q, seq, i + 1, 1 / math.sqrt(128), out, None, ws)
            else:
                gpu.quantize_append(plan, l, cache, kn, vn, seq)
        seq += 1
    torch.cuda.synchronize()
    _check(gpu, oq, plan, cache, ks, vs, L, hkv)


def _fp16_range_values(L, seed):
    """fp16 [L, 128] over the whole finite range: random bit patterns (every exponent, both
    signs, so denormals, signed zeros and values up to 65504) in the first 64 channels,
    denormals only in the next 32, and values packed near 1000 in the last 32 (tiny scales
    beside a large zero point)."""
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 16, (L, 128), dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7C00) != 0x7C00
    bits = np.where(finite, bits, bits & 0x83FF)  # exponent 31 -> denormal with the same sign
    x = bits.view(np.float16).copy()
    den = (rng.integers(0, 1 << 10, (L, 32)) | (rng.integers(0, 2, (L, 32)) << 15)).astype(np.uint16)
    x[:, 64:96] = den.view(np.float16)
    x[:, 96:] = (1000.0 + rng.integers(-40, 40, (L, 32)) * 0.5).astype(np.float16)
    return x


def test_prefill_append_full_fp16_range(gpu, oq):
    L, hkv = 96, 2
    plan = gpu.plan_layers(gpu.make_shape(hkv * 2, hkv, 1, max_tokens=L), CFGS)
    cache = torch.zeros(plan.total_bytes, dtype=torch.uint8, device="cuda")
    ks = [np.stack([_fp16_range_values(L, 300 + 10 * l + h) for h in range(hkv)]) for l in range(len(CFGS))]
    vs = [np.stack([_fp16_range_values(L, 400 + 10 * l + h) for h in range(hkv)]) for l in range(len(CFGS))]
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    for l in range(len(CFGS)):
        gpu.quantize_append(plan, l, cache, torch.from_numpy(ks[l][None]).cuda(), torch.from_numpy(vs[l][None]).cuda(),
                            z)
    torch.cuda.synchronize()
    _check(gpu, oq, plan, cache, ks, vs, L, hkv)
