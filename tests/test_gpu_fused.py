"""GPU tests of the fused append-and-decode entry point (kvq_append_decode_attention),
through the C ABI: after every step the cache bytes and the attention output and
log-sum-exp equal, bit for bit, those of kvq_quantize_append(n_new = 1) followed by
kvq_decode_attention on a copy of the same cache, and the output meets the oracle's
tolerance (rel L2 <= 1e-3, max abs <= 2e-3) on the oracle's own quantization of the
same token sequence. The lengths cover an empty stream, tail writes, single-token
flushes of the first, a middle and the last group, and a stream at capacity (no
append); the splits cover one split (final output from the split pass) and several
(the flush group and the tail in different splits)."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from test_gpu_parity import Case, check_attention

pytestmark = pytest.mark.gpu

# K8V8, K4V2, K4V4 per-token keys, K16V16, K2V8, K8V16 per-token keys
CFGS = [(8, 8), (4, 2), (4, 4, 1), (16, 16), (2, 8), (8, 16, 1)]
CAP = 160
LENS0 = [0, 30, 31, 62, 95, 158, 160]
SCALE = 1 / math.sqrt(128)


def _new_tokens(c, l, lens):
    """Token lens[r] of every request (the synthetic stream continues by position)."""
    ks = [syn.keys_fp16(c.seed, l, [r], range(c.hkv), lens[r], 1, outlier_count=c.outliers[0],
                        outlier_factor=c.outliers[1], num_kv_heads=c.hkv) for r in range(c.batch)]
    vs = [syn.values_fp16(c.seed, l, [r], range(c.hkv), lens[r], 1) for r in range(c.batch)]
    return torch.cat(ks).contiguous().cuda(), torch.cat(vs).contiguous().cuda()


def _buffers(gpu, c, max_len, splits):
    out = torch.full((c.batch, c.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((c.batch, c.hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu.workspace_bytes(c.plan, c.batch, max_len, splits) // 4 + 1, dtype=torch.float32,
                     device="cuda")
    return out, lse, ws


# G = 4 with one split and several, then every GQA group size class the split pass
# instantiates: 4 column slots (G <= 4), 2 slots (G 5..8, G = 8 filling all 16 columns) and
# one slot (G 9..16)
@pytest.mark.parametrize("hq,hkv,splits", [(8, 2, 1), (8, 2, 3), (7, 1, 0), (2, 1, 0), (6, 2, 2), (10, 2, 0),
                                           (12, 2, 0), (16, 2, 3), (9, 1, 0), (24, 2, 0), (16, 1, 2)])
def test_fused_equals_separate_calls_and_oracle(gpu, oq, hq, hkv, splits):
    a = Case(gpu, oq, hq=hq, hkv=hkv, batch=len(LENS0), cap=CAP, cfgs=CFGS, lens=LENS0, seed=11)
    b = Case(gpu, oq, hq=hq, hkv=hkv, batch=len(LENS0), cap=CAP, cfgs=CFGS, lens=LENS0, seed=11)
    assert torch.equal(a.cache, b.cache)
    lens = list(LENS0)
    for step in range(3):
        after = [min(L + 1, CAP) for L in lens]
        max_len = max(after)
        seq_before = torch.tensor(lens, dtype=torch.int32, device="cuda")
        seq_b = seq_before.clone()
        seq_after = torch.tensor(after, dtype=torch.int32, device="cuda")
        outs = []
        for l in range(len(CFGS)):
            q = syn.queries_fp16(a.seed, l, step, a.batch, hq).cuda()
            kn, vn = _new_tokens(a, l, lens)
            out_a, lse_a, ws_a = _buffers(gpu, a, max_len, splits)
            gpu.append_decode_attention(a.plan, l, a.cache, kn, vn, q, seq_before, max_len, SCALE, out_a, lse_a,
                                        ws_a, splits)
            out_b, lse_b, ws_b = _buffers(gpu, b, max_len, splits)
            gpu.quantize_append(b.plan, l, b.cache, kn, vn, seq_b)
            gpu.decode_attention(b.plan, l, b.cache, q, seq_after, max_len, SCALE, out_b, lse_b, ws_b, splits)
            torch.cuda.synchronize()
            oa, la, ob, lb = (t.cpu().numpy() for t in (out_a, lse_a, out_b, lse_b))
            assert np.array_equal(oa, ob) and np.array_equal(la, lb), f"step {step} layer {l} {CFGS[l]}"
            outs.append((q, oa, la))
        assert torch.equal(a.cache, b.cache), f"step {step}: cache bytes differ"
        # the oracle on the same token sequence, now `after` long
        a.lens = after
        for l in range(len(CFGS)):
            a.k[l] = syn.keys_fp16(a.seed, l, range(a.batch), range(hkv), 0, max_len, outlier_count=a.outliers[0],
                                   outlier_factor=a.outliers[1], num_kv_heads=hkv)
            a.v[l] = syn.values_fp16(a.seed, l, range(a.batch), range(hkv), 0, max_len)
            q, oa, la = outs[l]
            ref, ref_lse = a.oracle_decode(l, q)
            check_attention(oa, la, ref, ref_lse, after, hq, hkv)
        lens = after


def test_fused_every_tail_slot(gpu, oq):
    """One fused step per tail slot: the new token lands in slot 0 .. 30 of the tail (or
    completes the group), which the split pass merges into the tail pieces it reads; bit for
    bit the separate calls, and within the oracle's tolerance."""
    lens = [64 + t for t in range(32)]
    cfgs = [(8, 8), (4, 2), (16, 16)]
    a = Case(gpu, oq, hq=8, hkv=2, batch=len(lens), cap=100, cfgs=cfgs, lens=lens, seed=15)
    b = Case(gpu, oq, hq=8, hkv=2, batch=len(lens), cap=100, cfgs=cfgs, lens=lens, seed=15)
    after = [L + 1 for L in lens]
    seq_before = torch.tensor(lens, dtype=torch.int32, device="cuda")
    seq_after = torch.tensor(after, dtype=torch.int32, device="cuda")
    outs = []
    for l in range(len(cfgs)):
        q = syn.queries_fp16(a.seed, l, 0, a.batch, 8).cuda()
        kn, vn = _new_tokens(a, l, lens)
        out_a, lse_a, ws_a = _buffers(gpu, a, max(after), 0)
        gpu.append_decode_attention(a.plan, l, a.cache, kn, vn, q, seq_before.clone(), max(after), SCALE, out_a,
                                    lse_a, ws_a, 0)
        out_b, lse_b, ws_b = _buffers(gpu, b, max(after), 0)
        gpu.quantize_append(b.plan, l, b.cache, kn, vn, seq_before.clone())
        gpu.decode_attention(b.plan, l, b.cache, q, seq_after, max(after), SCALE, out_b, lse_b, ws_b, 0)
        torch.cuda.synchronize()
        oa, la, ob, lb = (t.cpu().numpy() for t in (out_a, lse_a, out_b, lse_b))
        assert np.array_equal(oa, ob) and np.array_equal(la, lb), f"layer {l} {cfgs[l]}"
        outs.append((q, oa, la))
    assert torch.equal(a.cache, b.cache)
    a.lens = after
    for l in range(len(cfgs)):
        a.k[l] = syn.keys_fp16(a.seed, l, range(a.batch), range(2), 0, max(after), outlier_count=a.outliers[0],
                               outlier_factor=a.outliers[1], num_kv_heads=2)
        a.v[l] = syn.values_fp16(a.seed, l, range(a.batch), range(2), 0, max(after))
        q, oa, la = outs[l]
        ref, ref_lse = a.oracle_decode(l, q)
        check_attention(oa, la, ref, ref_lse, after, 8)


def test_fused_packed_groups_match_oracle_packing(gpu, oq):
    """The groups the fused pass completes are packed exactly as the oracle packs them."""
    c = Case(gpu, oq, hq=8, hkv=2, batch=3, cap=96, cfgs=[(4, 2), (8, 4, 1)], lens=[31, 63, 95], seed=4)
    after = [32, 64, 96]
    seq = torch.tensor(c.lens, dtype=torch.int32, device="cuda")
    for l in range(2):
        q = syn.queries_fp16(4, l, 0, c.batch, c.hq).cuda()
        kn, vn = _new_tokens(c, l, c.lens)
        out, lse, ws = _buffers(gpu, c, 96, 0)
        gpu.append_decode_attention(c.plan, l, c.cache, kn, vn, q, seq, 96, SCALE, out, lse, ws, 0)
    torch.cuda.synchronize()
    c.lens = after
    for l in range(2):
        c.k[l] = syn.keys_fp16(4, l, range(3), range(2), 0, 96, num_kv_heads=2)
        c.v[l] = syn.values_fp16(4, l, range(3), range(2), 0, 96)
        for r in range(3):
            for h in range(2):
                want, mask = oq.pack_stream(c.oracle_stream(l, r, h), c.plan.layers[l].groups_cap)
                got = c.stream_bytes(l, r, h)
                bad = np.nonzero((want != got) & mask)[0]
                assert bad.size == 0, f"layer {l} r{r} h{h}: {bad.size} bytes differ"
