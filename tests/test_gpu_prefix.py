"""GPU parity of the prefix attention of chunked prefill (kvq_prefix_attention), through the
C ABI: every query row of a chunk attends to its request's whole cached prefix. Its output
and log-sum-exp meet the decode tolerance (rel L2 <= 1e-3, max abs <= 2e-3, lse 1e-4)
against the oracle's fp64 attention of the same rows over the oracle's own quantization of
the prefix; merged by log-sum-exp with the chunk's own causal attention they give the
oracle's chunked-prefill attention. The cases cover an empty prefix, one token, a group
less one, a whole group, ragged tails and a prefix at capacity; chunks of one token, of a
ragged last row tile and of several tiles; GQA groups of 1, 3, 4 and 16 query heads (16, 15,
16 and 16 rows a tile); one split and several (the merge pass)."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from test_gpu_parity import MIXED, Case, check_attention

pytestmark = pytest.mark.gpu

SCALE = 1 / math.sqrt(128)
LENS = [37, 0, 1, 31, 32, 150, 200]


def chunk_queries(seed, l, batch, hq, start, chunk):
    """q [batch, chunk, Hq, 128] of chunk tokens start .. start + chunk - 1."""
    return syn.queries_steps_fp16(seed, l, batch, hq, start, chunk).permute(0, 2, 1, 3).contiguous()


def run_prefix(gpu, c, l, q, splits, max_len=None):
    batch, chunk = q.shape[0], q.shape[1]
    max_len = max(c.lens) if max_len is None else max_len
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    wsb = gpu.prefix_workspace_bytes(c.plan, batch, chunk, max_len, splits)
    ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device="cuda") if wsb else None
    gpu.prefix_attention(c.plan, l, c.cache, q.cuda(), c.seq, max_len, SCALE, out, lse, ws, splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_prefix(oq, c, l, q):
    """fp64 (out, lse) of every chunk row over its request's quantized prefix."""
    batch, chunk = q.shape[0], q.shape[1]
    G = c.hq // c.hkv
    kb, vb, ka, _ = c.cfgs[l]
    out = np.zeros((batch, chunk, c.hq, 128))
    lse = np.zeros((batch, chunk, c.hq))
    for r in range(batch):
        L = c.lens[r]
        for h in range(c.hkv):
            rows = q[r, :, h * G:(h + 1) * G].reshape(chunk * G, 128).numpy()
            o, ls = oq.decode_stream(rows, c.k[l][r, h, :L].numpy(), c.v[l][r, h, :L].numpy(), kb, vb, ka == 1,
                                     SCALE)
            out[r, :, h * G:(h + 1) * G] = o.reshape(chunk, G, 128)
            lse[r, :, h * G:(h + 1) * G] = ls.reshape(chunk, G)
    return out, lse


@pytest.fixture(scope="module")
def cases(gpu, oq):
    return {(hq, hkv): Case(gpu, oq, hq=hq, hkv=hkv, batch=len(LENS), cap=200, cfgs=MIXED, lens=LENS, seed=21)
            for hq, hkv in [(8, 2), (6, 2), (16, 1), (2, 2)]}


@pytest.mark.parametrize("hq,hkv,chunk,splits", [(8, 2, 1, 1), (8, 2, 11, 0), (8, 2, 16, 3), (6, 2, 7, 1),
                                                 (16, 1, 3, 2), (2, 2, 17, 0)])
def test_prefix_matches_oracle(gpu, oq, cases, hq, hkv, chunk, splits):
    c = cases[(hq, hkv)]
    for l in range(len(c.cfgs)):
        q = chunk_queries(c.seed, l, c.batch, hq, 200, chunk)
        out, lse = run_prefix(gpu, c, l, q, splits)
        ref, ref_lse = oracle_prefix(oq, c, l, q)
        try:
            check_attention(out.reshape(c.batch, -1, 128), lse.reshape(c.batch, -1), ref.reshape(c.batch, -1, 128),
                            ref_lse.reshape(c.batch, -1), c.lens, hq)
        except AssertionError as e:
            raise AssertionError(f"layer {l} {c.cfgs[l]}: {e}") from None


def test_splits_agree(gpu, cases, oq):
    # one split and several give the same rows to within the operand rounding: the P.V
    # operands (weight and value) are each rounded once to fp16, at most 2^-11 relative, so
    # a row's output is within 2^-10 max|v| of exact and two of them within 2^-9 max|v|
    # (max over the request's dequantized values); the log-sum-exp comes from fp32 sums of
    # the unrounded weights and agrees to 1e-5
    c = cases[(8, 2)]
    q = chunk_queries(c.seed, 0, c.batch, 8, 200, 9)
    a, la = run_prefix(gpu, c, 0, q, 1)
    b, lb = run_prefix(gpu, c, 0, q, 4)
    kb, vb, ka, _ = c.cfgs[0]
    for r, L in enumerate(c.lens):
        if L == 0:
            continue
        vmax = max(np.abs(oq.dequant_stream(oq.quantize_stream(c.k[0][r, h, :L].numpy(), c.v[0][r, h, :L].numpy(),
                                                               kb, vb, ka == 1))[1]).max() for h in range(c.hkv))
        np.testing.assert_allclose(b[r], a[r], rtol=0, atol=2.0 ** -9 * vmax)
        np.testing.assert_allclose(lb[r], la[r], rtol=0, atol=1e-5)


def test_merged_with_chunk_part_is_chunked_prefill(gpu, oq, cases):
    # the prefix part merged (fp64, here) with the chunk's own causal part is the oracle's
    # attention of the chunk over the quantized prefix plus its own fp16 tokens
    c = cases[(8, 2)]
    G, chunk = 4, 5
    for l in (0, 1, 3):
        kb, vb, ka, _ = c.cfgs[l]
        q = chunk_queries(c.seed, l, c.batch, 8, 200, chunk)
        out, lse = run_prefix(gpu, c, l, q, 0)
        kc = syn.keys_fp16(c.seed, l, range(c.batch), range(c.hkv), 200, chunk, outlier_count=c.outliers[0],
                           outlier_factor=c.outliers[1], num_kv_heads=c.hkv)
        vc = syn.values_fp16(c.seed, l, range(c.batch), range(c.hkv), 200, chunk)
        got, want = [], []
        for r in range(c.batch):
            L = c.lens[r]
            for h in range(c.hkv):
                qr = q[r, :, h * G:(h + 1) * G].numpy()
                wo, _ = oq.chunk_prefill(qr, c.k[l][r, h, :L].numpy(), c.v[l][r, h, :L].numpy(), kc[r, h].numpy(),
                                         vc[r, h].numpy(), kb, vb, ka == 1, SCALE)
                for i in range(chunk):
                    oc, lc = oq.attention(qr[i], kc[r, h, :i + 1].float().numpy(), vc[r, h, :i + 1].float().numpy(),
                                          SCALE)
                    lp = lse[r, i, h * G:(h + 1) * G].astype(np.float64)
                    m = np.maximum(lp, lc)
                    wp, wc = np.exp(lp - m), np.exp(lc - m)
                    op = out[r, i, h * G:(h + 1) * G].astype(np.float64)
                    got.append((wp[:, None] * op + wc[:, None] * oc) / (wp + wc)[:, None])
                    want.append(wo[i])
        got, want = np.concatenate(got), np.concatenate(want)
        rel = np.linalg.norm(got - want) / np.linalg.norm(want)
        assert rel <= 1e-3 and np.abs(got - want).max() <= 2e-3, f"layer {l}: rel {rel:.3g}"


def test_large_chunk_sampled(gpu, oq):
    # a long prefix and a 256-token chunk (64 row tiles a KV head): sampled rows of a few
    # tiles against the oracle, every row finite and every lse within the prefix's range
    hq, hkv, L, chunk = 32, 8, 2048, 256
    c = Case(gpu, oq, hq=hq, hkv=hkv, batch=2, cap=L, cfgs=[(4, 2), (8, 8)], lens=[L, L - 45], seed=5)
    for l in range(2):
        q = chunk_queries(c.seed, l, 2, hq, L, chunk)
        out, lse = run_prefix(gpu, c, l, q, 0)
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        kb, vb, ka, _ = c.cfgs[l]
        G = hq // hkv
        for r in range(2):
            for h in (0, 5):
                for i in (0, 1, 129, 255):
                    rows = q[r, i, h * G:(h + 1) * G].numpy()
                    o, ls = oq.decode_stream(rows, c.k[l][r, h, :c.lens[r]].numpy(), c.v[l][r, h, :c.lens[r]].numpy(),
                                             kb, vb, ka == 1, SCALE)
                    got = out[r, i, h * G:(h + 1) * G]
                    rel = np.linalg.norm(got - o) / np.linalg.norm(o)
                    assert rel <= 1e-3 and np.abs(got - o).max() <= 2e-3, f"l{l} r{r} h{h} i{i}: rel {rel:.3g}"
                    assert np.abs(lse[r, i, h * G:(h + 1) * G] - ls).max() <= 1e-4


@pytest.mark.parametrize("hq,hkv,chunk,splits", [(14, 2, 100, 0), (6, 2, 200, 3), (28, 4, 40, 1)])
def test_row_blocks_split_a_token(gpu, oq, hq, hkv, chunk, splits):
    # a workgroup takes 256 rows; with G = 7 or 3 a chunk token's query heads straddle two
    # row blocks, and every row must still land in its own place
    c = Case(gpu, oq, hq=hq, hkv=hkv, batch=3, cap=160, cfgs=[(4, 2), (8, 4, 1), (2, 8)], lens=[160, 77, 5], seed=8)
    for l in range(len(c.cfgs)):
        q = chunk_queries(c.seed, l, c.batch, hq, 160, chunk)
        out, lse = run_prefix(gpu, c, l, q, splits)
        ref, ref_lse = oracle_prefix(oq, c, l, q)
        try:
            check_attention(out.reshape(c.batch, -1, 128), lse.reshape(c.batch, -1), ref.reshape(c.batch, -1, 128),
                            ref_lse.reshape(c.batch, -1), c.lens, hq)
        except AssertionError as e:
            raise AssertionError(f"layer {l} {c.cfgs[l]}: {e}") from None
