"""GPU parity of the whole chunked-prefill attention (kvq_chunk_prefill_attention), through the
C ABI: every query row of a chunk attends to its request's cached prefix as stored and, causally,
to the chunk's own fp16 tokens, in one softmax (the prefix splits and the chunk part merged by
log-sum-exp on the device). Checked against the oracle's chunk_prefill (fp64 softmax over the
dequantized prefix followed by the chunk's fp16 tokens 0..i) at rel L2 <= 1e-3 per (request, KV
head), max abs <= 2e-3 and lse within 1e-4. Cases: empty, one-token, group-less-one, one-group,
ragged and long prefixes; chunks of 1, 5, 33 (two key blocks) and 70 tokens (a ragged last row
block for G = 7); G = 1, 4 and 7; one prefix split and several."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from test_gpu_parity import Case, check_attention

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)


def _chunk_inputs(c, l, chunk):
    """The chunk's tokens are the tokens right after each request's prefix in the synthetic stream:
    q [B, chunk, Hq, 128]; k, v [B, Hkv, chunk, 128]."""
    B = c.batch
    q = syn.queries_steps_fp16(c.seed, l, B, c.hq, 500, chunk).permute(0, 2, 1, 3).contiguous()
    ks, vs = [], []
    for r in range(B):
        L = c.lens[r]
        ks.append(syn.keys_fp16(c.seed, l, [r], range(c.hkv), L, chunk, outlier_count=c.outliers[0],
                                outlier_factor=c.outliers[1], num_kv_heads=c.hkv))
        vs.append(syn.values_fp16(c.seed, l, [r], range(c.hkv), L, chunk))
    return q, torch.cat(ks).contiguous(), torch.cat(vs).contiguous()


@pytest.mark.parametrize("G,chunk,splits", [(4, 5, 0), (4, 33, 1), (1, 70, 3), (7, 70, 0), (4, 1, 2), (7, 33, 1)])
def test_chunk_prefill_matches_oracle(gpu, oq, G, chunk, splits):
    lens = [37, 0, 1, 31, 32, 150, 200]
    c = Case(gpu, oq, hq=2 * G, hkv=2, batch=len(lens), cap=224, cfgs=[(4, 2), (8, 4, 1), (16, 16)], lens=lens,
             seed=90 + G)
    for l in range(len(c.cfgs)):
        q, kc, vc = _chunk_inputs(c, l, chunk)
        ml = max(lens)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        wsb = gpu.chunk_prefill_workspace_bytes(c.plan, c.batch, chunk, ml, splits)
        ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device="cuda")
        gpu.chunk_prefill_attention(c.plan, l, c.cache, q.cuda(), kc.cuda(), vc.cuda(), c.seq, ml, SCALE, out, lse,
                                    ws, splits)
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        kb, vb, ka, _ = c.cfgs[l]
        ref = np.zeros(out.shape)
        ref_lse = np.zeros(lse.shape)
        for r in range(c.batch):
            L = lens[r]
            for h in range(c.hkv):
                o, ls = oq.chunk_prefill(q[r, :, h * G:(h + 1) * G].numpy(), c.k[l][r, h, :L].numpy(),
                                         c.v[l][r, h, :L].numpy(), kc[r, h].numpy(), vc[r, h].numpy(), kb, vb,
                                         ka == 1, SCALE)
                ref[r, :, h * G:(h + 1) * G] = o
                ref_lse[r, :, h * G:(h + 1) * G] = ls
        # rows of one (request, chunk token) as the "requests" of the batch-level check, then per
        # (request, KV head) over all chunk tokens
        n = c.batch * chunk
        try:
            check_attention(out.reshape(n, c.hq, 128), lse.reshape(n, c.hq), ref.reshape(n, c.hq, 128),
                            ref_lse.reshape(n, c.hq), [1] * n, c.hq, c.hkv)
        except AssertionError as e:
            raise AssertionError(f"layer {l} {c.cfgs[l]}: {e}") from None
        assert np.isfinite(out).all()


