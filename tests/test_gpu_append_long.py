"""GPU: a long append (a whole prompt for a full batch in one call) takes the append kernel's
run-per-workgroup path, where each workgroup quantizes a run of consecutive groups of its
stream with the next group's rows already loading. Sampled streams' packed bytes are bit-exact
against the oracle's packing, including the fp16 tail of the ragged end and a second append
that starts mid-group (its first group mixes tail and new tokens)."""
import numpy as np
import pytest
import torch

import synthetic as syn

pytestmark = pytest.mark.gpu

CFGS = [(4, 2, 0, 1), (8, 4, 1, 1), (2, 2, 0, 1)]


@pytest.mark.parametrize("batch,hkv,first,second", [(64, 8, 1090, 0), (16, 4, 700, 2000)])
def test_long_append_bytes(gpu, oq, batch, hkv, first, second):
    L = first + second
    plan = gpu.plan_layers(gpu.make_shape(hkv * 4, hkv, batch, max_tokens=L + 32), CFGS)
    cache = torch.zeros(plan.total_bytes, dtype=torch.uint8, device="cuda")
    seq = torch.zeros(batch, dtype=torch.int32, device="cuda")
    ks = [syn.keys_fp16(13, l, range(batch), range(hkv), 0, L, num_kv_heads=hkv) for l in range(len(CFGS))]
    vs = [syn.values_fp16(13, l, range(batch), range(hkv), 0, L) for l in range(len(CFGS))]
    for l in range(len(CFGS)):
        gpu.quantize_append(plan, l, cache, ks[l][:, :, :first].contiguous().cuda(),
                            vs[l][:, :, :first].contiguous().cuda(), seq)
    if second:
        seq += first
        for l in range(len(CFGS)):
            gpu.quantize_append(plan, l, cache, ks[l][:, :, first:].contiguous().cuda(),
                                vs[l][:, :, first:].contiguous().cuda(), seq)
    torch.cuda.synchronize()
    for l, (kb, vb, ka, _) in enumerate(CFGS):
        lp = plan.layers[l]
        for r in sorted({0, batch // 3, batch - 1}):
            for h in sorted({0, hkv - 1}):
                sq = oq.quantize_stream(ks[l][r, h].numpy(), vs[l][r, h].numpy(), kb, vb, ka == 1)
                want, mask = oq.pack_stream(sq, lp.groups_cap)
                a = lp.offset + (r * hkv + h) * lp.stream_bytes
                got = cache[a:a + lp.stream_bytes].cpu().numpy()
                bad = np.nonzero((want != got) & mask)[0]
                assert bad.size == 0, f"layer {l} K{kb}V{vb} r{r} h{h}: {bad.size} bytes differ"
