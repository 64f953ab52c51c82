"""GPU parity of the per-tag distortion and of the pool it drives (TriAxialKV page, "Facts":
D_k(b) as attention-output MSE, max over heads, mean over requests, sum over layers; INT2 or
INT4 per tag under an average-bit budget; INT2 tags' tokens in 32-token groups, leftovers
through the INT4 path).

D_k(b) measured with the library's kernels (paged pool + fp16 caches, log-sum-exp merge) must
equal the oracle's, written from the definition with its own quantizer and fp64 attention,
within 1e-3 relative (the kernels' attention is within ~1e-6 of fp64, and D is a mean of
squares of differences two orders larger). The allocation from the library's D must equal the
one from the oracle's, and the pool the library builds from it must be bit-exact with the
oracle's packing of the same tokens through the same page tables."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from layer_wise_mixed_amd import distortion
from layer_wise_mixed_amd.allocate import allocate, int2_tokens
from oracle import distortion as odist
from oracle import pack_paged

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)


def _layers(seed, B, hq, hkv, L, n_layers):
    out = []
    for li in range(n_layers):
        k = syn.keys_fp16(seed, li, range(B), range(hkv), 0, L, outlier_count=4, outlier_factor=10.0,
                          num_kv_heads=hkv)
        v = syn.values_fp16(seed, li, range(B), range(hkv), 0, L)
        q = syn.queries_fp16(seed, li, 0, B, hq)
        out.append((q, k, v))
    return out


@pytest.mark.parametrize("G", [1, 4, 7])
def test_tag_distortion_matches_oracle(gpu, G):
    B, hkv, L, K = 2, 2, 230, 5
    layers = _layers(30 + G, B, G * hkv, hkv, L, 2)
    tags = [np.array(syn.seeded_tags(30 + G, r, L, K, mean_run=24)) for r in range(B)]
    got = distortion.tag_distortion(layers, tags, K, SCALE)
    want = odist.tag_distortion([(q.numpy(), k.numpy(), v.numpy()) for q, k, v in layers], tags, K, SCALE)
    assert np.all(want >= 0) and want.max() > 0
    assert np.allclose(got, want, rtol=1e-3, atol=1e-12), (got, want)


def test_allocation_drives_the_pool(gpu, oq):
    """Calibrate on synthetic tags, allocate at 3.0 bits, append each request's tokens INT2 tags
    first (whole 32-token runs) and the rest INT4: the pool equals the oracle's packing."""
    B, hq, hkv, L, K = 2, 8, 2, 300, 6
    layers = _layers(77, B, hq, hkv, L, 1)
    tags = [np.array(syn.seeded_tags(77, r, L, K, mean_run=40)) for r in range(B)]
    D = distortion.tag_distortion(layers, tags, K, SCALE)
    Do = odist.tag_distortion([(q.numpy(), k.numpy(), v.numpy()) for q, k, v in layers], tags, K, SCALE)
    counts = np.bincount(np.concatenate(tags), minlength=K)
    bits = allocate(counts, D[:, 0], D[:, 1], 3.0)
    assert bits == allocate(counts, Do[:, 0], Do[:, 1], 3.0)
    assert sum(n * b for n, b in zip(counts, bits)) <= 3.0 * counts.sum()
    # the pool, one request at a time, INT2 runs first
    orders = [int2_tokens(tags[r], bits) for r in range(B)]
    n2 = [len(a) for a, _ in orders]
    n4 = [len(b) for _, b in orders]
    pairs = [x // 32 for x in n2]
    quads = [-(-x // 16) for x in n4]
    int2_pages, int4_pages = 2 * sum(pairs), sum(quads)
    max_pages = max(2 * p + qd for p, qd in zip(pairs, quads))
    plan = gpu.plan_layers(gpu.make_shape(hq, hkv, B, page_tokens=16, int2_pages=int2_pages, int4_pages=int4_pages),
                           [(2, 2, 0, 1)])
    pool = torch.zeros(plan.total_bytes, dtype=torch.uint8, device="cuda")
    table = np.zeros((B, max_pages), np.int32)
    p2, p4 = 0, int2_pages
    for r in range(B):
        row = [x for i in range(pairs[r]) for x in (p2 + 2 * i, p2 + 2 * i + 1)] + \
              list(range(p4, p4 + quads[r]))
        p2 += 2 * pairs[r]
        p4 += quads[r]
        table[r, :len(row)] = row
    dtable = torch.from_numpy(table).cuda()
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    _, k, v = layers[0]
    for r in range(B):
        order = torch.tensor(orders[r][0] + orders[r][1], dtype=torch.int64)
        kk = k[r:r + 1].index_select(2, order).contiguous().cuda()
        vv = v[r:r + 1].index_select(2, order).contiguous().cuda()
        add2 = torch.tensor([n2[r]], dtype=torch.int32, device="cuda")
        gpu.quantize_append(plan, 0, pool, kk, vv, None, gpu.make_pages(dtable[r], max_pages, zero[r:], zero[r:], add2))
    torch.cuda.synchronize()
    lp = plan.layers[0]
    want = np.zeros(lp.bytes, np.uint8)
    for r in range(B):
        order = orders[r][0] + orders[r][1]
        for h in range(hkv):
            pack_paged(want, k[r, h, order].numpy(), v[r, h, order].numpy(), n2[r], table[r], int2_pages, hkv, h)
    got = pool[lp.offset:lp.offset + lp.bytes].cpu().numpy()
    assert np.array_equal(got, want)
    assert sum(n2) > 0  # some tag took INT2 at 3.0 bits
