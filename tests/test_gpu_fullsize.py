"""Parity at full size. The benchmark's workloads are built exactly as the benchmark builds them
(a subset of their layers: each built layer has the benchmark's shapes, data, split count and
launches), stepped through their decode cycle with the benchmark's own step (the token append
fused into the decode split pass, for contiguous caches and for the paged pool),
and checked on sampled (request, KV head) streams: packed bytes bit-exact against the oracle's
packing of the regenerated stream, attention within the stated tolerance of the oracle's fp64
attention. Every other request of the batch is computed in the same launches. The fused step's
own output (fp16, last built layer) must equal bit for bit a separate decode over the cache it
left."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import synthetic as syn
from test_gpu_parity import MAX_ABS, REL_L2, lse_tolerance

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def _requests(B):
    return sorted({0, B // 2, B - 1})


def _decode32(wl, l, pos, pages=None, seq=None):
    kvq = wl.kvq
    out = torch.full((wl.B, wl.Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((wl.B, wl.Hq), float("nan"), dtype=torch.float32, device="cuda")
    kvq.decode_attention(wl.plan, l, wl.cache, wl.q[l][pos], seq, wl.max_len, wl.scale, out, lse, wl.ws, wl.splits,
                         pages=pages)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _compare(got, got_lse, ref, ref_lse, what, lse_tol):
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    mx = np.abs(got - ref).max()
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{what}: rel L2 {rel:.3g}, max abs {mx:.3g}"
    err = np.abs(got_lse - ref_lse)
    assert np.all(err <= lse_tol), f"{what}: lse error {err.max():.3g} > {lse_tol[np.argmax(err - lse_tol)]:.3g}"


def _keys(wl, li, r, h, n):
    cnt, fac = wl.outliers
    return syn.keys_fp16(wl.seed, li, [r], [h], 0, n, outlier_count=cnt, outlier_factor=fac,
                         num_kv_heads=wl.Hkv)[0, 0].numpy()


CONTIGUOUS = [
    # workload, layers to build, decode-cycle positions to check
    ("single-head-k8v4-l512", [0], [0]),
    ("llama31-8b-b64-kivi8-trace", [0, 31], [0, 31, 127]),
    ("llama31-8b-b64-mixed325-l2048", None, [0, 31]),
    ("qwen25-7b-b32-map396-l8192", None, [0, 31]),
]


def _mixed_layers(name, seed=0):
    """One layer of each (bK, bV) pair of the workload's map."""
    cfg = bench.WORKLOADS[name]["map"](seed)
    first = {}
    for i, c in enumerate(cfg):
        first.setdefault(tuple(c), i)
    return sorted(first.values())


@pytest.mark.parametrize("name,layers,positions", CONTIGUOUS, ids=[c[0] for c in CONTIGUOUS])
def test_fullsize_contiguous(gpu, oq, name, layers, positions):
    layers = layers if layers is not None else _mixed_layers(name)
    print(f"[fullsize] {name} layers {layers}", flush=True)
    wl = bench.Workload(name, layers=layers)
    wl.reset()
    G = wl.Hq // wl.Hkv
    for pos in range(max(positions) + 1):
        wl.step(pos)
        if pos not in positions:
            continue
        torch.cuda.synchronize()
        L = wl.P + pos + 1
        if wl.fused:
            last = wl.L - 1
            out16 = torch.full_like(wl.out, float("nan"))
            wl.kvq.decode_attention(wl.plan, last, wl.cache, wl.q[last][pos], wl.lens_before, wl.max_len, wl.scale,
                                    out16, None, wl.ws, wl.splits)
            torch.cuda.synchronize()
            assert torch.equal(out16, wl.out), f"{name} L{L}: fused step output differs from a decode after it"
        for l, li in enumerate(wl.layer_ids):
            lp = wl.plan.layers[l]
            kb, vb, kt = lp.k_bits, lp.v_bits, lp.k_axis == 1
            out, lse = _decode32(wl, l, pos, seq=wl.lens_before)
            q = wl.q[l][pos].cpu()
            for r in _requests(wl.B):
                for h in range(wl.Hkv):
                    k, v = _keys(wl, li, r, h, L), syn.values_fp16(wl.seed, li, [r], [h], 0, L)[0, 0].numpy()
                    sq = oq.quantize_stream(k, v, kb, vb, kt)
                    want, mask = oq.pack_stream(sq, lp.groups_cap)
                    a = lp.offset + (r * wl.Hkv + h) * lp.stream_bytes
                    got = wl.cache[a:a + lp.stream_bytes].cpu().numpy()
                    bad = np.nonzero((want != got) & mask)[0]
                    assert bad.size == 0, f"{name} layer {li} r{r} h{h} L{L}: {bad.size} bytes differ"
                    qr = q[r, h * G:(h + 1) * G].numpy()
                    kd, vd = oq.dequant_stream(sq)
                    ref, ref_lse = oq.attention(qr, kd, vd, wl.scale)
                    _compare(out[r, h * G:(h + 1) * G], lse[r, h * G:(h + 1) * G], ref, ref_lse,
                             f"{name} layer {li} r{r} h{h} L{L}", lse_tolerance(qr, kd, wl.scale))


@pytest.mark.parametrize("positions", [[0, 31]])
def test_fullsize_paged(gpu, oq, positions):
    name = "paged-b16-l32768-int2int4"
    print(f"[fullsize] {name} layer 0", flush=True)
    wl = bench.PagedWorkload(name, layers=[0])
    wl.reset()
    G = wl.Hq // wl.Hkv
    li = wl.layer_ids[0]
    lp = wl.plan.layers[0]
    table = wl.table.cpu().numpy()
    hkv = wl.Hkv
    for pos in range(max(positions) + 1):
        wl.step(pos)
        if pos not in positions:
            continue
        torch.cuda.synchronize()
        pages = wl.kvq.make_pages(wl.table, wl.max_pages, wl.n2_dev, wl.n4_before)
        out, lse = _decode32(wl, 0, pos, pages=pages)
        q = wl.q[0][pos].cpu()
        region = wl.cache[lp.offset:lp.offset + lp.bytes].cpu().numpy()
        for r in _requests(wl.B):
            n2, n4 = wl.n2s[r], wl.P - wl.n2s[r] + pos + 1
            order = wl._prompt_order(r) + list(range(wl.P, wl.P + pos + 1))
            np2, np4 = n2 // 16, -(-n4 // 16)
            compact = np.arange(np2 + np4, dtype=np.int32)  # the oracle's own placement
            pool = np.zeros(oq.paged_pool_bytes(hkv, np2, np4), np.uint8)
            mask = np.zeros_like(pool)
            for h in range(hkv):
                k = _keys(wl, li, r, h, wl.P + pos + 1)[order]
                v = syn.values_fp16(wl.seed, li, [r], [h], 0, wl.P + pos + 1)[0, 0].numpy()[order]
                oq.pack_paged(pool, k, v, n2, compact, np2, hkv, h, mask)
                kd, vd = oq.unpack_paged(pool, n2, n4, compact, np2, hkv, h)
                qr = q[r, h * G:(h + 1) * G].numpy()
                ref, ref_lse = oq.attention(qr, kd, vd, wl.scale)
                _compare(out[r, h * G:(h + 1) * G], lse[r, h * G:(h + 1) * G], ref, ref_lse,
                         f"paged r{r} h{h} n4 {n4}", lse_tolerance(qr, kd, wl.scale))
            # bytes: every INT2 record and INT4 page of the request, at its physical page
            for m in range(n2 // 32):
                g0 = int(table[r, 2 * m]) * lp.int2_page_bytes
                o0 = 2 * m * hkv * 2048
                assert np.array_equal(region[g0:g0 + hkv * 4096], pool[o0:o0 + hkv * 4096]), f"INT2 group {m}"
            int4_base = np2 * hkv * 2048
            for t in range(np4):
                g0 = lp.int4_offset + (int(table[r, np2 + t]) - wl.int2_pages) * lp.int4_page_bytes
                o0 = int4_base + t * hkv * 3072
                sl = slice(o0, o0 + hkv * 3072)
                bad = np.nonzero((region[g0:g0 + hkv * 3072] != pool[sl]) & (mask[sl] != 0))[0]
                assert bad.size == 0, f"INT4 page {t}: {bad.size} bytes differ"
