"""Pins of the oracle's paged INT2/INT4 pool (TriAxialKV page, "Facts": page pools split at an
offset, INT2 per-channel keys and per-token values, INT4 per-token keys and values, leftover
INT2 tokens routed to INT4, page tables listing INT2 pages before INT4 pages).

The page layout is this project's own. It is pinned three ways: hand-worked sites
(tests/golden/page_sites.json), its relation to the already pinned 32-token record layout (an
INT2 page pair is one K2V2 record per KV head; two INT4 pages are the two token halves of a
K4V4 per-token record, with V words interleaved bytewise), and invariants that do not depend
on any layout (page permutation, closed-form quantizer cases)."""
import json
import os

import numpy as np
import pytest

import synthetic as syn

HERE = os.path.dirname(os.path.abspath(__file__))
SITES = json.load(open(os.path.join(HERE, "golden", "page_sites.json")))
HKV = 2
PAGE = 16


def _tokens(seed, L, head=0):
    k = syn.keys_fp16(seed, 0, [0], [head], 0, L, outlier_count=4, outlier_factor=10.0, num_kv_heads=HKV)
    v = syn.values_fp16(seed, 0, [0], [head], 0, L)
    return k[0, 0].numpy(), v[0, 0].numpy()


def _pool(int2_pages, int4_pages, oq):
    return np.zeros(oq.paged_pool_bytes(HKV, int2_pages, int4_pages), np.uint8)


def _table(n2, n4, int2_pages, int4_pages, seed):
    """A shuffled page table: n2/32 INT2 pairs drawn from the INT2 region, then ceil(n4/16)
    INT4 pages drawn from the INT4 region."""
    pairs = syn.seeded_permutation(seed, syn.T_PAGE, int2_pages // 2)[: n2 // 32]
    quads = syn.seeded_permutation(seed, syn.T_PAGE, int4_pages, salt=1)[: (n4 + PAGE - 1) // PAGE]
    t = []
    for p in pairs:
        t += [2 * int(p), 2 * int(p) + 1]
    t += [int2_pages + int(x) for x in quads]
    return np.array(t, np.int32)


def test_worked_page_sites(oq):
    for s in SITES["k_sites"]:
        assert oq.page_k_site(s["p"], s["c"]) == (s["byte"], s["shift"]), s["why"]
    for s in SITES["v_sites"]:
        assert oq.page_v_site(s["p"], s["c"]) == (s["byte"], s["shift"]), s["why"]
    for s in SITES["meta"]:
        assert oq.page_meta_index(s["p"], s["n"]) == s["index"]


def test_page_sites_are_a_bijection(oq):
    """16 slots x 128 channels x 4 bits fill each 1 KiB code block exactly once."""
    for f, base in ((oq.page_k_site, 0), (oq.page_v_site, 1024)):
        bits = set()
        for p in range(16):
            for c in range(128):
                b, sh = f(p, c)
                assert base <= b < base + 1024 and b % 4 == 0 and sh % 4 == 0 and 0 <= sh <= 28
                bits.add((b, sh))
        assert len(bits) == 16 * 128
    assert sorted(oq.page_meta_index(p, n) for p in range(16) for n in range(4)) == list(range(64))


@pytest.mark.parametrize("site", SITES["k_sites"] + SITES["v_sites"], ids=lambda s: f"p{s['p']}c{s['c']}_{s['byte']}")
def test_single_code_lands_on_worked_page_site(oq, site):
    """One INT4 token whose only non-zero channel is c0 (value 1) has exactly one non-zero code,
    15, in that channel; every other code of the page is 0."""
    is_v = site["byte"] >= 1024
    k = np.zeros((PAGE, 128), np.float16)
    v = np.zeros((PAGE, 128), np.float16)
    (v if is_v else k)[site["p"], site["c"]] = 1.0
    int2_pages, int4_pages = 0, 1
    pool = _pool(int2_pages, int4_pages, oq)
    oq.pack_paged(pool, k, v, 0, [0], int2_pages, HKV, 0)
    page = pool[:3072]
    codes = page[:2048]
    word = int.from_bytes(bytes(codes[site["byte"]:site["byte"] + 4]), "little")
    assert word == 15 << site["shift"]
    assert int(np.count_nonzero(codes)) == 1


def test_int2_pair_is_a_k2v2_record(oq):
    """The record of an INT2 group in the pool equals the contiguous stream record of the same 32
    tokens at K2V2, keys per-channel."""
    int2_pages, int4_pages = 8, 2
    k, v = _tokens(3, 64)
    table = np.array([6, 7, 2, 3], np.int32)
    for h in range(HKV):
        pool = _pool(int2_pages, int4_pages, oq)
        oq.pack_paged(pool, k, v, 64, table, int2_pages, HKV, h)
        for m, pair in enumerate((6, 2)):
            sq = oq.quantize_stream(k[32 * m:32 * m + 32], v[32 * m:32 * m + 32], 2, 2, False)
            rec, _ = oq.pack_stream(sq, 1)
            at = pair * HKV * 2048 + h * 4096
            assert np.array_equal(pool[at:at + 4096], rec[:4096])


def test_int4_pages_are_the_halves_of_a_k4v4_token_record(oq):
    """Two INT4 pages holding 32 tokens carry exactly the contiguous K4V4 per-token record of
    those tokens: K code block = page a's then page b's; V record word u of a lane = bytes
    (a[h], b[h], a[2+h], b[2+h]) of the pages' word u/2 (h = u % 2); meta index 32 n + kappa(j)
    of the record = index 16 n + j % 16 of page j / 16."""
    k, v = _tokens(5, 32, head=1)
    sq = oq.quantize_stream(k, v, 4, 4, True)
    rec, _ = oq.pack_stream(sq, 1)
    int2_pages, int4_pages = 0, 4
    pool = _pool(int2_pages, int4_pages, oq)
    h = 1
    table = np.array([3, 1], np.int32)
    oq.pack_paged(pool, k, v, 0, table, int2_pages, HKV, h)
    pa = pool[3 * HKV * 3072 + h * 3072:][:3072]
    pb = pool[1 * HKV * 3072 + h * 3072:][:3072]
    assert np.array_equal(rec[:1024], pa[:1024])
    assert np.array_equal(rec[1024:2048], pb[:1024])
    vrec = rec[2048:4096]
    for lane in range(64):
        for u in range(8):
            ro = (u // 4) * 1024 + lane * 16 + (u % 4) * 4
            po = 1024 + lane * 16 + (u // 2) * 4
            hh = u % 2
            want = [pa[po + hh], pb[po + hh], pa[po + 2 + hh], pb[po + 2 + hh]]
            assert list(vrec[ro:ro + 4]) == want, (lane, u)
    f32 = lambda b: np.frombuffer(bytes(b), np.float32)
    for part, ro, po in (("k", 4096, 2048), ("v", 5120, 2560)):
        rm = f32(rec[ro:ro + 1024])
        ma, mb = f32(pa[po:po + 512]), f32(pb[po:po + 512])
        for j in range(32):
            src = ma if j < 16 else mb
            for n in range(4):
                ri = oq.meta_token_index(j, n)
                pi = oq.page_meta_index(j % 16, n)
                assert rm[ri] == src[pi] and rm[128 + ri] == src[64 + pi], (part, j, n)


def test_int4_closed_form(oq):
    """b = 4 per token, channels x_c = c mod 16: every 32-channel group has scale 1, zero 0, and
    dequantizes exactly (quantizer closed form, now through the page layout)."""
    x = np.tile((np.arange(128) % 16).astype(np.float16), (5, 1))
    pool = _pool(0, 1, oq)
    oq.pack_paged(pool, x, x, 0, [0], 0, HKV, 1)
    kd, vd = oq.unpack_paged(pool, 0, 5, [0], 0, HKV, 1)
    assert np.array_equal(kd, x.astype(np.float32)) and np.array_equal(vd, x.astype(np.float32))


def test_int2_closed_form(oq):
    """b = 2 per channel: a channel holding [0, .5, 1.5, 2.5, 3, then 27 x 1] gives codes
    [0, 0, 2, 2, 3, 1...] (ties to even), deq = code."""
    col = np.array([0, 0.5, 1.5, 2.5, 3] + [1.0] * 27, np.float16)
    k = np.tile(col[:, None], (1, 128))
    v = np.zeros((32, 128), np.float16)
    pool = _pool(2, 0, oq)
    oq.pack_paged(pool, k, v, 32, [0, 1], 2, HKV, 0)
    kd, vd = oq.unpack_paged(pool, 32, 0, [0, 1], 2, HKV, 0)
    want = np.array([0, 0, 2, 2, 3] + [1] * 27, np.float32)
    assert np.array_equal(kd, np.tile(want[:, None], (1, 128)))
    assert not vd.any()


@pytest.mark.parametrize("n2,n4", [(64, 40), (0, 17), (96, 0), (32, 1)])
def test_page_permutation_changes_nothing(oq, n2, n4):
    """Two different physical placements of the same tokens unpack to the same logical cache
    and the same attention (softmax attention is a function of the token set)."""
    int2_pages, int4_pages = 16, 8
    k, v = _tokens(7, n2 + n4)
    out = []
    for seed in (1, 2):
        pool = _pool(int2_pages, int4_pages, oq)
        t = _table(n2, n4, int2_pages, int4_pages, seed)
        oq.pack_paged(pool, k, v, n2, t, int2_pages, HKV, 1)
        out.append(oq.unpack_paged(pool, n2, n4, t, int2_pages, HKV, 1))
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])


def test_paged_tokens_follow_their_quantizers(oq):
    """The logical cache read back from the pool is the INT2 stream quantization (K2V2, keys
    per-channel) of the first n2 tokens followed by the per-token 4-bit quantization of the
    rest, dequantized as fmaf(code, scale, zero)."""
    n2, n4 = 64, 23
    k, v = _tokens(9, n2 + n4)
    pool = _pool(8, 4, oq)
    t = _table(n2, n4, 8, 4, 4)
    oq.pack_paged(pool, k, v, n2, t, 8, HKV, 0)
    kd, vd = oq.unpack_paged(pool, n2, n4, t, 8, HKV, 0)
    k2, v2 = oq.dequant_stream(oq.quantize_stream(k[:n2], v[:n2], 2, 2, False))
    assert np.array_equal(kd[:n2], k2) and np.array_equal(vd[:n2], v2)
    for x, got in ((k, kd), (v, vd)):
        codes, sc, zr = oq.quantize_tokens(x[n2:], 4)
        want = np.array([[oq.dequant(codes[j, c], sc[j, c // 32], zr[j, c // 32]) for c in range(128)]
                         for j in range(n4)], np.float32)
        assert np.array_equal(got[n2:], want)


def test_decode_paged_is_attention_over_the_logical_cache(oq):
    n2, n4, G = 32, 30, 3
    int2_pages, int4_pages = 4, 4
    pool = _pool(int2_pages, int4_pages, oq)
    tables = np.zeros((2, 8), np.int32)
    lens = [(32, 30), (0, 5)]
    t0 = _table(32, 30, int2_pages, int4_pages, 20)
    free4 = sorted(set(range(int2_pages, int2_pages + int4_pages)) - set(int(x) for x in t0[2:]))
    for r, (t, (a, b)) in enumerate(zip((t0, np.array(free4[:1], np.int32)), lens)):
        tables[r, :len(t)] = t
        k, v = _tokens(11 + r, a + b)
        oq.pack_paged(pool, k, v, a, t, int2_pages, HKV, 1)
    qs, want = [], []
    for r, (a, b) in enumerate(lens):
        q = syn.queries_fp16(1, 0, r, 1, G)[0].numpy()
        qs.append(q)
        kd, vd = oq.unpack_paged(pool, a, b, tables[r], int2_pages, HKV, 1)
        want.append(oq.attention(q, kd, vd, 0.125))
    out, lse, _ = oq.decode_paged(pool, [0, 1], [1, 1], [a for a, _ in lens], [b for _, b in lens], tables,
                                  int2_pages, HKV, np.stack(qs), G, 0.125, 2)
    for r in range(2):
        assert np.array_equal(out[r], want[r][0]) and np.array_equal(lse[r], want[r][1])


def test_int4_region_starts_at_the_pool_split(oq):
    """With 6 INT2 pages of 2 KV heads (2048 B per head each), the INT4 region starts at byte
    6 * 2 * 2048 = 24576; INT4 page id 7 is the second INT4 page, at 24576 + 2 * 3072 = 30720,
    and its KV head 1 at 30720 + 3072 = 33792."""
    k = np.zeros((1, 128), np.float16)
    k[0, 0] = 1.0
    pool = _pool(6, 2, oq)
    oq.pack_paged(pool, k, k, 0, [7], 6, HKV, 1)
    nz = np.nonzero(pool)[0]
    assert nz.min() >= 33792 and nz.max() < 33792 + 3072
    assert pool[33792] == 15  # K code of (slot 0, channel 0): lane 0, word 0, bits 0..3
