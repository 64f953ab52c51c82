"""Pins of the oracle's packer against hand-worked sites of the cache layout, and the
bijection property every block must have. The layout is this project's own (no page
prescribes one); tests/golden/layout_sites.json states its rules and the worked sites."""
import json
import os

import numpy as np
import pytest

import synthetic as syn

HERE = os.path.dirname(os.path.abspath(__file__))
SITES = json.load(open(os.path.join(HERE, "golden", "layout_sites.json")))


def test_worked_sites(oq):
    for s in SITES["k_sites"]:
        assert oq.k_site(s["j"], s["c"]) == (s["lane"], s["e"])
    for s in SITES["v_sites"]:
        assert oq.v_site(s["j"], s["c"]) == (s["lane"], s["e"])
    for s in SITES["meta_channel"]:
        assert oq.meta_channel_index(s["c"]) == s["index"]
    for s in SITES["meta_token"]:
        assert oq.meta_token_index(s["j"], s["n"]) == s["index"]


@pytest.mark.parametrize("which", ["k", "v"])
def test_sites_are_a_bijection(oq, which):
    """32 tokens x 128 channels map one-to-one onto 64 lanes x 64 positions."""
    f = oq.k_site if which == "k" else oq.v_site
    seen = set()
    for j in range(32):
        for c in range(128):
            lane, e = f(j, c)
            assert 0 <= lane < 64 and 0 <= e < 64
            seen.add((lane, e))
    assert len(seen) == 32 * 128
    assert len({oq.meta_channel_index(c) for c in range(128)}) == 128
    assert len({oq.meta_token_index(j, n) for j in range(32) for n in range(4)}) == 128


def _single_outlier_stream(j0, c0, value=1.0):
    k = np.zeros((32, 128), np.float16)
    k[j0, c0] = value
    v = np.zeros((32, 128), np.float16)
    return k, v


@pytest.mark.parametrize("site", [s for s in SITES["k_sites"]], ids=lambda s: f"k{s['j']}_{s['c']}_b{s['bits']}")
def test_single_code_lands_on_worked_site(oq, site):
    """A group whose only non-constant channel is c0, with its maximum at token j0, has exactly
    one non-zero K code, 2^b - 1 at (j0, c0); it must appear at the worked byte and bit."""
    b = site["bits"]
    k, v = _single_outlier_stream(site["j"], site["c"])
    sq = oq.quantize_stream(k, v, b, 4)
    buf, mask = oq.pack_stream(sq, 1)
    kblock = buf[:512 * b]
    nz = np.nonzero(kblock)[0]
    word = int.from_bytes(bytes(kblock[site["byte"]:site["byte"] + 4]), "little")
    assert word == ((2 ** b - 1) << site["shift"])
    assert set(nz.tolist()) <= set(range(site["byte"], site["byte"] + 4))
    assert mask[:oq.record_bytes(b, 4)].all()


def test_v_worked_site(oq):
    s = SITES["v_sites"][0]
    v = np.zeros((32, 128), np.float16)
    v[s["j"], (s["c"] // 32) * 32] = -1.0  # the group of channel c gets min -1, max 0 or 1
    v[s["j"], s["c"]] = 1.0
    k = np.zeros((32, 128), np.float16)
    sq = oq.quantize_stream(k, v, 4, s["bits"])
    buf, _ = oq.pack_stream(sq, 1)
    vblock = buf[512 * 4:512 * 4 + 512 * s["bits"]]
    word = int.from_bytes(bytes(vblock[s["byte"]:s["byte"] + 4]), "little")
    assert (word >> s["shift"]) & (2 ** s["bits"] - 1) == 2 ** s["bits"] - 1


@pytest.mark.parametrize("kb,vb,kt", [(8, 8, False), (4, 2, False), (2, 4, True), (16, 16, False), (8, 16, False)])
def test_pack_unpack_roundtrip(oq, kb, vb, kt):
    L = 101
    k = syn.keys_fp16(9, 0, [0], [0], 0, L, num_kv_heads=1)[0, 0].numpy()
    v = syn.values_fp16(9, 0, [0], [0], 0, L)[0, 0].numpy()
    sq = oq.quantize_stream(k, v, kb, vb, kt)
    kd, vd = oq.dequant_stream(sq)
    cap = 4
    buf, mask = oq.pack_stream(sq, cap)
    assert buf.size == cap * oq.record_bytes(kb, vb) + 16384
    kd2, vd2 = oq.unpack_stream(buf, L, kb, vb, kt, cap)
    assert np.array_equal(kd, kd2) and np.array_equal(vd, vd2)
    # defined bytes: 3 full records and 5 tail slots of 256 B each for K and for V
    assert mask.sum() == 3 * oq.record_bytes(kb, vb) + 5 * 512


def test_record_sizes(oq):
    # codes + 2 x 1 KiB meta: K8V8 2.5 B, K4V2 1.25 B per (token, channel) element
    assert oq.record_bytes(8, 8) == 10240 and oq.record_bytes(8, 8) / 4096 == 2.5
    assert oq.record_bytes(4, 2) == 5120 and oq.record_bytes(4, 2) / 4096 == 1.25
    assert oq.record_bytes(16, 16) == 16384
    assert oq.record_bytes(16, 4) == 8192 + 2048 + 1024
