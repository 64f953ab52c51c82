"""Pins of the oracle's quantizer against hand-worked cases, brute force and the
mathematics of nested grids. The quantizer is the asymmetric groupwise min/max
quantizer with group size 32 (TriAxialKV page, "Facts", quantizer bullet)."""
import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _f16(vals):
    return np.asarray(vals, dtype=np.float16)


def _f32_bits(s: str) -> np.float32:
    return np.array([int(s, 16)], dtype=np.uint32).view(np.float32)[0]


def test_half_to_float_all_values(oq):
    # every finite binary16 value converts exactly (numpy's conversion as the pin)
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allh.view(np.float16).astype(np.float32)
    for h in list(range(0, 65536, 97)) + [0, 1, 0x3FF, 0x400, 0x7BFF, 0x8001, 0xFBFF]:
        r = ref[h]
        if np.isnan(r):
            continue
        got = np.float32(oq.half_to_float(int(h)))
        assert got == r or (got == 0 and r == 0), (h, got, r)


@pytest.mark.parametrize("case", json.load(open(os.path.join(HERE, "golden", "quantizer_cases.json")))["cases"],
                         ids=lambda c: c["name"])
def test_golden_cases(oq, case):
    x = _f16(case["x"])
    scale, zero, codes = oq.quantize_group(x, case["bits"])
    if "scale_bits" in case:
        assert scale == _f32_bits(case["scale_bits"])
    else:
        assert scale == np.float32(case["scale"])
    assert zero == np.float32(case["zero"])
    assert codes.tolist() == case["codes"]
    if case.get("deq_exact"):
        for xi, ci in zip(x.astype(np.float32), codes):
            assert oq.dequant(ci, scale, zero) == xi
    if "deq_of_255_bits" in case:
        assert oq.dequant(255, scale, zero) == _f32_bits(case["deq_of_255_bits"])


def _levels_error(x64, scale, zero, bits):
    lv = zero + scale * np.arange(2 ** bits, dtype=np.float64)
    return np.min(np.abs(x64[:, None] - lv[None, :]), axis=1)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_brute_force_nearest_level(oq, bits):
    """Each code is a nearest grid level, checked exhaustively over all 2^b levels in fp64."""
    rng = np.random.default_rng(1000 + bits)
    for trial in range(300):
        n = int(rng.integers(2, 33))
        x = (rng.standard_normal(n) * rng.choice([0.01, 1.0, 30.0])).astype(np.float16)
        scale, zero, codes = oq.quantize_group(x, bits)
        x64 = x.astype(np.float64)
        assert zero == np.float32(x.astype(np.float32).min())
        assert codes.max() <= 2 ** bits - 1
        if scale == 0:
            assert (codes == 0).all()
            continue
        deq = zero + np.float64(scale) * codes.astype(np.float64)
        best = _levels_error(x64, np.float64(scale), np.float64(zero), bits)
        slack = 2 * np.spacing(np.float32(scale) * (2 ** bits)) + np.spacing(np.float32(np.abs(x64).max()))
        assert np.all(np.abs(x64 - deq) <= best + slack), trial


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_error_bound_half_scale(oq, bits):
    """|x - deq(code)| <= scale/2 + a few fp32 ulps, with deq = fmaf(code, scale, zero)."""
    rng = np.random.default_rng(7 + bits)
    for trial in range(200):
        x = (rng.standard_normal(32) * 3).astype(np.float16)
        x[rng.integers(0, 32)] *= 10  # an outlier
        scale, zero, codes = oq.quantize_group(x, bits)
        xf = x.astype(np.float32)
        deq = np.array([oq.dequant(c, scale, zero) for c in codes], dtype=np.float64)
        bound = np.float64(scale) / 2 + 4 * np.spacing(np.float32(np.abs(xf).max()))
        assert np.all(np.abs(xf.astype(np.float64) - deq) <= bound), trial


def test_error_monotone_in_bitwidth(oq):
    """3 | 15 | 255: the 2-bit grid is a subset of the 4-bit grid, which is a subset of the
    8-bit grid, so the per-element error cannot grow with the bit-width (up to fp32 slack)."""
    rng = np.random.default_rng(11)
    for trial in range(300):
        x = (rng.standard_normal(32) * rng.choice([0.1, 1.0, 20.0])).astype(np.float16)
        xf = x.astype(np.float64)
        errs = {}
        for b in (2, 4, 8):
            s, z, c = oq.quantize_group(x, b)
            deq = np.array([oq.dequant(ci, s, z) for ci in c], dtype=np.float64)
            errs[b] = np.abs(xf - deq)
        slack = 4 * np.spacing(np.float32(np.abs(xf).max()))
        assert np.all(errs[4] <= errs[2] + slack)
        assert np.all(errs[8] <= errs[4] + slack)
        assert np.mean(errs[8] ** 2) <= np.mean(errs[4] ** 2) <= np.mean(errs[2] ** 2) + 1e-30


def test_fp32_quotient_decides_ties(oq):
    """The code is the half-even rounding of the fp32 quotient (x - zero) / scale, not of
    the exact ratio. Case found by search over fp16 inputs, worked by hand: b = 4,
    zero = 0, max = 79 gives scale = fp32(79/15) = 0x40a88889 (5.2666669, just above
    79/15), so 39.5 / scale in fp32 is 7.4999995 and rounds to 7, although the exact
    ratio 39.5 * 15 / 79 = 7.5 is a tie that would round to the even 8."""
    x = _f16([0.0, 79.0, 39.5] + [0.0] * 29)
    scale, zero, codes = oq.quantize_group(x, 4)
    assert scale == _f32_bits("0x40a88889")
    assert codes[2] == 7
    assert codes[1] == 15 and codes[0] == 0


def test_stream_quantize_axes(oq):
    """Per-channel K groups run down a channel over 32 tokens; per-token groups across 32
    channels of one token; tokens past the last full group stay fp16."""
    import synthetic as syn

    k = syn.keys_fp16(3, 0, [0], [0], 0, 70, num_kv_heads=1)[0, 0].numpy()
    v = syn.values_fp16(3, 0, [0], [0], 0, 70)[0, 0].numpy()
    sq = oq.quantize_stream(k, v, 4, 2, k_token=False)
    assert sq.lq == 64
    for m in range(2):
        for c in (0, 17, 127):
            s, z, codes = oq.quantize_group(k[32 * m:32 * m + 32, c], 4)
            assert sq.kscale[m * 128 + c] == s and sq.kzero[m * 128 + c] == z
            assert sq.kcode[32 * m:32 * m + 32, c].tolist() == codes.tolist()
    for j in (0, 33, 63):
        for n in range(4):
            s, z, codes = oq.quantize_group(v[j, 32 * n:32 * n + 32], 2)
            assert sq.vscale[j * 4 + n] == s and sq.vzero[j * 4 + n] == z
            assert sq.vcode[j, 32 * n:32 * n + 32].tolist() == codes.tolist()
    kd, vd = oq.dequant_stream(sq)
    assert np.array_equal(kd[64:], k[64:].astype(np.float32))
    assert np.array_equal(vd[64:], v[64:].astype(np.float32))
    sqt = oq.quantize_stream(k, v, 4, 2, k_token=True)
    s, z, codes = oq.quantize_group(k[5, 32:64], 4)
    assert sqt.kscale[5 * 4 + 1] == s and sqt.kcode[5, 32:64].tolist() == codes.tolist()
    # b = 16 is a passthrough
    sq16 = oq.quantize_stream(k, v, 16, 16)
    kd16, vd16 = oq.dequant_stream(sq16)
    assert np.array_equal(kd16, k.astype(np.float32)) and np.array_equal(vd16, v.astype(np.float32))
