"""The append kernel's quantizer forms each code from q = RN(t RN(1/s)) instead of the IEEE
quotient Q = RN(t/s), and recodes an element with the IEEE division only when the distance
d = |RN(t y - rint(q))| (y = RN(1/s); one fused multiply-add) exceeds 1/2 - 2^-14. This checks,
in float32 arithmetic on the CPU (numpy rounds every float32 operation to nearest; the fused
operation is formed exactly in float64 and rounded once), the bound that makes this exact:
|q - Q| < 2^-14 for all quotients up to 255, and every element where rint(q) and rint(Q)
differ is flagged -- over groups shaped like the quantizer's (t = x - min >= 0,
s = (max - min) / (2^b - 1)). The fast codes never exceed 2^b - 1, so they need no clamp."""
import numpy as np


def _groups(rng, n, bits):
    x = rng.standard_normal((n, 32)) * rng.choice([1e-6, 1e-3, 1.0, 30.0, 1e4], size=(n, 1))
    x = np.clip(x, -65504, 65504).astype(np.float16).astype(np.float32)
    mn, mx = x.min(axis=1, keepdims=True), x.max(axis=1, keepdims=True)
    s = (mx - mn) / np.float32((1 << bits) - 1)
    keep = (s > 0)[:, 0]
    return (x - mn)[keep], s[keep]


def test_fast_quotient_within_bound_and_flags_every_difference():
    rng = np.random.default_rng(7)
    for bits in (2, 4, 8):
        t, s = _groups(rng, 20000, bits)
        y = np.float32(1.0) / s
        q = t * y
        Q = t / s
        assert q.dtype == np.float32 and Q.dtype == np.float32
        assert np.all(np.abs(q.astype(np.float64) - Q.astype(np.float64)) < 2.0 ** -14)
        r = np.rint(q)
        d = np.abs((t.astype(np.float64) * y.astype(np.float64) - r).astype(np.float32))
        flagged = d > np.float32(0.5) - np.float32(2.0 ** -14)
        differ = r != np.rint(Q)
        assert np.any(flagged)
        assert not np.any(differ & ~flagged)
        assert r.max() <= (1 << bits) - 1 and r.min() >= 0


def test_exact_half_quotients_are_flagged():
    # quotients that are exactly k + 1/2 (ties decided by the IEEE division, half to even)
    for levels in (3, 15, 255):
        s = np.float32(0.25)
        k = np.arange(levels, dtype=np.float32)
        t = (k + np.float32(0.5)) * s
        y = np.float32(1.0) / s
        q = t * y
        d = np.abs((t.astype(np.float64) * np.float64(y) - np.rint(q)).astype(np.float32))
        assert np.all(d > np.float32(0.5) - np.float32(2.0 ** -14))
