"""The append kernel's quantizer forms each code from q = RN(t RN(1/s)) instead of the IEEE
quotient Q = RN(t/s), and recodes an element with the IEEE division only when q lies within
2^-14 of a half-integer. This checks, in float32 arithmetic on the CPU (numpy rounds every
float32 operation to nearest), the bound that makes this exact: |q - Q| < 2^-14 for all
quotients up to 255 -- so wherever rint(q) and rint(Q) differ the element is flagged -- over
groups shaped like the quantizer's (t = x - min >= 0, s = (max - min) / (2^b - 1))."""
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
        flagged = np.abs((q - np.floor(q)) - np.float32(0.5)) < np.float32(2.0 ** -14)
        differ = np.rint(q) != np.rint(Q)
        assert not np.any(differ & ~flagged)


def test_exact_half_quotients_are_flagged():
    # quotients that are exactly k + 1/2 (ties decided by the IEEE division, half to even)
    for levels in (3, 15, 255):
        s = np.float32(0.25)
        k = np.arange(levels, dtype=np.float32)
        t = (k + np.float32(0.5)) * s
        q = t * (np.float32(1.0) / s)
        assert np.all(np.abs((q - np.floor(q)) - np.float32(0.5)) < np.float32(2.0 ** -14))
