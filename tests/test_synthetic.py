"""The seeded input generator: integer hash consistency and the N(0,1)-like shape."""
import numpy as np
import torch

import synthetic as syn


def test_tensor_hash_matches_scalar():
    xs = [0, 1, 2, 12345, 0xFFFFFFFF, 0x80000000, 0x7FFFFFFF, 987654321]
    t = syn.fmix32(torch.tensor(xs, dtype=torch.int64))
    assert t.tolist() == [syn.fmix32_int(x) for x in xs]


def test_distribution_and_outliers():
    x = syn.normal_fp16(0, syn.T_V, 0, range(2), range(2), 0, 512).float()
    assert abs(x.mean().item()) < 0.02 and abs(x.std().item() - 1.0) < 0.02
    assert x.abs().max().item() <= 6.0
    k = syn.keys_fp16(0, 3, range(2), range(2), 0, 256, outlier_count=4, outlier_factor=10.0,
                      num_kv_heads=2).float()
    chans = syn.outlier_channels(0, 3, 1, 4)
    assert len(set(chans)) == 4
    std = k[:, 1].std(dim=(0, 1))
    assert all(std[c] > 5 for c in chans)
    assert (np.delete(std.numpy(), chans) < 1.5).all()


def test_slices_are_consistent():
    """Any sub-range of tokens, requests or heads regenerates the same values."""
    full = syn.keys_fp16(5, 2, range(3), range(4), 0, 100, num_kv_heads=4)
    part = syn.keys_fp16(5, 2, [2], [1, 3], 40, 30, num_kv_heads=4)
    assert torch.equal(full[2, [1, 3], 40:70], part[0])
