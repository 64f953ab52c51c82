"""GPU test of kvq_decode_attention_noalloc, through the C ABI: the entry point for callers
that cannot allocate device memory keeps the split partials in the library's own device array.
Its output and log-sum-exp must equal, bit for bit, those of kvq_decode_attention with a
caller-given workspace on the same inputs (the same kernels and split count), on two calls in a
row, the second with a smaller input; and a call whose partials would not fit the array must be
refused before anything runs."""
import ctypes
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from test_gpu_parity import Case, check_attention

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)


def _call_noalloc(kvq, c, l, q, seq, batch, max_len, out, lse, splits):
    lib = kvq.load()
    st = lib.kvq_decode_attention_noalloc(ctypes.byref(c.plan), l, ctypes.c_void_p(c.cache.data_ptr()),
                                          ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(seq.data_ptr()), batch,
                                          max_len, ctypes.c_float(SCALE), ctypes.c_void_p(out.data_ptr()),
                                          kvq.OUT_F32, ctypes.c_void_p(lse.data_ptr()), splits, None,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.kvq_last_error().decode()


def _call_workspace(kvq, c, l, q, seq, max_len, out, lse, splits):
    batch = q.shape[0]
    ws = torch.empty(kvq.workspace_bytes(c.plan, batch, max_len, splits) // 4 + 1, dtype=torch.float32,
                     device="cuda")
    kvq.decode_attention(c.plan, l, c.cache, q, seq, max_len, SCALE, out, lse, ws, splits)


@pytest.mark.parametrize("splits", [3, 0])
def test_noalloc_equals_workspace_call_twice(gpu, oq, splits):
    lens = [150, 37, 96, 1, 64 + 17, 128]
    c = Case(gpu, oq, hq=8, hkv=2, batch=len(lens), cap=160, cfgs=[(4, 2), (8, 4, 1)], lens=lens, seed=61)
    # first call: the whole batch; second: the first three requests only and a shorter bound
    for l in range(len(c.cfgs)):
        for batch, max_len in ((len(lens), 150), (3, 150)):
            seq = c.seq[:batch].contiguous()
            q = syn.queries_fp16(c.seed, l, batch, batch, c.hq).cuda()
            outs = []
            for use_noalloc in (True, False):
                out = torch.full((batch, c.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
                lse = torch.full((batch, c.hq), float("nan"), dtype=torch.float32, device="cuda")
                if use_noalloc:
                    _call_noalloc(gpu, c, l, q, seq, batch, max_len, out, lse, splits)
                else:
                    _call_workspace(gpu, c, l, q, seq, max_len, out, lse, splits)
                torch.cuda.synchronize()
                outs.append((out.cpu().numpy(), lse.cpu().numpy()))
            assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1]), (l, batch)
            G = c.hq // c.hkv
            kb, vb, ka, _ = c.cfgs[l]
            ref = np.zeros((batch, c.hq, 128))
            ref_lse = np.zeros((batch, c.hq))
            for r in range(batch):
                for h in range(c.hkv):
                    L = lens[r]
                    o, ls = oq.decode_stream(q[r, h * G:(h + 1) * G].cpu().numpy(), c.k[l][r, h, :L].numpy(),
                                             c.v[l][r, h, :L].numpy(), kb, vb, ka == 1, SCALE)
                    ref[r, h * G:(h + 1) * G], ref_lse[r, h * G:(h + 1) * G] = o, ls
            check_attention(outs[0][0], outs[0][1], ref, ref_lse, lens[:batch], c.hq, c.hkv)


def test_noalloc_refuses_partials_beyond_the_array(gpu):
    plan = gpu.plan_layers(gpu.make_shape(32, 8, 64, max_tokens=4096), [(4, 2)])
    lib = gpu.load()
    # 64 requests x 32 q heads x 1024 splits x 129 fp32 > 16 MiB: refused on the host, nothing launched
    st = lib.kvq_decode_attention_noalloc(ctypes.byref(plan), 0, ctypes.c_void_p(256), ctypes.c_void_p(256),
                                          ctypes.c_void_p(256), 64, 4096, ctypes.c_float(SCALE),
                                          ctypes.c_void_p(256), gpu.OUT_F32, None, 1024, None, None)
    assert st == gpu.ERR_WORKSPACE
    assert b"scratch" in lib.kvq_last_error()
