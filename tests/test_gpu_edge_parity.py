"""GPU parity on the shapes and values the synthetic workloads do not reach, through the C ABI.

- Every GQA group size class the split pass instantiates (G = 2, 3, 5, 6, 8, 9, 12, 16: four,
  two and one column slots per tile, G = 8 filling all 16 columns), contiguous and paged.
- Degenerate and extreme groups (TriAxialKV page, "Facts", quantizer bullet: asymmetric
  min/max groups of 32): constant key and value groups (scale 0, every code 0, dequantized to
  the zero point exactly), a whole constant stream, q = 0 (attention = mean of the dequantized
  values), keys with |x| up to 3e4 in a few channels (scores far apart: softmax one-hot),
  values with |x| up to 6e4 in a few tokens, groups whose range is ~1e-4 around a moderate
  value, and groups of fp16 denormals (range ~1e-6 around zero).
- Every (bK, bV) in {2, 4, 8, 16}^2, keys per-channel and per-token.

Packed bytes are bit-exact with the oracle's own packing; attention is checked against the
oracle's fp64 attention on its own quantization, rel L2 <= 1e-3 on every (request, KV head)
stream and max abs <= 2e-3, with the log-sum-exp within the per-row bound derived for the
fp32 score sums (lse_tolerance)."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from test_gpu_parity import MAX_ABS, Case, check_attention, check_streams, lse_tolerance

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)
ALL_PAIRS = [(kb, vb, ax) for kb in (2, 4, 8, 16) for vb in (2, 4, 8, 16) for ax in ((0, 1) if kb < 16 else (0,))]


# ------------------------------------------------------------------ GQA sizes
@pytest.mark.parametrize("G", [2, 3, 5, 6, 8, 9, 12, 16])
@pytest.mark.parametrize("splits", [0, 3])
def test_decode_every_gqa_size(gpu, oq, G, splits):
    hkv = 2
    lens = [150, 1, 37, 96, 0, 64 + 31]
    c = Case(gpu, oq, hq=G * hkv, hkv=hkv, batch=len(lens), cap=160,
             cfgs=[(8, 4), (4, 2), (4, 4, 1), (16, 16), (2, 8)], lens=lens, seed=20 + G)
    for l in range(len(c.cfgs)):
        q = syn.queries_fp16(c.seed, l, splits, c.batch, c.hq).cuda()
        out, lse = c.decode(l, q, splits)
        ref, ref_lse = c.oracle_decode(l, q)
        try:
            check_attention(out, lse, ref, ref_lse, c.lens, c.hq, c.hkv)
        except AssertionError as e:
            raise AssertionError(f"G {G} layer {l} {c.cfgs[l]} splits {splits}: {e}") from None


# ----------------------------------------------------------- explicit values
class ExplicitCase:
    """A cache filled from given fp16 K and V ([batch][Hkv][L][128] numpy float16), each request
    with its own length, one append per request."""

    def __init__(self, kvq, oq, hq, hkv, cfgs, k, v, lens):
        self.kvq, self.oq = kvq, oq
        self.hq, self.hkv = hq, hkv
        self.batch = k.shape[0]
        self.cfgs = [tuple(cf) + (0, 1)[len(cf) - 2:] for cf in cfgs]
        self.k, self.v, self.lens = k, v, list(lens)
        cap = -(-max(lens) // 32) * 32 + 32
        self.plan = kvq.plan_layers(kvq.make_shape(hq, hkv, self.batch, max_tokens=cap), self.cfgs)
        self.cache = torch.zeros(self.plan.total_bytes, dtype=torch.uint8, device="cuda")
        z = torch.zeros(1, dtype=torch.int32, device="cuda")
        for l in range(len(self.cfgs)):
            for r in range(self.batch):
                if self.lens[r] == 0:
                    continue
                off = r * hkv * self.plan.layers[l].stream_bytes
                kk = torch.from_numpy(np.ascontiguousarray(k[r:r + 1, :, :self.lens[r]])).cuda()
                vv = torch.from_numpy(np.ascontiguousarray(v[r:r + 1, :, :self.lens[r]])).cuda()
                kvq.quantize_append(self.plan, l, self.cache[off:], kk, vv, z)
        self.seq = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

    def check_bytes(self, l):
        lp = self.plan.layers[l]
        kb, vb, ax, _ = self.cfgs[l]
        for r in range(self.batch):
            for h in range(self.hkv):
                L = self.lens[r]
                sq = self.oq.quantize_stream(self.k[r, h, :L], self.v[r, h, :L], kb, vb, ax == 1)
                want, mask = self.oq.pack_stream(sq, lp.groups_cap)
                a = lp.offset + (r * self.hkv + h) * lp.stream_bytes
                got = self.cache[a:a + lp.stream_bytes].cpu().numpy()
                bad = np.nonzero((want != got) & mask)[0]
                assert bad.size == 0, f"layer {l} {self.cfgs[l]} r{r} h{h}: {bad.size} bytes differ"

    def check_decode(self, l, q, splits):
        kvq, G = self.kvq, self.hq // self.hkv
        ml = max(self.lens)
        out = torch.full((self.batch, self.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((self.batch, self.hq), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(kvq.workspace_bytes(self.plan, self.batch, ml, splits) // 4 + 1, dtype=torch.float32,
                         device="cuda")
        kvq.decode_attention(self.plan, l, self.cache, torch.from_numpy(q).cuda(), self.seq, ml, SCALE, out, lse, ws,
                             splits)
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        kb, vb, ax, _ = self.cfgs[l]
        ref = np.zeros((self.batch, self.hq, 128))
        ref_lse = np.zeros((self.batch, self.hq))
        tol = np.zeros((self.batch, self.hq))
        for r in range(self.batch):
            L = self.lens[r]
            for h in range(self.hkv):
                qq = q[r, h * G:(h + 1) * G]
                sq = self.oq.quantize_stream(self.k[r, h, :L], self.v[r, h, :L], kb, vb, ax == 1)
                kd, vd = self.oq.dequant_stream(sq)
                o, ls = self.oq.attention(qq, kd, vd, SCALE)
                ref[r, h * G:(h + 1) * G], ref_lse[r, h * G:(h + 1) * G] = o, ls
                tol[r, h * G:(h + 1) * G] = lse_tolerance(qq, kd, SCALE, kb, ax == 1)
        where = f"layer {l} {self.cfgs[l]} splits {splits}"
        for r, L in enumerate(self.lens):
            if L == 0:
                assert np.all(out[r] == 0) and np.all(lse[r] == -np.inf), where
        full = [r for r, L in enumerate(self.lens) if L > 0]
        assert np.isfinite(out[full]).all(), f"{where}: non-finite output"
        # max abs 2e-3 on streams whose outputs are of unit scale; a stream whose reference
        # output reaches beyond 1 in magnitude (values of |x| ~ 6e4) is held to 2e-3 times
        # that magnitude: fp32 arithmetic carries relative, not absolute, error
        for r in full:
            for h in range(self.hkv):
                blk = slice(h * G, (h + 1) * G)
                scale = max(1.0, float(np.abs(ref[r, blk]).max()))
                err = float(np.abs(out[r, blk] - ref[r, blk]).max())
                assert err <= MAX_ABS * scale, \
                    f"{where}: request {r} KV head {h}: max abs {err:.3g} (output scale {scale:.3g})"
        dl = np.abs(lse[full] - ref_lse[full])
        bad = np.argwhere(dl > tol[full])
        if bad.size:
            i, row = bad[0]
            r = full[i]
            raise AssertionError(f"{where}: request {r} row {row}: lse {lse[r, row]:.7g} vs {ref_lse[r, row]:.7g}, "
                                 f"off by {dl[i, row]:.3g} (bound {tol[r, row]:.3g}); {len(bad)} rows over")
        try:
            check_streams(out, ref, self.lens, self.hkv)
        except AssertionError as e:
            raise AssertionError(f"{where}: {e}") from None


def edge_streams(seed, hkv, L):
    """fp16 K, V [6][hkv][L][128] and per-request notes:
    r0 every value 0.75 (a constant stream); r1 synthetic with constant groups planted (a key
    channel constant over a 32-token group, a token's 32-channel key and value slices
    constant); r2 keys with |x| up to 3e4 in channels 5 and 100; r3 values with |x| up to 6e4
    in a few tokens; r4 groups of range ~1e-4 around 0.01 (keys and values); r5 groups of fp16
    denormals (|x| < 1e-6)."""
    rng = np.random.default_rng(seed)
    B = 6
    k = syn.keys_fp16(seed, 0, range(B), range(hkv), 0, L, outlier_count=4, outlier_factor=10.0,
                      num_kv_heads=hkv).numpy().copy()
    v = syn.values_fp16(seed, 0, range(B), range(hkv), 0, L).numpy().copy()
    k[0] = 0.75
    v[0] = 0.75
    for h in range(hkv):
        for m in range(L // 32):
            k[1, h, 32 * m:32 * m + 32, (7 * m + h) % 128] = -1.5
            k[1, h, 32 * m + 3, 32:64] = 2.25
            v[1, h, 32 * m + 5, 64:96] = -0.5
            v[1, h, 32 * m + 9, :] = 1.0
    k[2, :, :, 5] = (rng.uniform(-3e4, 3e4, size=(hkv, L))).astype(np.float16)
    k[2, :, :, 100] = (rng.uniform(-3e4, 3e4, size=(hkv, L))).astype(np.float16)
    big = rng.choice(L, size=min(L, 4), replace=False)
    for h in range(hkv):
        for j in big:
            v[3, h, j, :] = rng.uniform(-6e4, 6e4, size=128).astype(np.float16)
    k[4] = (0.01 + rng.uniform(-5e-5, 5e-5, size=k[4].shape)).astype(np.float16)
    v[4] = (0.01 + rng.uniform(-5e-5, 5e-5, size=v[4].shape)).astype(np.float16)
    k[5] = rng.uniform(-5e-7, 5e-7, size=k[5].shape).astype(np.float16)
    v[5] = rng.uniform(-5e-7, 5e-7, size=v[5].shape).astype(np.float16)
    return k, v


@pytest.fixture(scope="module")
def edge(gpu, oq):
    hkv, G = 2, 4
    k, v = edge_streams(41, hkv, 131)
    lens = [131, 96, 70, 131, 64 + 17, 100]
    return ExplicitCase(gpu, oq, G * hkv, hkv, ALL_PAIRS, k, v, lens)


def test_edge_packed_bytes_bit_exact(edge):
    for l in range(len(edge.cfgs)):
        edge.check_bytes(l)


@pytest.mark.parametrize("splits", [0, 2])
def test_edge_decode(edge, splits):
    q = syn.queries_fp16(41, 0, splits, edge.batch, edge.hq).numpy().copy()
    q[1, :4] = 0.0  # q = 0 rows of request 1, KV head 0: the mean of the dequantized values
    for l in range(len(edge.cfgs)):
        edge.check_decode(l, q, splits)


def test_edge_zero_query_is_mean_of_values(edge, oq):
    """q = 0 everywhere: every row is the plain mean of its stream's dequantized values."""
    q = np.zeros((edge.batch, edge.hq, 128), np.float16)
    for l in (0, 5, 17):
        edge.check_decode(l, q, 0)


@pytest.mark.parametrize("G", [3, 8, 12])
def test_edge_values_other_group_sizes(gpu, oq, G):
    hkv = 2
    k, v = edge_streams(50 + G, hkv, 100)
    c = ExplicitCase(gpu, oq, G * hkv, hkv, [(4, 2), (8, 4), (2, 2, 1), (16, 8)], k, v, [100, 64, 33, 100, 95, 77])
    q = syn.queries_fp16(50 + G, 0, 0, c.batch, c.hq).numpy()
    for l in range(len(c.cfgs)):
        c.check_bytes(l)
        for splits in (0, 2):
            c.check_decode(l, q, splits)
