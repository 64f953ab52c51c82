"""GPU parity of libkvq against the CPU oracle, through the C ABI.

Packed codes, scales and zeros: bit-exact with the oracle's own packing of the same
fp16 inputs. Dequantized cache: bit-exact (both sides use one fmaf). Attention output:
relative L2 error <= 1e-3 and max abs error <= 2e-3 against the oracle's fp64 attention
on its own quantization."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn

pytestmark = pytest.mark.gpu

REL_L2 = 1e-3
MAX_ABS = 2e-3
LSE_ABS = 1e-4


def fold_magnitude(kdeq, kb, k_token):
    """Per (token, channel): the size of the terms the split pass adds in fp32 for that key
    element. It forms a score from the folded quantizer, scale * (q . codes) plus zero * sum(q),
    so a key element contributes |scale * code| + |zero| <= |k| + 2 |zero| (zero = the group's
    minimum, which code 0 dequantizes to exactly); fp16 tail tokens and 16-bit layers contribute
    |k|."""
    k = np.asarray(kdeq, dtype=np.float64).reshape(-1, 128)
    m = np.abs(k)
    lq = (k.shape[0] // 32) * 32
    if kb < 16 and lq:
        g = k[:lq].reshape(lq // 32, 32, 128)
        if k_token:  # a group is 32 channels of one token
            zero = k[:lq].reshape(lq, 4, 32).min(axis=2)
            m[:lq] += 2 * np.abs(np.repeat(zero, 32, axis=1))
        else:  # a group is 32 tokens of one channel
            zero = g.min(axis=1)
            m[:lq] += 2 * np.abs(np.repeat(zero, 32, axis=0))
    return m


def lse_tolerance(q_fp16, kdeq, scale, kb=16, k_token=False):
    """Per-row bound on |lse - lse_oracle|: 1e-4 plus 2^-19 times the largest sum over the
    channels of |q_c| times the fold magnitude of key element (j, c), times scale. The split pass
    forms scores in fp32 from ~22-bit products, and folding scales and zero points cancels terms
    of the fold magnitude's size, so its score error is a small multiple of 2^-22 of that sum;
    2^-19 leaves a factor 8."""
    q = np.abs(np.asarray(q_fp16, dtype=np.float64).reshape(-1, 128))
    k = fold_magnitude(kdeq, kb, k_token)
    if k.shape[0] == 0:
        return np.full(q.shape[0], LSE_ABS)
    return LSE_ABS + 2.0 ** -19 * (q @ k.T).max(axis=1) * scale


class Case:
    """A small cache built request by request (ragged lengths) with one append each."""

    def __init__(self, kvq, oq, hq, hkv, batch, cap, cfgs, lens, seed, outliers=(4, 10.0)):
        self.kvq, self.oq = kvq, oq
        self.hq, self.hkv, self.batch, self.cap = hq, hkv, batch, cap
        self.cfgs = [tuple(c) + (0, 1)[len(c) - 2:] for c in cfgs]
        self.lens = list(lens)
        self.seed = seed
        self.outliers = outliers
        self.plan = kvq.plan_layers(kvq.make_shape(hq, hkv, batch, max_tokens=cap), self.cfgs)
        self.cache = torch.zeros(self.plan.total_bytes, dtype=torch.uint8, device="cuda")
        self.k, self.v = {}, {}
        z = torch.zeros(1, dtype=torch.int32, device="cuda")
        for l in range(len(self.cfgs)):
            L = max(self.lens)
            self.k[l] = syn.keys_fp16(seed, l, range(batch), range(hkv), 0, L, outlier_count=outliers[0],
                                      outlier_factor=outliers[1], num_kv_heads=hkv)
            self.v[l] = syn.values_fp16(seed, l, range(batch), range(hkv), 0, L)
            for r in range(batch):
                if self.lens[r] == 0:
                    continue
                off = r * hkv * self.plan.layers[l].stream_bytes
                kk = self.k[l][r:r + 1, :, :self.lens[r]].contiguous().cuda()
                vv = self.v[l][r:r + 1, :, :self.lens[r]].contiguous().cuda()
                kvq.quantize_append(self.plan, l, self.cache[off:], kk, vv, z)
        self.seq = torch.tensor(self.lens, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

    def stream_bytes(self, l, r, h):
        lp = self.plan.layers[l]
        a = lp.offset + (r * self.hkv + h) * lp.stream_bytes
        return self.cache[a:a + lp.stream_bytes].cpu().numpy()

    def oracle_stream(self, l, r, h, L=None):
        L = self.lens[r] if L is None else L
        kb, vb, ka, _ = self.cfgs[l]
        return self.oq.quantize_stream(self.k[l][r, h, :L].numpy(), self.v[l][r, h, :L].numpy(), kb, vb, ka == 1)

    def decode(self, l, q, splits=0, out_dtype=torch.float32, max_len=None):
        kvq = self.kvq
        max_len = max(self.lens) if max_len is None else max_len
        out = torch.full((self.batch, self.hq, 128), float("nan"), dtype=out_dtype, device="cuda")
        lse = torch.full((self.batch, self.hq), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(kvq.workspace_bytes(self.plan, self.batch, max_len, splits) // 4 + 1, dtype=torch.float32,
                         device="cuda")
        kvq.decode_attention(self.plan, l, self.cache, q, self.seq, max_len, 1 / math.sqrt(128), out, lse, ws,
                             splits)
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), lse.cpu().numpy()

    def oracle_decode(self, l, q):
        G = self.hq // self.hkv
        kb, vb, ka, _ = self.cfgs[l]
        out = np.zeros((self.batch, self.hq, 128))
        lse = np.zeros((self.batch, self.hq))
        for r in range(self.batch):
            for h in range(self.hkv):
                L = self.lens[r]
                o, ls = self.oq.decode_stream(q[r, h * G:(h + 1) * G].cpu().numpy(), self.k[l][r, h, :L].numpy(),
                                              self.v[l][r, h, :L].numpy(), kb, vb, ka == 1, 1 / math.sqrt(128))
                out[r, h * G:(h + 1) * G] = o
                lse[r, h * G:(h + 1) * G] = ls
        return out, lse


def check_streams(out, ref, lens, hkv):
    """rel L2 <= 1e-3 on every (request, KV head) block of G query rows on its own, so that one
    bad stream cannot hide under the batch's aggregate (a tiny absolute floor of 1e-6 keeps
    blocks whose reference is exactly zero meaningful)."""
    G = out.shape[1] // hkv
    for r, L in enumerate(lens):
        if L == 0:
            continue
        for h in range(hkv):
            o = out[r, h * G:(h + 1) * G].astype(np.float64)
            rf = ref[r, h * G:(h + 1) * G]
            err = np.linalg.norm(o - rf)
            assert err <= REL_L2 * np.linalg.norm(rf) + 1e-6, \
                f"request {r} KV head {h} (L={L}): rel L2 {err / max(np.linalg.norm(rf), 1e-30):.3g}"


def check_attention(out, lse, ref, ref_lse, lens, hq, hkv=None):
    """The batch-level bar (rel L2 <= 1e-3, max abs <= 2e-3, lse within 1e-4), and with hkv the
    same rel L2 bar on every (request, KV head) stream."""
    empty = [r for r, L in enumerate(lens) if L == 0]
    full = [r for r, L in enumerate(lens) if L > 0]
    for r in empty:
        assert np.all(out[r] == 0) and np.all(lse[r] == -np.inf)
    o, rf = out[full], ref[full]
    rel = np.linalg.norm(o - rf) / np.linalg.norm(rf)
    mx = np.abs(o - rf).max()
    assert rel <= REL_L2, f"rel L2 {rel:.3g}"
    assert mx <= MAX_ABS, f"max abs {mx:.3g}"
    assert np.abs(lse[full] - ref_lse[full]).max() <= LSE_ABS
    if hkv is not None:
        check_streams(out, ref, lens, hkv)
    return rel, mx


MIXED = [(8, 8), (4, 2), (2, 4), (4, 4, 1), (16, 16), (8, 16), (2, 2), (16, 4), (8, 4, 1)]


@pytest.fixture(scope="module")
def ragged(gpu, oq):
    # ragged lengths: empty, 1, one short of a group, exactly a group, ragged tails, capacity
    return Case(gpu, oq, hq=8, hkv=2, batch=7, cap=200, cfgs=MIXED, lens=[37, 0, 1, 31, 32, 150, 200], seed=3)


def test_packed_bytes_bit_exact(ragged, oq):
    c = ragged
    for l in range(len(c.cfgs)):
        for r in range(c.batch):
            for h in range(c.hkv):
                want, mask = oq.pack_stream(c.oracle_stream(l, r, h), c.plan.layers[l].groups_cap)
                got = c.stream_bytes(l, r, h)
                bad = np.nonzero((want != got) & mask)[0]
                assert bad.size == 0, f"layer {l} {c.cfgs[l]} r{r} h{h}: {bad.size} bytes differ, first at {bad[:8]}"


def test_dequantize_bit_exact(ragged, oq, gpu):
    c = ragged
    maxL = max(c.lens)
    for l in range(len(c.cfgs)):
        ko = torch.full((c.batch, c.hkv, maxL, 128), float("nan"), device="cuda")
        vo = torch.full_like(ko, float("nan"))
        gpu.dequantize(c.plan, l, c.cache, c.seq, c.batch, maxL, ko, vo)
        torch.cuda.synchronize()
        ko, vo = ko.cpu().numpy(), vo.cpu().numpy()
        for r in range(c.batch):
            for h in range(c.hkv):
                L = c.lens[r]
                kd, vd = oq.dequant_stream(c.oracle_stream(l, r, h))
                assert np.array_equal(ko[r, h, :L], kd) and np.array_equal(vo[r, h, :L], vd), (l, r, h)


@pytest.mark.parametrize("splits", [0, 1, 3, 16])
def test_decode_attention_parity(ragged, splits):
    c = ragged
    for l in range(len(c.cfgs)):
        q = syn.queries_fp16(c.seed, l, 0, c.batch, c.hq).cuda()
        out, lse = c.decode(l, q, splits)
        ref, ref_lse = c.oracle_decode(l, q)
        check_attention(out, lse, ref, ref_lse, c.lens, c.hq, c.hkv)


def test_decode_fp16_output(ragged):
    c = ragged
    l = 1
    q = syn.queries_fp16(c.seed, l, 1, c.batch, c.hq).cuda()
    out, lse = c.decode(l, q, 0, torch.float16)
    ref, ref_lse = c.oracle_decode(l, q)
    check_attention(out, lse, ref, ref_lse, c.lens, c.hq, c.hkv)


def test_decode_deterministic(ragged):
    c = ragged
    q = syn.queries_fp16(c.seed, 0, 2, c.batch, c.hq).cuda()
    a, la = c.decode(0, q, 3)
    b, lb = c.decode(0, q, 3)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_every_tail_length(gpu, oq):
    # one request per tail length 0..31 after two packed groups: the split pass reads only the
    # tail's 16-byte pieces that hold tokens (key rows by token, value rows by groups of four
    # tokens), so every boundary (T = 4, 5, 16, 17, ...) is one of these rows
    lens = [64 + t for t in range(32)] + [16, 17]
    c = Case(gpu, oq, hq=8, hkv=2, batch=len(lens), cap=96, cfgs=[(8, 8), (4, 2), (2, 4, 1), (16, 16)], lens=lens,
             seed=14)
    for l in range(len(c.cfgs)):
        for splits in (0, 2):
            q = syn.queries_fp16(c.seed, l, splits, c.batch, c.hq).cuda()
            out, lse = c.decode(l, q, splits)
            ref, ref_lse = c.oracle_decode(l, q)
            try:
                check_attention(out, lse, ref, ref_lse, c.lens, c.hq, c.hkv)
            except AssertionError as e:
                raise AssertionError(f"layer {l} {c.cfgs[l]} splits {splits}: {e}") from None


@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 2), (7, 1), (28, 4)])
def test_gqa_shapes(gpu, oq, hq, hkv):
    c = Case(gpu, oq, hq=hq, hkv=hkv, batch=2, cap=130, cfgs=[(8, 4), (4, 2)], lens=[130, 45], seed=5,
             outliers=(8, 20.0))
    for l in range(2):
        q = syn.queries_fp16(5, l, 0, 2, hq).cuda()
        out, lse = c.decode(l, q)
        ref, ref_lse = c.oracle_decode(l, q)
        check_attention(out, lse, ref, ref_lse, c.lens, hq, hkv)


def test_incremental_appends_match_oracle(gpu, oq):
    """Tail writes, a flush that combines old tail tokens with new ones while new tail
    tokens are written in the same call, and single-token flushes."""
    hq, hkv, B, cap = 4, 2, 2, 160
    cfgs = [(4, 2), (8, 8, 1), (16, 16)]
    plan = gpu.plan_layers(gpu.make_shape(hq, hkv, B, max_tokens=cap), cfgs)
    cache = torch.zeros(plan.total_bytes, dtype=torch.uint8, device="cuda")
    seq = torch.zeros(B, dtype=torch.int32, device="cuda")
    total = 150
    K = {l: syn.keys_fp16(9, l, range(B), range(hkv), 0, total, num_kv_heads=hkv) for l in range(3)}
    V = {l: syn.values_fp16(9, l, range(B), range(hkv), 0, total) for l in range(3)}
    L = 0
    for n in [20, 1, 1, 9, 1, 1, 40, 33, 1, 31, 12]:
        for l in range(3):
            gpu.quantize_append(plan, l, cache, K[l][:, :, L:L + n].contiguous().cuda(),
                                V[l][:, :, L:L + n].contiguous().cuda(), seq)
        seq += n
        L += n
        torch.cuda.synchronize()
        for l in range(3):
            lp = plan.layers[l]
            for r in range(B):
                for h in range(hkv):
                    sq = oq.quantize_stream(K[l][r, h, :L].numpy(), V[l][r, h, :L].numpy(), cfgs[l][0], cfgs[l][1],
                                            len(cfgs[l]) > 2)
                    want, mask = oq.pack_stream(sq, lp.groups_cap)
                    a = lp.offset + (r * hkv + h) * lp.stream_bytes
                    got = cache[a:a + lp.stream_bytes].cpu().numpy()
                    assert np.array_equal(want[mask], got[mask]), (n, L, l, r, h)
    assert L == 150


def test_append_past_capacity_leaves_cache(gpu):
    plan = gpu.plan_layers(gpu.make_shape(2, 1, 1, max_tokens=64), [(4, 4)])
    cache = torch.zeros(plan.total_bytes, dtype=torch.uint8, device="cuda")
    seq = torch.tensor([60], dtype=torch.int32, device="cuda")
    k = torch.ones(1, 1, 8, 128, dtype=torch.float16, device="cuda")
    gpu.quantize_append(plan, 0, cache, k, k, seq)  # 60 + 8 > 64: no write
    torch.cuda.synchronize()
    assert int(cache.count_nonzero()) == 0
