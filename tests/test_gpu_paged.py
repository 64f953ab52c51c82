"""GPU parity of the paged INT2/INT4 pool (TriAxialKV page, "Facts": one pool split at an
offset into INT2 and INT4 pages, INT2 per-channel keys and per-token values, INT4 per-token keys
and values, leftover INT2 tokens through the INT4 path, page tables with INT2 pages first and
bitwidth-homogeneous splits merged by log-sum-exp), against the oracle, through the C ABI.

Pool bytes and the dequantized cache are bit-exact with the oracle's own packing of the same
tokens through the same page tables; attention is within relative L2 1e-3 and max abs 2e-3 of
the oracle's fp64 attention over its dequantized cache."""
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from test_gpu_parity import LSE_ABS, MAX_ABS, REL_L2, check_attention

pytestmark = pytest.mark.gpu
PAGE = 16


class PagedCase:
    """A paged pool filled by a schedule of appends. calls: list of (requests, n_new, add2) where
    add2 is the number of the n_new tokens (a multiple of 32) that go to INT2 groups; a call with
    several requests is one batched library call over requests 0 .. len-1."""

    def __init__(self, kvq, oq, hq, hkv, batch, int2_pages, int4_pages, max_pages, calls, seed, layers=2):
        self.kvq, self.oq = kvq, oq
        self.hq, self.hkv, self.batch, self.seed = hq, hkv, batch, seed
        self.int2_pages, self.int4_pages, self.max_pages = int2_pages, int4_pages, max_pages
        self.layers = layers
        shape = kvq.make_shape(hq, hkv, batch, page_tokens=PAGE, int2_pages=int2_pages, int4_pages=int4_pages)
        self.plan = kvq.plan_layers(shape, [(2, 2, 0, 1)] * layers)
        self.pool = torch.zeros(self.plan.total_bytes, dtype=torch.uint8, device="cuda")
        pairs = [2 * p for p in syn.seeded_permutation(seed, syn.T_PAGE, int2_pages // 2)]
        quads = [int2_pages + p for p in syn.seeded_permutation(seed, syn.T_PAGE, int4_pages, salt=1)]
        self.pairs = {r: [] for r in range(batch)}
        self.quads = {r: [] for r in range(batch)}
        self.n2 = [0] * batch
        self.n4 = [0] * batch
        self.arrived = [0] * batch
        self.int2_idx = {r: [] for r in range(batch)}  # arrival indices of INT2 tokens, in order
        self.int4_idx = {r: [] for r in range(batch)}
        total = max(sum(n for rs, n, _ in calls if r in rs) for r in range(batch)) or 1
        self.total = total
        self.k = [syn.keys_fp16(seed, l, range(batch), range(hkv), 0, total, outlier_count=4, outlier_factor=10.0,
                                num_kv_heads=hkv) for l in range(layers)]
        self.v = [syn.values_fp16(seed, l, range(batch), range(hkv), 0, total) for l in range(layers)]
        self.table = torch.zeros(batch, max_pages, dtype=torch.int32, device="cuda")
        self.d_n2 = torch.zeros(batch, dtype=torch.int32, device="cuda")
        self.d_n4 = torch.zeros(batch, dtype=torch.int32, device="cuda")
        self.d_add = torch.zeros(batch, dtype=torch.int32, device="cuda")
        for rs, n_new, add2 in calls:
            rs = list(rs)
            for r in rs:  # table state after the call
                while len(self.pairs[r]) < (self.n2[r] + add2) // 32:
                    self.pairs[r].append(pairs.pop())
                while len(self.quads[r]) * PAGE < self.n4[r] + n_new - add2:
                    self.quads[r].append(quads.pop())
                row = [x for p in self.pairs[r] for x in (p, p + 1)] + self.quads[r]
                assert len(row) <= max_pages
                self.table[r, :len(row)] = torch.tensor(row, dtype=torch.int32)
                self.d_add[r] = add2
            self.d_n2.copy_(torch.tensor(self.n2, dtype=torch.int32))
            self.d_n4.copy_(torch.tensor(self.n4, dtype=torch.int32))
            for l in range(layers):
                if rs == list(range(len(rs))) and len(rs) > 1:
                    self._append(l, rs, n_new, 0)
                else:
                    for r in rs:
                        self._append(l, [r], n_new, r)
            for r in rs:
                a0 = self.arrived[r]
                self.int2_idx[r] += list(range(a0, a0 + add2))
                self.int4_idx[r] += list(range(a0 + add2, a0 + n_new))
                self.arrived[r] += n_new
                self.n2[r] += add2
                self.n4[r] += n_new - add2
        self.d_n2.copy_(torch.tensor(self.n2, dtype=torch.int32))
        self.d_n4.copy_(torch.tensor(self.n4, dtype=torch.int32))
        torch.cuda.synchronize()

    def _append(self, l, rs, n_new, r0):
        kk = torch.stack([self.k[l][r, :, self.arrived[r]:self.arrived[r] + n_new] for r in rs]).contiguous().cuda()
        vv = torch.stack([self.v[l][r, :, self.arrived[r]:self.arrived[r] + n_new] for r in rs]).contiguous().cuda()
        pages = self.kvq.make_pages(self.table[r0], self.max_pages, self.d_n2[r0:], self.d_n4[r0:], self.d_add[r0:])
        self.kvq.quantize_append(self.plan, l, self.pool, kk, vv, None, pages)

    def pages(self):
        return self.kvq.make_pages(self.table, self.max_pages, self.d_n2, self.d_n4)

    def logical(self, l, r, h):
        idx = self.int2_idx[r] + self.int4_idx[r]
        return self.k[l][r, h, idx].numpy(), self.v[l][r, h, idx].numpy()

    def oracle_pool(self, l):
        lp = self.plan.layers[l]
        pool = np.zeros(lp.bytes, np.uint8)
        tb = self.table.cpu().numpy()
        for r in range(self.batch):
            for h in range(self.hkv):
                k, v = self.logical(l, r, h)
                self.oq.pack_paged(pool, k, v, self.n2[r], tb[r], self.int2_pages, self.hkv, h)
        return pool

    def layer_bytes(self, l):
        lp = self.plan.layers[l]
        return self.pool[lp.offset:lp.offset + lp.bytes].cpu().numpy()

    def max_len(self):
        return max(a + b for a, b in zip(self.n2, self.n4))

    def decode(self, l, q, splits=0, out_dtype=torch.float32):
        kvq = self.kvq
        ml = self.max_len()
        out = torch.full((self.batch, self.hq, 128), float("nan"), dtype=out_dtype, device="cuda")
        lse = torch.full((self.batch, self.hq), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(kvq.workspace_bytes(self.plan, self.batch, ml, splits) // 4 + 1, dtype=torch.float32,
                         device="cuda")
        kvq.decode_attention(self.plan, l, self.pool, q, None, ml, 1 / math.sqrt(128), out, lse, ws, splits,
                             pages=self.pages())
        torch.cuda.synchronize()
        return out.float().cpu().numpy(), lse.cpu().numpy()

    def oracle_decode(self, l, q, pool):
        G = self.hq // self.hkv
        out = np.zeros((self.batch, self.hq, 128))
        lse = np.zeros((self.batch, self.hq))
        tb = self.table.cpu().numpy()
        for r in range(self.batch):
            for h in range(self.hkv):
                kd, vd = self.oq.unpack_paged(pool, self.n2[r], self.n4[r], tb[r], self.int2_pages, self.hkv, h)
                o, ls = self.oq.attention(q[r, h * G:(h + 1) * G].cpu().numpy(), kd, vd, 1 / math.sqrt(128))
                out[r, h * G:(h + 1) * G] = o
                lse[r, h * G:(h + 1) * G] = ls
        return out, lse


def _check(out, lse, ref, ref_lse, lens):
    empty = [r for r, L in enumerate(lens) if L == 0]
    full = [r for r, L in enumerate(lens) if L > 0]
    for r in empty:
        assert np.all(out[r] == 0) and np.all(lse[r] == -np.inf)
    o, rf = out[full], ref[full]
    rel = np.linalg.norm(o - rf) / np.linalg.norm(rf)
    assert rel <= REL_L2, f"rel L2 {rel:.3g}"
    assert np.abs(o - rf).max() <= MAX_ABS, f"max abs {np.abs(o - rf).max():.3g}"
    assert np.abs(lse[full] - ref_lse[full]).max() <= LSE_ABS


# r0: INT2 + INT4, then more INT2 after INT4 tokens exist (its INT4 page moves in the table);
# r1: INT4 only; r2: INT2 only; r3: nothing before the decode appends; r4: stays empty.
# Then three one-token decode appends for requests 0..3 in one batched call each.
SCHEDULE = [([0], 40, 32), ([1], 17, 0), ([2], 64, 64), ([0], 65, 64),
            ([0, 1, 2, 3], 1, 0), ([0, 1, 2, 3], 1, 0), ([0, 1, 2, 3], 1, 0)]


@pytest.fixture(scope="module")
def small(gpu, oq):
    return PagedCase(gpu, oq, hq=8, hkv=2, batch=5, int2_pages=24, int4_pages=12, max_pages=16, calls=SCHEDULE,
                     seed=5)


@pytest.fixture(scope="module")
def long(gpu, oq):
    # G = 7; 40 INT2 groups and 300 INT4 tokens (a partial last page pair) for r0
    calls = [([0], 1580, 1280), ([1], 33, 32), ([0, 1], 1, 0)]
    return PagedCase(gpu, oq, hq=14, hkv=2, batch=2, int2_pages=96, int4_pages=32, max_pages=112, calls=calls,
                     seed=8, layers=1)


def test_paged_lengths(small):
    assert small.n2 == [96, 0, 64, 0, 0] and small.n4 == [12, 20, 3, 3, 0]


@pytest.mark.parametrize("case", ["small", "long"])
def test_paged_pool_bytes_bit_exact(case, request):
    c = request.getfixturevalue(case)
    for l in range(c.layers):
        want = c.oracle_pool(l)
        got = c.layer_bytes(l)
        bad = np.nonzero(want != got)[0]
        assert bad.size == 0, f"layer {l}: {bad.size} bytes differ, first at {bad[:8]}"


@pytest.mark.parametrize("case", ["small", "long"])
def test_paged_dequantize_bit_exact(case, request, oq):
    c = request.getfixturevalue(case)
    ml = c.max_len()
    tb = c.table.cpu().numpy()
    for l in range(c.layers):
        ko = torch.full((c.batch, c.hkv, ml, 128), float("nan"), device="cuda")
        vo = torch.full_like(ko, float("nan"))
        c.kvq.dequantize(c.plan, l, c.pool, None, c.batch, ml, ko, vo, pages=c.pages())
        torch.cuda.synchronize()
        ko, vo = ko.cpu().numpy(), vo.cpu().numpy()
        pool = c.oracle_pool(l)
        for r in range(c.batch):
            L = c.n2[r] + c.n4[r]
            for h in range(c.hkv):
                kd, vd = oq.unpack_paged(pool, c.n2[r], c.n4[r], tb[r], c.int2_pages, c.hkv, h)
                assert np.array_equal(ko[r, h, :L], kd) and np.array_equal(vo[r, h, :L], vd), (l, r, h)
                assert np.isnan(ko[r, h, L:]).all()


@pytest.mark.parametrize("splits", [0, 2, 3, 9])
def test_paged_decode_parity(small, splits):
    c = small
    for l in range(c.layers):
        q = syn.queries_fp16(c.seed, l, 0, c.batch, c.hq).cuda()
        out, lse = c.decode(l, q, splits)
        ref, ref_lse = c.oracle_decode(l, q, c.oracle_pool(l))
        _check(out, lse, ref, ref_lse, [a + b for a, b in zip(c.n2, c.n4)])


@pytest.mark.parametrize("splits", [0, 2, 5])
def test_paged_decode_long_g7(long, splits):
    c = long
    q = syn.queries_fp16(c.seed, 0, 0, c.batch, c.hq).cuda()
    out, lse = c.decode(0, q, splits, out_dtype=torch.float16)
    ref, ref_lse = c.oracle_decode(0, q, c.oracle_pool(0))
    _check(out, lse, ref, ref_lse, [a + b for a, b in zip(c.n2, c.n4)])


def test_paged_decode_deterministic(small):
    q = syn.queries_fp16(small.seed, 0, 1, small.batch, small.hq).cuda()
    a = small.decode(0, q)
    b = small.decode(0, q)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _fused_vs_separate(c, B, splits, steps=3):
    """steps one-token decode appends for requests 0 .. B-1: kvq_append_decode_attention on one
    copy of the pool against kvq_quantize_append(n_new = 1) then kvq_decode_attention on another;
    pool bytes, output and log-sum-exp must agree bit for bit."""
    kvq = c.kvq
    pool_a, pool_b = c.pool.clone(), c.pool.clone()
    n2 = torch.tensor(c.n2[:B], dtype=torch.int32, device="cuda")
    n4 = torch.tensor(c.n4[:B], dtype=torch.int32, device="cuda")
    table = c.table[:B].contiguous()
    for step in range(steps):
        before, after = n4.clone(), n4 + 1
        ml = max(a + b for a, b in zip(c.n2[:B], c.n4[:B])) + step + 1
        ws = torch.empty(kvq.workspace_bytes(c.plan, B, ml, splits) // 4 + 1, dtype=torch.float32, device="cuda")
        for l in range(c.layers):
            kn = syn.keys_fp16(c.seed + 1, l, range(B), range(c.hkv), 1000 + step, 1, num_kv_heads=c.hkv).cuda()
            vn = syn.values_fp16(c.seed + 1, l, range(B), range(c.hkv), 1000 + step, 1).cuda()
            q = syn.queries_fp16(c.seed + 1, l, step, B, c.hq).cuda()
            outs = []
            for fused, pool in ((True, pool_a), (False, pool_b)):
                out = torch.full((B, c.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
                lse = torch.full((B, c.hq), float("nan"), dtype=torch.float32, device="cuda")
                if fused:
                    pg = kvq.make_pages(table, c.max_pages, n2, before)
                    kvq.append_decode_attention(c.plan, l, pool, kn, vn, q, None, ml, 1 / math.sqrt(128), out, lse,
                                                ws, splits, pages=pg)
                else:
                    kvq.quantize_append(c.plan, l, pool, kn, vn, None, kvq.make_pages(table, c.max_pages, n2, before))
                    kvq.decode_attention(c.plan, l, pool, q, None, ml, 1 / math.sqrt(128), out, lse, ws, splits,
                                         pages=kvq.make_pages(table, c.max_pages, n2, after))
                torch.cuda.synchronize()
                outs.append((out.cpu().numpy(), lse.cpu().numpy()))
            assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1]), (step, l)
            assert np.isfinite(outs[0][0]).all()
        assert torch.equal(pool_a, pool_b), f"step {step}: pool bytes differ"
        n4 = after


@pytest.mark.parametrize("splits", [0, 3])
def test_fused_paged_step_equals_separate_calls(small, splits):
    """kvq_append_decode_attention on a paged pool: three decode steps of requests 0..3 (their
    new INT4 tokens land in pages the tables already hold) give, bit for bit, the pool bytes,
    output and log-sum-exp of kvq_quantize_append(n_new = 1) followed by kvq_decode_attention."""
    _fused_vs_separate(small, 4, splits)


@pytest.fixture(scope="module")
def bounds(gpu, oq):
    # INT4 lengths 30, 31, 127 and 159 (after 64 INT2 tokens): the fused steps write tokens
    # that complete a page pair (31, 127: the pair is then the first one its wave reads), open
    # a new pair (32) and land in a wave's second pair (159, one split); every table is then
    # extended by unused INT4 pages to hold three more tokens
    calls = [([0], 30, 0), ([1], 31, 0), ([2], 127, 0), ([3], 64 + 159, 64)]
    c = PagedCase(gpu, oq, hq=8, hkv=2, batch=4, int2_pages=8, int4_pages=32, max_pages=16, calls=calls, seed=12,
                  layers=1)
    used = {p for r in range(c.batch) for p in c.quads[r]}
    free = [p for p in range(c.int2_pages, c.int2_pages + c.int4_pages) if p not in used]
    for r in range(c.batch):
        have = len(c.pairs[r]) * 2 + len(c.quads[r])
        need = -(-(c.n4[r] + 3) // PAGE) - len(c.quads[r])
        for i in range(need):
            c.table[r, have + i] = free.pop()
    return c


def test_bounds_lengths(bounds):
    assert bounds.n2 == [0, 0, 0, 64] and bounds.n4 == [30, 31, 127, 159]


@pytest.mark.parametrize("splits", [0, 2, 3])
def test_fused_paged_step_at_pair_boundaries(bounds, splits):
    """The fused paged step where the new token completes a page pair, opens one, or lands in
    a pair its wave reads second: bit for bit the separate calls' pool, output and lse."""
    _fused_vs_separate(bounds, 4, splits)


@pytest.mark.parametrize("case,chunk,splits", [("small", 5, 0), ("small", 40, 3), ("long", 9, 0), ("long", 33, 2)])
def test_paged_prefix_and_chunk_prefill(case, chunk, splits, request, oq):
    """Chunked prefill over a paged pool: kvq_prefix_attention (every chunk row over the request's
    INT2 then INT4 tokens, no mask) and kvq_chunk_prefill_attention (plus the chunk's own fp16
    tokens, causally) against fp64 attention over the oracle's own unpacking of the same pool."""
    c = request.getfixturevalue(case)
    kvq = c.kvq
    G = c.hq // c.hkv
    ml = c.max_len()
    q = syn.queries_steps_fp16(c.seed, 0, c.batch, c.hq, 900, chunk).permute(0, 2, 1, 3).contiguous()
    kc = syn.keys_fp16(c.seed + 7, 0, range(c.batch), range(c.hkv), 0, chunk, num_kv_heads=c.hkv).contiguous()
    vc = syn.values_fp16(c.seed + 7, 0, range(c.batch), range(c.hkv), 0, chunk).contiguous()
    pool = c.oracle_pool(0)
    tb = c.table.cpu().numpy()
    scale = 1 / math.sqrt(128)
    ref_p = np.zeros((c.batch, chunk, c.hq, 128))
    lse_p = np.zeros((c.batch, chunk, c.hq))
    ref_c = np.zeros_like(ref_p)
    lse_c = np.zeros_like(lse_p)
    for r in range(c.batch):
        for h in range(c.hkv):
            kd, vd = oq.unpack_paged(pool, c.n2[r], c.n4[r], tb[r], c.int2_pages, c.hkv, h)
            rows = q[r, :, h * G:(h + 1) * G].reshape(chunk * G, 128).numpy()
            o, ls = oq.attention(rows, kd, vd, scale)
            ref_p[r, :, h * G:(h + 1) * G] = o.reshape(chunk, G, 128)
            lse_p[r, :, h * G:(h + 1) * G] = ls.reshape(chunk, G)
            kcf = kc[r, h].numpy().astype(np.float32)
            vcf = vc[r, h].numpy().astype(np.float32)
            for i in range(chunk):
                o, ls = oq.attention(q[r, i, h * G:(h + 1) * G].numpy(), np.concatenate([kd, kcf[:i + 1]]),
                                     np.concatenate([vd, vcf[:i + 1]]), scale)
                ref_c[r, i, h * G:(h + 1) * G] = o
                lse_c[r, i, h * G:(h + 1) * G] = ls
    n = c.batch * chunk
    lens = [c.n2[r] + c.n4[r] for r in range(c.batch) for _ in range(chunk)]
    # prefix part alone
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    wsb = kvq.prefix_workspace_bytes(c.plan, c.batch, chunk, ml, splits)
    ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device="cuda") if wsb else None
    kvq.prefix_attention(c.plan, 0, c.pool, q.cuda(), None, ml, scale, out, lse, ws, splits, pages=c.pages())
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy().reshape(n, c.hq, 128), lse.cpu().numpy().reshape(n, c.hq),
                    ref_p.reshape(n, c.hq, 128), lse_p.reshape(n, c.hq), lens, c.hq, c.hkv)
    # the whole chunked-prefill attention
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    wsb = kvq.chunk_prefill_workspace_bytes(c.plan, c.batch, chunk, ml, splits)
    ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device="cuda")
    kvq.chunk_prefill_attention(c.plan, 0, c.pool, q.cuda(), kc.cuda(), vc.cuda(), None, ml, scale, out, lse, ws,
                                splits, pages=c.pages())
    torch.cuda.synchronize()
    check_attention(out.cpu().numpy().reshape(n, c.hq, 128), lse.cpu().numpy().reshape(n, c.hq),
                    ref_c.reshape(n, c.hq, 128), lse_c.reshape(n, c.hq), [1] * n, c.hq, c.hkv)
