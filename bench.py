#!/usr/bin/env python3
"""Decode-attention benchmark of the layer-wise mixed-precision KV cache on one MI355X.

One step = one decode token for every request, through every layer: append the
token's fp16 K/V (tail write, and the 32-token group quantize-and-pack when the
tail fills), then split-KV decode attention over the packed cache and the
log-sum-exp merge. Inputs are seeded synthetic tensors (synthetic/), resident in
HBM before the timed region. Each step is replayed from a HIP graph captured
once per step position of the decode cycle.

Prints one JSON line (the benchmark contract), with a roofline object for the
split pass (algorithmic bytes per launch over its HIP-event duration) and a
CPU baseline (the oracle, timed on a bounded sample of the same step). Beside
the step, the line reports the append kernel at prefill size (HBM-bound) and
the chunked-prefill attention over the quantized prefix (matrix-core bound).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

# Kernel arguments in device memory (the HIP runtime's HIP_FORCE_DEV_KERNARG), set before the
# runtime starts; a value the caller set is kept. The graph-replayed step runs at the same
# speed either way, while an eagerly launched kernel otherwise fetches its arguments from host
# memory at the start of each dispatch: with them in device memory the eager per-dispatch
# event timing below measures the kernels as the timed graphs run them.
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthetic as syn  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak
METRIC = "decode-attention tokens/s and effective HBM GB/s (% of peak), batch 64, 1 GPU"


# ----------------------------------------------------------------- workloads
def _llama_mixed_map(seed):
    hi = set(syn.seeded_choice(seed, syn.T_MAP, 32, 8))
    return [(4, 4) if l in hi else (4, 2) for l in range(32)]


def _qwen_map(seed):
    hi = set(syn.seeded_choice(seed, syn.T_MAP, 28, 9, salt=1))
    return [(8, 4) if l in hi else (4, 2) for l in range(28)]


# prefill P tokens; a timed step appends token P + (i mod cycle), so the cache
# holds P + 1 .. P + cycle tokens over a cycle.
WORKLOADS = {
    "single-head-k8v4-l512": dict(layers=1, hq=1, hkv=1, batch=1, prefill=511, cycle=1,
                                  map=lambda s: [(8, 4)], outliers=(4, 10.0),
                                  desc="1 layer, 1 request, 1 q/KV head, 512 cached tokens, K8V4"),
    "llama31-8b-b64-kivi8-trace": dict(layers=32, hq=32, hkv=8, batch=64, prefill=128, cycle=128,
                                       map=lambda s: [(8, 8)] * 32, outliers=(4, 10.0),
                                       desc="Llama-3.1-8B attention shape, batch 64, 128-token prompt + "
                                            "128 decode steps, uniform K8V8"),
    "llama31-8b-b64-mixed325-l2048": dict(layers=32, hq=32, hkv=8, batch=64, prefill=2047, cycle=32,
                                          map=_llama_mixed_map, outliers=(4, 10.0),
                                          desc="Llama-3.1-8B shape, batch 64, context 2048..2079, seeded "
                                               "24 x K4V2 + 8 x K4V4 (3.25 bits)"),
    "qwen25-7b-b32-map396-l8192": dict(layers=28, hq=28, hkv=4, batch=32, prefill=8191, cycle=32,
                                       map=_qwen_map, outliers=(8, 20.0),
                                       desc="Qwen2.5-7B shape, batch 32, context 8192..8223, seeded "
                                            "9 x K8V4 + 19 x K4V2 (3.96 bits)"),
}
# Paged INT2/INT4 pool (TriAxialKV-style): every layer is a pool of 16-token pages; the prompt
# tokens of the tags the allocator sets to INT2, in 32-token groups, are INT2 (keys per-channel,
# values per-token), the rest and every decoded token INT4 per-token; tables in seeded page order.
PAGED_WORKLOADS = {
    "paged-b16-l32768-int2int4": dict(layers=36, hq=32, hkv=8, batch=16, prefill=32767, cycle=32,
                                      outliers=(4, 10.0), tags=8, budget=3.0,
                                      desc="36 layers, 32/8 heads, batch 16, context 32768..32799 in a paged pool: "
                                           "8 seeded role tags a request, each INT2 or INT4 by the allocator from "
                                           "D_k(b) measured with the library on a calibration sample at a 3.0-bit "
                                           "budget; the INT2 tags' tokens in 32-token groups, the rest and every "
                                           "decoded token INT4"),
}
WORKLOADS.update({k: dict(v, paged=True) for k, v in PAGED_WORKLOADS.items()})
DEFAULT_WORKLOAD = "llama31-8b-b64-mixed325-l2048"
# timed beside the headline, in the same JSON line: the uniform K8V8 (KIVI-8-like) baseline
SECONDARY_WORKLOAD = "llama31-8b-b64-kivi8-trace"


def capacity(w):
    return w["prefill"] + w["cycle"]


class Workload:
    """A planned, prefilled cache on the GPU plus the inputs of every decode step."""

    def __init__(self, name, seed=0, device="cuda", num_splits=0, gen_chunk=8, layers=None, fused=True):
        """layers: indices of the workload's layers to build (default all); a subset keeps every
        layer's shapes, data and launches, and is used by the full-size parity tests. fused: append
        through the fused append-and-decode call (else quantize_append, then decode_attention)."""
        self.fused = fused
        import torch

        import layer_wise_mixed_amd as kvq

        self.name, self.seed, self.kvq = name, seed, kvq
        w = self.w = WORKLOADS[name]
        self.layer_ids = list(range(w["layers"])) if layers is None else list(layers)
        self.L, self.B, self.Hq, self.Hkv = len(self.layer_ids), w["batch"], w["hq"], w["hkv"]
        self.P, self.C = w["prefill"], w["cycle"]
        self.cap = capacity(w)
        full_map = w["map"](seed)
        self.cfg = [full_map[i] for i in self.layer_ids]
        self.outliers = w["outliers"]
        self.shape = kvq.make_shape(self.Hq, self.Hkv, self.B, max_tokens=self.cap)
        self.plan = kvq.plan_layers(self.shape, self.cfg)
        self.cache = torch.empty(self.plan.total_bytes, dtype=torch.uint8, device=device)
        self.scale = 1.0 / math.sqrt(128.0)
        self.num_splits = num_splits
        zeros = torch.zeros(self.B, dtype=torch.int32, device=device)
        for l, li in enumerate(self.layer_ids):  # prefill, a few requests at a time
            for r0 in range(0, self.B, gen_chunk):
                rs = range(r0, min(self.B, r0 + gen_chunk))
                k = self.keys(li, rs, 0, self.P, device)
                v = syn.values_fp16(seed, li, rs, range(self.Hkv), 0, self.P, device=device)
                off = r0 * self.Hkv * self.plan.layers[l].stream_bytes
                kvq.quantize_append(self.plan, l, self.cache[off:], k, v, zeros[: len(rs)])
                del k, v
        torch.cuda.synchronize()
        # decode-step inputs: [cycle][batch][heads][1][128] and q [cycle][batch][Hq][128]
        self.k_dec, self.v_dec, self.q = [], [], []
        for li in self.layer_ids:
            k = self.keys(li, range(self.B), self.P, self.C, device)
            v = syn.values_fp16(seed, li, range(self.B), range(self.Hkv), self.P, self.C, device=device)
            self.k_dec.append(k.permute(2, 0, 1, 3).contiguous().unsqueeze(3))
            self.v_dec.append(v.permute(2, 0, 1, 3).contiguous().unsqueeze(3))
            qq = syn.queries_steps_fp16(seed, li, self.B, self.Hq, 0, self.C, device=device)
            self.q.append(qq.permute(2, 0, 1, 3).contiguous())
        self.lens_base = torch.full((self.B,), self.P, dtype=torch.int32, device=device)
        self.lens_before = self.lens_base.clone()
        self.lens_after = self.lens_base + 1
        self.max_len = self.cap
        self.splits = num_splits or kvq.num_splits(self.plan, 0, self.B, self.max_len)
        ws = kvq.workspace_bytes(self.plan, self.B, self.max_len, self.splits)
        self.ws = torch.empty(ws // 4 + 1, dtype=torch.float32, device=device)
        self.out = torch.empty(self.B, self.Hq, 128, dtype=torch.float16, device=device)
        torch.cuda.synchronize()

    def keys(self, layer, requests, t0, n, device):
        cnt, fac = self.outliers
        return syn.keys_fp16(self.seed, layer, requests, range(self.Hkv), t0, n, outlier_count=cnt,
                             outlier_factor=fac, num_kv_heads=self.Hkv, device=device)

    def prefill_append_rate(self, reps=10):
        """The first layer's prefill for the whole batch in one append call (every full group
        quantized and packed, the rest to the tail), timed with events around `reps` calls. It
        rewrites the same bytes the prefill wrote. Bytes: the fp16 K and V read, the records and
        tail slots written."""
        import torch

        kvq = self.kvq
        li = self.layer_ids[0]
        k = self.keys(li, range(self.B), 0, self.P, "cuda")
        v = syn.values_fp16(self.seed, li, range(self.B), range(self.Hkv), 0, self.P, device="cuda")
        zeros = torch.zeros(self.B, dtype=torch.int32, device="cuda")
        kvq.quantize_append(self.plan, 0, self.cache, k, v, zeros)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            kvq.quantize_append(self.plan, 0, self.cache, k, v, zeros)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps / 1e3
        lp = self.plan.layers[0]
        streams = self.B * self.Hkv
        nbytes = streams * self.P * 128 * 2 * 2 + streams * ((self.P // 32) * lp.record_bytes + (self.P % 32) * 512)
        return {"layer": li, "format": f"K{lp.k_bits}V{lp.v_bits}", "tokens": self.B * self.P, "us": t * 1e6,
                "bytes": nbytes, "GBps": nbytes / t / 1e9, "frac": nbytes / t / 1e9 / HBM_PEAK_GBS}

    def prefix_attention_rate(self, requests=4, chunk=256, reps=3):
        """Chunked prefill against the cache: `chunk` query tokens of each of the first
        `requests` requests attend over the first layer's cached prefix (P tokens) in one
        prefix-attention call; HIP events bound to the split pass time `reps` calls after one
        untimed call (timing only: by now the tail slots may hold later decode tokens). FLOPs:
        the two products, 2 * 2 * rows * P * 128, rows = requests * chunk * Hq."""
        import torch

        kvq = self.kvq
        li = self.layer_ids[0]
        nb = min(requests, self.B)
        q = syn.queries_steps_fp16(self.seed, li, nb, self.Hq, self.P, chunk, device="cuda")
        q = q.permute(0, 2, 1, 3).contiguous()
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        wsb = kvq.prefix_workspace_bytes(self.plan, nb, chunk, self.P)
        ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device="cuda") if wsb else None
        lens = torch.full((nb,), self.P, dtype=torch.int32, device="cuda")

        def call():
            kvq.prefix_attention(self.plan, 0, self.cache, q, lens, self.P, self.scale, out, lse, ws)

        call()
        torch.cuda.synchronize()
        kvq.timer_start(reps)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        ms, n = kvq.timer_read(kvq.TIMER_PREFIX)
        mms, mn = kvq.timer_read(kvq.TIMER_MERGE)
        kvq.timer_stop()
        t = ms / 1e3 / max(n, 1)
        tm = mms / 1e3 / max(mn, 1) if mn else 0.0
        rows = nb * chunk * self.Hq
        flops = 4.0 * rows * self.P * 128
        lp = self.plan.layers[0]
        return {"layer": li, "format": f"K{lp.k_bits}V{lp.v_bits}", "requests": nb, "chunk": chunk,
                "prefix": self.P, "rows": rows, "us": t * 1e6, "merge_us": tm * 1e6, "flops": flops,
                "TFLOPs": flops / t / 1e12, "bound": "mfma", "peak_TFLOPs": MFMA_F16_PEAK_TFLOPS,
                "frac": flops / t / 1e12 / MFMA_F16_PEAK_TFLOPS,
                "TFLOPs_with_merge": flops / (t + tm) / 1e12,
                "timing": "HIP events bound to the prefix kernel's dispatches (frac) and to the merge's"}

    def reset(self):
        self.lens_before.copy_(self.lens_base)
        self.lens_after.copy_(self.lens_base)
        self.lens_after.add_(1)

    def step(self, i):
        """Launch one decode step (all layers) for cycle position i: per layer, the token append
        fused into the decode split pass (one launch, plus the merge with several splits), or
        with fused=False the two calls."""
        kvq = self.kvq
        for l in range(self.L):
            if self.fused:
                kvq.append_decode_attention(self.plan, l, self.cache, self.k_dec[l][i], self.v_dec[l][i],
                                            self.q[l][i], self.lens_before, self.max_len, self.scale, self.out,
                                            None, self.ws, self.splits)
            else:
                kvq.quantize_append(self.plan, l, self.cache, self.k_dec[l][i], self.v_dec[l][i], self.lens_before)
                kvq.decode_attention(self.plan, l, self.cache, self.q[l][i], self.lens_after, self.max_len,
                                     self.scale, self.out, None, self.ws, self.splits)
        self.lens_before.add_(1)
        self.lens_after.add_(1)

    def split_bytes(self, i):
        """Algorithmic bytes the split passes of step i read: packed codes + scale/zero of the
        full groups, the fp16 tail, and q."""
        L = self.P + i + 1
        lq, t = (L // 32) * 32, L % 32
        total = 0
        for l in range(self.L):
            rb = self.plan.layers[l].record_bytes
            total += self.B * self.Hkv * ((lq // 32) * rb + t * 512) + self.B * self.Hq * 256
        return total


class PagedWorkload:
    """A prefilled paged pool on the GPU plus the inputs of every decode step (same interface as
    Workload). The prompt's INT2 runs go first in each request's page table, as the pool's page
    tables require; decoded tokens are INT4."""

    PAGE = 16

    def __init__(self, name, seed=0, device="cuda", num_splits=0, layers=None, fused=True):
        import torch

        import layer_wise_mixed_amd as kvq

        self.name, self.seed, self.kvq = name, seed, kvq
        self.fused = fused
        w = self.w = WORKLOADS[name]
        self.layer_ids = list(range(w["layers"])) if layers is None else list(layers)
        self.L, self.B, self.Hq, self.Hkv = len(self.layer_ids), w["batch"], w["hq"], w["hkv"]
        self.P, self.C = w["prefill"], w["cycle"]
        self.outliers = w["outliers"]
        self.scale = 1.0 / math.sqrt(128.0)
        # which prompt tokens are INT2: each request's tokens carry seeded role tags; D_k(b) of every
        # tag, measured with the library's kernels on a calibration sample (two requests, 2048
        # tokens, this workload's head shape), feeds the allocator at the workload's bit budget; the
        # INT2 tags' tokens form 32-token groups in arrival order, the rest go INT4
        from layer_wise_mixed_amd.allocate import int2_tokens
        from layer_wise_mixed_amd.distortion import calibrate

        self.num_tags, self.budget = w["tags"], w["budget"]
        self.D, self.tag_bits, _ = calibrate(self.Hq, self.Hkv, self.num_tags, self.budget, batch=2, seq_len=2048,
                                             seed=seed, outliers=self.outliers, device=device)
        self.orders, self.n2s = [], []
        for r in range(self.B):
            tags = syn.seeded_tags(seed, r, self.P, self.num_tags)
            a2, a4 = int2_tokens(tags, self.tag_bits)
            self.orders.append(a2 + a4)
            self.n2s.append(len(a2))
        pairs_r = [n2 // 32 for n2 in self.n2s]
        quads_r = [-(-(self.P - n2 + self.C) // self.PAGE) for n2 in self.n2s]
        self.int2_pages = 2 * sum(pairs_r)
        self.int4_pages = sum(quads_r)
        self.max_pages = max(2 * p + q for p, q in zip(pairs_r, quads_r))
        shape = kvq.make_shape(self.Hq, self.Hkv, self.B, page_tokens=self.PAGE, int2_pages=self.int2_pages,
                               int4_pages=self.int4_pages)
        self.plan = kvq.plan_layers(shape, [(2, 2, 0, 1)] * self.L)
        self.cache = torch.empty(self.plan.total_bytes, dtype=torch.uint8, device=device)
        # seeded physical page order, one table per request (shared by all layers)
        pairs = syn.seeded_permutation(seed, syn.T_PAGE, self.int2_pages // 2)
        quads = syn.seeded_permutation(seed, syn.T_PAGE, self.int4_pages, salt=1)
        table = np.zeros((self.B, self.max_pages), np.int32)
        p0, q0 = 0, 0
        for r in range(self.B):
            row = [x for p in pairs[p0:p0 + pairs_r[r]] for x in (2 * p, 2 * p + 1)]
            row += [self.int2_pages + q for q in quads[q0:q0 + quads_r[r]]]
            p0 += pairs_r[r]
            q0 += quads_r[r]
            table[r, :len(row)] = row
        self.table = torch.from_numpy(table).to(device)
        self.num_splits = num_splits
        zero = torch.zeros(self.B, dtype=torch.int32, device=device)
        add2 = torch.tensor(self.n2s, dtype=torch.int32, device=device)
        orders = [torch.tensor(self._prompt_order(r), dtype=torch.int64, device=device) for r in range(self.B)]
        for l, li in enumerate(self.layer_ids):  # prefill one request at a time: INT2 runs first, then the rest
            for r in range(self.B):
                order = orders[r]
                k = self.keys(li, [r], 0, self.P, device).index_select(2, order)
                v = syn.values_fp16(seed, li, [r], range(self.Hkv), 0, self.P, device=device).index_select(2, order)
                pages = kvq.make_pages(self.table[r], self.max_pages, zero[r:], zero[r:], add2[r:])
                kvq.quantize_append(self.plan, l, self.cache, k, v, None, pages)
                del k, v
        torch.cuda.synchronize()
        self.k_dec, self.v_dec, self.q = [], [], []
        for li in self.layer_ids:
            k = self.keys(li, range(self.B), self.P, self.C, device)
            v = syn.values_fp16(seed, li, range(self.B), range(self.Hkv), self.P, self.C, device=device)
            self.k_dec.append(k.permute(2, 0, 1, 3).contiguous().unsqueeze(3))
            self.v_dec.append(v.permute(2, 0, 1, 3).contiguous().unsqueeze(3))
            qq = syn.queries_steps_fp16(seed, li, self.B, self.Hq, 0, self.C, device=device)
            self.q.append(qq.permute(2, 0, 1, 3).contiguous())
        self.n2_dev = torch.tensor(self.n2s, dtype=torch.int32, device=device)
        self.n4_base = torch.tensor([self.P - n2 for n2 in self.n2s], dtype=torch.int32, device=device)
        self.n4_before = self.n4_base.clone()
        self.n4_after = self.n4_base + 1
        self.pages_append = kvq.make_pages(self.table, self.max_pages, self.n2_dev, self.n4_before)
        self.pages_decode = kvq.make_pages(self.table, self.max_pages, self.n2_dev, self.n4_after)
        self.max_len = self.P + self.C
        self.splits = num_splits or kvq.num_splits(self.plan, 0, self.B, self.max_len)
        ws = kvq.workspace_bytes(self.plan, self.B, self.max_len, self.splits)
        self.ws = torch.empty(ws // 4 + 1, dtype=torch.float32, device=device)
        self.out = torch.empty(self.B, self.Hq, 128, dtype=torch.float16, device=device)
        self.cfg = [(2, 2)] * self.L
        torch.cuda.synchronize()

    def _prompt_order(self, r):
        """Token indices of request r's prompt in append order: the tokens of its INT2 tags that fill
        whole 32-token groups, in arrival order, then every other token in arrival order."""
        return list(self.orders[r])

    def equiv_bits(self):
        """Mean code bits per cached token at the first decode step (INT2 2, INT4 4)."""
        n2 = sum(self.n2s)
        total = self.B * (self.P + 1)
        return (2.0 * n2 + 4.0 * (total - n2)) / total

    def keys(self, layer, requests, t0, n, device):
        cnt, fac = self.outliers
        return syn.keys_fp16(self.seed, layer, requests, range(self.Hkv), t0, n, outlier_count=cnt,
                             outlier_factor=fac, num_kv_heads=self.Hkv, device=device)

    def reset(self):
        self.n4_before.copy_(self.n4_base)
        self.n4_after.copy_(self.n4_base)
        self.n4_after.add_(1)

    def step(self, i):
        """One decode step: per layer, the new INT4 token appended inside the paged split pass
        (plus the merge), or with fused=False the append kernel, then the decode."""
        kvq = self.kvq
        for l in range(self.L):
            if self.fused:
                kvq.append_decode_attention(self.plan, l, self.cache, self.k_dec[l][i], self.v_dec[l][i],
                                            self.q[l][i], None, self.max_len, self.scale, self.out, None, self.ws,
                                            self.splits, pages=self.pages_append)
            else:
                kvq.quantize_append(self.plan, l, self.cache, self.k_dec[l][i], self.v_dec[l][i], None,
                                    self.pages_append)
                kvq.decode_attention(self.plan, l, self.cache, self.q[l][i], None, self.max_len, self.scale,
                                     self.out, None, self.ws, self.splits, pages=self.pages_decode)
        self.n4_before.add_(1)
        self.n4_after.add_(1)

    def split_bytes(self, i):
        """Algorithmic bytes the split passes of step i read: INT2 group records (codes + meta),
        INT4 tokens (codes + meta, 192 B per token and KV head), and q."""
        per_layer = self.B * self.Hq * 256
        for n2 in self.n2s:
            n4 = self.P - n2 + i + 1
            per_layer += self.Hkv * ((n2 // 32) * 4096 + n4 * 192)
        return per_layer * self.L


# the kernel sources of the decode step (the prefix-attention kernel is not part of it)
STEP_SOURCES = ["kvq_api.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_internal.h", "kvq_quantize.h",
                "kvq_split_mfma.hip"]


def _source_hash():
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        with open(os.path.join(ROOT, "layer_wise_mixed_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _traffic(workload, window):
    """HBM bytes per split launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources over the same window of cycle positions as this run's timed
    steps (`window` = [first, last] position, every position between them timed); else None."""
    path = os.path.join(ROOT, "profiles", "split_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        e = d.get(workload)
        if not e or e.get("source_hash") != _source_hash() or e.get("window") != list(window):
            return None
        return e["hbm_bytes_per_launch"]
    except Exception:
        return None


# -------------------------------------------------------------- CPU baseline
def _timed_reps(fn, max_seconds, max_reps=1000):
    """Call fn() until about max_seconds have passed: (seconds per call, calls, fn's last result)."""
    t0 = time.perf_counter()
    reps, res = 0, None
    while True:
        res = fn()
        reps += 1
        if time.perf_counter() - t0 > max_seconds or reps >= max_reps:
            break
    return (time.perf_counter() - t0) / reps, reps, res


def _threads():
    return min(os.cpu_count() or 1, 16)


def cpu_baseline_paged(wl, positions, max_seconds=15.0):
    """The oracle on a sample of the timed decode steps of a paged workload: it packs a sample of
    (request, KV head) streams of layer 0 into its own pool through the same page tables, each
    stream at the INT4 length of one of the timed cycle positions, then times unpack +
    dequantize + fp64 attention on all host threads (up to 16) and on one thread."""

    import oracle

    G = wl.Hq // wl.Hkv
    layer = wl.layer_ids[0]
    n_streams = min(wl.B * wl.Hkv, 16)
    pool = np.zeros(oracle.paged_pool_bytes(wl.Hkv, wl.int2_pages, wl.int4_pages), np.uint8)
    tables = wl.table.cpu().numpy()
    cnt, fac = wl.outliers
    req, head, n4s, qs = [], [], [], np.zeros((n_streams, G, 128), np.float16)
    for s in range(n_streams):
        r, h = divmod(s, wl.Hkv)
        pos = positions[s % len(positions)]
        n4 = wl.P - wl.n2s[r] + pos + 1
        order = wl._prompt_order(r) + list(range(wl.P, wl.P + pos + 1))
        k = syn.keys_fp16(wl.seed, layer, [r], [h], 0, wl.P + pos + 1, outlier_count=cnt, outlier_factor=fac,
                          num_kv_heads=wl.Hkv)[0, 0].numpy()[order]
        v = syn.values_fp16(wl.seed, layer, [r], [h], 0, wl.P + pos + 1)[0, 0].numpy()[order]
        oracle.pack_paged(pool, k, v, wl.n2s[r], tables[r], wl.int2_pages, wl.Hkv, h)
        req.append(r)
        head.append(h)
        n4s.append(n4)
        qs[s] = syn.queries_fp16(wl.seed, layer, pos, r + 1, wl.Hq)[r, h * G:(h + 1) * G].numpy()

    n2s = [wl.n2s[r] for r in req]

    def run(ns, threads):
        return oracle.decode_paged(pool, req[:ns], head[:ns], n2s[:ns], n4s[:ns], tables, wl.int2_pages,
                                   wl.Hkv, qs[:ns], G, wl.scale, threads)[2]

    dt, reps, used = _timed_reps(lambda: run(n_streams, _threads()), max_seconds)
    n1 = min(n_streams, 2)
    dt1, reps1, _ = _timed_reps(lambda: run(n1, 1), max_seconds / 3)
    scale = wl.B * wl.Hkv * wl.L
    t_step, t_step1 = dt / n_streams * scale, dt1 / n1 * scale
    return {"value": wl.B / t_step, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "value_1thread": wl.B / t_step1,
            "sample": f"{n_streams} (request, KV head) streams of layer 0, each at the length of one of the timed "
                      f"cycle positions ({min(n2s)}..{max(n2s)} INT2 + {min(n4s)}..{max(n4s)} INT4 tokens), "
                      f"repeated {reps}x "
                      f"({dt * 1e3:.1f} ms each) on {int(used)} threads, and {n1} streams {reps1}x on 1 thread; "
                      f"step time scaled to {wl.B * wl.Hkv} streams x {wl.L} layers"}


def cpu_baseline(wl, positions, max_seconds=15.0):
    """The oracle, timed on host cores on a sample of the timed decode steps: a sample of (request,
    KV head) streams of layer 0, each at the cache length of one of the timed cycle positions,
    packed by the oracle into its own layer; it unpacks + dequantizes them and runs fp64
    attention, on all host threads (up to 16) and on one thread."""

    import oracle

    if isinstance(wl, PagedWorkload):
        return cpu_baseline_paged(wl, positions, max_seconds)

    G = wl.Hq // wl.Hkv
    layer = wl.layer_ids[0]
    lp = wl.plan.layers[0]
    kb, vb, kt = lp.k_bits, lp.v_bits, lp.k_axis == 1
    cap_groups = wl.cap // 32
    stride = oracle.stream_bytes(kb, vb, cap_groups)
    # build the oracle's own packed cache for a sample of streams (not timed)
    n_streams = min(wl.B * wl.Hkv, 64)
    buf = np.zeros(n_streams * stride, np.uint8)
    qs = np.zeros((n_streams, G, 128), np.float16)
    lens = np.zeros(n_streams, np.int64)
    cnt, fac = wl.outliers
    for s in range(n_streams):
        r, h = divmod(s, wl.Hkv)
        pos = positions[s % len(positions)]
        L = wl.P + pos + 1  # the cache length a decode at this position attends over
        k = syn.keys_fp16(wl.seed, layer, [r], [h], 0, L, outlier_count=cnt, outlier_factor=fac,
                          num_kv_heads=wl.Hkv)[0, 0].numpy()
        v = syn.values_fp16(wl.seed, layer, [r], [h], 0, L)[0, 0].numpy()
        sq = oracle.quantize_stream(k, v, kb, vb, kt)
        b, _ = oracle.pack_stream(sq, cap_groups)
        buf[s * stride:(s + 1) * stride] = b
        lens[s] = L
        qs[s] = syn.queries_fp16(wl.seed, layer, pos, r + 1, wl.Hq)[r, h * G:(h + 1) * G].numpy()
    ids = np.arange(n_streams, dtype=np.int64)

    def run(ns, threads):
        return oracle.decode_packed(buf, stride, ids[:ns], lens[:ns], kb, vb, kt, cap_groups, qs[:ns], G, wl.scale,
                                    threads)[2]

    dt, reps, used = _timed_reps(lambda: run(n_streams, _threads()), max_seconds)
    n1 = min(n_streams, 8)
    dt1, reps1, _ = _timed_reps(lambda: run(n1, 1), max_seconds / 3)
    scale = wl.B * wl.Hkv * wl.L
    t_step, t_step1 = dt / n_streams * scale, dt1 / n1 * scale
    return {"value": wl.B / t_step, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "value_1thread": wl.B / t_step1,
            "sample": f"{n_streams} (request, KV head) streams of layer 0 ({lp.k_bits}/{lp.v_bits} bits), each at the "
                      f"length of one of the timed cycle positions (L = {int(lens.min())}..{int(lens.max())}), "
                      f"repeated {reps}x ({dt * 1e3:.1f} ms each) on {int(used)} threads, and {n1} streams {reps1}x "
                      f"on 1 thread; step time scaled to {wl.B * wl.Hkv} streams x {wl.L} layers"}


# ---------------------------------------------------------------------- main
def time_workload(wl, K, W, graph=True):
    """Time K decode steps of `wl` (after W untimed ones): HIP-graph replays between two events on
    the launch stream, then the same K steps launched eagerly with HIP events bound to each kernel
    dispatch for the per-kernel roofline. Returns the measured figures."""
    import torch

    kvq = wl.kvq
    stream = torch.cuda.Stream()
    graphs = None
    with torch.cuda.stream(stream):
        wl.reset()
        torch.cuda.synchronize()
        if graph:
            # capture one graph per cycle position; capture itself runs nothing
            graphs = []
            for i in range(min(wl.C, max(K, W, 1))):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    wl.step(i)
                graphs.append(g)
            wl.reset()
        torch.cuda.synchronize()

        def run(i, eager=False):
            pos = i % wl.C
            if pos == 0 and i > 0:
                wl.reset()
            if graphs is not None and not eager:
                graphs[pos].replay()
            else:
                wl.step(pos)

        for i in range(W):
            run(i)
        wl.reset()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(K):
            run(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = ev0.elapsed_time(ev1)
        # kernel-timing pass: the same K steps launched eagerly, with HIP events bound to
        # each kernel dispatch (the graph replays above carry no timer)
        wl.reset()
        torch.cuda.synchronize()
        kvq.timer_start(max(1, K * wl.L))
        for i in range(K):
            run(i, eager=True)
        torch.cuda.synchronize()
        split_ms, split_n = kvq.timer_read(kvq.TIMER_SPLIT)
        merge_ms, merge_n = kvq.timer_read(kvq.TIMER_MERGE)
        app_ms, app_n = kvq.timer_read(kvq.TIMER_APPEND)
        kvq.timer_stop()
    graph_used = graphs is not None
    del graphs
    positions = [i % wl.C for i in range(K)]
    bytes_total = sum(wl.split_bytes(p) for p in positions)
    n_launch = K * wl.L
    avg_split_s = (split_ms / 1e3) / max(split_n, 1)
    achieved = (bytes_total / n_launch) / avg_split_s / 1e9 if split_n else None
    window = [min(positions), max(positions)]
    return {"K": K, "W": W, "gpu_ms": gpu_ms, "wall_s": wall, "ms_per_step": gpu_ms / K,
            "value": wl.B * K / (gpu_ms / 1e3), "positions": positions, "window": window,
            "context": [wl.P + 1 + window[0], wl.P + 1 + window[1]],
            "bytes_total": bytes_total, "bytes_per_launch": bytes_total / max(n_launch, 1),
            "avg_split_s": avg_split_s, "split_n": split_n, "achieved": achieved,
            "merge_us": merge_ms * 1e3 / max(merge_n, 1), "merge_n": merge_n,
            "append_us": app_ms * 1e3 / max(app_n, 1), "append_n": app_n,
            "eff_gbs": bytes_total / (gpu_ms / 1e3) / 1e9,
            "traffic": _traffic(wl.name, window), "graph": graph_used}


def roofline_obj(m, fused):
    return {"bound": "hbm", "achieved": m["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": (m["achieved"] / HBM_PEAK_GBS) if m["achieved"] else None, "traffic": m["traffic"],
            "kernel": "decode split pass" + (" (with the fused token append)" if fused else ""),
            "avg_launch_us": m["avg_split_s"] * 1e6,
            "timing": "HIP events bound to each split dispatch, eager pass over the same K steps"
                      + (", kernel arguments in device memory" if os.environ.get("HIP_FORCE_DEV_KERNARG") == "1"
                         else ""),
            "bytes_per_launch": m["bytes_per_launch"],
            "traffic_window": "cycle positions %d..%d" % tuple(m["window"])}


def workload_config(wl, m, fused, graph):
    return {"workload": wl.name, "description": wl.w["desc"], "layers": wl.L, "batch": wl.B,
            "q_heads": wl.Hq, "kv_heads": wl.Hkv, "head_dim": 128, "context": m["context"],
            "equiv_bits": wl.equiv_bits() if hasattr(wl, "equiv_bits") else wl.plan.equiv_bits, "splits": wl.splits,
            "launch": ("hip-graph per step" if graph else "eager")
            + ("; token append fused into the split pass" if fused else "; append kernel, then split pass"),
            "effective_GBps_whole_step": m["eff_gbs"], "effective_frac_whole_step": m["eff_gbs"] / HBM_PEAK_GBS,
            **({"tag_bits": list(map(int, wl.tag_bits)), "int2_tokens_per_request": [min(wl.n2s), max(wl.n2s)]}
               if hasattr(wl, "tag_bits") else {})}


def make_workload(name, args):
    cls = PagedWorkload if WORKLOADS[name].get("paged") else Workload
    return cls(name, seed=args.seed, num_splits=args.splits, fused=not args.unfused)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: one decode cycle)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--secondary", default=None, choices=sorted(WORKLOADS) + ["none"],
                    help="workload timed after the headline one and reported beside it (default: the "
                         "uniform K8V8 trace when the headline is the default workload)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--unfused", action="store_true",
                    help="append with its own launch instead of inside the split pass")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the prefill-append and prefix-attention figures")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes 5 times (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU leg (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import layer_wise_mixed_amd as kvq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibrate:
        n = args.copy_calibrate
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}))
        return
    kvq.load()
    t_setup = time.perf_counter()
    wl = make_workload(args.workload, args)
    fused = getattr(wl, "fused", False)
    K = args.steps if args.steps is not None else wl.C
    W = args.warmup if args.warmup is not None else min(wl.C, 16)
    print(f"# setup {time.perf_counter() - t_setup:.1f}s: {wl.w['desc']}, splits={wl.splits}", file=sys.stderr,
          flush=True)
    m = time_workload(wl, K, W, graph=not args.no_graph)
    print(f"# {K} steps in {m['gpu_ms']:.3f} ms GPU ({m['wall_s'] * 1e3:.1f} ms wall); split {m['split_n']} launches "
          f"avg {m['avg_split_s'] * 1e6:.2f} us ({(m['achieved'] or 0) / HBM_PEAK_GBS:.3f} of HBM peak); merge avg "
          f"{m['merge_us']:.2f} us; append avg {m['append_us']:.2f} us; whole-step effective {m['eff_gbs']:.0f} GB/s",
          file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": m["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 mfma (hi+lo operand parts), f32 accumulate, f16 out",
        "data": "synthetic",
        "config": workload_config(wl, m, fused, not args.no_graph),
        "roofline": roofline_obj(m, fused),
    }
    if not args.no_extras and hasattr(wl, "prefill_append_rate"):
        # the quantize-and-pack kernel at prefill size (HBM-bound there), reported beside the step
        result["prefill_append"] = wl.prefill_append_rate()
        print(f"# prefill append, layer {result['prefill_append']['layer']}: "
              f"{result['prefill_append']['us']:.1f} us, {result['prefill_append']['GBps']:.0f} GB/s", file=sys.stderr,
              flush=True)
    if not args.no_extras and hasattr(wl, "prefix_attention_rate"):
        # chunked-prefill attention over the quantized prefix (matrix-core bound), beside the step
        pa = result["prefix_attention"] = wl.prefix_attention_rate()
        print(f"# prefix attention, layer {pa['layer']} {pa['format']}: {pa['rows']} rows x {pa['prefix']} tokens "
              f"in {pa['us']:.1f} us, {pa['TFLOPs']:.0f} TFLOP/s ({100 * pa['frac']:.1f}% of fp16 peak)",
              file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, m["positions"], args.cpu_seconds)
    sec = args.secondary or (SECONDARY_WORKLOAD if args.workload == DEFAULT_WORKLOAD else "none")
    if sec != "none" and sec != args.workload:
        del wl
        torch.cuda.empty_cache()
        wl2 = make_workload(sec, args)
        K2 = wl2.C if args.steps is None else args.steps
        W2 = min(wl2.C, 16) if args.warmup is None else args.warmup
        m2 = time_workload(wl2, K2, W2, graph=not args.no_graph)
        print(f"# secondary {sec}: {K2} steps, {m2['value']:.0f} tokens/s, split avg {m2['avg_split_s'] * 1e6:.2f} us "
              f"({(m2['achieved'] or 0) / HBM_PEAK_GBS:.3f} of HBM peak)", file=sys.stderr, flush=True)
        result["secondary"] = {"value": m2["value"], "unit": "tokens/s", "steps": K2, "warmup": W2,
                               "ms_per_step": m2["ms_per_step"],
                               "config": workload_config(wl2, m2, fused, not args.no_graph),
                               "roofline": roofline_obj(m2, fused)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
