"""CPU oracle of the layer-wise mixed-precision KV-cache path.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg import this package; the library it checks never
does. It shares no code with the HIP library: the arithmetic lives in
``kvq_oracle.c`` (plain loops, fp32 quantizer exactly as defined, fp64
attention), loaded here with ctypes and wrapped for numpy arrays.

Functions and the passages they follow:
  quantize_group      -- asymmetric groupwise min/max quantizer, group 32
                         (TriAxialKV page, "Facts": quantizer bullet)
  quantize_stream     -- K per-channel or per-token, V per-token
                         (KVTuner summary page, "Facts": per-channel keys;
                         TriAxialKV page, "Facts": quantizer bullet); tokens
                         that do not fill a group stay fp16
  attention           -- softmax attention of a decode query, fp64
  lse_merge           -- split merge by log-sum-exp (TriAxialKV page,
                         "Facts": split decode bullet)
  chunk_prefill       -- a prefill chunk's attention over the quantized
                         prefix plus its own fp16 tokens, causally (the
                         chunked-prefill reading: the prefix is what the
                         cache stores, the chunk is not yet quantized)
  pack_stream / unpack_stream -- this project's byte layout of the cache
  quantize_tokens / pack_paged / unpack_paged / decode_paged -- the paged
                         INT2/INT4 pool (TriAxialKV page, "Facts": page-pool,
                         leftover-routing and page-table bullets; INT4 keys
                         and values per-token)
  equiv_bits          -- mean over layers of (bK + bV) / 2 (KVTuner summary
                         page, "Experimental setup": equivalent precision;
                         first page, "Facts": K8V2 is called 5-bit, K4V8 6-bit)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvq_oracle.so")
_lib = None

D = 128
GROUP = 32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        L.oq_half_to_float.argtypes = [ctypes.c_uint16]
        L.oq_half_to_float.restype = ctypes.c_float
        L.oq_quantize_group.argtypes = [P, i64, i32, i32, P, P, P]
        L.oq_quantize_group.restype = None
        L.oq_dequant.argtypes = [ctypes.c_uint32, ctypes.c_float, ctypes.c_float]
        L.oq_dequant.restype = ctypes.c_float
        L.oq_quantize_stream.argtypes = [P, P, i64, i32, i32, i32, P, P, P, P, P, P]
        L.oq_quantize_stream.restype = None
        L.oq_dequant_stream.argtypes = [P, P, i64, i32, i32, i32, P, P, P, P, P, P, P, P]
        L.oq_dequant_stream.restype = None
        L.oq_record_bytes.argtypes = [i32, i32]
        L.oq_record_bytes.restype = i64
        L.oq_stream_bytes.argtypes = [i32, i32, i64]
        L.oq_stream_bytes.restype = i64
        L.oq_pack_stream.argtypes = [P, P, i64, i32, i32, i32, i64, P, P, P, P, P, P, P, P]
        L.oq_pack_stream.restype = None
        L.oq_unpack_stream.argtypes = [P, i64, i32, i32, i32, i64, P, P]
        L.oq_unpack_stream.restype = None
        L.oq_attention.argtypes = [P, i32, i32, P, P, i64, ctypes.c_double, P, P]
        L.oq_attention.restype = None
        L.oq_lse_merge.argtypes = [P, P, i32, i32, P, P]
        L.oq_lse_merge.restype = None
        L.oq_decode_packed.argtypes = [P, i64, i32, P, P, i32, i32, i32, i64, P, i32,
                                       ctypes.c_double, P, P, i32]
        L.oq_decode_packed.restype = i32
        for name in ("oq_k_site", "oq_v_site"):
            getattr(L, name).argtypes = [i32, i32, P, P]
            getattr(L, name).restype = None
        L.oq_meta_channel_index.argtypes = [i32]
        L.oq_meta_channel_index.restype = i32
        L.oq_meta_token_index.argtypes = [i32, i32]
        L.oq_meta_token_index.restype = i32
        for name in ("oq_page_k_site", "oq_page_v_site"):
            getattr(L, name).argtypes = [i32, i32, P, P]
            getattr(L, name).restype = None
        L.oq_page_meta_index.argtypes = [i32, i32]
        L.oq_page_meta_index.restype = i32
        L.oq_quantize_tokens.argtypes = [P, i64, i32, P, P, P]
        L.oq_quantize_tokens.restype = None
        L.oq_pack_paged.argtypes = [P, P, i64, i64, P, ctypes.c_int32, i32, i32, P, P]
        L.oq_pack_paged.restype = None
        L.oq_unpack_paged.argtypes = [P, i64, i64, P, ctypes.c_int32, i32, i32, P, P]
        L.oq_unpack_paged.restype = None
        L.oq_decode_paged.argtypes = [P, i32, P, P, P, P, P, i64, ctypes.c_int32, i32, P, i32,
                                      ctypes.c_double, P, P, i32]
        L.oq_decode_paged.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(x) -> np.ndarray:
    """fp16 data (torch tensor or numpy) as a C-contiguous uint16 array."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().contiguous().numpy()
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16
    return x


# ------------------------------------------------------------------ quantizer


def half_to_float(h: int) -> float:
    return lib().oq_half_to_float(h)


def quantize_group(x_fp16, bits: int):
    """(scale, zero, codes) of one group (any length) of fp16 values."""
    x = _u16(x_fp16).reshape(-1)
    codes = np.zeros(x.size, dtype=np.uint8)
    sc = ctypes.c_float()
    zr = ctypes.c_float()
    lib().oq_quantize_group(_p(x), 1, x.size, bits, ctypes.byref(sc), ctypes.byref(zr), _p(codes))
    return np.float32(sc.value), np.float32(zr.value), codes


def dequant(code: int, scale: float, zero: float) -> np.float32:
    return np.float32(lib().oq_dequant(int(code), float(scale), float(zero)))


class StreamQ:
    """Logical quantization of one stream (fields are numpy arrays)."""

    def __init__(self, k, v, L, kb, vb, k_token):
        self.k, self.v, self.L, self.kb, self.vb, self.k_token = k, v, L, kb, vb, k_token
        lq = (L // GROUP) * GROUP
        self.lq = lq
        self.kcode = np.zeros((lq, D), np.uint8)
        self.vcode = np.zeros((lq, D), np.uint8)
        nk = lq * 4 if k_token else (lq // GROUP) * D
        self.kscale = np.zeros(max(nk, 1), np.float32)
        self.kzero = np.zeros(max(nk, 1), np.float32)
        self.vscale = np.zeros(max(lq * 4, 1), np.float32)
        self.vzero = np.zeros(max(lq * 4, 1), np.float32)


def quantize_stream(k_fp16, v_fp16, kb: int, vb: int, k_token: bool = False) -> StreamQ:
    """Quantize one stream: k, v fp16 [L, 128]."""
    k = _u16(k_fp16).reshape(-1, D)
    v = _u16(v_fp16).reshape(-1, D)
    L = k.shape[0]
    q = StreamQ(k, v, L, kb, vb, k_token)
    lib().oq_quantize_stream(_p(k), _p(v), L, kb, vb, int(k_token), _p(q.kcode), _p(q.kscale),
                             _p(q.kzero), _p(q.vcode), _p(q.vscale), _p(q.vzero))
    return q


def dequant_stream(sq: StreamQ):
    """float32 (kdeq, vdeq) [L, 128] of a quantized stream."""
    kd = np.zeros((sq.L, D), np.float32)
    vd = np.zeros((sq.L, D), np.float32)
    lib().oq_dequant_stream(_p(sq.k), _p(sq.v), sq.L, sq.kb, sq.vb, int(sq.k_token), _p(sq.kcode),
                            _p(sq.kscale), _p(sq.kzero), _p(sq.vcode), _p(sq.vscale),
                            _p(sq.vzero), _p(kd), _p(vd))
    return kd, vd


# --------------------------------------------------------------------- layout


def record_bytes(kb: int, vb: int) -> int:
    return int(lib().oq_record_bytes(kb, vb))


def stream_bytes(kb: int, vb: int, groups_cap: int) -> int:
    return int(lib().oq_stream_bytes(kb, vb, groups_cap))


def pack_stream(sq: StreamQ, groups_cap: int):
    """(bytes, mask) of a stream in the cache layout; mask marks defined bytes."""
    n = stream_bytes(sq.kb, sq.vb, groups_cap)
    out = np.zeros(n, np.uint8)
    mask = np.zeros(n, np.uint8)
    lib().oq_pack_stream(_p(sq.k), _p(sq.v), sq.L, sq.kb, sq.vb, int(sq.k_token), groups_cap,
                         _p(sq.kcode), _p(sq.kscale), _p(sq.kzero), _p(sq.vcode), _p(sq.vscale),
                         _p(sq.vzero), _p(out), _p(mask))
    return out, mask.astype(bool)


def unpack_stream(buf: np.ndarray, L: int, kb: int, vb: int, k_token: bool, groups_cap: int):
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    kd = np.zeros((L, D), np.float32)
    vd = np.zeros((L, D), np.float32)
    lib().oq_unpack_stream(_p(buf), L, kb, vb, int(k_token), groups_cap, _p(kd), _p(vd))
    return kd, vd


def k_site(j: int, c: int):
    lane, e = ctypes.c_int(), ctypes.c_int()
    lib().oq_k_site(j, c, ctypes.byref(lane), ctypes.byref(e))
    return lane.value, e.value


def v_site(j: int, c: int):
    lane, e = ctypes.c_int(), ctypes.c_int()
    lib().oq_v_site(j, c, ctypes.byref(lane), ctypes.byref(e))
    return lane.value, e.value


def meta_channel_index(c: int) -> int:
    return int(lib().oq_meta_channel_index(c))


def meta_token_index(j: int, n: int) -> int:
    return int(lib().oq_meta_token_index(j, n))


# ----------------------------------------------------------------- paged pool

PAGE_TOKENS = 16


def page_k_site(p: int, c: int):
    """(byte, shift) of key (slot p, channel c) inside one KV head's INT4 page."""
    b, sh = ctypes.c_int(), ctypes.c_int()
    lib().oq_page_k_site(p, c, ctypes.byref(b), ctypes.byref(sh))
    return b.value, sh.value


def page_v_site(p: int, c: int):
    b, sh = ctypes.c_int(), ctypes.c_int()
    lib().oq_page_v_site(p, c, ctypes.byref(b), ctypes.byref(sh))
    return b.value, sh.value


def page_meta_index(p: int, n: int) -> int:
    return int(lib().oq_page_meta_index(p, n))


def quantize_tokens(x_fp16, bits: int):
    """Per-token quantization (four 32-channel groups per token) of fp16 [L, 128]:
    (codes [L, 128] uint8, scale [L, 4], zero [L, 4])."""
    x = _u16(x_fp16).reshape(-1, D)
    L = x.shape[0]
    codes = np.zeros((L, D), np.uint8)
    sc = np.zeros((max(L, 1), 4), np.float32)
    zr = np.zeros((max(L, 1), 4), np.float32)
    lib().oq_quantize_tokens(_p(x), L, bits, _p(codes), _p(sc), _p(zr))
    return codes, sc[:L], zr[:L]


def paged_pool_bytes(hkv: int, int2_pages: int, int4_pages: int) -> int:
    return int2_pages * hkv * 2048 + int4_pages * hkv * 3072


def pack_paged(pool: np.ndarray, k_fp16, v_fp16, n2: int, table, int2_pages: int, hkv: int, h: int,
               mask: np.ndarray | None = None):
    """Quantize one (request, KV head) -- fp16 [n2 + n4, 128] in logical order, INT2 tokens
    first -- into `pool` (uint8, modified in place) through its page table."""
    k = _u16(k_fp16).reshape(-1, D)
    v = _u16(v_fp16).reshape(-1, D)
    assert n2 % GROUP == 0 and 0 <= n2 <= k.shape[0]
    tb = np.ascontiguousarray(table, dtype=np.int32)
    lib().oq_pack_paged(_p(k), _p(v), n2, k.shape[0] - n2, _p(tb), int2_pages, hkv, h, _p(pool),
                        _p(mask) if mask is not None else None)


def unpack_paged(pool: np.ndarray, n2: int, n4: int, table, int2_pages: int, hkv: int, h: int):
    """float32 (kdeq, vdeq) [n2 + n4, 128] of one (request, KV head), logical order."""
    tb = np.ascontiguousarray(table, dtype=np.int32)
    kd = np.zeros((n2 + n4, D), np.float32)
    vd = np.zeros((n2 + n4, D), np.float32)
    lib().oq_unpack_paged(_p(pool), n2, n4, _p(tb), int2_pages, hkv, h, _p(kd), _p(vd))
    return kd, vd


def decode_paged(pool: np.ndarray, req, head, n2, n4, tables: np.ndarray, int2_pages: int, hkv: int,
                 q_fp16, G: int, scale: float, nthreads: int = 0):
    """One decode step over the oracle's own paged pool: (out, lse, threads)."""
    req = np.ascontiguousarray(req, dtype=np.int64)
    head = np.ascontiguousarray(head, dtype=np.int64)
    n2 = np.ascontiguousarray(n2, dtype=np.int64)
    n4 = np.ascontiguousarray(n4, dtype=np.int64)
    tb = np.ascontiguousarray(tables, dtype=np.int32)
    ns = len(req)
    q = _u16(q_fp16).reshape(ns, G, D)
    out = np.zeros((ns, G, D), np.float64)
    lse = np.zeros((ns, G), np.float64)
    used = lib().oq_decode_paged(_p(pool), ns, _p(req), _p(head), _p(n2), _p(n4), _p(tb), tb.shape[1],
                                 int2_pages, hkv, _p(q), G, float(scale), _p(out), _p(lse), nthreads)
    return out, lse, used


# ------------------------------------------------------------------ attention


def attention(q_fp16, kdeq: np.ndarray, vdeq: np.ndarray, scale: float):
    """fp64 (out [G, D], lse [G]) of G query rows over L cached tokens."""
    q = _u16(q_fp16).reshape(-1, D)
    G = q.shape[0]
    kd = np.ascontiguousarray(kdeq, dtype=np.float32).reshape(-1, D)
    vd = np.ascontiguousarray(vdeq, dtype=np.float32).reshape(-1, D)
    L = kd.shape[0]
    out = np.zeros((G, D), np.float64)
    lse = np.zeros(G, np.float64)
    lib().oq_attention(_p(q), G, D, _p(kd), _p(vd), L, float(scale), _p(out), _p(lse))
    return out, lse


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    o = np.ascontiguousarray(o_parts, dtype=np.float64)
    S, Dd = o.shape
    ls = np.ascontiguousarray(lse_parts, dtype=np.float64).reshape(S)
    out = np.zeros(Dd, np.float64)
    ol = ctypes.c_double()
    lib().oq_lse_merge(_p(o), _p(ls), S, Dd, _p(out), ctypes.byref(ol))
    return out, ol.value


def decode_stream(q_fp16, k_fp16, v_fp16, kb: int, vb: int, k_token: bool, scale: float):
    """Quantize a stream, dequantize it, and attend: fp64 (out [G, D], lse [G])."""
    sq = quantize_stream(k_fp16, v_fp16, kb, vb, k_token)
    kd, vd = dequant_stream(sq)
    return attention(q_fp16, kd, vd, scale)


def chunk_prefill(q_fp16, k_prefix, v_prefix, k_chunk, v_chunk, kb: int, vb: int, k_token: bool, scale: float):
    """Attention of a prefill chunk with a quantized cache in front of it: the
    query rows of chunk token i (q [C, G, D]) attend to the prefix as the cache
    stores it (k_prefix/v_prefix fp16 [L, D], quantized as by quantize_stream,
    the tail kept fp16) and, causally, to the chunk's own fp16 tokens 0..i
    (k_chunk/v_chunk [C, D]). One softmax over all those keys, fp64: (out
    [C, G, D], lse [C, G])."""
    q = _u16(q_fp16).reshape(len(k_chunk), -1, D)
    C, G = q.shape[0], q.shape[1]
    kp = vp = np.zeros((0, D), np.float32)
    if len(k_prefix):
        kp, vp = dequant_stream(quantize_stream(k_prefix, v_prefix, kb, vb, k_token))
    kc = _u16(k_chunk).reshape(C, D).view(np.float16).astype(np.float32)
    vc = _u16(v_chunk).reshape(C, D).view(np.float16).astype(np.float32)
    out = np.zeros((C, G, D))
    lse = np.zeros((C, G))
    for i in range(C):
        keys = np.concatenate([kp, kc[:i + 1]])
        vals = np.concatenate([vp, vc[:i + 1]])
        out[i], lse[i] = attention(q[i], keys, vals, scale)
    return out, lse


def decode_packed(cache_layer: np.ndarray, stream_stride: int, stream_ids, lens, kb, vb, k_token,
                  groups_cap, q_fp16, G, scale, nthreads=0):
    """One decode step over the oracle's own packed layer: returns (out, lse, threads)."""
    ids = np.ascontiguousarray(stream_ids, dtype=np.int64)
    ln = np.ascontiguousarray(lens, dtype=np.int64)
    q = _u16(q_fp16).reshape(len(ids), G, D)
    out = np.zeros((len(ids), G, D), np.float64)
    lse = np.zeros((len(ids), G), np.float64)
    used = lib().oq_decode_packed(_p(cache_layer), stream_stride, len(ids), _p(ids), _p(ln), kb, vb,
                                  int(k_token), groups_cap, _p(q), G, float(scale), _p(out),
                                  _p(lse), nthreads)
    return out, lse, used


# ---------------------------------------------------------------------- plan


def equiv_bits(pairs) -> float:
    """Mean over layers of (bK + bV) / 2, code bits only."""
    pairs = list(pairs)
    return sum((kb + vb) / 2.0 for kb, vb in pairs) / len(pairs)
