"""Python binding of libkvq (include/kvq.h): argument marshalling only.

Every step of the path runs in the HIP kernels of libkvq.so; this module maps
torch tensors (device memory, owned by the caller) and the current HIP stream
onto the C ABI. There is no fallback: if the library is not built, `load()`
raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

MAX_LAYERS = 256
HEAD_DIM = 128
GROUP = 32
OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_CAPACITY = -3
ERR_WORKSPACE = -4
ERR_HIP = -5
AXIS_CHANNEL = 0
AXIS_TOKEN = 1
OUT_F16 = 0
OUT_F32 = 1
TIMER_APPEND, TIMER_SPLIT, TIMER_MERGE, TIMER_PREFIX = 0, 1, 2, 3


class KvqError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"kvq error {code}: {message}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32), ("int2_pages", ctypes.c_int32),
                ("int4_pages", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class LayerCfg(ctypes.Structure):
    _fields_ = [("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("k_axis", ctypes.c_int32), ("v_axis", ctypes.c_int32)]


class LayerPlan(ctypes.Structure):
    _fields_ = [("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("k_axis", ctypes.c_int32), ("v_axis", ctypes.c_int32),
                ("offset", ctypes.c_uint64), ("bytes", ctypes.c_uint64),
                ("record_bytes", ctypes.c_uint64), ("groups_cap", ctypes.c_uint64),
                ("stream_bytes", ctypes.c_uint64), ("tail_offset", ctypes.c_uint64),
                ("int4_offset", ctypes.c_uint64), ("int2_page_bytes", ctypes.c_uint64),
                ("int4_page_bytes", ctypes.c_uint64)]


class Plan(ctypes.Structure):
    _fields_ = [("shape", Shape), ("num_layers", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("total_bytes", ctypes.c_uint64), ("equiv_bits", ctypes.c_double),
                ("int2_fraction", ctypes.c_double), ("layers", LayerPlan * MAX_LAYERS)]


class Pages(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("max_pages_per_req", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("int2_len", ctypes.c_void_p),
                ("int4_len", ctypes.c_void_p), ("int2_add", ctypes.c_void_p)]


SYMBOLS = ["kvq_plan_layers", "kvq_quantize_append", "kvq_decode_workspace_bytes", "kvq_decode_num_splits",
           "kvq_decode_attention", "kvq_decode_attention_noalloc", "kvq_append_decode_attention", "kvq_prefix_workspace_bytes",
           "kvq_prefix_attention", "kvq_chunk_prefill_workspace_bytes", "kvq_chunk_prefill_attention",
           "kvq_dequantize", "kvq_last_error", "kvq_timer_start", "kvq_timer_read",
           "kvq_timer_stop"]

_lib = None


def load():
    """Load libkvq.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (no fallback path exists)")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    L.kvq_plan_layers.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(LayerCfg), i32, ctypes.POINTER(Plan)]
    L.kvq_plan_layers.restype = ctypes.c_int
    L.kvq_quantize_append.argtypes = [ctypes.POINTER(Plan), i32, P, P, P, P, i32, i32, ctypes.POINTER(Pages), P]
    L.kvq_quantize_append.restype = ctypes.c_int
    L.kvq_decode_workspace_bytes.argtypes = [ctypes.POINTER(Plan), i32, i32, i32]
    L.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
    L.kvq_decode_num_splits.argtypes = [ctypes.POINTER(Plan), i32, i32, i32]
    L.kvq_decode_num_splits.restype = i32
    L.kvq_decode_attention.argtypes = [ctypes.POINTER(Plan), i32, P, P, P, i32, i32, ctypes.c_float, P, i32, P, P,
                                       ctypes.c_size_t, i32, ctypes.POINTER(Pages), P]
    L.kvq_decode_attention.restype = ctypes.c_int
    L.kvq_decode_attention_noalloc.argtypes = [ctypes.POINTER(Plan), i32, P, P, P, i32, i32, ctypes.c_float, P, i32,
                                               P, i32, ctypes.POINTER(Pages), P]
    L.kvq_decode_attention_noalloc.restype = ctypes.c_int
    L.kvq_append_decode_attention.argtypes = [ctypes.POINTER(Plan), i32, P, P, P, P, P, i32, i32, ctypes.c_float,
                                              P, i32, P, P, ctypes.c_size_t, i32, ctypes.POINTER(Pages), P]
    L.kvq_append_decode_attention.restype = ctypes.c_int
    L.kvq_prefix_workspace_bytes.argtypes = [ctypes.POINTER(Plan), i32, i32, i32, i32]
    L.kvq_prefix_workspace_bytes.restype = ctypes.c_size_t
    L.kvq_prefix_attention.argtypes = [ctypes.POINTER(Plan), i32, P, P, i32, P, i32, i32, ctypes.c_float, P, P, P,
                                       ctypes.c_size_t, i32, ctypes.POINTER(Pages), P]
    L.kvq_prefix_attention.restype = ctypes.c_int
    L.kvq_chunk_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Plan), i32, i32, i32, i32]
    L.kvq_chunk_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.kvq_chunk_prefill_attention.argtypes = [ctypes.POINTER(Plan), i32, P, P, P, P, i32, P, i32, i32, ctypes.c_float,
                                              P, P, P, ctypes.c_size_t, i32, ctypes.POINTER(Pages), P]
    L.kvq_chunk_prefill_attention.restype = ctypes.c_int
    L.kvq_dequantize.argtypes = [ctypes.POINTER(Plan), i32, P, P, i32, i32, P, P, ctypes.POINTER(Pages), P]
    L.kvq_dequantize.restype = ctypes.c_int
    L.kvq_last_error.argtypes = []
    L.kvq_last_error.restype = ctypes.c_char_p
    L.kvq_timer_start.argtypes = [i32]
    L.kvq_timer_start.restype = ctypes.c_int
    L.kvq_timer_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
    L.kvq_timer_read.restype = ctypes.c_int
    L.kvq_timer_stop.argtypes = []
    L.kvq_timer_stop.restype = ctypes.c_int
    _lib = L
    return _lib


def _check(code: int):
    if code != OK:
        raise KvqError(code, load().kvq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_i32(t, n, name):
    import torch

    assert t.dtype == torch.int32 and t.is_contiguous() and t.numel() >= n, f"{name}: int32 contiguous [>= {n}]"


def make_shape(num_q_heads, num_kv_heads, max_batch, max_tokens=0, page_tokens=0, int2_pages=0,
               int4_pages=0) -> Shape:
    return Shape(num_q_heads, num_kv_heads, HEAD_DIM, GROUP, max_batch, max_tokens, page_tokens, int2_pages,
                 int4_pages, 0)


def plan_layers(shape: Shape, cfgs) -> Plan:
    """cfgs: list of (k_bits, v_bits[, k_axis[, v_axis]])."""
    cfgs = list(cfgs)
    arr = (LayerCfg * max(len(cfgs), 1))()
    for i, c in enumerate(cfgs):
        c = tuple(c) + (AXIS_CHANNEL, AXIS_TOKEN)[len(c) - 2:]
        arr[i] = LayerCfg(*c[:4])
    plan = Plan()
    _check(load().kvq_plan_layers(ctypes.byref(shape), arr, len(cfgs), ctypes.byref(plan)))
    return plan


def make_pages(page_table=None, max_pages_per_req=0, int2_len=None, int4_len=None, int2_add=None) -> Pages:
    return Pages(None if page_table is None else page_table.data_ptr(), max_pages_per_req, 0,
                 None if int2_len is None else int2_len.data_ptr(), None if int4_len is None else int4_len.data_ptr(),
                 None if int2_add is None else int2_add.data_ptr())


def quantize_append(plan: Plan, layer: int, cache, k_new, v_new, seq_lens=None, pages: Pages | None = None,
                    stream=None):
    """k_new, v_new: fp16 [batch, Hkv, n_new, 128] device tensors."""
    import torch

    assert k_new.dtype == torch.float16 and v_new.dtype == torch.float16
    assert k_new.is_contiguous() and v_new.is_contiguous() and k_new.shape == v_new.shape
    batch, _, n_new, _ = k_new.shape
    if seq_lens is not None:
        _dev_i32(seq_lens, batch, "seq_lens")
    _check(load().kvq_quantize_append(ctypes.byref(plan), layer, _ptr(cache), _ptr(k_new), _ptr(v_new),
                                      _ptr(seq_lens), batch, n_new,
                                      None if pages is None else ctypes.byref(pages), _stream(stream)))


def workspace_bytes(plan: Plan, batch: int, max_seq_len: int, num_splits: int = 0) -> int:
    return int(load().kvq_decode_workspace_bytes(ctypes.byref(plan), batch, max_seq_len, num_splits))


def num_splits(plan: Plan, layer: int, batch: int, max_seq_len: int) -> int:
    return int(load().kvq_decode_num_splits(ctypes.byref(plan), layer, batch, max_seq_len))


def decode_attention(plan: Plan, layer: int, cache, q, seq_lens, max_seq_len: int, softmax_scale: float, out,
                     lse=None, workspace=None, num_splits: int = 0, pages: Pages | None = None, stream=None):
    """q: fp16 [batch, Hq, 128]; out: fp16 or fp32 [batch, Hq, 128]; lse: fp32 [batch, Hq] or None."""
    import torch

    assert q.dtype == torch.float16 and q.is_contiguous()
    assert out.is_contiguous() and out.dtype in (torch.float16, torch.float32)
    batch = q.shape[0]
    if seq_lens is not None:
        _dev_i32(seq_lens, batch, "seq_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kvq_decode_attention(ctypes.byref(plan), layer, _ptr(cache), _ptr(q), _ptr(seq_lens), batch,
                                       max_seq_len, float(softmax_scale), _ptr(out),
                                       OUT_F32 if out.dtype == torch.float32 else OUT_F16, _ptr(lse),
                                       _ptr(workspace), ws_bytes, num_splits,
                                       None if pages is None else ctypes.byref(pages), _stream(stream)))


def decode_attention_noalloc(plan: Plan, layer: int, cache, q, seq_lens, max_seq_len: int, softmax_scale: float,
                             out, lse=None, num_splits: int = 0, pages: Pages | None = None, stream=None):
    """decode_attention with the split partials in the library's own device array (no workspace;
    the library allocates nothing)."""
    import torch

    assert q.dtype == torch.float16 and q.is_contiguous()
    assert out.is_contiguous() and out.dtype in (torch.float16, torch.float32)
    batch = q.shape[0]
    if seq_lens is not None:
        _dev_i32(seq_lens, batch, "seq_lens")
    _check(load().kvq_decode_attention_noalloc(ctypes.byref(plan), layer, _ptr(cache), _ptr(q), _ptr(seq_lens), batch,
                                               max_seq_len, float(softmax_scale), _ptr(out),
                                               OUT_F32 if out.dtype == torch.float32 else OUT_F16, _ptr(lse),
                                               num_splits, None if pages is None else ctypes.byref(pages),
                                               _stream(stream)))


def append_decode_attention(plan: Plan, layer: int, cache, k_new, v_new, q, seq_lens, max_seq_len: int,
                            softmax_scale: float, out, lse=None, workspace=None, num_splits: int = 0,
                            pages: Pages | None = None, stream=None):
    """One token appended per request and the decode step over the cache with it, in one pass.
    k_new, v_new: fp16 [batch, Hkv, 1, 128]; seq_lens: lengths before the append (not advanced here;
    ignored with pages, whose int4_len holds the INT4 lengths before the append); max_seq_len: bound
    of the lengths + 1; q, out, lse, workspace, num_splits: as in decode_attention."""
    import torch

    assert k_new.dtype == torch.float16 and v_new.dtype == torch.float16
    assert k_new.is_contiguous() and v_new.is_contiguous() and k_new.shape == v_new.shape and k_new.shape[2] == 1
    assert q.dtype == torch.float16 and q.is_contiguous()
    assert out.is_contiguous() and out.dtype in (torch.float16, torch.float32)
    batch = q.shape[0]
    assert k_new.shape[0] == batch
    if pages is None:
        _dev_i32(seq_lens, batch, "seq_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kvq_append_decode_attention(ctypes.byref(plan), layer, _ptr(cache), _ptr(k_new), _ptr(v_new),
                                              _ptr(q), _ptr(seq_lens), batch, max_seq_len, float(softmax_scale),
                                              _ptr(out), OUT_F32 if out.dtype == torch.float32 else OUT_F16,
                                              _ptr(lse), _ptr(workspace), ws_bytes, num_splits,
                                              None if pages is None else ctypes.byref(pages), _stream(stream)))


def prefix_workspace_bytes(plan: Plan, batch: int, chunk: int, max_seq_len: int, num_splits: int = 0) -> int:
    return int(load().kvq_prefix_workspace_bytes(ctypes.byref(plan), batch, chunk, max_seq_len, num_splits))


def prefix_attention(plan: Plan, layer: int, cache, q, seq_lens, max_seq_len: int, softmax_scale: float, out,
                     lse=None, workspace=None, num_splits: int = 0, stream=None, pages: Pages | None = None):
    """Attention of a chunk of query tokens over each request's cached prefix (no mask).
    q: fp16 [batch, chunk, Hq, 128]; seq_lens: cached tokens per request; out: fp32 [batch, chunk, Hq, 128];
    lse: fp32 [batch, chunk, Hq] or None; workspace: prefix_workspace_bytes(...) bytes (None if 0)."""
    import torch

    assert q.dtype == torch.float16 and q.is_contiguous() and q.dim() == 4
    assert out.dtype == torch.float32 and out.is_contiguous() and out.shape == q.shape
    assert lse is None or (lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == q.shape[:3])
    batch, chunk = q.shape[0], q.shape[1]
    if pages is None:
        _dev_i32(seq_lens, batch, "seq_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kvq_prefix_attention(ctypes.byref(plan), layer, _ptr(cache), _ptr(q), chunk, _ptr(seq_lens), batch,
                                       max_seq_len, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                       ws_bytes, num_splits, None if pages is None else ctypes.byref(pages),
                                       _stream(stream)))


def chunk_prefill_workspace_bytes(plan: Plan, batch: int, chunk: int, max_seq_len: int, num_splits: int = 0) -> int:
    return int(load().kvq_chunk_prefill_workspace_bytes(ctypes.byref(plan), batch, chunk, max_seq_len, num_splits))


def chunk_prefill_attention(plan: Plan, layer: int, cache, q, k_chunk, v_chunk, seq_lens, max_seq_len: int,
                            softmax_scale: float, out, lse=None, workspace=None, num_splits: int = 0, stream=None,
                            pages: Pages | None = None):
    """A prefill chunk's whole attention: the cached prefix as stored plus the chunk's own fp16 tokens,
    causally. q: fp16 [batch, chunk, Hq, 128]; k_chunk, v_chunk: fp16 [batch, Hkv, chunk, 128];
    out: fp32 [batch, chunk, Hq, 128]; lse: fp32 [batch, chunk, Hq] or None; workspace:
    chunk_prefill_workspace_bytes(...) bytes."""
    import torch

    assert q.dtype == torch.float16 and q.is_contiguous() and q.dim() == 4
    assert k_chunk.dtype == torch.float16 and v_chunk.dtype == torch.float16
    assert k_chunk.is_contiguous() and v_chunk.is_contiguous() and k_chunk.shape == v_chunk.shape
    batch, chunk = q.shape[0], q.shape[1]
    assert k_chunk.shape[0] == batch and k_chunk.shape[2] == chunk
    assert out.dtype == torch.float32 and out.is_contiguous() and out.shape == q.shape
    assert lse is None or (lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == q.shape[:3])
    if pages is None:
        _dev_i32(seq_lens, batch, "seq_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().kvq_chunk_prefill_attention(ctypes.byref(plan), layer, _ptr(cache), _ptr(q), _ptr(k_chunk),
                                              _ptr(v_chunk), chunk, _ptr(seq_lens), batch, max_seq_len,
                                              float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                              num_splits, None if pages is None else ctypes.byref(pages),
                                              _stream(stream)))


def dequantize(plan: Plan, layer: int, cache, seq_lens, batch: int, max_seq_len: int, k_out, v_out,
               pages: Pages | None = None, stream=None):
    """k_out, v_out: fp32 [batch, Hkv, max_seq_len, 128]."""
    _check(load().kvq_dequantize(ctypes.byref(plan), layer, _ptr(cache), _ptr(seq_lens), batch, max_seq_len,
                                 _ptr(k_out), _ptr(v_out), None if pages is None else ctypes.byref(pages),
                                 _stream(stream)))


def timer_start(capacity: int):
    _check(load().kvq_timer_start(capacity))


def timer_read(kind: int):
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    _check(load().kvq_timer_read(kind, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def timer_stop():
    _check(load().kvq_timer_stop())
