"""Host-only checks of libkvq (no GPU needed): the library loads, exports every symbol
include/kvq.h declares, plans layer maps with the right byte geometry and equivalent
precision, and rejects bad arguments before any device work."""
import ctypes
import os
import re

import pytest

import layer_wise_mixed_amd as kvq
import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return kvq.load()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "kvq.h")).read()
    declared = set(re.findall(r"^[A-Za-z_0-9 ]+?\**\s*\**(kvq_\w+)\(", hdr, flags=re.M))
    assert declared >= {"kvq_plan_layers", "kvq_quantize_append", "kvq_decode_attention", "kvq_dequantize"}
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(kvq.SYMBOLS)


def test_struct_sizes_match_header():
    # kvq_shape: 10 int32; kvq_layer_plan: 4 int32 + 9 uint64; kvq_plan: shape + 2 int32 + u64 + 2 f64 + 256 layers
    assert ctypes.sizeof(kvq.Shape) == 40
    assert ctypes.sizeof(kvq.LayerPlan) == 16 + 9 * 8
    assert ctypes.sizeof(kvq.Plan) == 40 + 8 + 8 + 16 + 256 * ctypes.sizeof(kvq.LayerPlan)
    assert ctypes.sizeof(kvq.Pages) == 8 + 8 + 3 * 8


def _llama_mixed(seed=0):
    hi = set(syn.seeded_choice(seed, syn.T_MAP, 32, 8))
    return [(4, 4) if l in hi else (4, 2) for l in range(32)]


def test_plan_llama_mixed_325_bits():
    shape = kvq.make_shape(32, 8, 64, max_tokens=2080)
    plan = kvq.plan_layers(shape, _llama_mixed())
    assert plan.equiv_bits == 3.25
    assert plan.num_layers == 32
    prev_end = 0
    for l in range(32):
        lp = plan.layers[l]
        assert lp.offset % 4096 == 0 and lp.offset >= prev_end
        assert lp.groups_cap == 65
        assert lp.record_bytes == (5120 if (lp.k_bits, lp.v_bits) == (4, 2) else 6144)
        assert lp.stream_bytes == 65 * lp.record_bytes + 16384
        assert lp.tail_offset == 65 * lp.record_bytes
        assert lp.bytes == 64 * 8 * lp.stream_bytes
        prev_end = lp.offset + lp.bytes
    assert plan.total_bytes >= prev_end


def test_plan_qwen_map_and_kivi8():
    cfg = [(8, 4)] * 9 + [(4, 2)] * 19
    plan = kvq.plan_layers(kvq.make_shape(28, 4, 32, max_tokens=8192), cfg)
    assert abs(plan.equiv_bits - 111 / 28) < 1e-12
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 64, max_tokens=256), [(8, 8)] * 32)
    assert plan.equiv_bits == 8.0 and plan.layers[0].record_bytes == 10240
    # a layer left at 16 bits (skip-layer style) and K8V2 / K4V8 pairs
    plan = kvq.plan_layers(kvq.make_shape(8, 8, 1, max_tokens=64), [(16, 16), (8, 2), (4, 8)])
    assert plan.equiv_bits == (16 + 5 + 6) / 3


def test_plan_paged_pool_split():
    shape = kvq.make_shape(32, 8, 16, page_tokens=16, int2_pages=1024 * 16, int4_pages=1024 * 16 + 64)
    plan = kvq.plan_layers(shape, [(2, 2)] * 36)
    lp = plan.layers[0]
    assert lp.int2_page_bytes == 8 * 2048 and lp.int4_page_bytes == 8 * 3072
    assert lp.int4_offset == shape.int2_pages * lp.int2_page_bytes
    assert lp.bytes == lp.int4_offset + shape.int4_pages * lp.int4_page_bytes
    assert abs(plan.int2_fraction - shape.int2_pages / (shape.int2_pages + shape.int4_pages)) < 1e-15


@pytest.mark.parametrize("mutate,code", [
    (lambda s, c: setattr(s, "head_dim", 64), kvq.ERR_UNSUPPORTED),
    (lambda s, c: setattr(s, "group_size", 64), kvq.ERR_UNSUPPORTED),
    (lambda s, c: setattr(s, "num_q_heads", 30), kvq.ERR_UNSUPPORTED),
    (lambda s, c: setattr(s, "num_q_heads", 17 * 8), kvq.ERR_UNSUPPORTED),
    (lambda s, c: setattr(s, "max_tokens", 0), kvq.ERR_INVALID_ARG),
    (lambda s, c: setattr(s, "page_tokens", 32), kvq.ERR_UNSUPPORTED),
    (lambda s, c: c.__setitem__(0, (3, 4)), kvq.ERR_UNSUPPORTED),
    (lambda s, c: c.__setitem__(0, (4, 4, 0, 0)), kvq.ERR_UNSUPPORTED),
    (lambda s, c: c.__setitem__(0, (4, 4, 5, 1)), kvq.ERR_UNSUPPORTED),
])
def test_plan_rejects(mutate, code):
    shape = kvq.make_shape(32, 8, 4, max_tokens=256)
    cfg = [(8, 4)] * 4
    mutate(shape, cfg)
    with pytest.raises(kvq.KvqError) as ei:
        kvq.plan_layers(shape, cfg)
    assert ei.value.code == code


def test_plan_rejects_paged_odd_pages_and_non_k2v2():
    with pytest.raises(kvq.KvqError) as ei:
        kvq.plan_layers(kvq.make_shape(32, 8, 4, page_tokens=16, int2_pages=3, int4_pages=4), [(2, 2)])
    assert ei.value.code == kvq.ERR_INVALID_ARG
    with pytest.raises(kvq.KvqError) as ei:
        kvq.plan_layers(kvq.make_shape(32, 8, 4, page_tokens=16, int2_pages=4, int4_pages=4), [(4, 2)])
    assert ei.value.code == kvq.ERR_UNSUPPORTED


class _Fake:
    """A stand-in device pointer: the checks below fail before any device access."""

    def __init__(self, addr=0x1000):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _call_decode(lib, plan, layer=0, batch=2, max_seq_len=64, ws_bytes=1 << 30, splits=0, out_dtype=0, ws=True,
                 seq=True):
    f = ctypes.c_void_p(0x1000)
    return lib.kvq_decode_attention(ctypes.byref(plan), layer, f, f, f if seq else None, batch, max_seq_len,
                                    ctypes.c_float(0.088), f, out_dtype, None, f if ws else None, ws_bytes, splits,
                                    None, None)


def test_decode_argument_errors(lib):
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 4, max_tokens=256), [(8, 4)] * 2)
    assert _call_decode(lib, plan, layer=2) == kvq.ERR_INVALID_ARG
    assert _call_decode(lib, plan, layer=-1) == kvq.ERR_INVALID_ARG
    assert _call_decode(lib, plan, batch=5) == kvq.ERR_INVALID_ARG
    assert _call_decode(lib, plan, max_seq_len=257) == kvq.ERR_CAPACITY
    assert _call_decode(lib, plan, ws_bytes=16) == kvq.ERR_WORKSPACE
    assert _call_decode(lib, plan, ws=False) == kvq.ERR_WORKSPACE
    assert _call_decode(lib, plan, splits=2000) == kvq.ERR_INVALID_ARG
    assert _call_decode(lib, plan, out_dtype=7) == kvq.ERR_INVALID_ARG
    assert _call_decode(lib, plan, seq=False) == kvq.ERR_INVALID_ARG
    assert "seq_lens" in lib.kvq_last_error().decode()
    need = kvq.workspace_bytes(plan, 2, 64, 3)
    assert need == 2 * 32 * 3 * 129 * 4


def test_append_and_dequant_argument_errors(lib):
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 4, max_tokens=256), [(8, 4)])
    f = ctypes.c_void_p(0x1000)
    P = ctypes.byref(plan)
    assert lib.kvq_quantize_append(P, 0, f, f, f, f, 2, 300, None, None) == kvq.ERR_CAPACITY
    assert lib.kvq_quantize_append(P, 0, None, f, f, f, 2, 3, None, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_quantize_append(P, 0, f, f, f, f, 9, 3, None, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_quantize_append(P, 0, f, f, f, f, 2, -1, None, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_quantize_append(P, 0, f, f, f, f, 0, 3, None, None) == kvq.OK  # nothing to do
    assert lib.kvq_dequantize(P, 0, f, f, 2, 300, f, f, None, None) == kvq.ERR_CAPACITY
    assert lib.kvq_dequantize(P, 1, f, f, 2, 30, f, f, None, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_dequantize(None, 0, f, f, 2, 30, f, f, None, None) == kvq.ERR_INVALID_ARG


def test_fused_append_decode_argument_errors(lib):
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 4, max_tokens=256), [(8, 4)] * 2)
    f = ctypes.c_void_p(0x1000)

    def call(plan=plan, layer=0, batch=2, max_seq_len=64, ws_bytes=1 << 30, splits=0, seq=True, kn=True):
        return lib.kvq_append_decode_attention(ctypes.byref(plan), layer, f, f if kn else None, f, f,
                                               f if seq else None, batch, max_seq_len, ctypes.c_float(0.088), f, 0,
                                               None, f, ws_bytes, splits, None, None)

    assert call(layer=2) == kvq.ERR_INVALID_ARG
    assert call(batch=5) == kvq.ERR_INVALID_ARG
    assert call(max_seq_len=257) == kvq.ERR_CAPACITY
    assert call(max_seq_len=0) == kvq.ERR_INVALID_ARG  # it counts the appended token
    assert call(ws_bytes=16) == kvq.ERR_WORKSPACE
    assert call(splits=2000) == kvq.ERR_INVALID_ARG
    assert call(seq=False) == kvq.ERR_INVALID_ARG
    assert call(kn=False) == kvq.ERR_INVALID_ARG
    assert call(plan=_paged_plan()) == kvq.ERR_INVALID_ARG  # a paged plan needs pages
    assert "pages" in lib.kvq_last_error().decode()
    assert call(batch=0) == kvq.OK  # nothing to do


def test_auto_split_count():
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 64, max_tokens=2080), [(4, 2)])
    s = kvq.num_splits(plan, 0, 64, 2048)
    assert 1 <= s <= 64
    assert kvq.workspace_bytes(plan, 64, 2048) == 64 * 32 * s * 129 * 4


def _paged_plan():
    return kvq.plan_layers(kvq.make_shape(32, 8, 4, page_tokens=16, int2_pages=64, int4_pages=64), [(2, 2, 0, 1)])


def test_paged_argument_errors(lib):
    paged = _paged_plan()
    contig = kvq.plan_layers(kvq.make_shape(32, 8, 4, max_tokens=256), [(8, 4)])
    f = ctypes.c_void_p(0x1000)
    pages = kvq.make_pages(_Fake(), 128, _Fake(), _Fake())

    def dec(plan, pg, max_seq_len=64, splits=0):
        return lib.kvq_decode_attention(ctypes.byref(plan), 0, f, f, None, 2, max_seq_len, ctypes.c_float(0.088), f, 0,
                                        None, f, 1 << 30, splits, ctypes.byref(pg) if pg else None, None)

    assert dec(paged, None) == kvq.ERR_INVALID_ARG  # a paged plan needs pages
    assert dec(contig, pages) == kvq.ERR_INVALID_ARG  # pages for a contiguous plan
    assert dec(paged, kvq.make_pages(_Fake(), 128, None, _Fake())) == kvq.ERR_INVALID_ARG
    assert dec(paged, kvq.make_pages(_Fake(), 0, _Fake(), _Fake())) == kvq.ERR_INVALID_ARG
    assert dec(paged, pages, max_seq_len=128 * 16 + 1) == kvq.ERR_CAPACITY
    assert dec(paged, pages, splits=1) == kvq.ERR_INVALID_ARG  # one kind per split: at least 2
    big = kvq.make_pages(_Fake(), 4096, _Fake(), _Fake())
    assert dec(paged, big, max_seq_len=32 * 300, splits=2) == kvq.ERR_INVALID_ARG  # 300 groups in a split
    assert "256" in lib.kvq_last_error().decode()
    P = ctypes.byref(paged)
    assert lib.kvq_quantize_append(P, 0, f, f, f, None, 2, 3, None, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_quantize_append(P, 0, f, f, f, None, 2, 128 * 16 + 1, ctypes.byref(pages), None) == \
        kvq.ERR_CAPACITY
    assert lib.kvq_dequantize(P, 0, f, None, 2, 30, f, f, None, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_dequantize(P, 0, f, None, 2, 128 * 16 + 1, f, f, ctypes.byref(pages), None) == kvq.ERR_CAPACITY

    def fused(pg, max_seq_len=64, splits=0):
        return lib.kvq_append_decode_attention(P, 0, f, f, f, f, None, 2, max_seq_len, ctypes.c_float(0.088), f, 0,
                                               None, f, 1 << 30, splits, ctypes.byref(pg) if pg else None, None)

    assert fused(None) == kvq.ERR_INVALID_ARG  # a paged plan needs pages
    assert fused(pages, splits=1) == kvq.ERR_INVALID_ARG  # one kind per split: at least 2
    assert fused(pages, max_seq_len=128 * 16 + 1) == kvq.ERR_CAPACITY
    assert fused(pages, max_seq_len=0) == kvq.ERR_INVALID_ARG  # it counts the appended token
    assert fused(kvq.make_pages(_Fake(), 128, _Fake(), _Fake(), _Fake())) == kvq.ERR_INVALID_ARG  # int2_add
    assert "int2_add" in lib.kvq_last_error().decode()


@pytest.mark.parametrize("batch,max_seq_len", [(16, 32768), (1, 32768), (64, 100), (4, 1), (2, 0)])
def test_paged_auto_splits_hold_the_limits(batch, max_seq_len):
    """Automatic paged split count: at least 2, and ceil(groups / (splits - 1)) <= 256."""
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 64, page_tokens=16, int2_pages=64, int4_pages=64), [(2, 2, 0, 1)])
    s = kvq.num_splits(plan, 0, batch, max_seq_len)
    groups = (max_seq_len + 31) // 32
    if groups == 0:
        assert s >= 1
        return
    assert 2 <= s <= 1024
    assert -(-groups // (s - 1)) <= 256
    assert kvq.workspace_bytes(plan, batch, max_seq_len) == batch * 32 * s * 129 * 4


def test_misaligned_pointers_are_rejected(lib):
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 4, max_tokens=256), [(8, 4)])
    P = ctypes.byref(plan)
    f, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)
    assert lib.kvq_quantize_append(P, 0, f, odd, f, f, 2, 3, None, None) == kvq.ERR_INVALID_ARG
    assert "16-byte" in lib.kvq_last_error().decode()
    assert lib.kvq_quantize_append(P, 0, odd, f, f, f, 2, 3, None, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_decode_attention(P, 0, f, odd, f, 2, 64, ctypes.c_float(0.088), f, 0, None, f, 1 << 30, 0,
                                    None, None) == kvq.ERR_INVALID_ARG
    assert lib.kvq_append_decode_attention(P, 0, f, f, odd, f, f, 2, 64, ctypes.c_float(0.088), f, 0, None, f,
                                           1 << 30, 0, None, None) == kvq.ERR_INVALID_ARG


def test_prefix_attention_argument_errors(lib):
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 4, max_tokens=256), [(8, 4)] * 2)
    f, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)

    def call(plan=plan, layer=0, batch=2, chunk=64, max_seq_len=200, ws_bytes=1 << 30, splits=0, seq=True, q=f,
             ws=True):
        return lib.kvq_prefix_attention(ctypes.byref(plan), layer, f, q, chunk, f if seq else None, batch,
                                        max_seq_len, ctypes.c_float(0.088), f, None, f if ws else None, ws_bytes,
                                        splits, None, None)

    assert call(layer=2) == kvq.ERR_INVALID_ARG
    assert call(batch=5) == kvq.ERR_INVALID_ARG
    assert call(chunk=-1) == kvq.ERR_INVALID_ARG
    assert call(batch=4, chunk=1 << 20) == kvq.ERR_INVALID_ARG  # 4 * 2^20 * 32 rows > 2^26
    assert call(max_seq_len=257) == kvq.ERR_CAPACITY
    assert call(max_seq_len=-1) == kvq.ERR_INVALID_ARG
    assert call(splits=2000) == kvq.ERR_INVALID_ARG
    assert call(splits=3, ws_bytes=16) == kvq.ERR_WORKSPACE
    assert call(splits=3, ws=False) == kvq.ERR_WORKSPACE
    assert call(seq=False) == kvq.ERR_INVALID_ARG
    assert call(q=odd) == kvq.ERR_INVALID_ARG
    assert "16-byte" in lib.kvq_last_error().decode()
    assert call(plan=_paged_plan()) == kvq.ERR_INVALID_ARG  # a paged plan needs its pages
    assert call(batch=0) == kvq.OK and call(chunk=0) == kvq.OK  # nothing to do


def test_prefix_workspace_and_auto_splits():
    plan = kvq.plan_layers(kvq.make_shape(32, 8, 4, max_tokens=4096), [(4, 2)])
    # a workgroup takes 256 rows (64 tokens x 4 heads): 4 requests x 8 KV heads x 16 blocks
    # of a 1024-token chunk fill the chip with one split
    assert kvq.prefix_workspace_bytes(plan, 4, 1024, 4096) == 0
    # 2 x 8 x 4 blocks of a 256-token chunk: 64 workgroups, 4 splits make one round of 256
    assert kvq.prefix_workspace_bytes(plan, 2, 256, 4096) == 2 * 256 * 32 * 4 * 129 * 4
    # one 4-token chunk: 8 workgroups, so the prefix is split, into 16 splits of 8 groups (a
    # split keeps at least 8 of the 128)
    assert kvq.prefix_workspace_bytes(plan, 1, 4, 4096) == 1 * 4 * 32 * 16 * 129 * 4
    assert kvq.prefix_workspace_bytes(plan, 1, 4, 4096, 5) == 4 * 32 * 5 * 129 * 4
    assert kvq.prefix_workspace_bytes(plan, 1, 4, 4096, 1) == 0
    assert kvq.prefix_workspace_bytes(plan, 1, 4, 100) == 0  # 4 groups: no more than one split
