"""The C ABI on the CPU: the library loads, exports every call include/skv.h
declares, and rejects malformed arguments with the documented status before
touching the GPU (validation is host code; no kernel is launched here)."""
import ctypes
import os
import re

import pytest

import sparse_kv_cache_append_amd as skv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(skv.LIB_PATH):
        from sparse_kv_cache_append_amd import build
        build.build(verbose=False)
    return skv.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(skv_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(skv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def desc(**kw):
    base = dict(batch=1, n_kv_heads=8, head_dim=128, max_seq=1024, block=64,
                kv_dtype=skv.SKV_F16, k=0x1000, v=0x2000, k_scale=None, v_scale=None,
                kmin=0x3000, kmax=0x4000)
    base.update(kw)
    return skv.SkvCacheDesc(*[base[f] for f, _ in skv.SkvCacheDesc._fields_])


BAD = 0x10  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,expect", [
    (dict(batch=0), skv.SKV_EINVAL),
    (dict(n_kv_heads=0), skv.SKV_EINVAL),
    (dict(head_dim=100), skv.SKV_EINVAL),         # not a multiple of 16
    (dict(head_dim=2048), skv.SKV_EINVAL),        # above 1024
    (dict(head_dim=96), skv.SKV_EUNSUPPORTED),    # valid, not built
    (dict(head_dim=512), skv.SKV_EUNSUPPORTED),
    (dict(head_dim=96, kv_dtype=skv.SKV_Q8_0, k_scale=0x5000, v_scale=0x6000),
     skv.SKV_EUNSUPPORTED),                       # group-wise caches: 64, 128, 256
    (dict(block=40), skv.SKV_EINVAL),
    (dict(block=0), skv.SKV_EINVAL),
    (dict(kv_dtype=7), skv.SKV_EINVAL),
    (dict(k=None), skv.SKV_EINVAL),
    (dict(kv_dtype=skv.SKV_I8), skv.SKV_EINVAL),  # int8 without scales
    (dict(kmax=None), skv.SKV_EINVAL),            # half a side cache
    (dict(max_seq=0), skv.SKV_EINVAL),
    (dict(k=0x1008), skv.SKV_EINVAL),             # rows move in 16-byte vectors
    (dict(kmin=0x3004, kmax=0x4004), skv.SKV_EINVAL),
    (dict(kv_dtype=skv.SKV_I8, k_scale=0x5002, v_scale=0x6000), skv.SKV_EINVAL),
])
def test_cache_descriptor_validation(lib, kw, expect):
    d = desc(**kw)
    st = lib.skv_decode_attn(ctypes.byref(d), BAD, 32, BAD, 10, None, None, 0, 0.1, 4,
                             BAD, 1 << 30, None, None)
    assert st == expect


@pytest.mark.parametrize("dim", [64, 256])
def test_head_dims_64_256_core_calls_only(lib, dim):
    """Head dims 64 and 256 pass the descriptor check of every call (the
    calls below then stop at a later check, before any launch)."""
    d = desc(head_dim=dim)
    q = 0x7000
    # decode_attn: accepted, then the workspace is too small
    assert lib.skv_decode_attn(ctypes.byref(d), q, 32, BAD, 10, None, None, 0, 0.1, 4,
                               BAD, 16, None, None) == skv.SKV_EWORKSPACE
    # decode_attn_select and decode_step: the same
    assert lib.skv_decode_attn_select(ctypes.byref(d), q, 32, BAD, 10, BAD, BAD, 1, 2, 8,
                                      BAD, BAD, 0.1, 4, BAD, 16, None) == skv.SKV_EWORKSPACE
    assert lib.skv_decode_step(ctypes.byref(d), None, None, None, skv.SKV_F16, q, 32, BAD, 10,
                               None, 1, 2, 8, None, None, None, 0.1, 4, BAD, 16, BAD,
                               None) == skv.SKV_EWORKSPACE
    # block_bounds and kv_append: accepted, then a range check fails
    assert lib.skv_block_bounds(ctypes.byref(d), q, 32, BAD, 5000, BAD, None) == skv.SKV_ERANGE
    assert lib.skv_kv_append(ctypes.byref(d), BAD, 5000, q, q, skv.SKV_F16, None) == \
        skv.SKV_ERANGE
    # per-head bounds and token chunks: accepted, then a range check fails
    assert lib.skv_block_bounds_heads(ctypes.byref(d), q, 32, BAD, 5000, BAD, None) == \
        skv.SKV_ERANGE
    assert lib.skv_block_bounds_multi(ctypes.byref(d), q, 2, 32, BAD, 5000, BAD, None) == \
        skv.SKV_ERANGE
    # group-wise caches: accepted, then a range check fails
    g = desc(head_dim=dim, kv_dtype=skv.SKV_Q8_0, k_scale=0x5000, v_scale=0x6000)
    assert lib.skv_kv_append(ctypes.byref(g), BAD, 5000, q, q, skv.SKV_F32, None) == \
        skv.SKV_ERANGE
    # sparse-V: accepted, then the workspace is too small
    assert lib.skv_decode_attn_sparse_v(ctypes.byref(d), q, 32, BAD, 10, None, None, 0, 0.1,
                                        1e-3, 0.0, 4, BAD, 16, BAD, None) == \
        skv.SKV_EWORKSPACE
    # the scan: accepted, then a range check fails
    assert lib.skv_scan4_build(ctypes.byref(d), BAD, BAD, 5000, BAD, BAD, BAD, BAD, None) == \
        skv.SKV_ERANGE


def test_decode_argument_validation(lib):
    d = desc()
    call = lambda **a: lib.skv_decode_attn(
        ctypes.byref(d), a.get("q", BAD), a.get("H", 32), a.get("sl", BAD), a.get("ml", 10),
        a.get("si", None), a.get("sc", None), a.get("ms", 0), a.get("scale", 0.1),
        a.get("S", 4), a.get("ws", BAD), a.get("wb", 1 << 30), a.get("dbg", None), None)
    assert call(H=30) == skv.SKV_EINVAL               # H % Hkv != 0
    assert call(H=128) == skv.SKV_EUNSUPPORTED        # G = 16 not built
    assert call(q=None) == skv.SKV_EINVAL
    assert call(q=BAD + 4) == skv.SKV_EINVAL          # q not 16-byte aligned
    assert call(sl=None) == skv.SKV_EINVAL
    assert call(si=BAD) == skv.SKV_EINVAL             # sel_idx without sel_cnt
    assert call(si=BAD, sc=BAD, ms=0) == skv.SKV_EINVAL
    assert call(S=0) == skv.SKV_EINVAL
    assert call(S=5000) == skv.SKV_EINVAL
    assert call(scale=float("nan")) == skv.SKV_EINVAL
    assert call(ml=-1) == skv.SKV_ERANGE
    assert call(ml=1025) == skv.SKV_ERANGE            # above max_seq
    assert call(dbg=BAD) == skv.SKV_EINVAL            # dbg logits need an int8 cache
    assert call(ws=None) == skv.SKV_EWORKSPACE
    need = skv.workspace_bytes(1, 32, 128, 4)
    assert call(wb=need - 1) == skv.SKV_EWORKSPACE


def test_append_validation(lib):
    d = desc()
    f = lambda dd, **a: lib.skv_kv_append(ctypes.byref(dd), a.get("pos", BAD), a.get("n", 1),
                                          a.get("k", BAD), a.get("v", BAD),
                                          a.get("src", skv.SKV_F16), None)
    assert f(d, pos=None) == skv.SKV_EINVAL
    assert f(d, n=0) == skv.SKV_EINVAL
    assert f(d, k=None) == skv.SKV_EINVAL
    assert f(d, v=BAD + 8) == skv.SKV_EINVAL               # new rows 16-byte aligned
    assert f(d, n=1025) == skv.SKV_ERANGE
    assert f(d, src=skv.SKV_F32) == skv.SKV_EUNSUPPORTED   # f16 cache takes f16 rows
    assert f(d, src=99) == skv.SKV_EINVAL
    d8 = desc(kv_dtype=skv.SKV_I8, k_scale=0x5000, v_scale=0x6000)
    assert f(d8, src=skv.SKV_F16) == skv.SKV_EUNSUPPORTED  # int8 cache takes f32 rows


def test_bounds_and_select_validation(lib):
    nob = desc(kmin=None, kmax=None)
    assert lib.skv_block_bounds(ctypes.byref(nob), BAD, 32, BAD, 10, BAD, None) == skv.SKV_EINVAL
    d = desc()
    assert lib.skv_block_bounds(ctypes.byref(d), BAD, 31, BAD, 10, BAD, None) == skv.SKV_EINVAL
    assert lib.skv_block_bounds(ctypes.byref(d), BAD, 32, BAD, 2000, BAD, None) == skv.SKV_ERANGE
    assert lib.skv_block_bounds(ctypes.byref(d), None, 32, BAD, 10, BAD, None) == skv.SKV_EINVAL
    sel = lambda **a: lib.skv_select_topk(
        a.get("score", BAD), BAD, a.get("B", 1), 8, a.get("mb", 16), a.get("blk", 64), BAD,
        a.get("ns", 1), a.get("nr", 2), a.get("ms", 8), BAD, BAD, None, None)
    assert sel(score=None) == skv.SKV_EINVAL
    assert sel(B=0) == skv.SKV_EINVAL
    assert sel(blk=20) == skv.SKV_EINVAL
    assert sel(ns=-1) == skv.SKV_EINVAL
    assert sel(nr=-1) == skv.SKV_EINVAL
    assert sel(ms=0) == skv.SKV_EINVAL
    assert sel(mb=20000) == skv.SKV_EUNSUPPORTED


def test_combine_validation_and_sizes(lib):
    assert lib.skv_combine(None, 1, 32, 128, 4, BAD, None) == skv.SKV_EINVAL
    assert lib.skv_combine(BAD, 1, 32, 100, 4, BAD, None) == skv.SKV_EINVAL
    assert lib.skv_combine(BAD, 1, 32, 128, 0, BAD, None) == skv.SKV_EINVAL
    assert skv.workspace_bytes(2, 32, 128, 64) == 4 * 2 * 32 * 64 * 130
    assert skv.workspace_bytes(0, 32, 128, 64) == 0
    assert lib.skv_max_blocks(ctypes.byref(desc(max_seq=1000, block=64))) == 16
    assert skv.status_str(-3).startswith("SKV_EWORKSPACE")


def test_binding_fails_loudly_without_the_library(tmp_path):
    import importlib
    mod = importlib.import_module("sparse_kv_cache_append_amd")
    saved = mod._lib
    mod._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            mod.load(str(tmp_path / "nope.so"))
    finally:
        mod._lib = saved


def test_grid_size_limits(lib):
    """Launch grids that would not fit the hardware's grid dimensions are
    rejected on the host with SKV_ERANGE (1-D grids up to 2^31 - 1
    workgroups; the append keeps KV heads and sequences in y and z)."""
    big = desc(batch=65536, n_kv_heads=1, max_seq=64)
    assert lib.skv_decode_attn(ctypes.byref(big), BAD, 1, BAD, 10, None, None, 0, 0.1, 1,
                               BAD, 1 << 40, None, None) == skv.SKV_ERANGE
    wide = desc(batch=65535, n_kv_heads=16, max_seq=64)       # 1,048,560 rows x 4,096 parts
    assert lib.skv_decode_attn(ctypes.byref(wide), BAD, 16, BAD, 10, None, None, 0, 0.1, 4096,
                               BAD, 1 << 62, None, None) == skv.SKV_ERANGE
    assert lib.skv_select_topk(BAD, BAD, 70000, 40000, 16, 64, BAD, 1, 2, 8, BAD, BAD, None,
                               None) == skv.SKV_ERANGE
    assert lib.skv_combine(BAD, 70000, 40000, 128, 4, BAD, None) == skv.SKV_ERANGE


def test_default_split_rule():
    """Host-side split choice: about one workgroup per compute unit, at least
    one unit per part; dense int8 doubles that only while every part keeps at
    least 4 blocks; Quest parts run over the selected list."""
    ds = skv.default_split
    assert ds(1, 8, 512) == 32                              # 32K f16: 256 workgroups
    assert ds(1, 8, 8) == 8                                 # 512 tokens: one block per part
    assert ds(16, 8, 1024) == 2                             # 16 sequences x 8 KV heads
    assert ds(1, 4, 4096, kv_dtype="i8") == 128             # 262K int8: 512 workgroups
    assert ds(1, 8, 128, kv_dtype="i8") == 32               # 8K int8: 4-block parts kept
    assert ds(1, 8, 255, kv_dtype="i8") == 32               # 64 parts would hold < 4 blocks
    assert ds(1, 8, 256, kv_dtype="i8") == 64
    assert ds(1, 4, 517, kv_dtype="i8", sparse=True) == 64  # Quest: one workgroup per CU
    assert ds(1, 8, 512, kv_dtype="q4_0") == 64             # 32K q4_0 dense: two per CU
    assert ds(1, 8, 512, kv_dtype="q8_0") == 32             # q8_0 keeps one
    assert ds(1, 8, 131, kv_dtype="q4_0", sparse=True) == 32
    assert ds(1, 8, 131, sparse=True) == 32
    assert ds(1, 1, 10 ** 6) == 256 and ds(1, 1, 10 ** 9, target_wgs=10 ** 6) == 4096
    assert ds(4096, 16, 1000) == 1
    sc = skv.scan4_default_split
    assert sc(1, 8, 512) == 64                              # 32K scan: two per CU
    assert sc(1, 8, 255) == 32 and sc(1, 8, 256) == 64      # 4-block parts kept
    assert sc(1, 8, 8) == 8 and sc(16, 8, 1024) == 4


# ------------------------------------------------- binding argument checks
class _FakeCache:
    """The attributes the binding reads from a Cache (no device memory: every
    call below must be rejected before a pointer is taken)."""
    def __init__(self, kv_dtype="f16", batch=2, n_kv_heads=4, head_dim=128, max_blocks=8):
        self.kv_dtype, self.batch, self.n_kv_heads = kv_dtype, batch, n_kv_heads
        self.head_dim, self.max_blocks, self.block = head_dim, max_blocks, 64
        self.desc = desc(batch=batch, n_kv_heads=n_kv_heads)


def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _rejected(fn):
    with pytest.raises(skv.SkvError) as e:
        fn()
    assert e.value.status == skv.SKV_EINVAL


def _reaches_pointers(fn):
    """Validation passed: the binding got as far as taking device pointers
    of these CPU tensors."""
    with pytest.raises(ValueError, match="GPU"):
        fn()


def test_binding_checks_append_rows(lib):
    import torch
    c = _FakeCache("i8")
    pos = _t((2,), torch.int32)
    good = _t((2, 3, 4, 128), torch.float32)
    _reaches_pointers(lambda: skv.kv_append(c, pos, good, good.clone()))
    # the source dtype passed to C is the rows' own (a float16 row for an int8
    # cache is then rejected by the C side, not read as float32)
    _rejected(lambda: skv.kv_append(c, pos, good, _t((2, 3, 4, 128), torch.float16)))
    _rejected(lambda: skv.kv_append(c, pos, _t((2, 3, 4, 128), torch.float64),
                                    _t((2, 3, 4, 128), torch.float64)))
    _rejected(lambda: skv.kv_append(c, pos, _t((2, 3, 4, 64), torch.float32),
                                    _t((2, 3, 4, 64), torch.float32)))
    _rejected(lambda: skv.kv_append(c, pos, _t((1, 3, 4, 128), torch.float32),
                                    _t((1, 3, 4, 128), torch.float32)))
    _rejected(lambda: skv.kv_append(c, _t((2,), torch.int64), good, good.clone()))
    _rejected(lambda: skv.kv_append(c, _t((3,), torch.int32), good, good.clone()))


def test_binding_checks_query_lengths_and_lists(lib):
    import torch
    c = _FakeCache()
    q = _t((2, 8, 128), torch.float32)
    sl = _t((2,), torch.int32)
    ws = _t((1024,), torch.uint8)
    _reaches_pointers(lambda: skv.decode_attn(c, q, sl, 64, 0.1, 2, ws))
    _rejected(lambda: skv.decode_attn(c, q.half(), sl, 64, 0.1, 2, ws))
    _rejected(lambda: skv.decode_attn(c, q, sl.long(), 64, 0.1, 2, ws))
    _rejected(lambda: skv.decode_attn(c, _t((3, 8, 128), torch.float32), sl, 64, 0.1, 2, ws))
    si, sc = _t((2, 4, 5), torch.int32), _t((2, 4), torch.int32)
    _reaches_pointers(lambda: skv.decode_attn(c, q, sl, 64, 0.1, 2, ws, si, sc))
    _rejected(lambda: skv.decode_attn(c, q, sl, 64, 0.1, 2, ws, si.long(), sc))
    _rejected(lambda: skv.decode_attn(c, q, sl, 64, 0.1, 2, ws, si, None))
    _rejected(lambda: skv.decode_attn(c, q, sl, 64, 0.1, 2, ws,
                                      dbg_logits=_t((2, 8, 32), torch.int32)))
    score = _t((2, 4, 8), torch.float32)
    _reaches_pointers(lambda: skv.block_bounds(c, q, sl, 64, score))
    _rejected(lambda: skv.block_bounds(c, q, sl, 64, _t((2, 4, 7), torch.float32)))
    ks = _t((2,), torch.int32)
    _reaches_pointers(lambda: skv.select_topk(score, sl, 64, ks, 1, 2, si, sc))
    _rejected(lambda: skv.select_topk(score, sl, 64, ks.long(), 1, 2, si, sc))
    _rejected(lambda: skv.select_topk(score.double(), sl, 64, ks, 1, 2, si, sc))
    out = _t((2, 8, 128), torch.float32)
    _reaches_pointers(lambda: skv.combine(ws, 2, 8, 128, 2, out))
    _rejected(lambda: skv.combine(ws, 2, 8, 128, 2, out.half()))


def test_binding_checks_decode_step(lib):
    import torch
    c = _FakeCache("f16")
    q = _t((2, 8, 128), torch.float32)
    sl = _t((2,), torch.int32)
    ws = _t((1024,), torch.uint8)
    out = _t((2, 8, 128), torch.float32)
    rows = _t((2, 1, 4, 128), torch.float16)
    pos = _t((2,), torch.int32)
    _reaches_pointers(lambda: skv.decode_step(c, q, sl, 64, 0.1, 2, ws, out, pos0=pos,
                                              k_new=rows, v_new=rows.clone()))
    # two tokens where the step appends one
    two = _t((2, 2, 4, 128), torch.float16)
    _rejected(lambda: skv.decode_step(c, q, sl, 64, 0.1, 2, ws, out, pos0=pos, k_new=two,
                                      v_new=two.clone()))
    _rejected(lambda: skv.decode_step(c, q, sl, 64, 0.1, 2, ws, out, pos0=pos.long(),
                                      k_new=rows, v_new=rows.clone()))
    _rejected(lambda: skv.decode_step(c, q, sl, 64, 0.1, 2, ws, out.half()))
    score = _t((2, 4, 8), torch.float32)
    si, sc = _t((2, 4, 5), torch.int32), _t((2, 4), torch.int32)
    ks = _t((2,), torch.int32)
    _reaches_pointers(lambda: skv.decode_step(c, q, sl, 64, 0.1, 2, ws, out, k_sel=ks,
                                              score=score, sel_idx=si, sel_cnt=sc))
    _rejected(lambda: skv.decode_step(c, q, sl, 64, 0.1, 2, ws, out, k_sel=ks, score=score))
    _rejected(lambda: skv.decode_step(c, q, sl, 64, 0.1, 2, ws, out, k_sel=ks.long(),
                                      score=score, sel_idx=si, sel_cnt=sc))


def test_token_chunk_validation(lib):
    """Query-token chunks: T in {1, 2, 4, 8}, T x G <= 16, lists all-or-none,
    the workspace sized for T x n_heads rows; every failure before a launch."""
    d = desc()                                      # G = 32 / 8 = 4
    q, sl, score = 0x5000, 0x6000, 0x7000
    bb = lib.skv_block_bounds_multi
    assert bb(ctypes.byref(d), q, 3, 32, sl, 1024, score, None) == skv.SKV_EUNSUPPORTED
    assert bb(ctypes.byref(d), q, 8, 32, sl, 1024, score, None) == skv.SKV_EUNSUPPORTED  # 32 cols
    assert bb(ctypes.byref(d), q, 0, 32, sl, 1024, score, None) == skv.SKV_EINVAL
    assert bb(ctypes.byref(d), q, 4, 32, sl, 2048, score, None) == skv.SKV_ERANGE
    assert bb(ctypes.byref(d), None, 4, 32, sl, 1024, score, None) == skv.SKV_EINVAL
    st = lib.skv_select_topk_multi
    assert st(score, sl, 1, 3, 8, 16, 64, 0x8000, 1, 2, 8, 0x9000, 0xA000, None) == \
        skv.SKV_EUNSUPPORTED
    assert st(score, sl, 1, 0, 8, 16, 64, 0x8000, 1, 2, 8, 0x9000, 0xA000, None) == skv.SKV_EINVAL
    assert st(score, sl, 1, 4, 8, 16, 64, None, 1, 2, 8, 0x9000, 0xA000, None) == skv.SKV_EINVAL
    un = lib.skv_select_union_tokens
    assert un(0x9000, 0xA000, 1, 4, 8, 3, 8, 16, 32, 0xB000, 0xC000, 0xD000, None) == \
        skv.SKV_EUNSUPPORTED                        # group 3
    assert un(0x9000, 0xA000, 1, 8, 8, 4, 8, 16, 32, 0xB000, 0xC000, 0xD000, None) == \
        skv.SKV_EUNSUPPORTED                        # 32 bits
    assert un(0x9000, 0xA000, 1, 4, 8, 4, 8, 16, 32, 0xB000, 0xC000, None, None) == skv.SKV_EINVAL
    da = lib.skv_decode_attn_multi
    need = skv.workspace_bytes(1, 4 * 32, 128, 4)
    assert need == skv.workspace_bytes(1, 32, 128, 4) * 4
    assert da(ctypes.byref(d), q, 4, 32, sl, 1024, None, None, None, 0, 0.1, 4, 0xE000,
              need - 1, None) == skv.SKV_EWORKSPACE
    assert da(ctypes.byref(d), q, 8, 32, sl, 1024, None, None, None, 0, 0.1, 4, 0xE000,
              need * 2, None) == skv.SKV_EUNSUPPORTED
    assert da(ctypes.byref(d), q, 4, 32, sl, 1024, 0x9000, None, None, 8, 0.1, 4, 0xE000,
              need, None) == skv.SKV_EINVAL       # half a list
    assert da(ctypes.byref(d), q, 4, 32, sl, 1024, None, None, None, 0, -1.0, 4, 0xE000,
              need, None) == skv.SKV_EINVAL
    # group-wise caches: accepted, then the workspace is too small
    g = desc(kv_dtype=skv.SKV_Q8_0, k_scale=0xF000, v_scale=0xF100)
    assert da(ctypes.byref(g), q, 2, 32, sl, 1024, None, None, None, 0, 0.1, 4, 0xE000,
              16, None) == skv.SKV_EWORKSPACE
