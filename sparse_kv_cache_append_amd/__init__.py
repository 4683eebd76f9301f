"""Decode-step attention over dense, int8 and Quest block-sparse KV caches on
AMD MI355X (gfx950).

Python binding of ``libskv.so`` (declared in ``include/skv.h``).  This module
only marshals arguments: tensors become device pointers, the current torch
stream becomes the HIP stream, status codes become exceptions.  Every step of
the computation runs in the library's HIP kernels; there is no Python or CPU
fallback, and :func:`load` raises if the library is missing.

The five calls keep the C names: :func:`kv_append`, :func:`block_bounds`,
:func:`select_topk`, :func:`decode_attn`, :func:`combine`, and so does the
whole-step call :func:`decode_step` (plus :func:`workspace_bytes` and
:func:`status_str`).  :class:`Cache` owns the
cache tensors and the C descriptor; :func:`decode` chains the calls for one
decode step (dense, or Quest when ``k_sel`` is given), the shape of the
``Int8KVCache.append`` / ``decode`` interface on the cpu-attn kernel card
("Usage").
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = ["load", "Cache", "SkvError", "kv_append", "block_bounds", "select_topk",
           "decode_attn", "decode_attn_select", "decode_attn_sparse_v", "sparse_v_workspace_bytes",
           "block_bounds_heads", "select_union", "decode_attn_heads", "block_bounds_multi",
           "select_topk_multi", "select_union_tokens", "decode_attn_multi", "Scan4Index",
           "scan4_build", "scan4_candidates", "scan4_workspace_bytes", "scan4_default_split",
           "decode_step", "decode_step_static", "combine", "workspace_bytes", "status_str", "decode",
           "SKV_F16", "SKV_F32", "SKV_I8", "SKV_Q8_0", "SKV_Q4_0", "SKV_Q5_0", "LIB_PATH",
           "EXPORTS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libskv.so")

SKV_OK, SKV_EINVAL, SKV_ERANGE, SKV_EWORKSPACE, SKV_EUNSUPPORTED, SKV_EDEVICE = 0, -1, -2, -3, -4, -5
SKV_F16, SKV_F32, SKV_I8, SKV_Q8_0, SKV_Q4_0, SKV_Q5_0 = 1, 2, 3, 4, 5, 6
_KV_CODES = {"f16": SKV_F16, "i8": SKV_I8, "q8_0": SKV_Q8_0, "q4_0": SKV_Q4_0, "q5_0": SKV_Q5_0}
_GROUPED = ("q8_0", "q4_0", "q5_0")

EXPORTS = ("skv_max_blocks", "skv_kv_append", "skv_block_bounds", "skv_select_topk",
           "skv_decode_attn", "skv_decode_attn_select", "skv_decode_step",
           "skv_decode_step_static", "skv_static_scratch_bytes", "skv_decode_attn_sparse_v",
           "skv_sparse_v_workspace_bytes", "skv_block_bounds_heads", "skv_select_union",
           "skv_decode_attn_heads", "skv_block_bounds_multi", "skv_select_topk_multi",
           "skv_select_union_tokens", "skv_decode_attn_multi", "skv_scan4_build",
           "skv_scan4_workspace_bytes",
           "skv_scan4_candidates", "skv_combine",
           "skv_workspace_bytes", "skv_status_str")


class SkvCacheDesc(ctypes.Structure):
    """Mirror of ``skv_cache`` in include/skv.h."""
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("block", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("kmin", ctypes.c_void_p), ("kmax", ctypes.c_void_p)]


class SkvError(RuntimeError):
    def __init__(self, call: str, status: int, detail: str = ""):
        msg = f"{call} failed: {status_str(status)} ({status})"
        super().__init__(msg + (f": {detail}" if detail else ""))
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libskv.so once and declare the C signatures.  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_kv_cache_append_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    desc = ctypes.POINTER(SkvCacheDesc)
    sig = {
        "skv_max_blocks": (I32, [desc]),
        "skv_kv_append": (I32, [desc, P, I32, P, P, I32, P]),
        "skv_block_bounds": (I32, [desc, P, I32, P, I32, P, P]),
        "skv_select_topk": (I32, [P, P, I32, I32, I32, I32, P, I32, I32, I32, P, P, P, P]),
        "skv_decode_attn": (I32, [desc, P, I32, P, I32, P, P, I32, ctypes.c_float, I32, P, SZ, P, P]),
        "skv_decode_attn_select": (I32, [desc, P, I32, P, I32, P, P, I32, I32, I32, P, P,
                                         ctypes.c_float, I32, P, SZ, P]),
        "skv_decode_step": (I32, [desc, P, P, P, I32, P, I32, P, I32, P, I32, I32, I32, P, P, P,
                                   ctypes.c_float, I32, P, SZ, P, P]),
        "skv_decode_step_static": (I32, [desc, P, P, P, I32, P, I32, P, I32, P, I32, I32, I32,
                                         P, P, ctypes.c_float, I32, P, P]),
        "skv_static_scratch_bytes": (SZ, []),
        "skv_decode_attn_sparse_v": (I32, [desc, P, I32, P, I32, P, P, I32, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_float, I32, P, SZ, P, P]),
        "skv_sparse_v_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
        "skv_block_bounds_heads": (I32, [desc, P, I32, P, I32, P, P]),
        "skv_scan4_build": (I32, [desc, P, P, I32, P, P, P, P, P]),
        "skv_scan4_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "skv_scan4_candidates": (I32, [desc, P, P, P, P, P, I32, P, I32, ctypes.c_float, I32, P,
                                       SZ, P, P, P]),
        "skv_select_union": (I32, [P, P, I32, I32, I32, I32, I32, I32, P, P, P, P]),
        "skv_decode_attn_heads": (I32, [desc, P, I32, P, I32, P, P, P, I32, ctypes.c_float, I32,
                                        P, SZ, P]),
        "skv_block_bounds_multi": (I32, [desc, P, I32, I32, P, I32, P, P]),
        "skv_select_topk_multi": (I32, [P, P, I32, I32, I32, I32, I32, P, I32, I32, I32, P, P,
                                        P]),
        "skv_select_union_tokens": (I32, [P, P, I32, I32, I32, I32, I32, I32, I32, P, P, P, P]),
        "skv_decode_attn_multi": (I32, [desc, P, I32, I32, P, I32, P, P, P, I32, ctypes.c_float,
                                        I32, P, SZ, P]),
        "skv_combine": (I32, [P, I32, I32, I32, I32, P, P]),
        "skv_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "skv_status_str": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


_STATUS_NAMES = {SKV_OK: "SKV_OK", SKV_EINVAL: "SKV_EINVAL", SKV_ERANGE: "SKV_ERANGE",
                 SKV_EWORKSPACE: "SKV_EWORKSPACE", SKV_EUNSUPPORTED: "SKV_EUNSUPPORTED",
                 SKV_EDEVICE: "SKV_EDEVICE"}


def status_str(status: int) -> str:
    try:
        return load().skv_status_str(int(status)).decode()
    except RuntimeError:          # library missing: name the code only
        return _STATUS_NAMES.get(int(status), "unknown skv_status")


def workspace_bytes(batch: int, n_heads: int, head_dim: int, n_split: int) -> int:
    return int(load().skv_workspace_bytes(batch, n_heads, head_dim, n_split))


def _check(call: str, status: int):
    if status != SKV_OK:
        raise SkvError(call, status)


def _ptr(t) -> Optional[int]:
    """Device pointer of a CUDA tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _dtype_code(t) -> int:
    """skv_dtype of a tensor's element type (0, which the C side rejects, for
    any other type)."""
    import torch
    return {torch.float16: SKV_F16, torch.float32: SKV_F32, torch.int8: SKV_I8}.get(t.dtype, 0)


def _need(call: str, ok: bool, what: str):
    """Reject a malformed argument before anything is enqueued (SKV_EINVAL)."""
    if not ok:
        raise SkvError(call, SKV_EINVAL, what)


def _is(t, dtype, shape) -> bool:
    """t has element type dtype and the given shape (None entries: any size)."""
    if t is None or t.dtype != dtype or t.dim() != len(shape):
        return False
    return all(s is None or int(d) == s for d, s in zip(t.shape, shape))


def _check_rows(call: str, cache, k_new, v_new, n_new: Optional[int] = None):
    """New rows: [batch][n_new][Hkv][D], k_new and v_new alike, float16 for an
    f16 cache and float32 for an int8 cache (the C call checks the pair)."""
    import torch
    _need(call, k_new is not None and v_new is not None, "k_new and v_new are required")
    _need(call, k_new.dim() == 4 and tuple(k_new.shape) == tuple(v_new.shape)
          and k_new.dtype == v_new.dtype, "k_new and v_new must have one shape and dtype")
    _need(call, _is(k_new, k_new.dtype, (cache.batch, n_new, cache.n_kv_heads, cache.head_dim)),
          "k_new must be [batch][n_new][n_kv_heads][head_dim]")
    _need(call, k_new.dtype in (torch.float16, torch.float32), "k_new must be float16 or float32")


def _check_q(call: str, cache, q, seq_len):
    import torch
    _need(call, q is not None and _is(q, torch.float32, (cache.batch, None, cache.head_dim)),
          "q must be float32 [batch][n_heads][head_dim]")
    _need(call, _is(seq_len, torch.int32, (cache.batch,)), "seq_len must be int32 [batch]")


def _check_sel(call: str, batch: int, n_kv: int, sel_idx, sel_cnt):
    import torch
    _need(call, (sel_idx is None) == (sel_cnt is None), "sel_idx and sel_cnt go together")
    if sel_idx is not None:
        _need(call, _is(sel_idx, torch.int32, (batch, n_kv, None)),
              "sel_idx must be int32 [batch][n_kv_heads][max_sel]")
        _need(call, _is(sel_cnt, torch.int32, (batch, n_kv)),
              "sel_cnt must be int32 [batch][n_kv_heads]")


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Cache:
    """KV cache tensors plus the C descriptor.

    kv_dtype "f16": k, v [batch][n_kv_heads][max_seq][head_dim] float16.
    kv_dtype "i8": k, v int8 codes, same shape; k_scale, v_scale
    [batch][n_kv_heads][max_seq] float32.
    kv_dtype "q8_0" / "q4_0" / "q5_0" (groups of 32 channels): k, v uint8
    [batch][n_kv_heads][max_seq][head_dim] (q8_0 int8 codes) or [...][head_dim
    / 2] (q4_0 nibbles) or [batch][n_kv_heads][max_seq * 5 head_dim / 8]
    (q5_0: the nibble plane [max_seq][head_dim / 2], then the fifth-bit plane
    [max_seq][head_dim / 8]; ``q5_planes`` gives both views); k_scale,
    v_scale float16 [batch][n_kv_heads][max_seq][head_dim / 32].
    kmin, kmax: [batch][n_kv_heads][max_blocks][head_dim] float16 (Quest side
    cache, allocated when ``bounds``)."""

    def __init__(self, batch: int, n_kv_heads: int, max_seq: int, head_dim: int = 128,
                 kv_dtype: str = "f16", block: int = 64, bounds: bool = True, device="cuda"):
        import torch
        if kv_dtype not in _KV_CODES:
            raise ValueError("kv_dtype must be 'f16', 'i8', 'q8_0', 'q4_0' or 'q5_0'")
        self.batch, self.n_kv_heads, self.max_seq = batch, n_kv_heads, max_seq
        self.head_dim, self.block, self.kv_dtype = head_dim, block, kv_dtype
        self.max_blocks = -(-max_seq // block)
        shape = (batch, n_kv_heads, max_seq, head_dim)
        if kv_dtype == "q5_0":
            per = max_seq * (head_dim // 2 + head_dim // 8)
            self.k = torch.zeros(shape[:2] + (per,), dtype=torch.uint8, device=device)
            self.v = torch.zeros(shape[:2] + (per,), dtype=torch.uint8, device=device)
        elif kv_dtype in ("q8_0", "q4_0"):
            row = head_dim if kv_dtype == "q8_0" else head_dim // 2
            self.k = torch.zeros(shape[:3] + (row,), dtype=torch.uint8, device=device)
            self.v = torch.zeros(shape[:3] + (row,), dtype=torch.uint8, device=device)
        else:
            dt = torch.float16 if kv_dtype == "f16" else torch.int8
            self.k = torch.zeros(shape, dtype=dt, device=device)
            self.v = torch.zeros(shape, dtype=dt, device=device)
        self.k_scale = self.v_scale = None
        if kv_dtype == "i8":
            self.k_scale = torch.zeros(shape[:3], dtype=torch.float32, device=device)
            self.v_scale = torch.zeros(shape[:3], dtype=torch.float32, device=device)
        elif kv_dtype in _GROUPED:
            gshape = shape[:3] + (head_dim // 32,)
            self.k_scale = torch.zeros(gshape, dtype=torch.float16, device=device)
            self.v_scale = torch.zeros(gshape, dtype=torch.float16, device=device)
        self.kmin = self.kmax = None
        if bounds:
            bshape = (batch, n_kv_heads, self.max_blocks, head_dim)
            self.kmin = torch.zeros(bshape, dtype=torch.float16, device=device)
            self.kmax = torch.zeros(bshape, dtype=torch.float16, device=device)
        self.desc = SkvCacheDesc(batch, n_kv_heads, head_dim, max_seq, block, _KV_CODES[kv_dtype],
                                 _ptr(self.k), _ptr(self.v), _ptr(self.k_scale),
                                 _ptr(self.v_scale), _ptr(self.kmin), _ptr(self.kmax))

    def q5_planes(self, t):
        """The two planes of a q5_0 code tensor (self.k or self.v): the nibble
        plane [batch][n_kv_heads][max_seq][head_dim / 2] and the fifth-bit
        plane [batch][n_kv_heads][max_seq][head_dim / 8] (views)."""
        n = self.max_seq * (self.head_dim // 2)
        lo = t[:, :, :n].unflatten(2, (self.max_seq, self.head_dim // 2))
        hi = t[:, :, n:].unflatten(2, (self.max_seq, self.head_dim // 8))
        return lo, hi

    def src_dtype(self) -> int:
        return SKV_F16 if self.kv_dtype == "f16" else SKV_F32

    def clone(self) -> "Cache":
        """A second cache with copies of every tensor (same geometry)."""
        c = Cache.__new__(Cache)
        c.__dict__.update(self.__dict__)
        for name in ("k", "v", "k_scale", "v_scale", "kmin", "kmax"):
            t = getattr(self, name)
            setattr(c, name, None if t is None else t.clone())
        c.desc = SkvCacheDesc(self.batch, self.n_kv_heads, self.head_dim, self.max_seq,
                              self.block, self.desc.kv_dtype, _ptr(c.k), _ptr(c.v),
                              _ptr(c.k_scale), _ptr(c.v_scale), _ptr(c.kmin), _ptr(c.kmax))
        return c


def kv_append(cache: Cache, pos0, k_new, v_new, stream=None):
    """Append n_new tokens per sequence: k_new, v_new [batch][n_new][Hkv][D]
    (float16 for an f16 cache, float32 for an int8 cache); pos0 int32 [batch]."""
    import torch
    call = "skv_kv_append"
    _check_rows(call, cache, k_new, v_new)
    _need(call, _is(pos0, torch.int32, (cache.batch,)), "pos0 must be int32 [batch]")
    n_new = int(k_new.shape[1])
    _check(call, load().skv_kv_append(
        ctypes.byref(cache.desc), _ptr(pos0), n_new, _ptr(k_new), _ptr(v_new),
        _dtype_code(k_new), _stream(stream)))


def block_bounds(cache: Cache, q, seq_len, max_len: int, score, stream=None):
    """score [batch][Hkv][max_blocks] <- group-max Quest bound of every block."""
    import torch
    _check_q("skv_block_bounds", cache, q, seq_len)
    _need("skv_block_bounds", _is(score, torch.float32,
                                  (cache.batch, cache.n_kv_heads, cache.max_blocks)),
          "score must be float32 [batch][n_kv_heads][max_blocks]")
    _check("skv_block_bounds", load().skv_block_bounds(
        ctypes.byref(cache.desc), _ptr(q), int(q.shape[1]), _ptr(seq_len), int(max_len),
        _ptr(score), _stream(stream)))


def select_topk(score, seq_len, block: int, k_sel, n_sink: int, n_recent: int,
                sel_idx, sel_cnt, sel_mask=None, stream=None):
    """Fixed top-K + sink + recent; sel_idx [batch][Hkv][max_sel] int32 ascending."""
    import torch
    call = "skv_select_topk"
    _need(call, _is(score, torch.float32, (None, None, None)),
          "score must be float32 [batch][n_kv_heads][max_blocks]")
    B, Hkv, max_blocks = (int(x) for x in score.shape)
    _need(call, _is(seq_len, torch.int32, (B,)), "seq_len must be int32 [batch]")
    _need(call, _is(k_sel, torch.int32, (B,)), "k_sel must be int32 [batch]")
    _need(call, sel_idx is not None, "sel_idx and sel_cnt are required")
    _check_sel(call, B, Hkv, sel_idx, sel_cnt)
    if sel_mask is not None:
        _need(call, sel_mask.dtype in (torch.int32, getattr(torch, "uint32", torch.int32))
              and _is(sel_mask, sel_mask.dtype, (B, Hkv, -(-max_blocks // 32))),
              "sel_mask must be 32-bit [batch][n_kv_heads][ceil(max_blocks/32)]")
    _check("skv_select_topk", load().skv_select_topk(
        _ptr(score), _ptr(seq_len), B, Hkv, max_blocks, int(block), _ptr(k_sel), int(n_sink),
        int(n_recent), int(sel_idx.shape[2]), _ptr(sel_idx), _ptr(sel_cnt), _ptr(sel_mask),
        _stream(stream)))


def decode_attn(cache: Cache, q, seq_len, max_len: int, softmax_scale: float, n_split: int,
                workspace, sel_idx=None, sel_cnt=None, dbg_logits=None, stream=None):
    """Split-K partial states into ``workspace`` (uint8/float tensor of at least
    workspace_bytes(...) bytes)."""
    import torch
    call = "skv_decode_attn"
    _check_q(call, cache, q, seq_len)
    _check_sel(call, cache.batch, cache.n_kv_heads, sel_idx, sel_cnt)
    if dbg_logits is not None:
        _need(call, _is(dbg_logits, torch.int32, (cache.batch, int(q.shape[1]), None))
              and int(dbg_logits.shape[2]) >= int(max_len),
              "dbg_logits must be int32 [batch][n_heads][>= max_len]")
    max_sel = int(sel_idx.shape[2]) if sel_idx is not None else 0
    _check(call, load().skv_decode_attn(
        ctypes.byref(cache.desc), _ptr(q), int(q.shape[1]), _ptr(seq_len), int(max_len),
        _ptr(sel_idx), _ptr(sel_cnt), max_sel, float(softmax_scale), int(n_split),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(dbg_logits),
        _stream(stream)))


def decode_attn_select(cache: Cache, q, seq_len, max_len: int, softmax_scale: float,
                       n_split: int, workspace, score, k_sel, n_sink: int, n_recent: int,
                       sel_idx, sel_cnt, stream=None):
    """select_topk + decode_attn in one launch (the selection in the attention
    kernel's prologue): sel_idx/sel_cnt receive the list, ``workspace`` the
    split-K partial states."""
    import torch
    call = "skv_decode_attn_select"
    _check_q(call, cache, q, seq_len)
    _need(call, _is(k_sel, torch.int32, (cache.batch,)), "k_sel must be int32 [batch]")
    _need(call, _is(score, torch.float32, (cache.batch, cache.n_kv_heads, cache.max_blocks)),
          "score must be float32 [batch][n_kv_heads][max_blocks]")
    _need(call, sel_idx is not None, "sel_idx and sel_cnt are required")
    _check_sel(call, cache.batch, cache.n_kv_heads, sel_idx, sel_cnt)
    _check(call, load().skv_decode_attn_select(
        ctypes.byref(cache.desc), _ptr(q), int(q.shape[1]), _ptr(seq_len), int(max_len),
        _ptr(score), _ptr(k_sel), int(n_sink), int(n_recent), int(sel_idx.shape[2]),
        _ptr(sel_idx), _ptr(sel_cnt), float(softmax_scale), int(n_split), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_step(cache: Cache, q, seq_len, max_len: int, softmax_scale: float, n_split: int,
                workspace, out, pos0=None, k_new=None, v_new=None, k_sel=None, n_sink: int = 1,
                n_recent: int = 2, score=None, sel_idx=None, sel_cnt=None, stream=None):
    """One decode step in three launches, two when dense (skv_decode_step): optional one-token
    append (k_new, v_new [batch][1][Hkv][D] at pos0), dense or Quest (k_sel)
    attention, combine into ``out``.  Quest needs score [batch][Hkv][max_blocks]
    scratch and sel_idx [batch][Hkv][max_sel] / sel_cnt [batch][Hkv] outputs."""
    import torch
    call = "skv_decode_step"
    _check_q(call, cache, q, seq_len)
    _need(call, _is(out, torch.float32, tuple(q.shape)), "out must be float32 like q")
    src = 0
    if k_new is not None:
        _check_rows(call, cache, k_new, v_new, 1)
        _need(call, _is(pos0, torch.int32, (cache.batch,)), "pos0 must be int32 [batch]")
        src = _dtype_code(k_new)
    if k_sel is not None:
        _need(call, _is(k_sel, torch.int32, (cache.batch,)), "k_sel must be int32 [batch]")
        _need(call, _is(score, torch.float32, (cache.batch, cache.n_kv_heads, cache.max_blocks)),
              "score must be float32 [batch][n_kv_heads][max_blocks]")
        _need(call, sel_idx is not None, "sel_idx and sel_cnt are required for Quest")
        _check_sel(call, cache.batch, cache.n_kv_heads, sel_idx, sel_cnt)
    max_sel = int(sel_idx.shape[2]) if sel_idx is not None else 0
    _check(call, load().skv_decode_step(
        ctypes.byref(cache.desc), _ptr(pos0), _ptr(k_new), _ptr(v_new), src,
        _ptr(q), int(q.shape[1]), _ptr(seq_len), int(max_len), _ptr(k_sel), int(n_sink),
        int(n_recent), max_sel, _ptr(score), _ptr(sel_idx), _ptr(sel_cnt),
        float(softmax_scale), int(n_split), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))


def block_bounds_heads(cache: Cache, q, seq_len, max_len: int, score, stream=None):
    """score [batch][H][max_blocks] <- each query head's own Quest bound."""
    import torch
    call = "skv_block_bounds_heads"
    _check_q(call, cache, q, seq_len)
    _need(call, _is(score, torch.float32, (cache.batch, int(q.shape[1]), cache.max_blocks)),
          "score must be float32 [batch][n_heads][max_blocks]")
    _check(call, load().skv_block_bounds_heads(
        ctypes.byref(cache.desc), _ptr(q), int(q.shape[1]), _ptr(seq_len), int(max_len),
        _ptr(score), _stream(stream)))


def select_union(sel_idx, sel_cnt, n_kv_heads: int, max_blocks: int, uni_idx, uni_cnt,
                 uni_mask, stream=None):
    """Per KV head, the ascending union of its query heads' lists
    (sel_idx [batch][H][max_sel]) with a head bit mask per block."""
    import torch
    call = "skv_select_union"
    _need(call, _is(sel_idx, torch.int32, (None, None, None)), "sel_idx must be int32 3-D")
    B, H, max_sel = (int(x) for x in sel_idx.shape)
    _need(call, _is(sel_cnt, torch.int32, (B, H)), "sel_cnt must be int32 [batch][n_heads]")
    _need(call, _is(uni_idx, torch.int32, (B, n_kv_heads, None)),
          "uni_idx must be int32 [batch][n_kv_heads][max_union]")
    max_union = int(uni_idx.shape[2])
    _need(call, _is(uni_cnt, torch.int32, (B, n_kv_heads)), "uni_cnt must be int32 [batch][Hkv]")
    _need(call, _is(uni_mask, uni_mask.dtype, (B, n_kv_heads, max_union))
          and uni_mask.element_size() == 4, "uni_mask must be 32-bit like uni_idx")
    _check(call, load().skv_select_union(
        _ptr(sel_idx), _ptr(sel_cnt), B, H, int(n_kv_heads), max_sel, int(max_blocks), max_union,
        _ptr(uni_idx), _ptr(uni_cnt), _ptr(uni_mask), _stream(stream)))


def decode_attn_heads(cache: Cache, q, seq_len, max_len: int, softmax_scale: float,
                      n_split: int, workspace, uni_idx, uni_cnt, uni_mask, stream=None):
    """Split-K partial states with each query head over its own blocks (the
    union list with head masks from select_union)."""
    call = "skv_decode_attn_heads"
    _check_q(call, cache, q, seq_len)
    _check_sel(call, cache.batch, cache.n_kv_heads, uni_idx, uni_cnt)
    _need(call, uni_mask is not None and tuple(uni_mask.shape) == tuple(uni_idx.shape)
          and uni_mask.element_size() == 4, "uni_mask must be 32-bit like uni_idx")
    _check(call, load().skv_decode_attn_heads(
        ctypes.byref(cache.desc), _ptr(q), int(q.shape[1]), _ptr(seq_len), int(max_len),
        _ptr(uni_idx), _ptr(uni_cnt), _ptr(uni_mask), int(uni_idx.shape[2]),
        float(softmax_scale), int(n_split), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


# ----------------------------------------------------------- token chunks
def _check_qt(call: str, cache, q, seq_len):
    """q float32 [batch][T][n_heads][head_dim], seq_len int32 [batch]."""
    import torch
    _need(call, q is not None and _is(q, torch.float32, (cache.batch, None, None, cache.head_dim)),
          "q must be float32 [batch][n_tokens][n_heads][head_dim]")
    _need(call, _is(seq_len, torch.int32, (cache.batch,)), "seq_len must be int32 [batch]")
    return int(q.shape[1]), int(q.shape[2])


def block_bounds_multi(cache: Cache, q, seq_len, max_len: int, score, stream=None):
    """score [batch][Hkv][T][max_blocks] <- each chunk token's group-max bound."""
    import torch
    call = "skv_block_bounds_multi"
    T, H = _check_qt(call, cache, q, seq_len)
    _need(call, _is(score, torch.float32, (cache.batch, cache.n_kv_heads, T, cache.max_blocks)),
          "score must be float32 [batch][n_kv_heads][n_tokens][max_blocks]")
    _check(call, load().skv_block_bounds_multi(
        ctypes.byref(cache.desc), _ptr(q), T, H, _ptr(seq_len), int(max_len), _ptr(score),
        _stream(stream)))


def select_topk_multi(score, seq_len, block: int, k_sel, n_sink: int, n_recent: int,
                      sel_idx, sel_cnt, stream=None):
    """Each chunk token's top-K (score [batch][Hkv][T][max_blocks]) into
    sel_idx [batch][Hkv][T][max_sel], sel_cnt [batch][Hkv][T]."""
    import torch
    call = "skv_select_topk_multi"
    _need(call, _is(score, torch.float32, (None, None, None, None)), "score must be float32 4-D")
    B, Hkv, T, max_blocks = (int(x) for x in score.shape)
    _need(call, _is(seq_len, torch.int32, (B,)) and _is(k_sel, torch.int32, (B,)),
          "seq_len and k_sel must be int32 [batch]")
    _need(call, _is(sel_idx, torch.int32, (B, Hkv, T, None)),
          "sel_idx must be int32 [batch][n_kv_heads][n_tokens][max_sel]")
    _need(call, _is(sel_cnt, torch.int32, (B, Hkv, T)),
          "sel_cnt must be int32 [batch][n_kv_heads][n_tokens]")
    _check(call, load().skv_select_topk_multi(
        _ptr(score), _ptr(seq_len), B, T, Hkv, max_blocks, int(block), _ptr(k_sel), int(n_sink),
        int(n_recent), int(sel_idx.shape[3]), _ptr(sel_idx), _ptr(sel_cnt), _stream(stream)))


def select_union_tokens(sel_idx, sel_cnt, group: int, max_blocks: int, uni_idx, uni_cnt,
                        uni_mask, stream=None):
    """Per KV head, the ascending union of its chunk tokens' lists, token t's
    blocks tagged with bits [t * group, (t + 1) * group)."""
    import torch
    call = "skv_select_union_tokens"
    _need(call, _is(sel_idx, torch.int32, (None, None, None, None)), "sel_idx must be int32 4-D")
    B, Hkv, T, max_sel = (int(x) for x in sel_idx.shape)
    _need(call, _is(sel_cnt, torch.int32, (B, Hkv, T)),
          "sel_cnt must be int32 [batch][n_kv_heads][n_tokens]")
    _need(call, _is(uni_idx, torch.int32, (B, Hkv, None)),
          "uni_idx must be int32 [batch][n_kv_heads][max_union]")
    max_union = int(uni_idx.shape[2])
    _need(call, _is(uni_cnt, torch.int32, (B, Hkv)), "uni_cnt must be int32 [batch][Hkv]")
    _need(call, _is(uni_mask, uni_mask.dtype, (B, Hkv, max_union))
          and uni_mask.element_size() == 4, "uni_mask must be 32-bit like uni_idx")
    _check(call, load().skv_select_union_tokens(
        _ptr(sel_idx), _ptr(sel_cnt), B, T, Hkv, int(group), max_sel, int(max_blocks),
        max_union, _ptr(uni_idx), _ptr(uni_cnt), _ptr(uni_mask), _stream(stream)))


def decode_attn_multi(cache: Cache, q, seq_len, max_len: int, softmax_scale: float,
                      n_split: int, workspace, uni_idx=None, uni_cnt=None, uni_mask=None,
                      stream=None):
    """Split-K partial states of a chunk of query tokens (q [batch][T][H][D]),
    each token causal over its prefix, densely (no lists) or over its own
    blocks (the union list with token masks from select_union_tokens).
    combine(workspace, batch, T * H, D, n_split, out) then gives
    out [batch][T][H][D]."""
    call = "skv_decode_attn_multi"
    T, H = _check_qt(call, cache, q, seq_len)
    _check_sel(call, cache.batch, cache.n_kv_heads, uni_idx, uni_cnt)
    _need(call, (uni_mask is None) == (uni_idx is None), "uni_mask goes with uni_idx")
    if uni_mask is not None:
        _need(call, tuple(uni_mask.shape) == tuple(uni_idx.shape)
              and uni_mask.element_size() == 4, "uni_mask must be 32-bit like uni_idx")
    _check(call, load().skv_decode_attn_multi(
        ctypes.byref(cache.desc), _ptr(q), T, H, _ptr(seq_len), int(max_len), _ptr(uni_idx),
        _ptr(uni_cnt), _ptr(uni_mask), int(uni_idx.shape[2]) if uni_idx is not None else 0,
        float(softmax_scale), int(n_split), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


class Scan4Index:
    """The 4-bit key index of an f16 cache: codes4 uint8
    [batch][n_kv_heads][max_seq][head_dim / 2], lo / step / err float32
    [batch][n_kv_heads][max_blocks][head_dim]."""

    def __init__(self, cache: Cache, device="cuda"):
        import torch
        B, Hkv, D = cache.batch, cache.n_kv_heads, cache.head_dim
        self.codes4 = torch.zeros((B, Hkv, cache.max_seq, D // 2), dtype=torch.uint8,
                                  device=device)
        shape = (B, Hkv, cache.max_blocks, D)
        self.lo = torch.zeros(shape, dtype=torch.float32, device=device)
        self.step = torch.zeros(shape, dtype=torch.float32, device=device)
        self.err = torch.zeros(shape, dtype=torch.float32, device=device)


def scan4_build(cache: Cache, index: Scan4Index, pos0, seq_len, max_len: int, stream=None):
    """(Re)build the index blocks from the one holding pos0[b] to the end of
    sequence b."""
    import torch
    call = "skv_scan4_build"
    _need(call, _is(pos0, torch.int32, (cache.batch,)), "pos0 must be int32 [batch]")
    _need(call, _is(seq_len, torch.int32, (cache.batch,)), "seq_len must be int32 [batch]")
    _check(call, load().skv_scan4_build(
        ctypes.byref(cache.desc), _ptr(pos0), _ptr(seq_len), int(max_len), _ptr(index.codes4),
        _ptr(index.lo), _ptr(index.step), _ptr(index.err), _stream(stream)))


def scan4_workspace_bytes(batch: int, n_heads: int, n_split: int, max_len: int) -> int:
    return int(load().skv_scan4_workspace_bytes(batch, n_heads, n_split, max_len))


def scan4_candidates(cache: Cache, index: Scan4Index, q, seq_len, max_len: int, delta: float,
                     n_split: int, workspace, cand, cand_cnt, stream=None):
    """Per query head, the tokens whose exact q.k could be within delta of the
    largest (cand: 32-bit [batch][H][ceil(max_len/32)], cand_cnt: int32
    [batch][H]); workspace then holds UB [batch][H][max_len] first."""
    import torch
    call = "skv_scan4_candidates"
    _check_q(call, cache, q, seq_len)
    H = int(q.shape[1])
    _need(call, _is(cand, cand.dtype, (cache.batch, H, -(-int(max_len) // 32)))
          and cand.element_size() == 4, "cand must be 32-bit [batch][H][ceil(max_len/32)]")
    _need(call, _is(cand_cnt, torch.int32, (cache.batch, H)), "cand_cnt must be int32 [batch][H]")
    _check(call, load().skv_scan4_candidates(
        ctypes.byref(cache.desc), _ptr(index.codes4), _ptr(index.lo), _ptr(index.step),
        _ptr(index.err), _ptr(q), H, _ptr(seq_len), int(max_len), float(delta), int(n_split),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(cand),
        _ptr(cand_cnt), _stream(stream)))


def sparse_v_workspace_bytes(batch: int, n_heads: int, n_kv_heads: int, head_dim: int,
                             n_split: int, max_len: int) -> int:
    return int(load().skv_sparse_v_workspace_bytes(batch, n_heads, n_kv_heads, head_dim,
                                                   n_split, max_len))


def decode_attn_sparse_v(cache: Cache, q, seq_len, max_len: int, softmax_scale: float,
                         n_split: int, workspace, tau: float = 0.0, eps: float = 0.0,
                         sel_idx=None, sel_cnt=None, keep_mask=None, stream=None):
    """Split-K partial states with sparse-V (value rows of normalized weight
    below tau, or below eps / n, left out) into ``workspace`` (at least
    sparse_v_workspace_bytes(...) bytes); combine() then gives the output.
    keep_mask: optional zeroed int32 [batch][n_heads][ceil(max_len/32)]
    receiving the kept-row bits."""
    import torch
    call = "skv_decode_attn_sparse_v"
    _check_q(call, cache, q, seq_len)
    _check_sel(call, cache.batch, cache.n_kv_heads, sel_idx, sel_cnt)
    if keep_mask is not None:
        _need(call, _is(keep_mask, keep_mask.dtype, (cache.batch, int(q.shape[1]),
                                                     -(-int(max_len) // 32)))
              and keep_mask.element_size() == 4, "keep_mask must be 32-bit "
              "[batch][n_heads][ceil(max_len/32)]")
    max_sel = int(sel_idx.shape[2]) if sel_idx is not None else 0
    _check(call, load().skv_decode_attn_sparse_v(
        ctypes.byref(cache.desc), _ptr(q), int(q.shape[1]), _ptr(seq_len), int(max_len),
        _ptr(sel_idx), _ptr(sel_cnt), max_sel, float(softmax_scale), float(tau), float(eps),
        int(n_split), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(keep_mask), _stream(stream)))


def decode_step_static(cache: Cache, q, seq_len, max_len: int, softmax_scale: float,
                       n_split: int, out, pos0=None, k_new=None, v_new=None, k_sel=None,
                       n_sink: int = 1, n_recent: int = 2, sel_idx=None, sel_cnt=None,
                       stream=None):
    """decode_step with its scratch (scores, split-K partials) in the library's
    fixed per-GPU array (skv_decode_step_static): allocates nothing.  Calls that
    overlap on one GPU race on that array."""
    import torch
    call = "skv_decode_step_static"
    _check_q(call, cache, q, seq_len)
    _need(call, _is(out, torch.float32, tuple(q.shape)), "out must be float32 like q")
    src = 0
    if k_new is not None:
        _check_rows(call, cache, k_new, v_new, 1)
        _need(call, _is(pos0, torch.int32, (cache.batch,)), "pos0 must be int32 [batch]")
        src = _dtype_code(k_new)
    if k_sel is not None:
        _need(call, _is(k_sel, torch.int32, (cache.batch,)), "k_sel must be int32 [batch]")
        _need(call, sel_idx is not None, "sel_idx and sel_cnt are required for Quest")
        _check_sel(call, cache.batch, cache.n_kv_heads, sel_idx, sel_cnt)
    max_sel = int(sel_idx.shape[2]) if sel_idx is not None else 0
    _check(call, load().skv_decode_step_static(
        ctypes.byref(cache.desc), _ptr(pos0), _ptr(k_new), _ptr(v_new), src,
        _ptr(q), int(q.shape[1]), _ptr(seq_len), int(max_len), _ptr(k_sel), int(n_sink),
        int(n_recent), max_sel, _ptr(sel_idx), _ptr(sel_cnt), float(softmax_scale),
        int(n_split), _ptr(out), _stream(stream)))


def static_scratch_bytes() -> int:
    return int(load().skv_static_scratch_bytes())


def combine(workspace, batch: int, n_heads: int, head_dim: int, n_split: int, out, stream=None):
    """out [batch][n_heads][head_dim] float32 from the split-K partials."""
    import torch
    _need("skv_combine", _is(out, torch.float32, (batch, n_heads, head_dim)),
          "out must be float32 [batch][n_heads][head_dim]")
    _check("skv_combine", load().skv_combine(
        _ptr(workspace), int(batch), int(n_heads), int(head_dim), int(n_split), _ptr(out),
        _stream(stream)))


def default_split(batch: int, n_kv_heads: int, n_units: int, target_wgs: Optional[int] = None,
                  kv_dtype: str = "f16", sparse: bool = False) -> int:
    """Parts per (sequence, KV head) so the grid has about ``target_wgs``
    workgroups, at least one block (or selected entry) per part.  Default:
    one workgroup per compute unit, or two for dense decode over an int8
    cache while every part still gets at least 4 blocks: its tiles cost more
    arithmetic per byte and gain from a second workgroup hiding the first
    one's loads (262K context, 4 KV heads: 128 parts of 32 blocks), but short
    parts are dominated by their fixed cost (8K context, 8 KV heads: the step
    takes 12.1 us with 64 parts of 2 blocks, 11.5 us with 32 parts of 4).
    Sparse decode keeps one: every part of a row also runs the block
    selection.  Dense q4_0 takes two as well (32K context, 8 KV heads: 16.9 us
    at 64 parts against 18.6 us at 32); dense q8_0 keeps one (19.6 against
    18.9 us)."""
    if target_wgs is None:
        target_wgs = 256
        two = math.ceil(512 / max(1, batch * n_kv_heads))
        if kv_dtype in ("i8", "q4_0", "q5_0") and not sparse and n_units >= 4 * two:
            target_wgs = 512
    n = max(1, math.ceil(target_wgs / max(1, batch * n_kv_heads)))
    return int(max(1, min(n, n_units, 4096)))


def scan4_default_split(batch: int, n_kv_heads: int, n_blocks: int) -> int:
    """Parts per (sequence, KV head) for scan4_candidates: two workgroups per
    compute unit while every part keeps at least 4 blocks.  A scan tile
    carries the bound arithmetic of all G heads of its KV head, so a second
    workgroup per compute unit hides the first one's loads (32K context, 8
    KV heads, warm cache: 16.0 us at 64 parts against 17.6 us at 32)."""
    two = math.ceil(512 / max(1, batch * n_kv_heads))
    target = 512 if n_blocks >= 4 * two else 256
    return default_split(batch, n_kv_heads, n_blocks, target_wgs=target)


def decode(cache: Cache, q, seq_len, max_len: int, softmax_scale: Optional[float] = None,
           k_sel=None, n_sink: int = 1, n_recent: int = 2, max_sel: Optional[int] = None,
           n_split: Optional[int] = None, stream=None):
    """One decode step: dense (k_sel None) or Quest (k_sel int32 [batch]).
    Returns out [batch][H][D] float32.  Allocates its scratch tensors."""
    import torch
    B, H, D = (int(x) for x in q.shape)
    dev = q.device
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale
    sel_idx = sel_cnt = None
    nb_max = -(-max_len // cache.block)
    if k_sel is not None:
        if max_sel is None:
            max_sel = int(k_sel.max().item()) + n_sink + n_recent
        max_sel = max(1, min(max_sel, nb_max if nb_max > 0 else 1))
        score = torch.empty((B, cache.n_kv_heads, cache.max_blocks), dtype=torch.float32, device=dev)
        sel_idx = torch.empty((B, cache.n_kv_heads, max_sel), dtype=torch.int32, device=dev)
        sel_cnt = torch.empty((B, cache.n_kv_heads), dtype=torch.int32, device=dev)
        block_bounds(cache, q, seq_len, max_len, score, stream)
        select_topk(score, seq_len, cache.block, k_sel, n_sink, n_recent, sel_idx, sel_cnt,
                    stream=stream)
    units = max_sel if k_sel is not None else max(nb_max, 1)
    S = n_split or default_split(B, cache.n_kv_heads, units, kv_dtype=cache.kv_dtype,
                                 sparse=k_sel is not None)
    ws = torch.empty(workspace_bytes(B, H, D, S), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    decode_attn(cache, q, seq_len, max_len, scale, S, ws, sel_idx, sel_cnt, stream=stream)
    combine(ws, B, H, D, S, out, stream)
    return out
