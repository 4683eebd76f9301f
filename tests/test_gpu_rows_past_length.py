"""Rows past a sequence's length never count, however far max_len lies
above it: the dense walk's parts are laid out over max_len, each tile's
buffer resource reads zeros past the length, and the int8 scales of those
rows are clamped to the last valid token.  Every row past the length L is
poisoned here (f16: NaN; int8: code -128 and NaN scales) and the call's
max_len lies above L by a row, a tile, a block or the whole cache, with L
ending inside a part's first tile, its second tile, or past every part but
the first; with many parts, most of them lie wholly past L.  Bars as for the
dense decode: f16 within 1e-3 of the oracle over the first L tokens (per head
and per element), int8 logit dots exact and the output within 1e-4 of the
method; every output finite.  The folded append of the dense step is covered
by the step tests (a new token at L - 1 with max_len above it)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_append_amd as skv
import workloads
from gpu_harness import DEV, assert_close, build_cache, quantized_host

pytestmark = pytest.mark.gpu

CASES = [
    # (L, max_len - L, block, n_split)
    (1, 1, 64, None),
    (5, 200, 16, None),
    (17, 13, 64, 64),
    (40, 960, 64, 8),
    (300, 1, 64, None),
    (1000, 24, 16, 32),
    (2049, 2047, 128, None),
]


def _print(*a):
    print("[dense entry]", *a, flush=True)


def _poison_tail(cache, L):
    if cache.kv_dtype == "f16":
        cache.k[0, :, L:] = float("nan")
        cache.v[0, :, L:] = float("nan")
    else:
        cache.k[0, :, L:] = -128
        cache.v[0, :, L:] = -128
        cache.k_scale[0, :, L:] = float("nan")
        cache.v_scale[0, :, L:] = float("nan")
    torch.cuda.synchronize()


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("kv", ["f16", "i8"])
@pytest.mark.parametrize("L,extra,block,S", CASES)
def test_rows_past_the_length_never_count(gpu_lib, D, kv, L, extra, block, S):
    _print(D, kv, L, extra, block, S)
    w = workloads.gaussian(1100 + L + D, 1, 32, 8, D, [L], kv, block=block)
    max_len = L + extra
    cache = build_cache(w, max_seq=max_len)
    _poison_tail(cache, L)
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    seq_len = torch.tensor([L], dtype=torch.int32, device=DEV)
    nb = -(-max_len // block)
    S = S or skv.default_split(1, w.Hkv, nb, kv_dtype=kv)
    ws = torch.empty(skv.workspace_bytes(1, w.H, D, S), dtype=torch.uint8, device=DEV)
    out = torch.empty((1, w.H, D), dtype=torch.float32, device=DEV)
    dl = None
    if kv == "i8":
        dl = torch.full((1, w.H, max_len), -2 ** 31, dtype=torch.int32, device=DEV)
    skv.decode_attn(cache, q, seq_len, max_len, w.softmax_scale, S, ws, dbg_logits=dl)
    skv.combine(ws, 1, w.H, D, S, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()[0]
    assert np.all(np.isfinite(o))
    if kv == "f16":
        ref = oracle.attend_f16(w.q[0], w.k[0], w.v[0], w.softmax_scale)
        assert_close(o, ref, 1e-3, D, L, extra)
    else:
        kc, ks, vc, vs = quantized_host(w, 0)
        dots, _, _ = oracle.int8_logit_dots(w.q[0], kc)
        got = dl.cpu().numpy()[0]
        assert np.array_equal(got[:, :L].astype(np.int64), dots)
        assert np.all(got[:, L:] == -2 ** 31)          # nothing written past the length
        ref = oracle.attend_i8(w.q[0], kc, ks, vc, vs, w.softmax_scale)
        assert_close(o, ref, 1e-4, D, L, extra)
