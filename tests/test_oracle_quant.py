"""Pins for oracle.quant: absmax int8 invariants and directed f16 rounding."""
import numpy as np
import pytest

import oracle


def test_absmax_element_maps_to_127_and_error_within_half_step():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((500, 128)) * rng.uniform(1e-3, 50, (500, 1))).astype(np.float32)
    codes, scale = oracle.quantize_rows(x)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    assert np.all(np.max(np.abs(codes.astype(int)), axis=1) == 127)
    err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * scale.astype(np.float64)[:, None])
    # rint error <= 0.5 code step, plus the float32 rounding of x/scale at |code| <= 127
    assert np.all(err <= scale.astype(np.float64)[:, None] * (0.5 + 2.0 ** -17))


def test_scale_is_float32_division_of_absmax_by_127():
    x = np.array([[0.5, -2.0, 1.0, 0.0]], np.float32)
    codes, scale = oracle.quantize_rows(x)
    assert scale[0] == np.float32(2.0) / np.float32(127)
    # 0.5/scale = 31.75 -> 32 ; -2/scale -> -127 ; 1/scale = 63.5 -> 64 (half to even) ; 0 -> 0
    assert codes.tolist() == [[32, -127, 64, 0]]


def test_round_half_to_even():
    # absmax 127 gives scale 1.0 exactly, so codes are rint(x)
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, 3.49999]], np.float32)
    codes, scale = oracle.quantize_rows(x)
    assert scale[0] == 1.0
    assert codes.tolist() == [[127, 0, 2, 2, 0, -2, 3]]


def test_zero_row_gives_zero_scale_and_codes():
    codes, scale = oracle.quantize_rows(np.zeros((3, 16), np.float32))
    assert np.all(codes == 0) and np.all(scale == 0)


def test_subnormal_scale_row_follows_ieee():
    # absmax 1e-37: a/127 is a float32 subnormal; no flush to zero
    x = np.array([[1e-37, -5e-38, 2.5e-38, 0.0]], np.float32)
    codes, scale = oracle.quantize_rows(x)
    assert 0 < scale[0] < np.finfo(np.float32).tiny
    assert codes[0, 0] == 127


def test_requantizing_the_dequantized_row_is_idempotent():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((200, 64)).astype(np.float32)
    codes, scale = oracle.quantize_rows(x)
    deq = (codes.astype(np.float32) * scale[:, None]).astype(np.float32)
    codes2, scale2 = oracle.quantize_rows(deq)
    assert np.array_equal(codes, codes2)


@pytest.mark.parametrize("fn,side", [(oracle.f16_round_down, -1), (oracle.f16_round_up, 1)])
def test_directed_f16_rounding_is_sound_and_tightest(fn, side):
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10,
                        np.float32([0.0, -0.0, 1.0, 65504.0, 65519.0, 65520.0, 70000.0,
                                    -70000.0, 6e-8, -6e-8, 1e-9, 2049.0, -2049.0])]).astype(np.float32)
    r = fn(x)
    assert r.dtype == np.float16
    r32 = r.astype(np.float32)
    if side < 0:
        assert np.all(r32 <= x)
        nxt = np.nextafter(r, np.float16(np.inf)).astype(np.float32)
        assert np.all(nxt > x)          # the next f16 inward already violates it
    else:
        assert np.all(r32 >= x)
        nxt = np.nextafter(r, np.float16(-np.inf)).astype(np.float32)
        assert np.all(nxt < x)
    exact = x.astype(np.float16).astype(np.float32) == x
    assert np.array_equal(r32[exact], x[exact])      # exactly representable values stay
