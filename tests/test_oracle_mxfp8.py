"""Pins for the MXFP8 oracle (oracle/mxfp8.py): E4M3FN decoding and rounding
against torch's float8_e4m3fn, block scales and saturation in closed form.

Each pin targets a plausible mistake: a wrong exponent bias or scale offset,
round-half-away instead of half-even, no saturation, lost subnormals or signs.
"""
import numpy as np
import pytest
import torch

from oracle import mxfp8 as mx


def torch_e4m3_value(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decoding_matches_torch_for_every_code():
    codes = np.arange(256)
    ours, ref = mx.e4m3fn_value(codes), torch_e4m3_value(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # a few landmarks of the format: max 448, min normal 2^-6, min subnormal 2^-9, 256 = 0x78
    assert mx.e4m3fn_value(0x7E) == 448 and mx.e4m3fn_value(0x08) == 2.0 ** -6
    assert mx.e4m3fn_value(0x01) == 2.0 ** -9 and mx.e4m3fn_value(0x78) == 256


def test_nearest_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(mx.e4m3_nearest(mx.e4m3fn_value(codes)), codes)


def test_nearest_ties_go_to_even_like_torch():
    # midpoints between consecutive finite magnitudes (all exact in fp32)
    v = mx.e4m3fn_value(np.arange(0x7F))
    mids = np.concatenate([(v[:-1] + v[1:]) / 2, -(v[:-1] + v[1:]) / 2])
    ref = torch.from_numpy(mids.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mx.e4m3_nearest(mids), ref)
    assert mx.e4m3_nearest(np.array([1.0625]))[0] == 0x38  # between 1.0 (0x38) and 1.125 (0x39)
    assert mx.e4m3_nearest(np.array([1.1875]))[0] == 0x3A  # between 1.125 and 1.25 (0x3A)


def test_nearest_saturates_past_448():
    y = np.array([449.0, 464.0, 480.0, 510.0, -500.0])
    assert list(mx.e4m3_nearest(y)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


@pytest.mark.parametrize("k", [-133, -126, -20, -1, 0, 1, 7, 8, 9, 40, 127])
def test_scale_exponent_closed_form(k):
    for f in (1.0, 1.5, 1.9921875):  # floor(log2(f * 2^k)) = k for f in [1, 2)
        assert mx.scale_exponent(np.array([f * 2.0 ** k]))[0] == max(k - 8, -127)


def test_zero_block_takes_code_zero():
    q, s = mx.quantize(np.zeros((1, 64)))
    assert np.all(q == 0) and np.all(s == 0)


@pytest.mark.parametrize("k", [-100, -7, 0, 3, 60])
def test_power_of_two_block(k):
    q, s = mx.quantize(np.full((2, 32), 2.0 ** k))
    assert np.all(s == 127 + k - 8) and np.all(q == 0x78)  # 2^k / 2^(k-8) = 256


@pytest.mark.parametrize("s_exp", [-20, 0, 11])
def test_block_of_every_code_round_trips(s_exp):
    # a block whose max is 448 * 2^s has scale 2^s (floor(log2 448) = 8), so
    # every E4M3 value times 2^s is represented exactly
    pos = np.array([c for c in range(0x7F)], dtype=np.int64)
    vals = mx.e4m3fn_value(pos)
    allv = np.concatenate([vals, -vals[1:]])  # every finite value but -0
    nblk = -(-len(allv) // 31)
    allv = np.concatenate([allv, np.zeros(nblk * 31 - len(allv))]).reshape(nblk, 31)
    x = np.concatenate([allv, np.full((nblk, 1), 448.0)], axis=1) * 2.0 ** s_exp  # 448 in each block
    q, s = mx.quantize(x.reshape(1, -1))
    assert np.all(s == 127 + s_exp)
    back = mx.dequantize(q, s)
    assert np.array_equal(back, x.reshape(1, -1))


def test_dequantized_error_bound_on_random_blocks():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, 256)) * np.exp2(rng.integers(-30, 30, size=(16, 8)).repeat(32, axis=1))
    x = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()  # bf16 inputs
    q, s = mx.quantize(x)
    back = mx.dequantize(q, s)
    unit = np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    y = np.abs(x) / unit
    # half a unit in the last place: 2^-4 relative for normals, 2^-10 * scale for subnormals;
    # past 448 the element saturates
    bound = np.where(y <= 448, np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * unit),
                     np.abs(x) - 448 * unit)
    assert np.all(np.abs(back - x) <= bound * (1 + 1e-12))


def test_signs_are_kept():
    x = np.array([[-1.0, 1.0, -0.0, 0.0] * 8])
    q, _ = mx.quantize(x)
    assert list(q[0, :4]) == [0xF8, 0x78, 0x80, 0x00]  # amax 1 -> scale 2^-8: +-1 -> +-256
