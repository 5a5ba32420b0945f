"""MXFP8 quantisation of bf16 values: E4M3 elements with one E8M0 scale per 32.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may use this module; the product path never
does.  Plain numpy, brute force, for small inputs.

What it computes (vLLM MiniMax-M3 page, MiniMaxM3SparseRocmNvfp4Impl,
forward_decode_mxfp8): a decode output emitted as E4M3 values
``[tokens, H*D]`` with row-major E8M0 scales ``[tokens, H*D/32]``, equal to
the MXFP8 E4M3 quantisation of the bf16 output.  The page does not spell
the quantisation out; this follows the OCP Microscaling format:

- elements are grouped in blocks of 32 consecutive values along a row;
- a block's scale is the power of two 2**s with s = floor(log2(amax)) - 8,
  amax the largest magnitude in the block and 8 the exponent of the largest
  power of two that E4M3 represents (256); s is clamped to E8M0's range
  [-127, 127] and stored as the byte s + 127; an all-zero block takes code 0;
- each element x is replaced by the E4M3FN value nearest to x / 2**s (ties
  to the even code, i.e. the even mantissa), among the finite values, so
  magnitudes past 448 saturate to 448; the sign bit of x is kept.
"""
from __future__ import annotations

import numpy as np

E8M0_BIAS = 127
ELEM_EMAX = 8  # exponent of the largest power of two in E4M3 (2**8 = 256)
BLOCK = 32


def e4m3fn_value(code) -> np.ndarray:
    """fp64 value of E4M3FN bytes (sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal m * 2**-9; S.1111.111 is NaN; no infinities)."""
    code = np.asarray(code, dtype=np.int64)
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((code & 0x7F) == 0x7F, np.nan, val)


_POS_CODES = np.arange(0x7F, dtype=np.int64)  # 0x00..0x7E: every finite non-negative value
_POS_VALUES = e4m3fn_value(_POS_CODES)


def e4m3_nearest(y: np.ndarray) -> np.ndarray:
    """E4M3FN code of the finite value nearest to each |y| (ties to the even
    code), with the sign bit of y.  y must be exactly representable in fp64."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y).reshape(-1, 1)
    dist = np.abs(a - _POS_VALUES.reshape(1, -1))
    best = dist.min(axis=1, keepdims=True)
    tied = dist == best
    # among the nearest codes prefer an even one (at most two are tied, and
    # two neighbours always differ in their last bit)
    even = tied & ((_POS_CODES.reshape(1, -1) & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), tied.argmax(axis=1))
    codes = _POS_CODES[pick].reshape(y.shape)
    return np.where(np.signbit(y), codes | 0x80, codes).astype(np.uint8)


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Block scale exponent s (int) for block maxima amax >= 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, k = np.frexp(amax)  # amax = f * 2**k with f in [0.5, 1)  ->  floor(log2 amax) = k - 1
    s = np.where(amax > 0, k - 1 - ELEM_EMAX, -E8M0_BIAS)
    return np.clip(s, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize(x: np.ndarray):
    """MXFP8 of a [rows, cols] array of bf16-representable values (cols % 32 == 0).

    Returns (q uint8 [rows, cols] E4M3FN codes, scale uint8 [rows, cols/32]
    E8M0 codes)."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    blocks = x.reshape(rows, cols // BLOCK, BLOCK)
    s = scale_exponent(np.abs(blocks).max(axis=2))
    y = blocks * np.exp2(-s.astype(np.float64))[..., None]  # exact: a power-of-two shift
    q = e4m3_nearest(y).reshape(rows, cols)
    return q, (s + E8M0_BIAS).astype(np.uint8)


def dequantize(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp64 values of MXFP8 data (inverse of the encoding up to rounding)."""
    rows, cols = q.shape
    v = e4m3fn_value(q).reshape(rows, cols // BLOCK, BLOCK)
    return (v * np.exp2(scale.astype(np.float64) - E8M0_BIAS)[..., None]).reshape(rows, cols)
