"""MXFP8 (E4M3 elements, one E8M0 scale per 32 elements) quantiser of the oracle.
TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say only that MoK trains in MXFP8 with the format handled inside the
kernel and no separate conversion kernel (sebask.de, "Mixture-of-Kittens: Cursors
Open-Source-Ansatz für effizientes MoE-Training auf NVL72", § Determinismus und
MXFP8-Unterstützung; stamatios.com, "Cursor abre código de megakernel MoE para GPUs
NVL72", § Outras características).  The block rule is therefore taken from the
OCP Microscaling Formats (MX) v1.0 specification, written here from its text:

  * a block is 32 consecutive elements along the contraction axis;
  * shared exponent X = floor(log2(max |v|)) - 8  (8 = exponent of E4M3's largest
    normal, 448 = 1.75 * 2^8), clamped to [-127, 127]; an all-zero block takes
    X = -127; the scale byte is X + 127 (E8M0);
  * each element is v / 2^X converted to E4M3 with round-to-nearest-even and
    saturation to +-448.

E4M3 ("FN" variant: no infinities, one NaN pattern S.1111.111): sign bit, 4
exponent bits with bias 7, 3 mantissa bits; normals (1 + m/8) 2^(E-7) for E >= 1,
subnormals (m/8) 2^-6 for E = 0.  The sign bit of the input is kept, also when
the magnitude rounds to zero.  NaN/Inf inputs are out of scope.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_encode(v) -> np.ndarray:
    """Codes of the values ``v`` (|v| <= 448, finite), round-to-nearest-even."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or not np.all(np.isfinite(a)):
        raise ValueError("e4m3_encode expects finite values within +-448")
    code = np.zeros(v.shape, dtype=np.int64)
    normal = a >= 2.0 ** -6
    # normal range: a = mant * 2^e with mant in [1, 2)
    fr, ex = np.frexp(np.where(normal, a, 1.0))          # a = fr * 2^ex, fr in [0.5, 1)
    e = ex - 1
    mant = fr * 2.0                                        # in [1, 2), exact
    q = np.rint((mant - 1.0) * 8.0).astype(np.int64)       # rint = round half to even
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    code_norm = ((e + 7) << 3) | q
    # subnormal range: multiples of 2^-9; rounding up to 8 * 2^-9 gives the smallest normal
    qs = np.rint(np.where(normal, 0.0, a) / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_norm, qs)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def _e4m3_value(c: np.ndarray) -> np.ndarray:
    """Value of each code from its bit fields (NaN codes give NaN)."""
    c = np.asarray(c, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(E == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(E - 7.0))
    return np.where((E == 15) & (m == 7), np.nan, s * val)


# the 256 code values, looked up by code (the same bit-field rule, evaluated once)
_E4M3_TABLE = _e4m3_value(np.arange(256))


def e4m3_decode(code) -> np.ndarray:
    v = _E4M3_TABLE[np.asarray(code, dtype=np.uint8)]
    if np.isnan(v).any():
        raise ValueError("NaN code")
    return v


def _blocks(a: np.ndarray, axis: int):
    a = np.moveaxis(np.asarray(a, dtype=np.float64), axis, -1)
    n = a.shape[-1]
    if n % BLOCK:
        raise ValueError(f"axis length {n} is not a multiple of {BLOCK}")
    return a.reshape(a.shape[:-1] + (n // BLOCK, BLOCK))


def mx_quantize(a, axis: int = -1):
    """Quantise ``a`` in blocks of 32 along ``axis``.

    Returns (codes uint8 with the shape of ``a``, scales uint8 with ``axis``
    divided by 32), both laid out like ``a`` with ``axis`` in place.
    """
    a = np.asarray(a, dtype=np.float64)
    ax = axis % a.ndim
    b = _blocks(a, ax)
    amax = np.max(np.abs(b), axis=-1)
    fr, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    X = np.where(amax > 0, (ex - 1) - 8, -127)
    X = np.clip(X, -127, 127)
    scaled = b / np.exp2(X.astype(np.float64))[..., None]
    q = e4m3_encode(np.clip(scaled, -E4M3_MAX, E4M3_MAX))
    codes = np.moveaxis(q.reshape(q.shape[:-2] + (-1,)), -1, ax)
    scales = np.moveaxis((X + 127).astype(np.uint8), -1, ax)
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


def mx_dequantize(codes, scales, axis: int = -1) -> np.ndarray:
    codes = np.asarray(codes)
    ax = axis % codes.ndim
    vals = _blocks(e4m3_decode(codes), ax)
    X = np.moveaxis(np.asarray(scales, dtype=np.float64), ax, -1) - 127.0
    out = vals * np.exp2(X)[..., None]
    return np.ascontiguousarray(np.moveaxis(out.reshape(out.shape[:-2] + (-1,)), -1, ax))


def mx_roundtrip(a, axis: int = -1) -> np.ndarray:
    """dequant(quant(a)) along ``axis``: the value an MX GEMM operand stands for."""
    c, s = mx_quantize(a, axis)
    return mx_dequantize(c, s, axis)
