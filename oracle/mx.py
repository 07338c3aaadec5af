"""MXFP8 block quantisation (oracle).

[AREX] closing paragraph of the design section and [AIGWX] "详细发生了什么":
the layer has a BF16 mode and an MXFP8 mode; in MXFP8 mode the weights are
quantised ahead of time and the activations are quantised inside dispatch,
the expert GEMM and SwiGLU.  [ALPHA] section 三: weight quantisation happens
outside the timed region.

The pages name the format only.  The rule below is the OCP Microscaling (MX)
v1.0 specification's, for the MXFP8 (E4M3) element type:
  * blocks of 32 consecutive elements along the GEMM's reduction axis share one
    scale X = 2**s stored as E8M0 (biased exponent s + 127);
  * s = floor(log2(amax)) - 8, where 8 is the largest exponent of a normal E4M3
    value, clamped to [-127, 127]; an all-zero block gets s = -127;
  * each element is v / X rounded to nearest-even on the E4M3 grid and
    saturated to +-448 (E4M3 has no infinity; its one NaN code is never made).
A trailing partial block behaves as if zero-padded (zeros do not change amax).
"""
from __future__ import annotations

import numpy as np

MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal E4M3 value (1.75 * 2**8)
E4M3_EMIN = -6         # exponent of the smallest normal E4M3 value
E4M3_MBITS = 3


def e4m3_round(v):
    """Round float64 values to the nearest-even E4M3 value, saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, q = np.frexp(a)                      # a = f * 2**q, f in [0.5, 1)
    e = np.maximum(q - 1, E4M3_EMIN)        # subnormals share the quantum of the min normal
    quantum = np.ldexp(1.0, e - E4M3_MBITS)
    r = np.round(a / quantum) * quantum     # np.round rounds halves to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, v)


def e4m3_encode(r):
    """Bit pattern (uint8) of E4M3 values r (which must lie on the grid)."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.signbit(r).astype(np.uint8) << 7
    a = np.abs(r)
    _, q = np.frexp(a)
    e = q - 1
    normal = a >= 2.0 ** E4M3_EMIN
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, (a / np.ldexp(1.0, e) - 1.0) * 8.0, a / 2.0 ** (E4M3_EMIN - E4M3_MBITS))
    if not np.all(mant == np.round(mant)):
        raise ValueError("value not on the E4M3 grid")
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    return sign | code.astype(np.uint8)


def _e4m3_decode_fields(code):
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(ef == 0, m * 2.0 ** (E4M3_EMIN - E4M3_MBITS), (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


# every byte's value, decoded field by field by the function above
_E4M3_VALUES = _e4m3_decode_fields(np.arange(256))


def e4m3_decode(code):
    """float64 values of E4M3 bit patterns (0x7F / 0xFF, the NaN codes, decode to NaN)."""
    return _E4M3_VALUES[np.asarray(code).astype(np.intp)]


def _blocks_last(v):
    n = v.shape[-1]
    nb = -(-n // MX_BLOCK)
    pad = nb * MX_BLOCK - n
    if pad:
        v = np.concatenate([v, np.zeros(v.shape[:-1] + (pad,), v.dtype)], axis=-1)
    return v.reshape(v.shape[:-1] + (nb, MX_BLOCK)), n


def _block_scale_exp(b, emax):
    """Scale exponent s of each block (last axis of b): floor(log2 amax) - emax,
    clamped to [-127, 127]; -127 for an all-zero block."""
    amax = np.max(np.abs(b), axis=-1)
    _, q = np.frexp(amax)
    s = np.where(amax > 0, (q - 1) - emax, -127)
    return np.clip(s, -127, 127)


def mx_quantize(v, axis: int = -1):
    """Quantise v along `axis` in blocks of 32.

    Returns (codes uint8, same shape as v; scales uint8 E8M0, with the axis
    length replaced by the number of blocks).
    """
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    b, n = _blocks_last(v)
    s = _block_scale_exp(b, E4M3_EMAX)
    X = np.ldexp(1.0, s)[..., None]
    r = e4m3_round(b / X)
    codes = e4m3_encode(r).reshape(b.shape[:-2] + (-1,))[..., :n]
    scales = (s + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def mx_dequantize(codes, scales, axis: int = -1):
    """float64 values of an MX tensor (inverse of the layout of mx_quantize)."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    sc = np.moveaxis(np.asarray(scales), axis, -1).astype(np.int64)
    n = c.shape[-1]
    val = e4m3_decode(c)
    X = np.ldexp(1.0, sc - 127)
    Xe = np.repeat(X, MX_BLOCK, axis=-1)[..., :n]
    return np.moveaxis(val * Xe, -1, axis)


def mx_roundtrip(v, axis: int = -1):
    """Quantise then dequantise v along `axis` (float64 result).

    The value an element takes is its grid value times its block's scale; the
    bit patterns in between (encode, then decode) are exact inverses on the
    grid, so they are skipped here.  A CPU test checks that this equals
    mx_dequantize(*mx_quantize(v)) bit for bit."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    b, n = _blocks_last(v)
    X = np.ldexp(1.0, _block_scale_exp(b, E4M3_EMAX))[..., None]
    r = (e4m3_round(b / X) * X).reshape(b.shape[:-2] + (-1,))[..., :n]
    return np.moveaxis(r, -1, axis)


# ------------------------------------------------------------------ MXFP4
# The same block structure with E2M1 elements (OCP MX v1.0, MXFP4): 1 sign
# bit, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5,
# 2, 3, 4, 6; scale 2**(floor(log2(amax)) - 2), 2 being the exponent of the
# largest value (6 = 1.5 * 2**2); round to nearest even, saturate to +-6.
E2M1_MAX = 6.0
E2M1_EMAX = 2
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_round(v):
    """Round float64 values to the nearest-even E2M1 value, saturating at 6."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, q = np.frexp(a)                      # a = f * 2**q, f in [0.5, 1)
    e = np.maximum(q - 1, 0)                # below 1 the quantum is that of [1, 2)
    quantum = np.ldexp(1.0, e - 1)          # one mantissa bit
    r = np.round(a / quantum) * quantum     # np.round rounds halves to even
    r = np.minimum(r, E2M1_MAX)
    return np.copysign(r, v)


def e2m1_encode(r):
    """Code (uint8, 0..15) of E2M1 values r (which must lie on the grid)."""
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    idx = np.searchsorted(E2M1_GRID, a)
    if not np.all((idx < 8) & (E2M1_GRID[np.minimum(idx, 7)] == a)):
        raise ValueError("value not on the E2M1 grid")
    return (np.signbit(r).astype(np.uint8) << 3) | idx.astype(np.uint8)


def e2m1_decode(code):
    c = np.asarray(code, dtype=np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_GRID[c & 7]


def mxfp4_quantize(v, axis: int = -1):
    """MXFP4 along `axis` in blocks of 32: (codes uint8 0..15, same shape as v;
    E8M0 scales uint8 with the axis length replaced by the number of blocks)."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    b, n = _blocks_last(v)
    s = _block_scale_exp(b, E2M1_EMAX)
    X = np.ldexp(1.0, s)[..., None]
    codes = e2m1_encode(e2m1_round(b / X)).reshape(b.shape[:-2] + (-1,))[..., :n]
    return np.moveaxis(codes, -1, axis), np.moveaxis((s + 127).astype(np.uint8), -1, axis)


def mxfp4_dequantize(codes, scales, axis: int = -1):
    c = np.moveaxis(np.asarray(codes), axis, -1)
    sc = np.moveaxis(np.asarray(scales), axis, -1).astype(np.int64)
    n = c.shape[-1]
    Xe = np.repeat(np.ldexp(1.0, sc - 127), MX_BLOCK, axis=-1)[..., :n]
    return np.moveaxis(e2m1_decode(c) * Xe, -1, axis)


def mxfp4_roundtrip(v, axis: int = -1):
    """Quantise to MXFP4 then dequantise (float64); as mx_roundtrip, the grid
    value times the block scale, checked against the codes' round trip."""
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    b, n = _blocks_last(v)
    X = np.ldexp(1.0, _block_scale_exp(b, E2M1_EMAX))[..., None]
    r = (e2m1_round(b / X) * X).reshape(b.shape[:-2] + (-1,))[..., :n]
    return np.moveaxis(r, -1, axis)
