"""Read-copy quantisers, emulated exactly in numpy (oracle; test infrastructure only).

Pages: page 1 (section on low precision) and page 4 ("What shipped",
quantisation paragraph) describe a low-precision copy of the checkpoint that
serves output reads and never re-enters the recurrence; the pages use NVFP4 on
their hardware.  The two formats here are the published OCP ones:

* fp8 E4M3FN (OCP 8-bit floating point, v1.0): 1 sign, 4 exponent (bias 7),
  3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448.
  Block layout (reading): one float32 scale per 32 consecutive elements along
  the contiguous N axis, scale = amax / 448 computed in float32; element code =
  E4M3 round-to-nearest-even of (x / scale) computed in float32, saturating to
  +-448.  amax == 0 gives scale 0 and all-zero codes.
* MXFP4 (OCP Microscaling v1.0): E2M1 elements (1 sign, 2 exponent bits with
  bias 1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6) sharing one E8M0
  scale 2^E per 32 elements, E = floor(log2(amax)) - 2 (2 = largest E2M1
  exponent), clamped to [-126, 127] so that the scale is a normal float32
  (reading: E8M0 can also encode 2^-127, which is not used); element code =
  E2M1 round-to-nearest-even of x / 2^E, saturating to +-6.  amax == 0 gives
  E = -126.  Two codes per byte, even element in the low nibble.

The rounding here is done on exact float64 values (quantum = 2^(e - mbits)),
not with bit tricks, so it is an independent statement of the format rules.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _rne_to_format(a: np.ndarray, mbits: int, emin: int) -> np.ndarray:
    """Round non-negative float64 ``a`` to a binary format with ``mbits`` mantissa
    bits and smallest normal exponent ``emin`` (unbounded above), ties to even."""
    a = np.asarray(a, np.float64)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)              # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, emin)          # floor(log2 a), clamped to the normal range
    quantum = np.ldexp(1.0, e - mbits)
    m = a / quantum                        # exact (power-of-two division)
    r = np.round(m)                        # numpy rounds half to even
    return r * quantum


def e4m3_encode(x) -> np.ndarray:
    """float values -> uint8 E4M3FN codes (RNE, saturating to +-448)."""
    x = np.asarray(x, np.float64)
    sign = np.signbit(x)
    v = _rne_to_format(np.abs(x), mbits=3, emin=-6)
    v = np.minimum(v, E4M3_MAX)
    code = np.zeros(v.shape, np.int64)
    sub = v < 2.0 ** -6
    code[sub] = (v[sub] / 2.0 ** -9).astype(np.int64)          # 0..7 (0.0 -> 0)
    nz = ~sub
    _, ex = np.frexp(v[nz])
    e = ex - 1
    mant = (v[nz] / np.ldexp(1.0, e - 3)).astype(np.int64) - 8
    code[nz] = ((e + 7) << 3) | mant
    code = code | (sign.astype(np.int64) << 7)
    return code.astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """uint8 E4M3FN codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e2m1_encode(x) -> np.ndarray:
    """float values -> uint8 E2M1 codes 0..15 (RNE, saturating to +-6)."""
    x = np.asarray(x, np.float64)
    sign = np.signbit(x)
    v = _rne_to_format(np.abs(x), mbits=1, emin=0)
    v = np.minimum(v, E2M1_MAX)
    code = np.zeros(v.shape, np.int64)
    sub = v < 1.0
    code[sub] = (v[sub] / 0.5).astype(np.int64)                  # 0 or 1
    nz = ~sub
    _, ex = np.frexp(v[nz])
    e = ex - 1
    mant = (v[nz] / np.ldexp(1.0, e - 1)).astype(np.int64) - 2
    code[nz] = ((e + 1) << 1) | mant
    code = code | (sign.astype(np.int64) << 3)
    return code.astype(np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    val = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return s * val


def _blocks(x32: np.ndarray) -> np.ndarray:
    x32 = np.asarray(x32)
    if x32.dtype != np.float32:
        raise TypeError("read copies are made from float32 values")
    if x32.shape[-1] % BLOCK:
        raise ValueError("N must be a multiple of 32")
    return x32.reshape(x32.shape[:-1] + (x32.shape[-1] // BLOCK, BLOCK))


def quantize_fp8_blocks(x32: np.ndarray, amax=None):
    """float32 [..., N] -> (codes uint8 [..., N], scales float32 [..., N/32]).

    ``amax`` (float32 [..., N/32]) overrides the block maxima (used to bound ambiguity)."""
    xb = _blocks(x32)
    if amax is None:
        amax = np.max(np.abs(xb), axis=-1)                           # float32
    amax = np.asarray(amax, np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)         # float32 division
    safe = np.where(scale == 0, np.float32(1), scale).astype(np.float32)
    y = (xb / safe[..., None]).astype(np.float32)                    # float32 division
    codes = e4m3_encode(y)
    codes = np.where((scale == 0)[..., None], np.uint8(0), codes)
    return codes.reshape(x32.shape), scale


def dequantize_fp8_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    cb = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // BLOCK, BLOCK))
    val = e4m3_decode(cb) * scales.astype(np.float64)[..., None]     # exact in float64
    return val.reshape(codes.shape)


def _mx_exponent(amax: np.ndarray) -> np.ndarray:
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(amax)
    E = np.where(amax > 0, (ex - 1) - 2, -126)
    return np.clip(E, -126, 127)


def quantize_mxfp4_blocks(x32: np.ndarray, amax=None):
    """float32 [..., N] -> (packed codes uint8 [..., N/2], E8M0 uint8 [..., N/32]).

    ``amax`` overrides the block maxima (used to bound ambiguity)."""
    xb = _blocks(x32).astype(np.float64)
    if amax is None:
        amax = np.max(np.abs(xb), axis=-1)
    E = _mx_exponent(np.asarray(amax, np.float64))
    y = xb / np.ldexp(1.0, E)[..., None]                              # exact
    codes = e2m1_encode(y).reshape(x32.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (E + 127).astype(np.uint8)


def dequantize_mxfp4_blocks(packed: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    lo = packed & 0xF
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    cb = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // BLOCK, BLOCK))
    scale = np.ldexp(1.0, e8m0.astype(np.int64) - 127)
    return (e2m1_decode(cb) * scale[..., None]).reshape(codes.shape)


def read_copy_dequant(fmt: str, x32: np.ndarray) -> np.ndarray:
    """Quantise float32 values with ``fmt`` and return the dequantised float64 values."""
    if fmt == "fp8":
        return dequantize_fp8_blocks(*quantize_fp8_blocks(x32))
    if fmt == "mxfp4":
        return dequantize_mxfp4_blocks(*quantize_mxfp4_blocks(x32))
    raise ValueError(fmt)


def read_copy_ambiguity(fmt: str, x32: np.ndarray, delta) -> np.ndarray:
    """Bound on |dequant(x') - dequant(x)| per element when every float32 input may differ
    by at most ``delta`` (absolute, broadcast against x) from x.

    Reading: the copy is made from the fp32 checkpoint the GPU holds, which agrees with the
    oracle's only up to fp32 reassociation; an element (or, for MXFP4, a block maximum) that
    lies that close to a rounding boundary has two correct codes.  Codes are monotone in x
    for a fixed scale and in the scale for a fixed x, so the extreme codes come from the
    corners x +- delta, amax +- delta, and the extreme dequantised values from the extreme
    codes times the extreme scales.
    """
    x32 = np.asarray(x32, np.float32)
    delta = np.broadcast_to(np.asarray(delta, np.float64), x32.shape)
    xb = _blocks(x32).astype(np.float64)
    db = delta.reshape(xb.shape)
    amax = np.max(np.abs(xb), axis=-1)
    damax = np.max(db, axis=-1)
    base = read_copy_dequant(fmt, x32)
    lo_c = hi_c = None
    scales = []
    for sa in (-1.0, 1.0):
        am = np.maximum(amax + sa * damax, 0.0)
        if fmt == "fp8":
            am32 = am.astype(np.float32)
            scales.append((am32 / np.float32(E4M3_MAX)).astype(np.float32).astype(np.float64))
        else:
            scales.append(np.ldexp(1.0, _mx_exponent(am)))
        for sx in (-1.0, 1.0):
            xp = (xb + sx * db).astype(np.float32).reshape(x32.shape)
            if fmt == "fp8":
                codes, _ = quantize_fp8_blocks(xp, amax=am.astype(np.float32))
                val = e4m3_decode(codes.reshape(xb.shape))
                val = np.where((am.astype(np.float32) / np.float32(E4M3_MAX) == 0)[..., None], 0.0, val)
            else:
                packed, _ = quantize_mxfp4_blocks(xp, amax=am)
                lo = packed & 0xF
                hi = packed >> 4
                c = np.stack([lo, hi], axis=-1).reshape(x32.shape)
                val = e2m1_decode(c.reshape(xb.shape))
            lo_c = val if lo_c is None else np.minimum(lo_c, val)
            hi_c = val if hi_c is None else np.maximum(hi_c, val)
    s_lo = np.minimum(scales[0], scales[1])[..., None]
    s_hi = np.maximum(scales[0], scales[1])[..., None]
    b = base.reshape(xb.shape)
    worst = np.zeros_like(b)
    for c in (lo_c, hi_c):
        for sc in (s_lo, s_hi):
            worst = np.maximum(worst, np.abs(c * sc - b))
    # a block whose maximum is within delta of zero has no determined scale: any dequantised
    # value is within 1.5 (amax + delta) of zero (E2M1 saturation; E4M3 rounds by < 2^-4)
    degenerate = (amax - damax) <= 0
    worst = np.where(degenerate[..., None], 3.0 * (amax + damax)[..., None], worst)
    return worst.reshape(x32.shape)
