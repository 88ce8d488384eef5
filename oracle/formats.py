"""Oracle number formats: bf16 (RNE), E4M3FN (RNE), E2M1 and E8M0.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.

Each conversion is the format's definition written out: the set of values the
format can hold is enumerated (or described by sign, exponent and mantissa),
and rounding picks the nearest member, ties to the member whose code is even.
Distances are taken in float64, where every difference used here is exact
(all operands are float32 or narrower values of nearby magnitude).

Sources:
* bf16 round-to-nearest-even packing of two floats into one word, low half
  first: page ``vllm.models.muse_spark.amd.mono.kernels.dev``, ``bf16_pair``;
  packed-word unpacking: page ``vllm.models.deepseek_v41.amd.mono.common.ops``,
  ``bf_lo`` / ``bf_hi``.
* E4M3 packing of four floats, byte order a, b, c, d from the low byte, RNE,
  inputs already in range: the ``...common.ops`` page, ``fp8_pack4``. The
  variant is OCP E4M3FN (bias 7, no infinities, NaN = S.1111.111, max 448).
* E2M1 nibbles, low nibble first, times a power-of-two scale: the
  ``...kernels.dev`` page, ``fp4x8_bf16``; the scale's E8M0 code c stands for
  2**(c - 127): same page, ``e8m0_f32``. E2M1 itself (1 sign, 2 exponent bits
  with bias 1, 1 mantissa bit, subnormal when the exponent field is 0) is the
  OCP Microscaling (MX) v1.0 element format; the pages name it but give no
  table.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 pattern is the high half of the float32 with the same value
    (``bf_lo`` / ``bf_hi`` on the ``...common.ops`` page move the half into the
    top 16 bits of a float32), so the widening is exact.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def _bf16_value(hi_bits: np.ndarray) -> np.ndarray:
    """Value of bf16 patterns given as uint32 in the range 0..0xFFFF, as f64.

    The pattern one past the largest finite magnitude (0x7F80, infinity) is
    given the value 2**128 here: that is the point the round-to-nearest rule
    treats as the next representable magnitude when deciding overflow.
    """
    mag = hi_bits & np.uint32(0x7FFF)
    sign = np.where((hi_bits & np.uint32(0x8000)) != 0, -1.0, 1.0)
    with np.errstate(invalid="ignore"):
        val = ((mag << np.uint32(16)).astype(np.uint32)).view(np.float32).astype(np.float64)
    val = np.where(mag == 0x7F80, 2.0**128, val)
    return sign * val


def f32_to_bf16_rne(x) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Definition: of the two bf16 values that bracket x (the one obtained by
    dropping the low 16 bits, and the next one away from zero), take the
    nearer; on a tie take the one whose pattern is even. Infinities stay
    infinities; NaN maps to a quiet NaN of the same sign. Magnitudes at or
    beyond the midpoint between the largest finite bf16 and 2**128 round to
    infinity, as IEEE round-to-nearest does.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint32)
    lo = (u >> np.uint32(16)).astype(np.uint32)  # truncation toward zero
    hi = lo + np.uint32(1)  # next magnitude away from zero (same sign bit)
    with np.errstate(invalid="ignore", over="ignore"):
        xv = x.astype(np.float64)
        d_lo = np.abs(xv - _bf16_value(lo))
        d_hi = np.abs(_bf16_value(hi & np.uint32(0xFFFF)) - xv)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint32(1)) == 1))
    out = np.where(take_hi, hi, lo)
    finite = np.isfinite(x)
    is_nan = np.isnan(x)
    out = np.where(finite, out, lo)  # +-inf: the truncation is exact
    out = np.where(is_nan, (lo | np.uint32(0x0040)), out)  # quiet NaN
    return (out & np.uint32(0xFFFF)).astype(np.uint16)


def bf16_pair_word(a, b) -> np.ndarray:
    """Two float32 -> one uint32 word: bf16(a) in the low half, bf16(b) high.

    The word layout of ``bf16_pair`` (``...kernels.dev`` page), rounding RNE.
    """
    lo = f32_to_bf16_rne(a).astype(np.uint32)
    hi = f32_to_bf16_rne(b).astype(np.uint32)
    return (lo | (hi << np.uint32(16))).astype(np.uint32)


# ---------------------------------------------------------------------------
# E4M3FN
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """E4M3FN code (0..255) -> float64 value (NaN for S.1111.111).

    Fields: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
    Exponent field 0 is subnormal: m * 2**-9. Otherwise 2**(e-7) * (1 + m/8).
    """
    c = np.asarray(code, dtype=np.int64)
    s = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = m * 2.0**-9
    nrm = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    v = np.where(e == 0, sub, nrm)
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def f32_to_e4m3_rne(x) -> np.ndarray:
    """float32 values with |x| <= 448 -> E4M3FN codes (uint8), RNE.

    Definition: the nearest of the 127 non-negative finite E4M3FN magnitudes
    (codes 0x00..0x7E), ties to the even code; the sign goes to bit 7 (so -0.0
    gives 0x80). Inputs outside [-448, 448] (or NaN) are outside the contract
    of the packing helper ("already in range") and are rejected.
    """
    x = np.asarray(x, dtype=np.float32)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("E4M3 packing is defined here for |x| <= 448 only")
    codes = np.arange(0x7F, dtype=np.int64)  # 0x00..0x7E, increasing magnitude
    mags = e4m3_value(codes)
    a = np.abs(x.astype(np.float64))
    hi = np.searchsorted(mags, a, side="left")  # first magnitude >= a
    hi = np.minimum(hi, len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(a - mags[lo])
    d_hi = np.abs(mags[hi] - a)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    c = np.where(take_hi, codes[hi], codes[lo])
    sign = np.signbit(x)
    return (c | np.where(sign, 0x80, 0)).astype(np.uint8)


def e4m3_rne_sat(x) -> np.ndarray:
    """float64 values -> E4M3FN codes (uint8) of the values saturated to the
    format's range: each value is first clamped to [-448, 448] (448 is the
    largest finite E4M3FN magnitude), then rounded to the nearest of the 127
    non-negative finite magnitudes, ties to the even code, with the sign in
    bit 7 (-0.0 gives 0x80). This is the output stage of the E4M3-output
    GEMM: the pages' ``fp8_pack4`` packs values "already in range", and the
    saturation is what brings a scaled sum into that range. NaN is rejected.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("E4M3 output of NaN is outside the contract")
    y = np.clip(x, -E4M3_MAX, E4M3_MAX)
    codes = np.arange(0x7F, dtype=np.int64)
    mags = e4m3_value(codes)
    a = np.abs(y)
    hi = np.minimum(np.searchsorted(mags, a, side="left"), len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(a - mags[lo])
    d_hi = np.abs(mags[hi] - a)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    c = np.where(take_hi, codes[hi], codes[lo])
    return (c | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def e4m3_pack4_word(a, b, c, d) -> np.ndarray:
    """Four float32 (in range) -> one uint32 of E4M3 bytes a, b, c, d, low first.

    The byte order of ``fp8_pack4`` on the ``...common.ops`` page.
    """
    parts = [f32_to_e4m3_rne(v).astype(np.uint32) for v in (a, b, c, d)]
    return (parts[0] | (parts[1] << 8) | (parts[2] << 16) | (parts[3] << 24)).astype(np.uint32)


# ---------------------------------------------------------------------------
# E2M1 / E8M0 / MXFP4
# ---------------------------------------------------------------------------


def e2m1_value(code) -> np.ndarray:
    """E2M1 code (0..15) -> float64.

    Fields: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0. An
    exponent field of 0 is subnormal: m * 0.5. Otherwise 2**(e-1) * (1 + m/2).
    Code 8 is -0.0.
    """
    c = np.asarray(code, dtype=np.int64)
    s = np.where((c & 0x8) != 0, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    v = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return s * v


def e8m0_value(code) -> np.ndarray:
    """E8M0 scale code (0..255) -> float64: 2**(code - 127); code 255 is NaN.

    The ``e8m0_f32`` helper on the ``...kernels.dev`` page maps a biased
    exponent to the float32 power of two it stands for.
    """
    c = np.asarray(code, dtype=np.int64)
    v = np.ldexp(np.ones(c.shape, dtype=np.float64), (c - 127).astype(np.int64))
    return np.where(c == 255, np.nan, v)


def mxfp4_nibbles(wq: np.ndarray) -> np.ndarray:
    """Packed E2M1 bytes [N, K/2] -> codes [N, K], low nibble first.

    Element k of a row sits in byte k // 2 of that row: the low nibble when k
    is even, the high nibble when k is odd (``fp4x8_bf16`` on the
    ``...kernels.dev`` page reads a dword of 8 E2M1 low nibble first, so a
    little-endian dword's element j is nibble j counted from bit 0).
    """
    wq = np.asarray(wq, dtype=np.uint8)
    n, kh = wq.shape
    out = np.empty((n, 2 * kh), dtype=np.uint8)
    out[:, 0::2] = wq & 0x0F
    out[:, 1::2] = wq >> 4
    return out


def mxfp4_dequant_f64(wq: np.ndarray, wscale: np.ndarray) -> np.ndarray:
    """MXFP4 weights -> float64 [N, K]: w[n, k] = E2M1(nib(n, k)) * 2**(s[n, k//32] - 127).

    ``wq`` is uint8 [N, K/2] (two E2M1 codes a byte, low nibble first) and
    ``wscale`` uint8 [N, K/32] (one E8M0 code per 32-element K block, rows
    in the same order as ``wq``).
    """
    codes = mxfp4_nibbles(wq)
    n, k = codes.shape
    wscale = np.asarray(wscale, dtype=np.uint8)
    if wscale.shape != (n, k // 32) or k % 32:
        raise ValueError(f"scale shape {wscale.shape} does not match weights [{n}, {k}]")
    scale = np.repeat(e8m0_value(wscale), 32, axis=1)
    return e2m1_value(codes) * scale


def mxfp4_dequant_bf16_bits(wq: np.ndarray, wscale: np.ndarray) -> np.ndarray:
    """MXFP4 weights -> bf16 bit patterns [N, K], requiring the result to be exact.

    The decode is exact whenever every product is a bf16 value (true for scale
    codes whose products stay normal and finite in bf16). The rounding step
    below is then the identity, which is asserted.
    """
    w = mxfp4_dequant_f64(wq, wscale)
    bits = f32_to_bf16_rne(w.astype(np.float32))
    back = bf16_bits_to_f64(bits)
    both_nan = np.isnan(back) & np.isnan(w)
    if not np.all((back == w) | both_nan):
        raise ValueError("MXFP4 decode is not exact in bf16 for these scale codes")
    # signed zeros: E2M1 -0 times a scale is -0, which the bit pattern keeps
    return bits


def mxfp8_dequant_f64(wq8: np.ndarray, wscale: np.ndarray) -> np.ndarray:
    """MXFP8 weights -> float64 [N, K]: w[n, k] = E4M3(wq8[n, k]) * 2**(s[n, k//32] - 127).

    ``wq8`` is uint8 [N, K], one OCP E4M3FN code per byte (element k in byte
    k); ``wscale`` is uint8 [N, K/32], one E8M0 code per 32-element K block.
    This is the block scaling of the MXFP4 path (page
    vllm.models.muse_spark.amd.mono.kernels.dev, e8m0_f32) with eight-bit E4M3
    elements, the format of that page family's fp8_pack4 helper (page
    vllm.models.deepseek_v41.amd.mono.common.ops). Code 0x7F / 0xFF is NaN.
    """
    codes = np.asarray(wq8, dtype=np.uint8)
    n, k = codes.shape
    wscale = np.asarray(wscale, dtype=np.uint8)
    if wscale.shape != (n, k // 32) or k % 32:
        raise ValueError(f"scale shape {wscale.shape} does not match weights [{n}, {k}]")
    scale = np.repeat(e8m0_value(wscale), 32, axis=1)
    return e4m3_value(codes) * scale


def mxfp8_dequant_bf16_bits(wq8: np.ndarray, wscale: np.ndarray) -> np.ndarray:
    """MXFP8 weights -> bf16 bit patterns [N, K], requiring the result to be exact.

    E4M3 values have at most four significant bits, so every product with a
    power of two that stays normal and finite is a bf16 value; the rounding
    below is then the identity, which is asserted (NaN codes stay NaN).
    """
    w = mxfp8_dequant_f64(wq8, wscale)
    bits = f32_to_bf16_rne(w.astype(np.float32))
    back = bf16_bits_to_f64(bits)
    both_nan = np.isnan(back) & np.isnan(w)
    if not np.all((back == w) | both_nan):
        raise ValueError("MXFP8 decode is not exact in bf16 for these scale codes")
    return bits
