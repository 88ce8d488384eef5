"""Pins for oracle/formats.py against things other than itself.

Each conversion is checked against hand-worked fixtures under tests/golden/,
an independent closed form, and (where one exists) a library routine, so that
a plausible mistake (a wrong tie rule, nibble order, sign or bias) fails here.
"""

import math

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.conftest import golden_rows

# ---------------------------------------------------------------- bf16 -----


def _torch_bf16_bits(x_f32):
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _structured_f32_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(7)
    rnd = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([pats, rnd])


def test_bf16_golden_cases():
    for f32_hex, bf16_hex, *_ in golden_rows("bf16_rne_cases.txt"):
        x = np.array([int(f32_hex, 16)], dtype=np.uint32).view(np.float32)
        got = int(F.f32_to_bf16_rne(x)[0])
        assert got == int(bf16_hex, 16), (f32_hex, hex(got), bf16_hex)


def test_bf16_matches_torch_and_integer_form():
    pats = _structured_f32_patterns()
    x = pats.view(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        got = F.f32_to_bf16_rne(x)
    nan = np.isnan(x)
    # library routine: torch's float32 -> bfloat16 cast rounds to nearest even
    ref = _torch_bf16_bits(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # an independent closed form of RNE on the bit pattern (non-NaN inputs)
    u = pats[~nan].astype(np.uint64)
    closed = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(got[~nan], closed)
    # NaN stays NaN
    assert np.all(np.isnan(F.bf16_bits_to_f64(got[nan])))


def test_bf16_widening_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = F.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert np.all(same)
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def test_bf16_pair_word_layout():
    # bf16(a) in the low half, bf16(b) in the high half (bf16_pair)
    w = F.bf16_pair_word(np.float32([1.0]), np.float32([-2.0]))
    assert int(w[0]) == 0xC0003F80


# ---------------------------------------------------------------- E4M3 -----


def test_e4m3_golden_cases():
    for val, code, *_ in golden_rows("e4m3_cases.txt"):
        got = int(F.f32_to_e4m3_rne(np.float32([float(val)]))[0])
        assert got == int(code, 16), (val, hex(got), code)


def test_e4m3_pack4_golden():
    for a, b, c, d, word in golden_rows("e4m3_pack4_cases.txt"):
        got = int(F.e4m3_pack4_word(*[np.float32([float(v)]) for v in (a, b, c, d)])[0])
        assert got == int(word, 16), (a, b, c, d, hex(got), word)


def test_e4m3_values_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = F.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert np.all(same)
    assert F.e4m3_value(np.array([0x7E]))[0] == 448.0


def _e4m3_probe_values():
    mags = F.e4m3_value(np.arange(0x7F))  # all finite non-negative values
    mids = (mags[:-1] + mags[1:]) / 2
    vals = np.concatenate([mags, mids]).astype(np.float32)
    up = np.nextafter(vals, np.float32(np.inf))
    dn = np.nextafter(vals, np.float32(0))
    rng = np.random.default_rng(3)
    rnd = (rng.random(1 << 16) * 448).astype(np.float32)
    v = np.concatenate([vals, up, dn, rnd])
    v = v[np.abs(v) <= 448]
    return np.concatenate([v, -v])


def test_e4m3_rne_matches_torch():
    v = _e4m3_probe_values()
    got = F.f32_to_e4m3_rne(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.f32_to_e4m3_rne(np.float32([449.0]))


# ------------------------------------------------------- E2M1 / E8M0 -------


def test_e2m1_all_codes():
    vals = F.e2m1_value(np.arange(16))
    assert list(vals[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(vals[8:]) == [-v for v in vals[:8]]
    assert math.copysign(1.0, vals[8]) == -1.0  # code 8 is -0
    assert np.all(np.diff(vals[:8]) > 0)
    # torch's E2M1 pair type as a library cross-check (unpack by its own rule)
    if hasattr(torch, "float4_e2m1fn_x2"):
        try:
            t = torch.arange(16, dtype=torch.uint8).view(torch.float4_e2m1fn_x2)
            ref = t.to(torch.float32)  # not every build implements this cast
        except (RuntimeError, TypeError, NotImplementedError):
            ref = None
        if ref is not None and ref.numel() == 16:
            assert np.array_equal(ref.numpy().astype(np.float64), vals)


def test_e8m0_closed_form_and_library():
    codes = np.arange(255)
    got = F.e8m0_value(codes)
    for c in range(255):
        assert got[c] == math.ldexp(1.0, c - 127)
    # the helper's bit form: code << 23 read as float32, for codes 1..254
    bits = (np.arange(1, 255, dtype=np.uint32) << np.uint32(23)).view(np.float32)
    assert np.array_equal(got[1:255], bits.astype(np.float64))
    assert np.isnan(F.e8m0_value(np.array([255]))[0])
    if hasattr(torch, "float8_e8m0fnu"):
        ref = torch.arange(1, 256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu)
        ref = ref.double().numpy()
        g = F.e8m0_value(np.arange(1, 256))
        assert np.all((g == ref) | (np.isnan(g) & np.isnan(ref)))


# ------------------------------------------------------------- MXFP4 -------


def _dword_rows(word_hex):
    w = np.array([int(word_hex, 16)], dtype=np.uint32)
    return w.view(np.uint8).reshape(1, 4)  # little-endian bytes of one dword


def test_mxfp4_golden_cases():
    for row in golden_rows("mxfp4_cases.txt"):
        word, code, vals = row[0], int(row[1]), [float(v) for v in row[2:]]
        wq = np.tile(_dword_rows(word), (1, 4))  # 32 elements: the dword 4 times
        ws = np.array([[code]], dtype=np.uint8)
        got = F.mxfp4_dequant_f64(wq, ws)[0, :8]
        assert list(got) == vals, (word, code, list(got))
        assert list(np.signbit(got)) == [math.copysign(1.0, v) < 0 for v in vals]


def test_mxfp4_bruteforce_small():
    rng = np.random.default_rng(11)
    n, k = 3, 64
    wq = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    ws = rng.integers(110, 140, size=(n, k // 32), dtype=np.uint8)
    table = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}
    got = F.mxfp4_dequant_f64(wq, ws)
    for r in range(n):
        for c in range(k):
            byte = int(wq[r][c // 2])
            nib = (byte & 15) if c % 2 == 0 else (byte >> 4)
            mag = table[nib & 7]
            val = (-mag if nib & 8 else mag) * 2.0 ** (int(ws[r][c // 32]) - 127)
            assert got[r][c] == val


def test_mxfp4_bf16_exact_range():
    # every (code, scale) pair with scale in [2, 252] decodes exactly to bf16
    codes = np.arange(16, dtype=np.uint8)
    scales = np.arange(2, 253, dtype=np.uint8)
    n = len(scales)
    nib = np.tile(codes, 2)  # 32 elements per row: each code twice
    wq = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    wq = np.tile(wq, (n, 1))
    ws = scales.reshape(n, 1)
    bits = F.mxfp4_dequant_bf16_bits(wq, ws)
    vals = F.bf16_bits_to_f64(bits)
    expect = F.e2m1_value(nib)[None, :] * np.ldexp(1.0, (scales.astype(int) - 127))[:, None]
    assert np.array_equal(vals, expect)


# ------------------------------------------------ planted mistakes ---------


def test_pins_catch_planted_mistakes():
    """Wrong variants of the oracle, planted here on the CPU, must fail the pins."""
    # truncation instead of RNE fails the bf16 fixtures
    x = np.array([0x3F818000], dtype=np.uint32).view(np.float32)
    trunc = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert int(trunc[0]) != 0x3F82 and int(F.f32_to_bf16_rne(x)[0]) == 0x3F82
    # high-nibble-first decode fails the MXFP4 fixture
    wq = np.tile(_dword_rows("0x76543210"), (1, 4))
    swapped = np.empty((1, 32), dtype=np.uint8)
    swapped[:, 0::2] = wq >> 4
    swapped[:, 1::2] = wq & 15
    assert list(F.e2m1_value(swapped[0, :8])) != [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    # a scale bias of 128 instead of 127 fails the E8M0 closed form
    assert F.e8m0_value(np.array([127]))[0] == 1.0 != 2.0 ** (127 - 128)


def _e4m3_fields(code: int) -> float:
    """E4M3FN from its bit fields, written out for the pins below."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def test_mxfp8_golden_cases():
    for row in golden_rows("mxfp8_cases.txt"):
        codes = [int(b, 16) for b in row[:8]]
        scale = int(row[8])
        vals = [float(v) for v in row[9:]]
        wq8 = np.tile(np.array(codes, dtype=np.uint8), 4).reshape(1, 32)
        got = F.mxfp8_dequant_f64(wq8, np.array([[scale]], dtype=np.uint8))[0, :8]
        for g, v in zip(got, vals):
            if math.isnan(v):
                assert math.isnan(g)
            else:
                assert g == v and math.copysign(1.0, g) == math.copysign(1.0, v), (row, list(got))


def test_mxfp8_bruteforce_small():
    rng = np.random.default_rng(12)
    n, k = 3, 96
    wq8 = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    ws = rng.integers(110, 140, size=(n, k // 32), dtype=np.uint8)
    got = F.mxfp8_dequant_f64(wq8, ws)
    for r in range(n):
        for c in range(k):
            want = _e4m3_fields(int(wq8[r][c])) * 2.0 ** (int(ws[r][c // 32]) - 127)
            if math.isnan(want):
                assert math.isnan(got[r][c])
            else:
                assert got[r][c] == want


def test_mxfp8_bf16_exact_range():
    # every non-NaN code with every scale in [10, 246] decodes exactly to bf16
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    codes = np.concatenate([codes, codes[: (-len(codes)) % 32]])
    scales = np.arange(10, 247, dtype=np.uint8)
    n, k = len(scales), len(codes)
    wq8 = np.tile(codes, (n, 1))
    ws = np.repeat(scales.reshape(n, 1), k // 32, axis=1)
    vals = F.bf16_bits_to_f64(F.mxfp8_dequant_bf16_bits(wq8, ws))
    expect = np.array([[_e4m3_fields(int(c)) * 2.0 ** (int(sc) - 127) for c in codes] for sc in scales])
    assert np.array_equal(vals, expect)


def test_mxfp8_planted_mistakes_fail():
    """A decode that reads codes as E5M2, or applies the scale of the wrong
    block, must differ from the oracle on the golden rows."""
    wq8 = np.tile(np.array([0x38, 0x40, 0x48, 0x30, 0x3C, 0x01, 0x08, 0x7E], dtype=np.uint8), 8).reshape(1, 64)
    ws = np.array([[127, 129]], dtype=np.uint8)
    good = F.mxfp8_dequant_f64(wq8, ws)
    wrong_block = F.e4m3_value(wq8) * np.ldexp(1.0, np.repeat(ws[:, ::-1].astype(int) - 127, 32, axis=1))
    assert not np.array_equal(good, wrong_block)
    e5m2 = np.array([[(-1.0) ** (int(c) >> 7) * (1 + (int(c) & 3) / 4) * 2.0 ** (((int(c) >> 2) & 31) - 15) for c in row]
                     for row in wq8])
    assert not np.allclose(good[:, :32], e5m2[:, :32])


# ------------------------------------------------ E4M3 output (saturated) ---


def test_e4m3_rne_sat_agrees_in_range():
    """In range, the float64 output rounding is the packing helper's rounding
    (pinned to torch above) on every probe value."""
    v = _e4m3_probe_values()
    assert np.array_equal(F.e4m3_rne_sat(v.astype(np.float64)), F.f32_to_e4m3_rne(v))
    for val, code, *_ in golden_rows("e4m3_cases.txt"):
        assert int(F.e4m3_rne_sat(np.float64([float(val)]))[0]) == int(code, 16), val


def test_e4m3_rne_sat_saturates_and_rounds_in_float64():
    # saturation: anything beyond 448 in magnitude is +-448 (0x7E / 0xFE)
    big = np.array([448.0, 448.0000001, 464.0, 500.0, 1e30, -449.0, -1e300])
    assert list(F.e4m3_rne_sat(big)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    # midpoints decided by float64 values that float32 cannot hold:
    # 17 is the tie of 16 (0x58, even) and 18 (0x59); 19 the tie of 18 and 20 (0x5A)
    eps = 1e-12
    cases = {17.0: 0x58, 17.0 + eps: 0x59, 17.0 - eps: 0x58, 19.0: 0x5A, 19.0 - eps: 0x59,
             25.0: 0x5C, 25.0 + eps: 0x5D, -17.0: 0xD8, 0.0009765625 + eps: 0x01}
    for x, code in cases.items():
        assert int(F.e4m3_rne_sat(np.float64([x]))[0]) == code, (x, code)


def test_e4m3_rne_sat_planted_mistakes_fail():
    """Truncation instead of nearest, or no saturation, would fail the pins."""
    mags = F.e4m3_value(np.arange(0x7F))

    def truncating(x):
        a = np.clip(np.abs(x), 0, 448)
        c = np.searchsorted(mags, a, side="right") - 1
        return (c | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)

    x = np.float64([17.0 + 1e-12, 19.0])
    assert not np.array_equal(truncating(x), F.e4m3_rne_sat(x))
    with pytest.raises(ValueError):
        F.f32_to_e4m3_rne(np.float32([500.0]))  # the unsaturated rounding rejects it
    with pytest.raises(ValueError):
        F.e4m3_rne_sat(np.float64([np.nan]))
