"""Pins for oracle/gemm.py against things other than itself.

The fp64 product is checked against a hand-worked fixture, a pure-Python brute
force on tiny shapes, exact special cases (identity, one-hot permutation, K=1,
integer operands) and the MXFP4 decode; the acceptance bound and the
fixed-order butterfly against hand-derived values.
"""

import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as G
from tests.conftest import golden_rows
import workloads


def _bits(vals):
    return workloads.to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_gemm_tiny_golden():
    rows = {r[0]: r[1:] for r in golden_rows("gemm_tiny.txt")}
    T, K, N = int(rows["T"][0]), int(rows["K"][0]), int(rows["N"][0])
    x = np.array([float(v) for v in rows["X"]]).reshape(T, K)
    w = np.array([float(v) for v in rows["W"]]).reshape(N, K)
    c = np.array([float(v) for v in rows["C"]]).reshape(T, N)
    got = G.gemm_bf16_ref(_bits(x), _bits(w))
    assert np.array_equal(got, c)
    assert G.gemm_bruteforce(x.tolist(), w.tolist()) == c.tolist()


def test_gemm_matches_bruteforce_small_shapes():
    rng = np.random.default_rng(5)
    for T, N, K in [(1, 1, 1), (1, 3, 7), (3, 5, 7), (2, 32, 256), (3, 17, 96)]:
        xb = _bits(rng.standard_normal((T, K)))
        wb = _bits(rng.standard_normal((N, K)) * 0.02)
        got = G.gemm_bf16_ref(xb, wb)
        bf = G.gemm_bruteforce(F.bf16_bits_to_f64(xb).tolist(), F.bf16_bits_to_f64(wb).tolist())
        # both are float64 sums of exact products; they differ only by the
        # order of float64 rounding
        np.testing.assert_allclose(got, np.array(bf), rtol=1e-12, atol=1e-12)


def test_gemm_identity_and_permutation():
    rng = np.random.default_rng(6)
    T, K = 3, 64
    xb = _bits(rng.standard_normal((T, K)))
    x = F.bf16_bits_to_f64(xb)
    assert np.array_equal(G.gemm_bf16_ref(xb, _bits(np.eye(K))), x)
    # one-hot rows: W[n, perm[n]] = 1 with N != K, so a transposed operand fails
    N = 40
    perm = rng.permutation(K)[:N]
    w = np.zeros((N, K))
    w[np.arange(N), perm] = 1.0
    assert np.array_equal(G.gemm_bf16_ref(xb, _bits(w)), x[:, perm])


def test_gemm_k1_is_outer_product():
    rng = np.random.default_rng(8)
    xb = _bits(rng.standard_normal((4, 1)))
    wb = _bits(rng.standard_normal((6, 1)))
    x = F.bf16_bits_to_f64(xb)[:, 0]
    w = F.bf16_bits_to_f64(wb)[:, 0]
    assert np.array_equal(G.gemm_bf16_ref(xb, wb), np.outer(x, w))


def test_gemm_integer_operands_exact():
    xb, wb = workloads.integer_bf16_case(5, 300, 7, seed=9)
    got = G.gemm_bf16_ref(xb, wb)
    xi = F.bf16_bits_to_f64(xb).astype(np.int64).tolist()
    wi = F.bf16_bits_to_f64(wb).astype(np.int64).tolist()
    exact = [[sum(a * b for a, b in zip(xr, wr)) for wr in wi] for xr in xi]
    assert got.tolist() == [[float(v) for v in r] for r in exact]


def test_gemm_mxfp4_two_routes():
    x, wq, ws = workloads.small_mxfp4_case(3, 128, 5, seed=10)
    a = G.gemm_mxfp4_ref(x, wq, ws)
    b = G.gemm_bf16_ref(x, F.mxfp4_dequant_bf16_bits(wq, ws))
    assert np.array_equal(a, b)
    bf = G.gemm_bruteforce(F.bf16_bits_to_f64(x).tolist(), F.mxfp4_dequant_f64(wq, ws).tolist())
    np.testing.assert_allclose(a, np.array(bf), rtol=1e-12, atol=1e-12)


def test_tolerance_bound_values():
    ref = np.array([[1.0, -2.0], [0.0, 4.0]])
    rms = math.sqrt((1 + 4 + 0 + 16) / 4)
    b = G.tolerance_bound(ref, 100)
    expect = 2.0**-7 * np.abs(ref) + 1e-3 * 10 * rms
    assert np.allclose(b, expect, rtol=0, atol=0)
    assert G.violation_ratio(ref, ref, 100) == 0.0
    assert G.violation_ratio(ref + b, ref, 100) <= 1.0 + 1e-12
    assert G.violation_ratio(ref + 1.01 * b, ref, 100) > 1.0
    bad = ref.copy()
    bad[0, 0] = np.nan
    assert G.violation_ratio(bad, ref, 100) == math.inf


def test_tolerance_catches_a_dropped_term():
    # a planted mistake on the CPU: dropping the last K column of a random
    # product at workload scale exceeds the bound somewhere
    x, w = workloads.small_bf16_case(8, 1024, 256, seed=12)
    ref = G.gemm_bf16_ref(x, w)
    bad = G.gemm_bf16_ref(x[:, :-1], w[:, :-1])
    assert G.violation_ratio(bad, ref, 1024) > 1.0
    # and a bf16 rounding of the exact result passes, as it must
    rounded = F.bf16_bits_to_f64(F.f32_to_bf16_rne(ref.astype(np.float32)))
    assert G.violation_ratio(rounded, ref, 1024) <= 1.0


def test_butterfly_order_is_the_contract():
    v = np.zeros((1, 64), dtype=np.float32)
    v[0, 0] = 2.0**24
    v[0, 1] = 1.0
    v[0, 33] = 1.0
    # offsets 32 first: lane 1 + lane 33 = 2 before meeting 2^24 -> exact 2^24 + 2
    assert np.all(G.butterfly_f32(v) == 2.0**24 + 2)
    # offsets 1 first: 2^24 + 1 rounds to 2^24 twice -> 2^24
    assert np.all(G.butterfly_f32(v, offsets=(1, 2, 4, 8, 16, 32)) == 2.0**24)


def test_butterfly_integer_sum_exact():
    rng = np.random.default_rng(13)
    v = rng.integers(-1000, 1000, size=(50, 64)).astype(np.float32)
    out = G.butterfly_f32(v)
    assert np.array_equal(out, np.repeat(v.sum(axis=1, dtype=np.float64)[:, None], 64, axis=1))


def test_mxfp8_gemm_matches_bruteforce_and_integer_exact():
    """The MXFP8 GEMM on decoded weights equals the pure-Python triple loop,
    and with integer E4M3 values, integer X and scale 1 it is exact."""
    rng = np.random.default_rng(21)
    T, N, K = 2, 3, 64
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4], dtype=np.uint8)  # 0 1 2 3 4 -1 -2 -3
    wq8 = rng.choice(ints, size=(N, K))
    ws = np.full((N, K // 32), 127, dtype=np.uint8)
    xv = rng.integers(-3, 4, size=(T, K)).astype(np.float32)
    x = F.f32_to_bf16_rne(xv)
    got = G.gemm_mxfp8_ref(x, wq8, ws)
    wv = F.mxfp8_dequant_f64(wq8, ws)
    assert set(np.unique(wv)) <= {0.0, 1.0, 2.0, 3.0, 4.0, -1.0, -2.0, -3.0}
    bf = G.gemm_bruteforce(F.bf16_bits_to_f64(x).tolist(), wv.tolist())
    assert np.array_equal(got, np.array(bf))
    assert np.array_equal(got, np.round(got))


def test_e4m3_output_reference_and_bound():
    """The E4M3-output GEMM reference: integer operands give exact sums, so
    with a power-of-two scale the codes are the rounding of exact values
    (checked against the brute force), saturation caps them at +-448, and the
    acceptance bound passes the exact codes and fails codes one step off."""
    rng = np.random.default_rng(11)
    T, N, K = 3, 8, 96
    x = rng.integers(-3, 4, size=(T, K)).astype(np.float32)
    w = rng.integers(-3, 4, size=(N, K)).astype(np.float32)
    xb, wb = workloads.to_bf16_bits(x), workloads.to_bf16_bits(w)
    brute = np.array(G.gemm_bruteforce(x.tolist(), w.tolist()))
    for scale in (1.0, 0.25, 8.0):
        y, codes = G.gemm_bf16_e4m3_ref(xb, wb, scale)
        assert np.array_equal(y, np.clip(brute * scale, -448, 448))
        assert np.array_equal(codes, F.e4m3_rne_sat(np.clip(brute * scale, -448, 448)))
        assert G.e4m3_out_violation_ratio(codes, brute, K, scale) <= 1.0
    y, codes = G.gemm_bf16_e4m3_ref(xb, wb, 8.0)
    assert np.all(np.abs(F.e4m3_value(codes)) <= 448) and np.any(np.abs(brute * 8.0) > 448)
    # a code one step away from a large value breaks the bound
    big = np.array([[300.0]])
    good = F.e4m3_rne_sat(big)
    off = (good.astype(np.int64) + 2).astype(np.uint8)  # two E4M3 steps up: 352 instead of 288/320
    assert G.e4m3_out_violation_ratio(good, big, 1, 1.0) <= 1.0
    assert G.e4m3_out_violation_ratio(off, big, 1, 1.0) > 1.0


def test_chain_reference_is_the_composed_product():
    """Signed two-term selections keep every chain value a small integer, so
    the chain's outputs are exactly the composition of the plain products
    (brute force, step by step), and a value that bf16 cannot hold is refused."""
    rng = np.random.default_rng(12)
    T, dims = 3, [64, 32, 96, 64]
    x = rng.integers(-1, 2, size=(T, dims[0])).astype(np.float32)
    ws = []
    for i in range(len(dims) - 1):
        w = np.zeros((dims[i + 1], dims[i]), dtype=np.float32)
        for n in range(dims[i + 1]):
            a, b = rng.choice(dims[i], size=2, replace=False)
            w[n, a], w[n, b] = rng.choice([-1.0, 1.0]), rng.choice([-1.0, 1.0])
        ws.append(w)
    outs = G.gemm_chain_ref(workloads.to_bf16_bits(x), [workloads.to_bf16_bits(w) for w in ws])
    a = x.astype(np.float64)
    for i, w in enumerate(ws):
        a = np.array(G.gemm_bruteforce(a.tolist(), w.tolist()))
        assert np.array_equal(outs[i], a)
    ones_x = workloads.to_bf16_bits(np.ones((1, 257), dtype=np.float32))
    ones_w = workloads.to_bf16_bits(np.ones((16, 257), dtype=np.float32))
    with pytest.raises(ValueError):  # 257 needs nine significant bits
        G.gemm_chain_ref(ones_x, [ones_w])
