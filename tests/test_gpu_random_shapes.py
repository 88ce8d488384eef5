"""Parity against the oracle on seeded random shapes.

Every call goes through the C ABI with the library's own kernel choice, over
token counts 1..130, output widths that are multiples of 16, rank slices of
several lengths and split_k in {1, 2, 4, 8}, for the three weight formats.
The outputs start as a NaN sentinel, so an output element that no kernel
writes fails the test as surely as a wrong one.
"""

import numpy as np
import pytest

import split_reduction_amd as sk
from oracle import gemm as G
from tests.gpu_util import assert_parity, log, run_bf16, run_mxfp4, run_mxfp8
import workloads

pytestmark = pytest.mark.gpu

N_CASES = 96


def _shapes():
    """(fmt, T, N, K, S) drawn from one seeded generator; K a multiple of
    128 * S (every format's shape rule), at most 8192."""
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(N_CASES):
        fmt = ("bf16", "mxfp4", "mxfp8")[i % 3]
        S = int(rng.choice([1, 2, 4, 8]))
        T = int(rng.choice([1, 2, 3, 5, 8, 9, 15, 16, 17, 24, 31, 32, 33, 48, 64, 100, 128, 130]))
        N = 16 * int(rng.integers(1, 257))            # 16 .. 4096
        K = 128 * S * int(rng.integers(1, 64 // S + 1))  # up to 8192
        out.append((fmt, T, N, K, S))
    return out


@pytest.mark.parametrize("case", list(enumerate(_shapes())), ids=lambda c: f"{c[0]}-{c[1][0]}-T{c[1][1]}-N{c[1][2]}-K{c[1][3]}-S{c[1][4]}")
def test_random_shape_parity(case):
    i, (fmt, T, N, K, S) = case
    wf = {"bf16": 0, "mxfp4": 1, "mxfp8": 2}[fmt]
    log(f"random shape {i}: {fmt} T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S, wf)}")
    seed = 90000 + i
    if fmt == "bf16":
        x, w = workloads.small_bf16_case(T, K, N, seed)
        c, ref = run_bf16(x, w, S), G.gemm_bf16_ref(x, w)
    elif fmt == "mxfp4":
        x, wq, ws = workloads.small_mxfp4_case(T, K, N, seed)
        c, ref = run_mxfp4(x, wq, ws, S), G.gemm_mxfp4_ref(x, wq, ws)
    else:
        x, wq8, ws = workloads.small_mxfp8_case(T, K, N, seed)
        c, ref = run_mxfp8(x, wq8, ws, S), G.gemm_mxfp8_ref(x, wq8, ws)
    assert_parity(c, ref, K, f"random shape {i}")
