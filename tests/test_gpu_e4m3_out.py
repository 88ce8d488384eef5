"""GPU parity of the E4M3-output GEMM (skgemm_bf16_e4m3) against the oracle.

The codes C8 are the E4M3FN rounding of the FP32 sum times the caller's
scale, saturated to +-448. Integer operands with a power-of-two scale make
every FP32 step exact, so there the codes must equal the oracle's rounding of
the exact values, bit for bit (ties included: integer sums land on E4M3
midpoints); random operands are held to the bound derived in
oracle.gemm.e4m3_out_violation_ratio. Every kernel kind's output stage is
pinned in turn.
"""

import numpy as np
import pytest

import split_reduction_amd as sk
from oracle import formats as F
from oracle import gemm as G
from tests.gpu_util import DEV, log, to_dev_bf16, torch
import workloads

pytestmark = pytest.mark.gpu

SENT8 = 0x7F  # an E4M3 NaN code: the output stage never writes it (values are saturated)


def run_e4m3(x, w, S, scale, W=None):
    t = torch()
    T, K = x.shape
    N = w.shape[0] if W is None else W.shape[0]
    C8 = t.full((T, N), SENT8, dtype=t.uint8, device=DEV)
    sk.skgemm_bf16_e4m3(to_dev_bf16(w) if W is None else W, to_dev_bf16(x), C8, scale, T, N, K, S)
    t.cuda.synchronize()
    c = C8.cpu().numpy()
    assert not np.any(c == SENT8), f"{int(np.count_nonzero(c == SENT8))} outputs never written"
    return c


def same_values(a, b):
    """Codes equal as values (+0 and -0 are the same zero)."""
    return np.array_equal(F.e4m3_value(a), F.e4m3_value(b))


# (T, N, K, split_k, pinned kind): every kernel's output stage
KINDS = [(5, 512, 1024, 4, 2), (1, 256, 1024, 2, 2), (24, 1024, 2048, 8, 1), (8, 2048, 2048, 4, 1),
         (40, 512, 2048, 4, 3), (100, 256, 1024, 2, 3), (17, 160, 1024, 2, 0), (3, 96, 512, 1, 0)]


@pytest.mark.parametrize("T,N,K,S,kind", KINDS)
def test_e4m3_out_integer_exact(T, N, K, S, kind, tune):
    tune("kind", kind)
    tac = sk.skgemm_tactic_for(T, N, K, S)
    log(f"e4m3 out exact T={T} N={N} K={K} S={S} kind={kind} tactic={tac}")
    x, w = workloads.integer_bf16_case(T, K, N, seed=9800 + T + S, mag=3)
    for scale in (0.0625, 1.0):  # at 1.0 many sums exceed 448: saturation
        _, want = G.gemm_bf16_e4m3_ref(x, w, scale)
        got = run_e4m3(x, w, S, scale)
        assert same_values(got, want), f"kind {kind} scale {scale}"


@pytest.mark.parametrize("name", ["bf16_t8_k7168_n2048", "bf16_t32_k7168_n18432", "bf16_t1_k1024_n1024"])
def test_e4m3_out_workload_parity(name):
    w = workloads.WORKLOADS[name]
    x = workloads.gen_x(w)
    wb = workloads.gen_w_bf16(w)
    ref = G.gemm_bf16_ref(x, wb)
    scale = 448.0 / float(np.max(np.abs(ref)))  # the largest output maps to the top of the range
    scale = float(np.float32(scale))
    log(f"e4m3 out {name} scale={scale:.6g} tactic={sk.skgemm_tactic_for(w.T, w.N, w.K, w.split_k)}")
    got = run_e4m3(x, wb, w.split_k, scale)
    ratio = G.e4m3_out_violation_ratio(got, ref, w.K, scale)
    log(f"  max |err|/bound = {ratio:.4f}")
    assert ratio <= 1.0
    # most codes are the rounding of the exact value (a few near midpoints may not be)
    _, want = G.gemm_bf16_e4m3_ref(x, wb, scale)
    agree = np.mean(F.e4m3_value(got) == F.e4m3_value(want))
    log(f"  codes equal to the rounded exact value: {agree:.4f}")
    assert agree > 0.99


def test_e4m3_out_rejects_bad_scale():
    t = torch()
    W = t.zeros((32, 64), dtype=t.bfloat16, device=DEV)
    X = t.zeros((2, 64), dtype=t.bfloat16, device=DEV)
    C8 = t.full((2, 32), 5, dtype=t.uint8, device=DEV)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(sk.SkgemmError) as e:
            sk.skgemm_bf16_e4m3(W, X, C8, bad, 2, 32, 64, 1)
        assert e.value.code == sk.SKGEMM_EINVAL
    t.cuda.synchronize()
    assert np.all(C8.cpu().numpy() == 5)
