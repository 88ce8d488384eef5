"""GPU parity of the chained GEMM launch (skgemm_bf16_chain).

A chain multiplies each step's stored bf16 output by the next step's
weights. Integer chains (signed two-term selections of small integers) keep
every value exactly representable, so the whole chain must equal the oracle's
chain bit for bit; random chains of the decode shapes are checked step by step
against the oracle applied to the GPU's own stored input of that step.
"""

import numpy as np
import pytest

import split_reduction_amd as sk
from oracle import formats as F
from oracle import gemm as G
from tests.gpu_util import DEV, SENTINEL, assert_parity, bf16_bits, log, to_dev_bf16, torch
import workloads

pytestmark = pytest.mark.gpu


def selection_weights(rng, n, k, terms=2):
    w = np.zeros((n, k), dtype=np.float32)
    for r in range(n):
        cols = rng.choice(k, size=terms, replace=False)
        w[r, cols] = rng.choice([-1.0, 1.0], size=terms)
    return workloads.to_bf16_bits(w)


def run_chain(x_bits, w_bits, dims, S):
    t = torch()
    T = x_bits.shape[0]
    Ws = [to_dev_bf16(w) for w in w_bits]
    Cs = [t.full((T, d), SENTINEL, dtype=t.int16, device=DEV).view(t.bfloat16) for d in dims[1:]]
    sk.skgemm_bf16_chain(Ws, to_dev_bf16(x_bits), Cs, dims, T, S)
    t.cuda.synchronize()
    outs = [bf16_bits(c) for c in Cs]
    for i, o in enumerate(outs):
        assert not np.any(o == SENTINEL), f"step {i}: outputs never written"
    return outs


# (T, dims, split_k): both folds (T <= 8 and 9..16), every split, steps with
# fewer tiles than workgroups and tile counts that are not a multiple of the
# grid, growing and shrinking widths, a single step.
EXACT = [
    (8, [7168, 2048, 7168, 2048, 7168, 2048, 7168, 2048, 7168], 4),
    (1, [1024, 4096, 512, 2048], 1),
    (5, [2048, 1024, 3072, 256, 2048], 2),
    (12, [1024, 7168, 1024, 1536], 8),
    (16, [4096, 768, 4096], 4),
    (3, [512, 9216], 8),
]


@pytest.mark.parametrize("T,dims,S", EXACT)
def test_chain_integer_exact(T, dims, S):
    rng = np.random.default_rng(9900 + T + len(dims) + S)
    log(f"chain exact T={T} dims={dims} S={S}")
    x = workloads.to_bf16_bits(rng.integers(-1, 2, size=(T, dims[0])).astype(np.float32))
    ws = [selection_weights(rng, dims[i + 1], dims[i]) for i in range(len(dims) - 1)]
    want = G.gemm_chain_ref(x, ws)
    got = run_chain(x, ws, dims, S)
    for i in range(len(ws)):
        assert np.array_equal(F.bf16_bits_to_f64(got[i]), want[i]), f"step {i}"


def test_chain_dense_single_step_exact():
    """One step with dense small integers: every FP32 order is exact, so the
    rank-order sum must give the rounded exact value everywhere."""
    for (T, K, N, S) in [(8, 1024, 2048, 4), (16, 1024, 512, 8), (1, 512, 256, 1)]:
        log(f"chain one dense step T={T} K={K} N={N} S={S}")
        x, w = workloads.integer_bf16_case(T, K, N, seed=9950 + T + S)
        exact = G.gemm_bf16_ref(x, w)
        want = F.f32_to_bf16_rne(exact.astype(np.float32))
        got = run_chain(x, [w], [K, N], S)[0]
        assert np.array_equal(F.bf16_bits_to_f64(got), F.bf16_bits_to_f64(want))


@pytest.mark.parametrize("T,S", [(8, 4), (16, 4), (2, 8)])
def test_chain_decode_shapes_stepwise(T, S):
    """Eight steps alternating K=7168 -> N=2048 and K=2048 -> N=7168 (the
    T=8, K=7168, N=2048 decode shape and its transpose), random weights:
    every step within the bound of the oracle applied to its stored input."""
    dims = [7168, 2048] * 4 + [7168]
    rng = np.random.default_rng(9970 + T)
    x = workloads.to_bf16_bits(rng.standard_normal((T, dims[0]), dtype=np.float32))
    ws = [workloads.to_bf16_bits(rng.standard_normal((dims[i + 1], dims[i]), dtype=np.float32)
                                 * np.float32(1.0 / np.sqrt(dims[i]))) for i in range(len(dims) - 1)]
    log(f"chain decode shapes T={T} S={S}")
    got = run_chain(x, ws, dims, S)
    a = x
    for i, w in enumerate(ws):
        assert_parity(got[i], G.gemm_bf16_ref(a, w), dims[i], f"chain step {i}")
        a = got[i]


def test_chain_repeated_launches_and_health():
    """The barrier words return to their start state: back-to-back chains on
    one stream give identical bits, and no barrier wait runs out."""
    T, dims, S = 8, [2048, 1024, 2048, 512], 2
    rng = np.random.default_rng(9990)
    x = workloads.to_bf16_bits(rng.standard_normal((T, dims[0]), dtype=np.float32))
    ws = [workloads.to_bf16_bits(rng.standard_normal((dims[i + 1], dims[i]), dtype=np.float32) * np.float32(0.03))
          for i in range(len(dims) - 1)]
    sk.skgemm_health()
    first = run_chain(x, ws, dims, S)
    for rep in range(4):
        again = run_chain(x, ws, dims, S)
        for i in range(len(ws)):
            assert np.array_equal(again[i], first[i]), f"rep {rep} step {i}"
    assert sk.skgemm_health()["timeouts"] == 0


@pytest.mark.parametrize("T,dims,S", [
    (8, [7168, 2048, 7168, 2048, 7168, 2048, 7168, 2048, 7168], 4),
    (5, [1024, 2048, 1024, 3072, 512, 2048], 2),
    (16, [2048, 1024, 2048, 1024], 8),
])
def test_chain_ping_pong_buffers(T, dims, S):
    """Outputs alternate between two buffers, so step i overwrites the memory
    that step i-1 read as its activations (every step's C overlaps the C of
    two steps before). Integer chains: the last two outputs, still held in the
    two buffers, equal the oracle's chain bit for bit, launch after launch."""
    t = torch()
    rng = np.random.default_rng(9990 + T + S)
    log(f"chain ping-pong T={T} dims={dims} S={S}")
    x = workloads.to_bf16_bits(rng.integers(-1, 2, size=(T, dims[0])).astype(np.float32))
    ws = [selection_weights(rng, dims[i + 1], dims[i]) for i in range(len(dims) - 1)]
    want = G.gemm_chain_ref(x, ws)
    L = len(ws)
    width = max(dims[1:])
    bufs = [t.full((T * width,), SENTINEL, dtype=t.int16, device=DEV) for _ in range(2)]
    Cs = [bufs[i % 2][:T * dims[i + 1]].view(T, dims[i + 1]).view(t.bfloat16) for i in range(L)]
    Wd = [to_dev_bf16(w) for w in ws]
    for rep in range(3):
        sk.skgemm_bf16_chain(Wd, to_dev_bf16(x), Cs, dims, T, S)
        t.cuda.synchronize()
        for i in (L - 2, L - 1):
            if i < 0:
                continue
            got = bf16_bits(Cs[i])
            assert np.array_equal(F.bf16_bits_to_f64(got), want[i]), f"rep {rep} step {i}"
