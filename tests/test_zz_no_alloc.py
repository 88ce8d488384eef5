"""skgemm_bf16_noalloc: the entry point that allocates nothing.

Its split-K partials and counters live in a fixed per-GPU scratch array. The
GPU test calls it through the C ABI and checks it against skgemm_bf16 (the
same kernels: identical bits) and the fp64 oracle, on calls in a row whose
sizes shrink, and inside a captured graph replayed between eager calls. The
CPU test checks that a call the scratch cannot serve fails before any device
work.
"""

import numpy as np
import pytest

import split_reduction_amd as sk
from oracle import gemm as G
from tests.gpu_util import (assert_parity, checked_bits, log, sentinel_bf16, to_dev_bf16, torch)
import workloads


def test_noalloc_rejects_oversized_calls_before_device_work():
    lib = sk.lib()
    a = 1 << 20  # an aligned fake address: these calls fail their checks first
    # 8 ranks x 128 rows x 16384 features x 4 bytes = 64 MiB of partials
    assert lib.skgemm_bf16_noalloc(a, a, a, 128, 16384, 16384, 8, None) == sk.SKGEMM_ESCRATCH
    assert lib.skgemm_bf16_noalloc(a, a, a, 1, 16, 96, 3, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_bf16_noalloc(a + 8, a, a, 1, 16, 64, 1, None) == sk.SKGEMM_EALIGN
    assert lib.skgemm_bf16_noalloc(None, None, None, 0, 16, 64, 1, None) == sk.SKGEMM_OK
    assert "scratch" in sk.strerror(sk.SKGEMM_ESCRATCH)


# (T, N, K, split_k), largest first: the persistent kernel (T=32 K=7168
# N=18432), the wide kernel over two token blocks (T=200), the wide kernel
# (T=64), and a persistent call with a smaller N.
CASES = [(32, 18432, 7168, 8), (200, 2048, 2048, 4), (64, 4096, 2048, 4), (12, 1024, 7168, 4)]


@pytest.mark.gpu
def test_noalloc_matches_bf16_on_calls_in_a_row():
    t = torch()
    for i, (T, N, K, S) in enumerate(CASES):
        tac = sk.skgemm_tactic_for(T, N, K, S)
        log(f"noalloc call {i}: T={T} N={N} K={K} S={S} tactic={tac}")
        assert tac["kind"] in ("stream", "wide"), tac  # kernels with a split-K workspace
        x, w = workloads.small_bf16_case(T, K, N, seed=9700 + i)
        W, X = to_dev_bf16(w), to_dev_bf16(x)
        C0, C1 = sentinel_bf16(T, N), sentinel_bf16(T, N)
        sk.skgemm_bf16_noalloc(W, X, C0, T, N, K, S)
        sk.skgemm_bf16(W, X, C1, T, N, K, S)
        t.cuda.synchronize()
        got, want = checked_bits(C0), checked_bits(C1)
        assert np.array_equal(got, want), f"call {i}: differs from skgemm_bf16"
        assert_parity(got, G.gemm_bf16_ref(x, w), K, f"noalloc call {i}")


@pytest.mark.gpu
def test_noalloc_in_a_graph_between_eager_calls():
    """Captured without any reserve; every replay gives the eager bits, with
    eager no-allocation calls of another size between the replays."""
    t = torch()
    T, N, K, S = 32, 4096, 7168, 8
    x, w = workloads.small_bf16_case(T, K, N, seed=9710)
    W, X = to_dev_bf16(w), to_dev_bf16(x)
    s = t.cuda.Stream()
    log(f"noalloc graph: T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S)}")
    with t.cuda.stream(s):
        eager = sentinel_bf16(T, N)
        sk.skgemm_bf16_noalloc(W, X, eager, T, N, K, S, s)
    t.cuda.synchronize()
    eager_bits = checked_bits(eager)
    assert_parity(eager_bits, G.gemm_bf16_ref(x, w), K, "noalloc eager")
    C = sentinel_bf16(T, N)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=s):
        sk.skgemm_bf16_noalloc(W, X, C, T, N, K, S, s)
    x2, w2 = workloads.small_bf16_case(12, 1024, 1024, seed=9711)
    W2, X2 = to_dev_bf16(w2), to_dev_bf16(x2)
    C2 = sentinel_bf16(12, 1024)
    for rep in range(3):
        with t.cuda.stream(s):
            C.fill_(float("nan"))
            g.replay()
        t.cuda.synchronize()
        assert np.array_equal(checked_bits(C), eager_bits), f"replay {rep}"
        with t.cuda.stream(s):
            sk.skgemm_bf16_noalloc(W2, X2, C2, 12, 1024, 1024, 4, s)
        t.cuda.synchronize()
        assert_parity(checked_bits(C2), G.gemm_bf16_ref(x2, w2), 1024, f"eager between replays {rep}")
    del g
