"""GPU parity of the split-K GEMM against the fp64 oracle.

Every case goes through the C ABI (``split_reduction_amd`` binding). The
acceptance bound is |C - ref| <= 2^-7 |ref| + 1e-3 sqrt(K) rms(ref), element
by element; exact special cases (integer operands, identity, one-hot rows)
must match bit for bit.
"""

import numpy as np
import pytest

import split_reduction_amd as sk
from oracle import formats as F
from oracle import gemm as G
from tests.gpu_util import (DEV, assert_parity, bf16_bits, checked_bits, empty_bf16, log, run_bf16,
                            run_mxfp4, run_mxfp8, sentinel_bf16, to_dev_bf16, to_dev_u8, torch)
import workloads

pytestmark = pytest.mark.gpu

# (T, N, K, split_k): shapes chosen to reach every instantiated workgroup
# shape (tile 16 / 32 / 64 and the X-sharing tile), ragged T, several LDS
# chunks per K slice, uneven step counts per wave, T above one 128-row block,
# and K = 0.
BF16_CASES = [
    (1, 1024, 1024, 4),
    (3, 4096, 512, 4),
    (24, 8192, 512, 4),
    (40, 8192, 1024, 8),
    (64, 8192, 512, 4),
    (100, 8192, 512, 4),
    (128, 2048, 2048, 1),
    (17, 256, 4096, 2),
    (128, 512, 8192, 2),
    (5, 160, 96, 1),
    (9, 48, 192, 2),
    (200, 96, 256, 2),
    (2, 64, 0, 1),
    (2, 64, 0, 4),
]


@pytest.mark.parametrize("T,N,K,S", BF16_CASES)
def test_bf16_parity_small(T, N, K, S):
    log(f"bf16 parity T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S)}")
    x, w = workloads.small_bf16_case(T, K, N, seed=1000 + T + N + K + S)
    c = run_bf16(x, w, S)
    ref = G.gemm_bf16_ref(x, w)
    if K == 0:
        assert np.all(F.bf16_bits_to_f64(c) == 0.0)
        return
    assert_parity(c, ref, K, f"T={T} N={N} K={K} S={S}")


@pytest.mark.parametrize("S", [1, 2, 4, 8])
@pytest.mark.parametrize("T", [1, 5, 16, 33, 128])
def test_bf16_integer_operands_bit_exact(T, S):
    N, K = 512, 1024
    log(f"bf16 integer exact T={T} S={S}")
    x, w = workloads.integer_bf16_case(T, K, N, seed=2000 + T * 10 + S)
    c = run_bf16(x, w, S)
    exact = G.gemm_bf16_ref(x, w)  # integers below 2^24: every FP32 order is exact
    assert np.max(np.abs(exact)) < 2**24
    ref = F.f32_to_bf16_rne(exact.astype(np.float32))
    assert np.array_equal(c, ref)


def test_bf16_identity_and_permutation_bit_exact():
    rng = np.random.default_rng(31)
    T, K = 7, 512
    x = workloads.to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    log("bf16 identity")
    eye = workloads.to_bf16_bits(np.eye(K, dtype=np.float32))
    c = run_bf16(x, eye, 2)
    assert np.array_equal(F.bf16_bits_to_f64(c), F.bf16_bits_to_f64(x))
    log("bf16 one-hot permutation")
    N = 256
    perm = rng.permutation(K)[:N]
    w = np.zeros((N, K), dtype=np.float32)
    w[np.arange(N), perm] = 1.0
    c = run_bf16(x, workloads.to_bf16_bits(w), 4)
    assert np.array_equal(F.bf16_bits_to_f64(c), F.bf16_bits_to_f64(x)[:, perm])


def test_bf16_repeatable_bits():
    w = workloads.WORKLOADS["bf16_t8_k7168_n2048"]
    x = workloads.gen_x(w)
    wb = workloads.gen_w_bf16(w)
    log("bf16 determinism on the T=8 K=7168 N=2048 workload")
    W = to_dev_bf16(wb)
    first = run_bf16(x, None, w.split_k, W=W)
    for _ in range(3):
        assert np.array_equal(run_bf16(x, None, w.split_k, W=W), first)


def test_bf16_writes_only_c_once():
    T, N, K, S = 5, 320, 1024, 4
    log("bf16 write bounds")
    x, w = workloads.small_bf16_case(T, K, N, seed=41)
    t = torch()
    sentinel = 0x7FC1  # a NaN pattern the kernel never produces from finite inputs
    buf = t.full((T + 3, N), sentinel, dtype=t.int16, device=DEV).view(t.bfloat16)
    C = buf[:T]
    sk.skgemm_bf16(to_dev_bf16(w), to_dev_bf16(x), C, T, N, K, S)
    t.cuda.synchronize()
    allb = bf16_bits(buf)
    assert np.all(allb[T:] == sentinel)
    assert not np.any(allb[:T] == sentinel)
    assert_parity(allb[:T], G.gemm_bf16_ref(x, w), K, "bounded write")


def test_bf16_rejects_bad_arguments_without_touching_c():
    t = torch()
    log("bf16 argument errors")
    W = t.zeros((32, 96), dtype=t.bfloat16, device=DEV)
    X = t.zeros((2, 96), dtype=t.bfloat16, device=DEV)
    C = t.full((2, 32), 7, dtype=t.int16, device=DEV).view(t.bfloat16)
    for args, code in [((2, 32, 96, 2), sk.SKGEMM_ESHAPE), ((2, 32, 96, 3), sk.SKGEMM_EINVAL),
                       ((2, 30, 96, 1), sk.SKGEMM_ESHAPE)]:
        with pytest.raises(sk.SkgemmError) as e:
            sk.skgemm_bf16(W, X, C, *args)
        assert e.value.code == code
    with pytest.raises(sk.SkgemmError) as e:
        sk.skgemm_bf16(W.data_ptr() + 2, X, C, 2, 32, 96, 1)
    assert e.value.code == sk.SKGEMM_EALIGN
    # tensors the binding cannot pass: host memory, a strided view, a short buffer
    for args in [(W, X.cpu(), C), (W, X, C.t()), (W[:31], X, C), (W, X, C.view(-1)[:63])]:
        with pytest.raises(sk.SkgemmError) as e:
            sk.skgemm_bf16(*args, 2, 32, 96, 1)
        assert e.value.code == sk.SKGEMM_EINVAL
    t.cuda.synchronize()
    assert np.all(bf16_bits(C) == 7)


def test_bf16_two_streams():
    t = torch()
    w = workloads.WORKLOADS["bf16_t8_k7168_n2048"]
    x = workloads.gen_x(w)
    wb = workloads.gen_w_bf16(w)
    ref = G.gemm_bf16_ref(x, wb)
    log("bf16 on two streams at once")
    W, X = to_dev_bf16(wb), to_dev_bf16(x)
    s1, s2 = t.cuda.Stream(), t.cuda.Stream()
    outs = []
    t.cuda.synchronize()
    for s in (s1, s2):
        with t.cuda.stream(s):
            C = empty_bf16(w.T, w.N)
            for _ in range(4):
                sk.skgemm_bf16(W, X, C, w.T, w.N, w.K, w.split_k)
            outs.append(C)
    t.cuda.synchronize()
    for C in outs:
        assert_parity(bf16_bits(C), ref, w.K, "two streams")


# ---------------------------------------------------------------- MXFP4 ----

MX_CASES = [
    (1, 256, 512, 1),
    (3, 4096, 512, 4),
    (16, 1024, 1024, 2),
    (40, 2048, 1024, 4),
    (128, 512, 2048, 2),
    (130, 64, 256, 1),
    (2, 64, 0, 4),  # empty sum: zeros
]


def assert_zero_or_parity(c, ref, K, what):
    """K == 0 is an empty sum, stored as +0 everywhere; otherwise parity."""
    if K == 0:
        assert np.all(c == 0), f"{what}: an empty sum must store +0"
        return
    assert_parity(c, ref, K, what)


@pytest.mark.parametrize("T,N,K,S", MX_CASES)
def test_mxfp4_parity_small(T, N, K, S):
    log(f"mxfp4 parity T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S, True)}")
    x, wq, ws = workloads.small_mxfp4_case(T, K, N, seed=3000 + T + N + K + S)
    c = run_mxfp4(x, wq, ws, S)
    assert_zero_or_parity(c, G.gemm_mxfp4_ref(x, wq, ws), K, f"mxfp4 T={T} N={N} K={K} S={S}")


@pytest.mark.parametrize("S", [1, 4])
def test_mxfp4_integer_operands_bit_exact(S):
    T, N, K = 20, 256, 1024
    log(f"mxfp4 integer exact S={S}")
    rng = np.random.default_rng(50 + S)
    x = workloads.to_bf16_bits(rng.integers(-3, 4, size=(T, K)).astype(np.float32))
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ws = np.full((N, K // 32), 127, dtype=np.uint8)  # scale 1: weights in {0, +-0.5, ..., +-6}
    c = run_mxfp4(x, wq, ws, S)
    exact = G.gemm_mxfp4_ref(x, wq, ws)  # multiples of 0.5 below 2^22: exact in FP32
    assert np.max(np.abs(exact)) < 2**22
    assert np.array_equal(c, F.f32_to_bf16_rne(exact.astype(np.float32)))


MX8_CASES = [
    (1, 256, 512, 1),
    (3, 4096, 512, 4),
    (16, 1024, 1024, 2),
    (40, 2048, 1024, 4),
    (128, 512, 2048, 2),
    (130, 64, 256, 1),
    (2, 64, 0, 4),  # empty sum: zeros
]


@pytest.mark.parametrize("T,N,K,S", MX8_CASES)
def test_mxfp8_parity_small(T, N, K, S):
    log(f"mxfp8 parity T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S, 2)}")
    x, wq8, ws = workloads.small_mxfp8_case(T, K, N, seed=3500 + T + N + K + S)
    assert_zero_or_parity(run_mxfp8(x, wq8, ws, S), G.gemm_mxfp8_ref(x, wq8, ws), K,
                          f"mxfp8 T={T} N={N} K={K} S={S}")


@pytest.mark.parametrize("S", [1, 4])
def test_mxfp8_integer_operands_bit_exact(S):
    T, N, K = 20, 256, 1024
    log(f"mxfp8 integer exact S={S}")
    rng = np.random.default_rng(60 + S)
    x = workloads.to_bf16_bits(rng.integers(-3, 4, size=(T, K)).astype(np.float32))
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4, 0x80], dtype=np.uint8)  # 0 +-1..4, -0
    wq8 = rng.choice(ints, size=(N, K))
    ws = np.full((N, K // 32), 127, dtype=np.uint8)
    exact = G.gemm_mxfp8_ref(x, wq8, ws)
    c = run_mxfp8(x, wq8, ws, S)
    assert np.array_equal(F.bf16_bits_to_f64(c), F.bf16_bits_to_f64(F.f32_to_bf16_rne(exact.astype(np.float32))))


# Unfolded block-scaled tiles of the cluster kernel (T = 9..32) at slices of
# several lengths. The scales change from block to block, so a scale taken
# from the wrong block, row or rank slice changes the exact result.
BLOCK_SCALE_CASES = [
    # (T, K, S): rank slice ks = K / S
    (16, 1024, 2),   # ks 512
    (16, 1280, 2),   # ks 640
    (9, 3584, 4),    # ks 896
    (16, 4096, 2),   # ks 2048
    (20, 4352, 2),   # ks 2176, two token tiles
    (16, 768, 2),    # ks 384
    (12, 1152, 2),   # ks 576: MXFP8 only (MXFP4 needs K % (128 * split_k) == 0)
]


def _block_scale_case(fmt, T, K, N, seed):
    rng = np.random.default_rng(seed)
    x = workloads.to_bf16_bits(rng.integers(-3, 4, size=(T, K)).astype(np.float32))
    ws = rng.integers(125, 130, size=(N, K // 32), dtype=np.uint8)  # 2^-2 .. 2^2 per block
    if fmt == "mxfp4":
        wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        return x, wq, ws, G.gemm_mxfp4_ref(x, wq, ws)
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0, 0xC4, 0x80], dtype=np.uint8)
    wq8 = rng.choice(ints, size=(N, K))
    return x, wq8, ws, G.gemm_mxfp8_ref(x, wq8, ws)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("T,K,S", BLOCK_SCALE_CASES)
def test_cluster_block_scales_bit_exact(fmt, T, K, S, tune):
    """Integer activations, small-integer weights and per-block power-of-two
    scales: every product and partial sum is exact in FP32, so the bf16
    output is the RNE rounding of the exact result, bit for bit."""
    N = 256
    step = 128 if fmt == "mxfp4" else 64
    if (K // S) % step:
        pytest.skip("slice not a whole number of load steps")
    tune("kind", 2)
    wf = 1 if fmt == "mxfp4" else 2
    tac = sk.skgemm_tactic_for(T, N, K, S, wf)
    log(f"{fmt} block scales T={T} K={K} S={S} ks={K // S} tactic={tac}")
    assert tac["kind"] == "cluster" and tac["fold"] == 1
    x, wq, ws, exact = _block_scale_case(fmt, T, K, N, seed=7100 + T + K + S + wf)
    assert np.max(np.abs(exact)) < 2**22
    c = run_mxfp4(x, wq, ws, S) if fmt == "mxfp4" else run_mxfp8(x, wq, ws, S)
    want = F.f32_to_bf16_rne(exact.astype(np.float32))
    assert np.array_equal(F.bf16_bits_to_f64(c), F.bf16_bits_to_f64(want))


def test_mxfp8_batched_and_workload():
    t = torch()
    T, N, K, S, L = 16, 512, 2048, 4, 3
    cases = [workloads.small_mxfp8_case(T, K, N, seed=9600 + l) for l in range(L)]
    log(f"batched mxfp8 L={L} T={T} N={N} K={K} S={S}")
    Wq = to_dev_u8(np.stack([c[1] for c in cases]))
    Ws = to_dev_u8(np.stack([c[2] for c in cases]))
    X = to_dev_bf16(np.stack([c[0] for c in cases]))
    C = t.empty((L, T, N), dtype=t.bfloat16, device=DEV)
    sk.skgemm_mxfp8_batched(Wq, Ws, X, C, T, N, K, S, L, N * K, N * K // 32, T * K * 2, T * N * 2)
    t.cuda.synchronize()
    cb = bf16_bits(C)
    for l, (x, wq8, ws) in enumerate(cases):
        assert_parity(cb[l], G.gemm_mxfp8_ref(x, wq8, ws), K, f"mxfp8 batch {l}")
    w = workloads.WORKLOADS["mxfp8_t16_k7168_n4096"]
    log(f"workload {w.name} tactic={sk.skgemm_tactic_for(w.T, w.N, w.K, w.split_k, 2)}")
    x = workloads.gen_x(w)
    wq8, ws = workloads.gen_w_mxfp8(w)
    assert_parity(run_mxfp8(x, wq8, ws, w.split_k), G.gemm_mxfp8_ref(x, wq8, ws), w.K, w.name)


# ------------------------------------------------------ full workloads -----


@pytest.mark.parametrize("name", ["bf16_t1_k1024_n1024", "bf16_t8_k7168_n2048", "bf16_t32_k7168_n18432"])
def test_bf16_workload_full_parity(name):
    w = workloads.WORKLOADS[name]
    log(f"workload {name} tactic={sk.skgemm_tactic_for(w.T, w.N, w.K, w.split_k)}")
    x = workloads.gen_x(w)
    wb = workloads.gen_w_bf16(w)
    c = run_bf16(x, wb, w.split_k)
    assert_parity(c, G.gemm_bf16_ref(x, wb), w.K, name)


def test_mxfp4_workload_full_parity():
    w = workloads.WORKLOADS["mxfp4_t16_k7168_n4096"]
    log(f"workload {w.name} tactic={sk.skgemm_tactic_for(w.T, w.N, w.K, w.split_k, True)}")
    x = workloads.gen_x(w)
    wq, ws = workloads.gen_w_mxfp4(w)
    c = run_mxfp4(x, wq, ws, w.split_k)
    assert_parity(c, G.gemm_mxfp4_ref(x, wq, ws), w.K, w.name)


@pytest.fixture(scope="module")
def sweep_weights():
    """The K = N = 16384 sweep weights: bf16 bits on the host, the same on the
    device, and their exact float64 values (2 GiB, converted once for all T)."""
    w = workloads.sweep_workload(1)
    log("generating the K = N = 16384 sweep weights")
    wb = workloads.gen_w_bf16(w)
    w64 = F.bf16_bits_to_f64(wb)
    return wb, to_dev_bf16(wb), w64


@pytest.mark.parametrize("T", list(workloads.SWEEP_T))
def test_bf16_sweep_full_parity(T, sweep_weights):
    """Every one of the T x 16384 outputs of each sweep point against the fp64
    oracle, with the rms taken over the whole output (the kernels and split
    that the benchmark times: the library's own choice at split_k per T)."""
    wb, W, w64 = sweep_weights
    w = workloads.sweep_workload(T)
    log(f"sweep T={T} S={w.split_k} tactic={sk.skgemm_tactic_for(T, w.N, w.K, w.split_k)}")
    x = workloads.gen_x(w)
    c = run_bf16(x, None, w.split_k, W=W)
    ref = G.gemm_decoded_ref(x, w64)
    assert ref.shape == (T, w.N)
    assert_parity(c, ref, w.K, f"sweep T={T} (all {T * w.N} outputs)")


def test_graph_replays_match_eager():
    """Captured into a HIP graph (workspace reserved first), every replay gives
    the eager bits, with eager work and synchronisations between replays."""
    t = torch()
    w = workloads.WORKLOADS["bf16_t32_k7168_n18432"]
    T, N, K, S = 32, 2048, 7168, 8
    log("graph capture and replays, T=32 N=2048 K=7168 S=8")
    x, wb = workloads.small_bf16_case(T, K, N, seed=71)
    W, X = to_dev_bf16(wb), to_dev_bf16(x)
    eager = run_bf16(x, None, S, W=W)
    s = t.cuda.Stream()
    sk.skgemm_reserve(T, N, S, s)
    C = empty_bf16(T, N)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=s):
        sk.skgemm_bf16(W, X, C, T, N, K, S, s)
    for rep in range(4):
        C.zero_()
        g.replay()
        t.cuda.synchronize()
        assert np.array_equal(bf16_bits(C), eager), f"replay {rep}"
        # eager work on the default stream between replays
        other = run_bf16(x[:5], None, 4, W=W)
        assert other.shape == (5, N)
    assert w.K == K


def test_graph_replay_after_workspace_growth(tune):
    """A graph captured after skgemm_reserve keeps the workspace it was
    captured with: a later eager call that needs more space replaces the
    stream's workspace but must not free the old one, so later replays still
    give the eager bits."""
    t = torch()
    tune("kind", 1)  # the persistent kernel: a split-K workspace in every call
    T, N, K, S = 8, 1024, 4096, 4
    log(f"graph replay after workspace growth, T={T} N={N} K={K} S={S} "
        f"tactic={sk.skgemm_tactic_for(T, N, K, S)}")
    x, wb = workloads.small_bf16_case(T, K, N, seed=72)
    W, X = to_dev_bf16(wb), to_dev_bf16(x)
    s = t.cuda.Stream()
    sk.skgemm_reserve(T, N, S, s)
    C = empty_bf16(T, N)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=s):
        sk.skgemm_bf16(W, X, C, T, N, K, S, s)
    with t.cuda.stream(s):
        eager = sentinel_bf16(T, N)
        sk.skgemm_bf16(W, X, eager, T, N, K, S, s)
    t.cuda.synchronize()
    eager_bits = checked_bits(eager)
    # a larger call on the same stream grows (replaces) the workspace
    T2, N2, K2, S2 = 32, 8192, 4096, 8
    x2, w2 = workloads.small_bf16_case(T2, K2, N2, seed=73)
    W2, X2 = to_dev_bf16(w2), to_dev_bf16(x2)
    C2 = sentinel_bf16(T2, N2)
    with t.cuda.stream(s):
        sk.skgemm_bf16(W2, X2, C2, T2, N2, K2, S2, s)
    t.cuda.synchronize()
    assert_parity(checked_bits(C2), G.gemm_bf16_ref(x2, w2), K2, "the larger call")
    for rep in range(3):
        with t.cuda.stream(s):
            C.fill_(float("nan"))
            g.replay()
        t.cuda.synchronize()
        assert np.array_equal(bf16_bits(C), eager_bits), f"replay {rep}"
        with t.cuda.stream(s):  # eager work on the grown workspace between replays
            sk.skgemm_bf16(W2, X2, C2, T2, N2, K2, S2, s)
        t.cuda.synchronize()
    del g


# Every instantiated kernel shape, pinned through skgemm_set_override (the
# "stream" knob selects a persistent-kernel shape, "shape" a
# one-tile-per-workgroup shape), on shapes with ragged T, uneven step counts
# per wave and several tiles per wave column.
FORCED = (
    [{"kind": 1, "stream": i} for i in range(7)]
    + [{"kind": 0, "shape": i} for i in range(6)]
    + [{"kind": 2, "fold": f, "cluster_c": c} for f in (1, 2, 4, 8) for c in (1, 2)]
)


@pytest.mark.parametrize("env", FORCED, ids=lambda e: ",".join(f"{k}={v}" for k, v in e.items()))
def test_every_kernel_shape(env, tune):
    for k, v in env.items():
        tune(k, v)
    kind = {0: "tiled", 1: "stream", 2: "cluster"}[env["kind"]]
    bf16_cases = [(3, 512, 1792, 4), (24, 1024, 2048, 8), (17, 256, 7168, 2), (1, 4096, 512, 1),
                  (7, 96, 2048, 2), (2, 64, 1024, 8)]
    ran = 0

    def tactic(T, N, K, S, mx):
        # A forced kind that cannot take the shape (slice too short for its
        # waves, T beyond its token tiles) refuses it rather than falling back.
        try:
            return sk.skgemm_tactic_for(T, N, K, S, mx)
        except sk.SkgemmError as e:
            assert e.code == sk.SKGEMM_ESHAPE
            log(f"forced {env}: T={T} N={N} K={K} S={S} mx={mx} not applicable")
            return None

    for (T, N, K, S) in bf16_cases:
        tac = tactic(T, N, K, S, False)
        if tac is None:
            continue
        log(f"forced {env}: bf16 T={T} N={N} K={K} S={S} tactic={tac}")
        assert tac["kind"] == kind
        x, w = workloads.small_bf16_case(T, K, N, seed=5000 + T + S)
        assert_parity(run_bf16(x, w, S), G.gemm_bf16_ref(x, w), K, f"{env} T={T} S={S}")
        ran += 1
    for (T, N, K, S) in [(5, 512, 2048, 4), (30, 256, 1024, 2), (1, 128, 1024, 2), (5, 512, 8192, 2),
                         (20, 256, 2048, 1)]:
        tac = tactic(T, N, K, S, True)
        if tac is None:
            continue
        log(f"forced {env}: mxfp4 T={T} N={N} K={K} S={S} tactic={tac}")
        assert tac["kind"] == kind
        x, wq, ws = workloads.small_mxfp4_case(T, K, N, seed=6000 + T + S)
        assert_parity(run_mxfp4(x, wq, ws, S), G.gemm_mxfp4_ref(x, wq, ws), K, f"{env} mx T={T}")
        ran += 1
    for (T, N, K, S) in [(5, 512, 1024, 4), (30, 256, 512, 2), (1, 128, 1024, 2), (5, 512, 4096, 2),
                         (20, 256, 1024, 1)]:
        try:
            tac = sk.skgemm_tactic_for(T, N, K, S, 2)
        except sk.SkgemmError as e:
            assert e.code == sk.SKGEMM_ESHAPE
            continue
        log(f"forced {env}: mxfp8 T={T} N={N} K={K} S={S} tactic={tac}")
        assert tac["kind"] == kind
        x, wq8, ws = workloads.small_mxfp8_case(T, K, N, seed=6100 + T + S)
        assert_parity(run_mxfp8(x, wq8, ws, S), G.gemm_mxfp8_ref(x, wq8, ws), K, f"{env} mx8 T={T}")
        ran += 1
    assert ran >= 4


def test_cluster_integer_exact(tune):
    """The one-workgroup-per-tile kernel at every fold and split: integer
    operands make every FP32 order exact, so C is the RNE of the exact sum."""
    tune("kind", "2")
    for f in (1, 2, 4, 8):
        tune("fold", str(f))
        for (T, N, K, S) in [(1, 64, 1024, 4), (3, 32, 512, 2), (8, 48, 2048, 8), (16, 16, 256, 1),
                             (29, 32, 1024, 4)]:
            tac = sk.skgemm_tactic_for(T, N, K, S)
            log(f"cluster exact fold<={f}: T={T} N={N} K={K} S={S} tactic={tac}")
            x, w = workloads.integer_bf16_case(T, K, N, seed=7000 + 10 * f + T)
            got = run_bf16(x, w, S)
            exact = G.gemm_bf16_ref(x, w)
            assert np.max(np.abs(exact)) < 2**24
            want = F.f32_to_bf16_rne(exact.astype(np.float32))
            assert np.array_equal(F.bf16_bits_to_f64(got), F.bf16_bits_to_f64(want)), \
                f"fold<={f} T={T} S={S}"


@pytest.mark.parametrize("shape", ["1", "4", "5", "6"])
@pytest.mark.parametrize("wait", ["0", "1", "10000"])
def test_owner_handover(wait, shape, tune):
    """The persistent kernel's tile owners wait as usual, give up at once, or
    after one tick and hand their tiles to the last rank to arrive: results
    must be unchanged, several launches in a row (the counters end each
    launch at 0), and the health report holds well-formed records of the
    waits that ran out (none for the normal wait)."""
    tune("kind", "1")
    tune("stream", shape)
    tune("owner_wait", wait)
    # K slices of 1792, 512 and 512: every forced shape gives each of its
    # streaming waves at least one ring slot (two load steps) per tile.
    for (T, N, K, S) in [(8, 2048, 7168, 4), (24, 1024, 4096, 8), (3, 4096, 1024, 2)]:
        tac = sk.skgemm_tactic_for(T, N, K, S)
        log(f"owner hand-over wait={wait}: T={T} N={N} K={K} S={S} tactic={tac}")
        assert tac["kind"] == "stream" and tac["shape"] == int(shape)
        x, w = workloads.small_bf16_case(T, K, N, seed=8000 + T + S)
        ref = G.gemm_bf16_ref(x, w)
        W = to_dev_bf16(w)
        sk.skgemm_health()  # clear
        for rep in range(3):
            assert_parity(run_bf16(x, None, S, W=W), ref, K, f"hand-over T={T} S={S} rep {rep}")
        h = sk.skgemm_health()
        log(f"  health: {h['timeouts']} time-outs, first records {h['records'][:3]}")
        # Every record names a real tile group and owner rank; a time-out is
        # recorded only for a wait that was armed and ran out.
        for (group, rank, problem, ticks) in h["records"]:
            assert group < N // 16 and rank < S and problem == 0 and ticks == int(wait)
        if wait in ("0", "10000"):
            assert h["timeouts"] == 0


WIDE_CASES = [(40, 512, 4096, 4), (100, 256, 2048, 2), (128, 768, 1024, 1), (64, 512, 8192, 8),
              (33, 256, 512, 1), (77, 512, 2048, 4)]
WIDE_MX_CASES = [(48, 256, 2048, 2), (120, 512, 4096, 8), (65, 256, 1024, 1)]


@pytest.mark.parametrize("wait", [None, "0"])
def test_wide_kernel(wait, tune):
    """The wide-tile kernel (33..128 tokens): every token-tile count it is
    built for, ragged T, every split, bf16 and MXFP4; with the owner wait at
    0 the columns go to the last rank to arrive instead."""
    tune("kind", "3")
    if wait is not None:
        tune("owner_wait", wait)
    for (T, N, K, S) in WIDE_CASES:
        tac = sk.skgemm_tactic_for(T, N, K, S)
        log(f"wide wait={wait}: bf16 T={T} N={N} K={K} S={S} tactic={tac}")
        assert tac["kind"] == "wide"
        x, w = workloads.small_bf16_case(T, K, N, seed=9000 + T + S)
        ref = G.gemm_bf16_ref(x, w)
        W = to_dev_bf16(w)
        for rep in range(2):
            assert_parity(run_bf16(x, None, S, W=W), ref, K, f"wide T={T} S={S} rep {rep}")
    for (T, N, K, S) in WIDE_MX_CASES:
        tac = sk.skgemm_tactic_for(T, N, K, S, True)
        log(f"wide wait={wait}: mxfp4 T={T} N={N} K={K} S={S} tactic={tac}")
        assert tac["kind"] == "wide"
        x, wq, ws = workloads.small_mxfp4_case(T, K, N, seed=9100 + T + S)
        assert_parity(run_mxfp4(x, wq, ws, S), G.gemm_mxfp4_ref(x, wq, ws), K, f"wide mx T={T} S={S}")
    for (T, N, K, S) in WIDE_MX_CASES:
        tac = sk.skgemm_tactic_for(T, N, K, S, 2)
        log(f"wide wait={wait}: mxfp8 T={T} N={N} K={K} S={S} tactic={tac}")
        assert tac["kind"] == "wide"
        x, wq8, ws = workloads.small_mxfp8_case(T, K, N, seed=9150 + T + S)
        assert_parity(run_mxfp8(x, wq8, ws, S), G.gemm_mxfp8_ref(x, wq8, ws), K, f"wide mx8 T={T} S={S}")


@pytest.mark.parametrize("S", [1, 2, 4, 8])
def test_wide_integer_exact(S, tune):
    tune("kind", "3")
    for T in (33, 64, 97, 128):
        N, K = 512, 4096
        log(f"wide integer exact T={T} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S)}")
        x, w = workloads.integer_bf16_case(T, K, N, seed=9200 + T + S, mag=2)
        exact = G.gemm_bf16_ref(x, w)
        assert np.max(np.abs(exact)) < 2**24
        want = F.f32_to_bf16_rne(exact.astype(np.float32))
        assert np.array_equal(F.bf16_bits_to_f64(run_bf16(x, w, S)), F.bf16_bits_to_f64(want))


# bf16 wide tiles of up to 64 tokens pass activation chunks of 256 elements
# through three LDS buffers with a handshake; n chunks per rank slice covers
# the prologue's one and two chunks, a partial turn of the buffers and many.
@pytest.mark.parametrize("T,n,S", [(33, 1, 1), (64, 1, 4), (48, 2, 2), (40, 3, 1), (64, 5, 2), (57, 16, 4)])
def test_wide_chunk_handshake_integer_exact(T, n, S, tune):
    tune("kind", "3")
    N, K = 512, 256 * n * S
    tac = sk.skgemm_tactic_for(T, N, K, S)
    log(f"wide handshake T={T} chunks={n} S={S} K={K} tactic={tac}")
    assert tac["kind"] == "wide" and tac["kc"] == 256
    x, w = workloads.integer_bf16_case(T, K, N, seed=9300 + T + n + S, mag=2)
    exact = G.gemm_bf16_ref(x, w)
    assert np.max(np.abs(exact)) < 2**24
    want = F.f32_to_bf16_rne(exact.astype(np.float32))
    for rep in range(2):
        assert np.array_equal(F.bf16_bits_to_f64(run_bf16(x, w, S)), F.bf16_bits_to_f64(want)), f"rep {rep}"


@pytest.mark.parametrize("shape", ["0", "6"])
def test_partials_held_in_lds_bit_identical(shape, tune):
    """The persistent kernel holds tile partials in LDS until its stream ends
    where they fit (pdefer); otherwise it stores them tile by tile (deferred
    organisation, shape 0) or from the storer wave's registers in bursts
    (shape 6). The same sums in the same order: identical bits either way,
    and both meet the oracle's bound (one and two token tiles, S = 4 and 8)."""
    # (the last: 1029 tiles over 32 workgroups, 32-33 each: register batches of 16, 16 and 1)
    cases = [(32, 2304, 7168, 8), (16, 4096, 4096, 8), (8, 8192, 8192, 4), (5, 4096, 4096, 8),
             (12, 16464, 4096, 8)]
    tune("kind", "1")
    tune("stream", shape)
    for (T, N, K, S) in cases:
        x, w = workloads.small_bf16_case(T, K, N, seed=9400 + T + S)
        ref = G.gemm_bf16_ref(x, w)
        W = to_dev_bf16(w)
        got = {}
        for flag in ("1", "0"):
            tune("pdefer", flag)
            tac = sk.skgemm_tactic_for(T, N, K, S)
            log(f"shape {shape} pdefer={flag}: T={T} N={N} K={K} S={S} tactic={tac}")
            assert tac["kind"] == "stream" and tac["shape"] == int(shape) and tac["pdefer"] == int(flag)
            got[flag] = run_bf16(x, None, S, W=W)
            assert_parity(got[flag], ref, K, f"shape {shape} pdefer={flag} T={T} S={S}")
        assert np.array_equal(got["1"], got["0"])


def test_kinds_share_counters(tune):
    """The persistent, wide and tiled kernels hand off through the same
    arrival-counter area of one stream's workspace (one counter line per 16
    output rows). Interleaved twice over one N, every launch must return its
    counters to zero for the next kind: bit-exact results on integer operands."""
    N, K, S = 1024, 4096, 8
    runs = [("1", 32), ("3", 64), ("0", 32), ("1", 8), ("0", 80), ("3", 128)]
    for rep in range(2):
        for kind, T in runs:
            tune("kind", kind)
            tac = sk.skgemm_tactic_for(T, N, K, S)
            log(f"shared counters rep={rep} kind={kind} T={T} N={N} K={K} S={S} tactic={tac}")
            x, w = workloads.integer_bf16_case(T, K, N, seed=9300 + 10 * rep + T, mag=2)
            want = F.f32_to_bf16_rne(G.gemm_bf16_ref(x, w).astype(np.float32))
            assert np.array_equal(F.bf16_bits_to_f64(run_bf16(x, w, S)), F.bf16_bits_to_f64(want))


BATCH_KINDS = [("2", [(3, 512, 1024, 4), (16, 256, 2048, 2)]),   # cluster
               ("1", [(8, 2048, 4096, 4), (24, 1024, 2048, 8)]),  # stream
               ("3", [(40, 512, 4096, 4), (128, 256, 2048, 2)]),  # wide
               ("0", [(5, 160, 512, 2), (70, 64, 1024, 4)])]      # tiled


@pytest.mark.parametrize("kind,cases", BATCH_KINDS, ids=["cluster", "stream", "wide", "tiled"])
def test_batched_bf16(kind, cases, tune):
    """L problems in one launch equal L single calls: every problem against
    the oracle, padded strides (gaps in C untouched), L = 1 bit-equal to the
    single call, and weights shared across the batch (stride 0)."""
    tune("kind", kind)
    t = torch()
    for (T, N, K, S) in cases:
        L = 3
        log(f"batched kind={kind} L={L} T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S)}")
        xs, ws = zip(*[workloads.small_bf16_case(T, K, N, seed=9300 + 7 * l + T) for l in range(L)])
        wpad, xpad, cpad = 256, 512, 64  # elements of padding after each problem
        Wb = t.zeros(L, N * K + wpad, dtype=t.int16, device=DEV)
        Xb = t.zeros(L, T * K + xpad, dtype=t.int16, device=DEV)
        for l in range(L):
            Wb[l, :N * K] = to_dev_bf16(ws[l]).view(t.int16).reshape(-1)
            Xb[l, :T * K] = to_dev_bf16(xs[l]).view(t.int16).reshape(-1)
        sentinel = 0x7FC1
        Cb = t.full((L, T * N + cpad), sentinel, dtype=t.int16, device=DEV)
        sk.skgemm_bf16_batched(Wb, Xb, Cb, T, N, K, S, L, (N * K + wpad) * 2, (T * K + xpad) * 2,
                               (T * N + cpad) * 2)
        t.cuda.synchronize()
        cb = Cb.cpu().numpy().view(np.uint16)
        assert np.all(cb[:, T * N:] == sentinel)
        for l in range(L):
            assert_parity(cb[l, :T * N].reshape(T, N), G.gemm_bf16_ref(xs[l], ws[l]), K, f"batch {l}")
        # L = 1 is the single call, bit for bit
        one = t.empty((T, N), dtype=t.bfloat16, device=DEV)
        sk.skgemm_bf16_batched(Wb, Xb, one, T, N, K, S, 1, 0, 0, 0)
        t.cuda.synchronize()
        single = run_bf16(xs[0], ws[0], S)
        assert np.array_equal(bf16_bits(one), single)
        # weights shared by every problem
        Cs = t.empty((L, T * N), dtype=t.bfloat16, device=DEV)
        sk.skgemm_bf16_batched(Wb, Xb, Cs, T, N, K, S, L, 0, (T * K + xpad) * 2, T * N * 2)
        t.cuda.synchronize()
        cs = bf16_bits(Cs)
        for l in range(L):
            assert_parity(cs[l].reshape(T, N), G.gemm_bf16_ref(xs[l], ws[0]), K, f"shared W, batch {l}")


def test_batched_mxfp4_and_oversized_grid():
    """MXFP4 batches, and a batch whose grid exceeds what the GPU holds at once
    (owners then hand over at once): still one correct result per problem."""
    t = torch()
    for (T, N, K, S, L) in [(16, 512, 2048, 4, 3), (48, 512, 2048, 4, 12)]:
        log(f"batched mxfp4 L={L} T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S, True)}")
        cases = [workloads.small_mxfp4_case(T, K, N, seed=9400 + l) for l in range(L)]
        Wq = to_dev_u8(np.stack([c[1] for c in cases]))
        Ws = to_dev_u8(np.stack([c[2] for c in cases]))
        X = to_dev_bf16(np.stack([c[0] for c in cases]))
        C = t.empty((L, T, N), dtype=t.bfloat16, device=DEV)
        sk.skgemm_mxfp4_batched(Wq, Ws, X, C, T, N, K, S, L, N * K // 2, N * K // 32, T * K * 2, T * N * 2)
        t.cuda.synchronize()
        cb = bf16_bits(C)
        for l, (x, wq, ws) in enumerate(cases):
            assert_parity(cb[l], G.gemm_mxfp4_ref(x, wq, ws), K, f"mx batch {l}")
    for (T, N, K, S, L) in [(64, 1024, 2048, 4, 40)]:  # wide kernel, 640 workgroups
        log(f"batched bf16 oversized L={L} T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S)}")
        cases = [workloads.small_bf16_case(T, K, N, seed=9500 + l) for l in range(L)]
        W = to_dev_bf16(np.stack([c[1] for c in cases]))
        X = to_dev_bf16(np.stack([c[0] for c in cases]))
        C = t.empty((L, T, N), dtype=t.bfloat16, device=DEV)
        sk.skgemm_bf16_batched(W, X, C, T, N, K, S, L, N * K * 2, T * K * 2, T * N * 2)
        t.cuda.synchronize()
        cb = bf16_bits(C)
        for l in (0, 7, L - 1):
            x, w = cases[l]
            assert_parity(cb[l], G.gemm_bf16_ref(x, w), K, f"oversized batch {l}")


def test_timeline_stamps(tune):
    """Opt-in phase stamps: five non-decreasing device-clock values per
    workgroup, the counter hand-off's two (where reached) between the own
    stores and the exit, results unchanged, nothing written once turned off."""
    tune("kind", "1")
    t = torch()
    w = workloads.WORKLOADS["bf16_t8_k7168_n2048"]
    x = workloads.gen_x(w)
    wb = workloads.gen_w_bf16(w)
    tac = sk.skgemm_tactic_for(w.T, w.N, w.K, w.split_k)
    log(f"timeline stamps on {w.name}, tactic={tac}")
    assert tac["kind"] == "stream"
    buf = t.zeros(tac["grid"] * 8, dtype=t.int64, device=DEV)
    sk.skgemm_set_timeline(buf, buf.numel())
    try:
        c = run_bf16(x, wb, w.split_k)
    finally:
        sk.skgemm_set_timeline(None, 0)
    st = buf.view(tac["grid"], 8).cpu().numpy()
    assert np.all(st[:, :5] > 0) and np.all(st[:, 7] == 0)
    assert np.all(np.diff(st[:, :5], axis=1) >= 0)
    for j in (5, 6):  # arrivals done, owned polls done: 0 where not reached
        m = st[:, j] > 0
        assert np.all(st[m, j] >= st[m, 3]) and np.all(st[m, j] <= st[m, 4])
    m = (st[:, 5] > 0) & (st[:, 6] > 0)
    assert np.all(st[m, 6] >= st[m, 5])
    span_us = (st[:, 4].max() - st[:, 0].min()) * 0.01
    log(f"  workgroup span {span_us:.2f} us")
    assert 0 < span_us < 1e4
    assert_parity(c, G.gemm_bf16_ref(x, wb), w.K, "with stamps")
    buf.zero_()
    run_bf16(x, wb, w.split_k)
    assert int(buf.abs().sum().item()) == 0


def test_health_records_timeouts(tune):
    """With a one-tick owner wait on a shape with many tiles per owner, some
    waits run out: the report counts them, names their tiles and clears."""
    t = torch()
    tune("owner_wait", 1)
    tune("kind", 1)
    tune("stream", 0)
    T, N, K, S = 8, 8192, 4096, 8
    x, w = workloads.small_bf16_case(T, K, N, seed=8100)
    W, X = to_dev_bf16(w), to_dev_bf16(x)
    C = empty_bf16(T, N)
    sk.skgemm_health()
    log(f"health: T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S)}")
    for _ in range(5):
        sk.skgemm_bf16(W, X, C, T, N, K, S)
    t.cuda.synchronize()
    h = sk.skgemm_health()
    log(f"  {h['timeouts']} time-outs, records {h['records'][:4]}")
    assert h["timeouts"] >= 1 and len(h["records"]) == min(h["timeouts"], 15)
    assert_parity(bf16_bits(C), G.gemm_bf16_ref(x, w), K, "after time-outs")
    assert sk.skgemm_health()["timeouts"] == 0  # cleared


MAILBOX_CASES = [(32, 2304, 7168, 8), (16, 4096, 4096, 8), (8, 8192, 8192, 4), (5, 4096, 4096, 8),
                 (24, 1024, 4096, 8), (3, 4096, 1024, 2), (12, 16464, 4096, 8)]


@pytest.mark.parametrize("shape", ["0", "1", "4", "5", "6"])
@pytest.mark.parametrize("wait", ["0", "1", "10000"])
def test_mailbox_handoff_bit_identical(shape, wait, tune):
    """The tagged-mailbox hand-off sums the same partials in the same order
    as the arrival counter: identical bits, within the oracle's bound, over
    launches in a row (each with the next epoch's tag), with the owner wait
    at its bound, at one tick (owners give up, peers take over) and at zero;
    also with partials held in LDS or not (pdefer)."""
    tune("kind", 1)
    tune("stream", shape)
    tune("owner_wait", wait)
    ran = 0
    for (T, N, K, S) in MAILBOX_CASES:
        for pdefer in ("1", "0"):
            tune("pdefer", pdefer)
            tune("handoff", 0)
            try:
                tac = sk.skgemm_tactic_for(T, N, K, S)
            except sk.SkgemmError:
                continue
            x, w = workloads.small_bf16_case(T, K, N, seed=9600 + T + S)
            W = to_dev_bf16(w)
            counter = run_bf16(x, None, S, W=W)
            tune("handoff", 1)
            tac = sk.skgemm_tactic_for(T, N, K, S)
            assert tac["handoff"] == "mailbox", tac
            log(f"mailbox shape={shape} wait={wait} pdefer={tac['pdefer']}: T={T} N={N} K={K} S={S}")
            sk.skgemm_health()
            for rep in range(3):
                got = run_bf16(x, None, S, W=W)
                assert np.array_equal(got, counter), f"rep {rep}: mailbox bits differ from the counter's"
            h = sk.skgemm_health()
            for (group, rank, problem, ticks) in h["records"]:
                assert rank != 0xFFFF, "a take-over's poll ran out"
                assert group < N // 16 and rank < S and ticks == int(wait)
            if wait in ("0", "10000"):
                assert h["timeouts"] == 0
            assert_parity(got, G.gemm_bf16_ref(x, w), K, f"mailbox T={T} S={S}")
            ran += 1
    assert ran >= 4


def test_mailbox_graph_replays_match_eager(tune):
    """The mailbox tag comes from a device epoch word, not from the launch's
    arguments: a captured launch replayed several times (eager mailbox calls
    between) gives the eager bits every time."""
    t = torch()
    tune("handoff", 1)
    T, N, K, S = 32, 4096, 7168, 8
    tune("kind", 1)
    log(f"mailbox graph T={T} N={N} K={K} S={S} tactic={sk.skgemm_tactic_for(T, N, K, S)}")
    x, wb = workloads.small_bf16_case(T, K, N, seed=9650)
    W, X = to_dev_bf16(wb), to_dev_bf16(x)
    s = t.cuda.Stream()
    sk.skgemm_reserve(T, N, S, s)
    with t.cuda.stream(s):
        eager = sentinel_bf16(T, N)
        sk.skgemm_bf16(W, X, eager, T, N, K, S, s)
    t.cuda.synchronize()
    eager_bits = checked_bits(eager)
    assert_parity(eager_bits, G.gemm_bf16_ref(x, wb), K, "mailbox eager")
    C = sentinel_bf16(T, N)
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=s):
        sk.skgemm_bf16(W, X, C, T, N, K, S, s)
    for rep in range(4):
        with t.cuda.stream(s):
            C.fill_(float("nan"))
            g.replay()
            sk.skgemm_bf16(W, X, eager, T, N, K, S, s)  # an eager call between replays
        t.cuda.synchronize()
        assert np.array_equal(checked_bits(C), eager_bits), f"replay {rep}"
        assert np.array_equal(checked_bits(eager), eager_bits), f"eager after replay {rep}"
    del g
