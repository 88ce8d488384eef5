"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and its host-side argument checks and tactic choice behave as the
header states. No call here reaches the GPU (every call below is rejected, or
has nothing to do, before any HIP runtime call)."""

import ctypes
import os
import re
import subprocess

import pytest

import split_reduction_amd as sk
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "skgemm.h")


def _ensure_built():
    if not os.path.exists(sk.LIB_PATH):
        from split_reduction_amd import build

        build.build()


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"SKGEMM_API\s+[\w\s\*]+?\b(skgemm_\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = set(declared_symbols())
    for must in ("skgemm_bf16", "skgemm_mxfp4", "skgemm_reserve", "skgemm_mxfp4_dequant",
                 "skgemm_pack_bf16", "skgemm_pack_e4m3", "skgemm_wave_sum", "skgemm_tactic_for",
                 "skgemm_strerror", "skgemm_last_hip_error", "skgemm_release"):
        assert must in names


def test_library_exports_every_declared_symbol():
    _ensure_built()
    lib = ctypes.CDLL(sk.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sk.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (skgemm_\w+)", out))
    assert set(declared_symbols()) <= exported
    # nothing else of ours leaks out of the library
    assert {s for s in exported if s.startswith("skgemm")} == set(declared_symbols())


def test_argument_checks_before_any_device_work():
    _ensure_built()
    lib = sk.lib()
    a = 1 << 20  # a 16-byte aligned fake address: the checks below never dereference it
    # split_k outside {1,2,4,8}
    assert lib.skgemm_bf16(a, a, a, 1, 16, 96, 3, None) == sk.SKGEMM_EINVAL
    # negative sizes
    assert lib.skgemm_bf16(a, a, a, -1, 16, 64, 1, None) == sk.SKGEMM_EINVAL
    # N not a multiple of 16, K not a multiple of 32*split_k
    assert lib.skgemm_bf16(a, a, a, 1, 24, 64, 1, None) == sk.SKGEMM_ESHAPE
    assert lib.skgemm_bf16(a, a, a, 1, 16, 96, 2, None) == sk.SKGEMM_ESHAPE
    # MXFP4 needs K % (128 * split_k) == 0
    assert lib.skgemm_mxfp4(a, a, a, a, 1, 16, 256, 4, None) == sk.SKGEMM_ESHAPE
    # null and misaligned pointers
    assert lib.skgemm_bf16(None, a, a, 1, 16, 64, 1, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_bf16(a + 8, a, a, 1, 16, 64, 1, None) == sk.SKGEMM_EALIGN
    assert lib.skgemm_mxfp4(a, None, a, a, 1, 16, 128, 1, None) == sk.SKGEMM_EINVAL
    # size limits
    assert lib.skgemm_bf16(a, a, a, 1, 1 << 19, 64, 1, None) == sk.SKGEMM_ESHAPE
    # empty work: nothing enqueued, success, pointers not needed
    assert lib.skgemm_bf16(None, None, None, 0, 16, 64, 1, None) == sk.SKGEMM_OK
    assert lib.skgemm_bf16(None, None, None, 4, 0, 64, 1, None) == sk.SKGEMM_OK
    assert lib.skgemm_pack_bf16(None, None, 0, None) == sk.SKGEMM_OK
    assert lib.skgemm_wave_sum(a, None, 1, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_mxfp4_dequant(a, a, a, 16, 48, None) == sk.SKGEMM_ESHAPE
    # batched calls: L range, stride alignment, overlapping outputs
    assert lib.skgemm_bf16_batched(a, a, a, 2, 16, 64, 1, 0, 0, 0, 64, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_bf16_batched(a, a, a, 2, 16, 64, 1, 5000, 0, 0, 64, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_bf16_batched(a, a, a, 2, 16, 64, 1, 2, 8, 0, 64, None) == sk.SKGEMM_EALIGN
    assert lib.skgemm_bf16_batched(a, a, a, 2, 16, 64, 1, 2, 0, 0, 48, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_mxfp4_batched(a, a, a, a, 2, 16, 128, 1, 2, 0, 7, 16, 48, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_reserve_batched(1, 16, 1, 0, None) == sk.SKGEMM_EINVAL
    # the streaming-read reference
    assert lib.skgemm_read_probe(None, 64, a, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_read_probe(a, 24, a, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_read_probe(a + 8, 64, a, None) == sk.SKGEMM_EALIGN


class _FakeGpuTensor:
    """Stands in for a GPU tensor on a machine without one. Every call below has
    an operand that the binding rejects, so the library is never called and the
    fake address is never used."""

    def __init__(self, nbytes, contiguous=True):
        self.device = type("D", (), {"type": "cuda"})()
        self._nbytes, self._contiguous = nbytes, contiguous

    def is_contiguous(self):
        return self._contiguous

    def numel(self):
        return self._nbytes // 2

    def element_size(self):
        return 2

    def data_ptr(self):
        return 1 << 20


def test_binding_rejects_tensors_it_cannot_pass():
    """The binding refuses host tensors, strided views and buffers shorter than
    the call reads or writes, with SKGEMM_EINVAL, before anything is launched."""
    _ensure_built()
    import torch

    T, N, K = 2, 32, 64
    host = torch.zeros((N, K), dtype=torch.bfloat16)
    with pytest.raises(sk.SkgemmError) as e:
        sk.skgemm_bf16(host, _FakeGpuTensor(2 * T * K), _FakeGpuTensor(2 * T * N), T, N, K, 1)
    assert e.value.code == sk.SKGEMM_EINVAL and "not on the GPU" in str(e.value)
    with pytest.raises(sk.SkgemmError) as e:
        sk.skgemm_bf16(_FakeGpuTensor(2 * N * K, contiguous=False), _FakeGpuTensor(2 * T * K),
                       _FakeGpuTensor(2 * T * N), T, N, K, 1)
    assert e.value.code == sk.SKGEMM_EINVAL and "contiguous" in str(e.value)
    # one byte short, for each operand of each format
    full = {"W": 2 * N * K, "X": 2 * T * K, "C": 2 * T * N}
    for short in full:
        args = {k: _FakeGpuTensor(v - (2 if k == short else 0)) for k, v in full.items()}
        with pytest.raises(sk.SkgemmError) as e:
            sk.skgemm_bf16(args["W"], args["X"], args["C"], T, N, K, 1)
        assert e.value.code == sk.SKGEMM_EINVAL and e.value.args[0].startswith(short + ":")
    with pytest.raises(sk.SkgemmError) as e:
        sk.skgemm_mxfp4(_FakeGpuTensor(N * K // 2), _FakeGpuTensor(N * K // 32 - 2), _FakeGpuTensor(2 * T * K),
                        _FakeGpuTensor(2 * T * N), T, N, 128, 1)
    assert e.value.args[0].startswith("Wq:")  # K = 128 needs twice the nibbles
    with pytest.raises(sk.SkgemmError) as e:
        sk.skgemm_mxfp8(_FakeGpuTensor(N * K), _FakeGpuTensor(N * K // 32 - 2), _FakeGpuTensor(2 * T * K),
                        _FakeGpuTensor(2 * T * N), T, N, K, 1)
    assert e.value.args[0].startswith("Wscale:")
    # batched: the last problem's C ends (L-1)*stride + T*N*2 bytes in
    L, cs = 3, 2 * T * N + 64
    with pytest.raises(sk.SkgemmError) as e:
        sk.skgemm_bf16_batched(_FakeGpuTensor(2 * N * K), _FakeGpuTensor(2 * T * K),
                               _FakeGpuTensor((L - 1) * cs + 2 * T * N - 2), T, N, K, 1, L, 0, 0, cs)
    assert e.value.args[0].startswith("C:")


def test_strerror_covers_every_code():
    _ensure_built()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert sk.strerror(code) and "unknown" not in sk.strerror(code)
    assert "unknown" in sk.strerror(-99)


@pytest.mark.parametrize("T,N,K,S,mx", [
    (1, 1024, 1024, 4, False),
    (8, 2048, 7168, 4, False),
    (32, 18432, 7168, 8, False),
    (16, 4096, 7168, 4, True),
    (24, 16384, 16384, 4, False),
    (128, 16384, 16384, 2, False),
    (300, 256, 1024, 1, False),
    (200, 96, 256, 2, False),
    (130, 64, 256, 1, True),
])
def test_tactics_cover_the_workloads(T, N, K, S, mx):
    _ensure_built()
    t = sk.skgemm_tactic_for(T, N, K, S, mx)
    assert t["nt"] == min((min(T, 128) + 15) // 16, 8)
    assert N % t["tile_n"] == 0
    if t["kind"] == "tiled":
        assert t["grid"] == (N // t["tile_n"]) * S
    elif t["kind"] == "wide":  # 256-row tiles, one per workgroup per split rank, X in chunks
        assert t["tile_n"] == 256 and t["grid"] == (N // 256) * S and 33 <= min(T, 128)
        assert (K // S) % t["kc"] == 0 and t["lds"] == 2 * 16 * t["nt"] * t["kc"] * 2
    elif t["kind"] == "cluster":  # one workgroup per tile of 16/fold rows, S rank groups of waves
        assert t["tile_n"] * t["fold"] == 16 and t["grid"] == N // t["tile_n"]
        assert t["threads"] % (64 * S) == 0 and t["threads"] <= 1024
        assert T <= 16 // t["fold"] or (t["fold"] == 1 and T <= 32)
        assert t["kc"] == K // S and t["lds"] == 0
    else:  # persistent: G workgroups per split rank, every wave column owns a tile
        assert t["grid"] % S == 0 and t["tile_n"] == 16
        assert 1 <= (t["grid"] // S - 1) * t["wn"] < N // 16
        assert t["kc"] == K // S
    assert (K // S) % t["kc"] == 0
    assert t["lds"] <= 159 * 1024
    assert t["token_blocks"] == (T + 127) // 128
    step = 128 if mx else 32
    assert t["kc"] % step == 0
    assert min(T, 128) * t["kc"] * 2 <= 128 * 1024


# The kernel choices the tactic makes, each fixed by a measurement on MI355X
# (cold weights, graph replay): folded cluster tiles take one piece per lane
# when S * (one-piece steps per rank slice) >= 64; the cluster fold shrinks
# while the grid still covers the 256 CUs; an unfolded cluster grid below 256
# workgroups gives way to the persistent kernel; a single problem runs the
# persistent kernel at one workgroup per CU; cluster workgroups have at most
# four waves for a single bf16 problem and eight for block-scaled weights and
# batches. Load steps in flight per wave (d): 6 for one-piece bf16 cluster
# tiles in four-wave workgroups, 2 for two-piece tiles at folds of 4 and 8, 3
# for block-scaled tiles, 3 / 4 for the persistent storer shape at one / two
# token tiles, 4 (two ring slots) in the wide kernel. Persistent organisation: 7 streaming waves and a storer wave
# (shape 6) for single problems with many tiles per workgroup, the partials
# held in LDS until the stream ends wherever they fit (pdefer) and in the
# storer's registers where they do not (K=N=16384 T=24/32); the
# epilogue-wave shape (2) for few tiles per workgroup.
@pytest.mark.parametrize("T,N,K,S,wf,want", [
    (8, 2048, 7168, 4, 0, {"kind": "cluster", "fold": 2, "c": 1, "wk": 4, "d": 6, "grid": 256}),
    (8, 1024, 2048, 2, 0, {"kind": "cluster", "fold": 2, "c": 2}),
    (8, 4096, 7168, 4, 0, {"kind": "cluster", "fold": 1, "c": 2, "grid": 256}),
    (5, 1024, 7168, 4, 0, {"kind": "cluster", "fold": 2, "grid": 128}),
    (1, 1024, 1024, 4, 0, {"kind": "cluster", "fold": 4, "c": 2, "d": 2, "grid": 256}),
    (16, 4096, 7168, 4, 1, {"kind": "cluster", "fold": 1, "wk": 8, "d": 3}),
    (16, 4096, 7168, 4, 2, {"kind": "cluster", "fold": 1, "wk": 8, "d": 3}),
    (12, 1024, 7168, 4, 0, {"kind": "stream", "grid": 256}),
    (32, 2048, 7168, 4, 0, {"kind": "stream", "grid": 256}),
    (32, 18432, 7168, 8, 0, {"kind": "stream", "grid": 256, "shape": 6, "pdefer": 1}),
    (8, 16384, 16384, 8, 0, {"kind": "stream", "shape": 6, "pdefer": 1, "d": 3}),
    (16, 16384, 16384, 8, 0, {"kind": "stream", "shape": 6, "pdefer": 1}),
    (24, 16384, 16384, 8, 0, {"kind": "stream", "shape": 6, "pdefer": 0}),
    (32, 16384, 16384, 8, 0, {"kind": "stream", "shape": 6, "pdefer": 0, "d": 4}),
    (12, 1024, 7168, 4, 0, {"kind": "stream", "shape": 2, "pdefer": 0}),
    (64, 16384, 16384, 4, 0, {"kind": "wide", "d": 4}),
])
def test_tactic_rules(T, N, K, S, wf, want):
    _ensure_built()
    t = sk.skgemm_tactic_for(T, N, K, S, wf)
    got = {k: t[k] for k in want}
    assert got == want, (T, N, K, S, wf, t)
    if t["kind"] == "cluster":
        assert t["wk"] <= 8


def _row_bytes(wf, K):
    return K // 2 if wf == 1 else K if wf == 2 else 2 * K


@pytest.mark.parametrize("T,N,K,S,wf", [
    (1, 262144, 16384, 8, 0),     # 8 GiB of bf16 weights
    (8, 131072, 8192, 4, 0),      # exactly 2 GiB
    (8, 65536, 16384, 8, 0),      # exactly 2 GiB
    (16, 262144, 32768, 4, 1),    # MXFP4, 4 GiB of codes
    (32, 262144, 16384, 8, 2),    # MXFP8, 4 GiB of codes
    (1, 16384, 16384, 8, 0),      # 512 MiB: the persistent kernel
])
def test_weight_span_fits_the_chosen_kernel(T, N, K, S, wf):
    """A kernel that addresses the whole weight matrix through one buffer
    resource (the persistent kernel) is chosen only while that span stays
    below 2^31 bytes; larger matrices go to kernels that rebase the resource
    per tile, and the call is still accepted."""
    _ensure_built()
    t = sk.skgemm_tactic_for(T, N, K, S, wf)
    span = N * _row_bytes(wf, K)
    if t["kind"] == "stream":
        assert span < 2**31 and (wf == 0 or N * (K // 32) < 2**31)
    else:
        # per-tile resources: at most 256 rows of one tile
        assert t["tile_n"] * _row_bytes(wf, K) <= 2**31
    if span >= 2**31:
        assert t["kind"] != "stream"


def test_override_pins_and_restores():
    """skgemm_set_override pins a choice for later calls and the tactic
    query; -1 restores the library's own choice; bad knobs and values are
    rejected. No environment variable changes the choice."""
    _ensure_built()
    lib = sk.lib()
    own = sk.skgemm_tactic_for(8, 2048, 7168, 4)
    assert own["kind"] == "cluster"
    os.environ["SKGEMM_KIND"] = "1"  # ignored: only the override pins a kind
    try:
        assert sk.skgemm_tactic_for(8, 2048, 7168, 4) == own
        sk.skgemm_set_override("kind", 1)
        assert sk.skgemm_tactic_for(8, 2048, 7168, 4)["kind"] == "stream"
        sk.skgemm_set_override("kind", 3)  # the wide kernel cannot take T = 8
        with pytest.raises(sk.SkgemmError) as e:
            sk.skgemm_tactic_for(8, 2048, 7168, 4)
        assert e.value.code == sk.SKGEMM_ESHAPE
        sk.skgemm_set_override("kind", -1)
        assert sk.skgemm_tactic_for(8, 2048, 7168, 4) == own
    finally:
        os.environ.pop("SKGEMM_KIND", None)
        sk.clear_overrides()
    assert lib.skgemm_set_override(99, 0) == sk.SKGEMM_EINVAL
    assert lib.skgemm_set_override(-1, 0) == sk.SKGEMM_EINVAL
    assert lib.skgemm_set_override(0, -2) == sk.SKGEMM_EINVAL


def test_e4m3_output_scale_checked_before_device_work():
    _ensure_built()
    lib = sk.lib()
    a = 1 << 20
    f = ctypes.c_float
    for bad in (0.0, -2.0, float("nan"), float("inf")):
        assert lib.skgemm_bf16_e4m3(a, a, a, f(bad), 1, 16, 64, 1, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_bf16_e4m3(a, a, a, f(1.0), 1, 24, 64, 1, None) == sk.SKGEMM_ESHAPE
    assert lib.skgemm_bf16_e4m3(None, None, None, f(1.0), 0, 16, 64, 1, None) == sk.SKGEMM_OK


def test_chain_arguments_checked_before_device_work():
    _ensure_built()
    lib = sk.lib()
    a = 1 << 20
    P = ctypes.c_void_p

    def arrs(L, dims, cbase=1 << 30):
        w = (P * L)(*([a] * L))
        c = (P * L)(*[cbase + (i << 24) for i in range(L)])
        d = (ctypes.c_int * (L + 1))(*dims)
        return w, c, d

    w, c, d = arrs(2, [7168, 2048, 7168])
    assert lib.skgemm_bf16_chain(w, a, c, d, 0, 8, 4, None) == sk.SKGEMM_EINVAL    # L = 0
    assert lib.skgemm_bf16_chain(w, a, c, d, 2, 17, 4, None) == sk.SKGEMM_EINVAL   # T > 16
    assert lib.skgemm_bf16_chain(w, a, c, d, 2, 8, 3, None) == sk.SKGEMM_EINVAL    # split_k
    assert lib.skgemm_bf16_chain(None, a, c, d, 2, 8, 4, None) == sk.SKGEMM_EINVAL
    assert lib.skgemm_bf16_chain(w, a + 8, c, d, 2, 8, 4, None) == sk.SKGEMM_EALIGN
    w, c, d = arrs(2, [7168, 2040, 7168])
    assert lib.skgemm_bf16_chain(w, a, c, d, 2, 8, 4, None) == sk.SKGEMM_ESHAPE    # N % 16
    w, c, d = arrs(1, [1088, 2048])
    assert lib.skgemm_bf16_chain(w, a, c, d, 1, 8, 4, None) == sk.SKGEMM_ESHAPE    # K % (64 * 4) at T <= 8
    w, c, d = arrs(1, [1024, 2048], cbase=a)  # C[0] on top of X
    assert lib.skgemm_bf16_chain(w, a, c, d, 1, 8, 4, None) == sk.SKGEMM_EINVAL
    w, c, d = arrs(65, [1024] * 66)
    assert lib.skgemm_bf16_chain(w, a, c, d, 65, 8, 4, None) == sk.SKGEMM_EINVAL   # L > 64
