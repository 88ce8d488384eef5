"""Python binding of libskgemm.so, the split-K decode GEMM for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/skgemm.h``. Functions carry the
C names and argument order; array arguments may be torch tensors on the GPU
(their storage address is passed) or plain integer device addresses. The
stream defaults to torch's current stream on the current device.

The library is loaded on first use. If it is missing or fails to load, every
call raises ``SkgemmError``: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import json
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libskgemm.so")

SKGEMM_OK = 0
SKGEMM_EINVAL = -1
SKGEMM_EALIGN = -2
SKGEMM_ESHAPE = -3
SKGEMM_ENOMEM = -4
SKGEMM_EHIP = -5
SKGEMM_ESCRATCH = -6

# skgemm_set_override knobs (include/skgemm.h, enum skgemm_knob)
KNOBS = {"kind": 0, "stream": 1, "shape": 2, "fold": 3, "cluster_c": 4, "wg_per_cu": 5,
         "pdefer": 6, "owner_wait": 7, "handoff": 8}

_lib = None


class SkgemmError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(what)


def _declare(lib):
    vp, i, sz, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    sig = {
        "skgemm_bf16": [vp, vp, vp, i, i, i, i, st],
        "skgemm_mxfp4": [vp, vp, vp, vp, i, i, i, i, st],
        "skgemm_mxfp8": [vp, vp, vp, vp, i, i, i, i, st],
        "skgemm_mxfp8_batched": [vp, vp, vp, vp, i, i, i, i, i, sz, sz, sz, sz, st],
        "skgemm_mxfp8_dequant": [vp, vp, vp, i, i, st],
        "skgemm_reserve": [i, i, i, st],
        "skgemm_reserve_batched": [i, i, i, i, st],
        "skgemm_bf16_batched": [vp, vp, vp, i, i, i, i, i, sz, sz, sz, st],
        "skgemm_mxfp4_batched": [vp, vp, vp, vp, i, i, i, i, i, sz, sz, sz, sz, st],
        "skgemm_release": [],
        "skgemm_mxfp4_dequant": [vp, vp, vp, i, i, st],
        "skgemm_pack_bf16": [vp, vp, sz, st],
        "skgemm_pack_e4m3": [vp, vp, sz, st],
        "skgemm_wave_sum": [vp, vp, sz, st],
        "skgemm_tactic_for": [i, i, i, i, i, ctypes.c_char_p, sz],
        "skgemm_last_hip_error": [],
        "skgemm_set_timeline": [vp, sz],
        "skgemm_read_probe": [vp, sz, vp, st],
        "skgemm_health": [vp, sz, st],
        "skgemm_set_override": [i, i],
        "skgemm_bf16_noalloc": [vp, vp, vp, i, i, i, i, st],
        "skgemm_bf16_e4m3": [vp, vp, vp, ctypes.c_float, i, i, i, i, st],
        "skgemm_bf16_chain": [vp, vp, vp, vp, i, i, i, st],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.skgemm_strerror.argtypes = [ctypes.c_int]
    lib.skgemm_strerror.restype = ctypes.c_char_p


def lib():
    """The loaded libskgemm.so (raises SkgemmError if it is not built).

    torch is imported first: its wheel carries its own HIP runtime under the
    same soname (libamdhip64.so.7) but loads it by file name, so if this
    library pulled in the system runtime first, the process would hold two
    HIP runtimes and launches from here would fail (hipErrorNoDevice). With
    torch's runtime already loaded, this library binds to that one instance.
    """
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SkgemmError(SKGEMM_EHIP, f"{LIB_PATH} is not built (run split_reduction_amd/build.py)")
        import torch  # noqa: F401  (one HIP runtime per process: torch's)

        try:
            handle = ctypes.CDLL(LIB_PATH)
        except OSError as e:
            raise SkgemmError(SKGEMM_EHIP, f"cannot load {LIB_PATH}: {e}") from e
        _declare(handle)
        _lib = handle
    return _lib


def strerror(code: int) -> str:
    return lib().skgemm_strerror(code).decode()


def _check(code: int, name: str) -> None:
    if code != SKGEMM_OK:
        extra = ""
        if code == SKGEMM_EHIP:
            extra = f" (hipError {lib().skgemm_last_hip_error()})"
        raise SkgemmError(code, f"{name}: {strerror(code)}{extra}")


def _ptr(a, nbytes: int = 0, what: str = "argument") -> int:
    """Device address of a tensor or of a plain integer address (None is 0).

    A tensor must live on the GPU, be contiguous and hold at least `nbytes`
    from its first element: the kernels read or write that dense block at the
    address, so a host tensor, a strided view or a short buffer would reach the
    device as a bad address. Such tensors raise SkgemmError(SKGEMM_EINVAL) here,
    before anything is launched. Integer addresses are passed through unchecked
    (the caller vouches for them)."""
    if a is None:
        return 0
    if isinstance(a, int):
        return a
    if a.device.type != "cuda":
        raise SkgemmError(SKGEMM_EINVAL, f"{what}: a tensor on {a.device}, not on the GPU")
    if not a.is_contiguous():
        raise SkgemmError(SKGEMM_EINVAL, f"{what}: not contiguous")
    have = a.numel() * a.element_size()
    if have < nbytes:
        raise SkgemmError(SKGEMM_EINVAL, f"{what}: holds {have} bytes, the call needs {nbytes}")
    return a.data_ptr()


def _n(*dims) -> int:
    """Product of the sizes, 0 if any is not positive (the library rejects or
    skips such calls itself, so they need no bytes)."""
    out = 1
    for d in dims:
        if d <= 0:
            return 0
        out *= d
    return out


def _batched(L: int, stride: int, one: int) -> int:
    """Bytes spanned by L problems `stride` bytes apart, each `one` bytes."""
    return 0 if L <= 0 or one == 0 else (L - 1) * max(stride, 0) + one


def _stream(stream) -> int:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def skgemm_bf16(W, X, C, T: int, N: int, K: int, split_k: int, stream=None) -> None:
    """C[T, N] = X[T, K] . W[N, K]^T (bf16 in and out, FP32 accumulation)."""
    code = lib().skgemm_bf16(_ptr(W, 2 * _n(N, K), "W"), _ptr(X, 2 * _n(T, K), "X"),
                             _ptr(C, 2 * _n(T, N), "C"), T, N, K, split_k, _stream(stream))
    _check(code, "skgemm_bf16")


def skgemm_bf16_e4m3(W, X, C8, c_scale: float, T: int, N: int, K: int, split_k: int, stream=None) -> None:
    """C8[T, N] (uint8 E4M3FN codes) of (X . W^T) * c_scale, saturated to +-448."""
    code = lib().skgemm_bf16_e4m3(_ptr(W, 2 * _n(N, K), "W"), _ptr(X, 2 * _n(T, K), "X"),
                                  _ptr(C8, _n(T, N), "C8"), float(c_scale), T, N, K, split_k, _stream(stream))
    _check(code, "skgemm_bf16_e4m3")


def skgemm_bf16_chain(Ws, X, Cs, dims, T: int, split_k: int, stream=None) -> None:
    """L GEMMs in one launch, C[i] = A_i . W[i]^T with A_0 = X, A_i = C[i-1];
    Ws and Cs are sequences of L tensors (or addresses), dims L + 1 sizes."""
    L = len(Ws)
    if len(Cs) != L or len(dims) != L + 1:
        raise SkgemmError(SKGEMM_EINVAL, "skgemm_bf16_chain: need L weights, L outputs and L + 1 dims")
    wp = (ctypes.c_void_p * max(L, 1))(*[_ptr(Ws[i], 2 * _n(dims[i + 1], dims[i]), f"W[{i}]") for i in range(L)])
    cp = (ctypes.c_void_p * max(L, 1))(*[_ptr(Cs[i], 2 * _n(T, dims[i + 1]), f"C[{i}]") for i in range(L)])
    dp = (ctypes.c_int * (L + 1))(*[int(d) for d in dims])
    code = lib().skgemm_bf16_chain(wp, _ptr(X, 2 * _n(T, dims[0]) if dims else 0, "X"), cp, dp, L, T, split_k,
                                   _stream(stream))
    _check(code, "skgemm_bf16_chain")


def skgemm_bf16_noalloc(W, X, C, T: int, N: int, K: int, split_k: int, stream=None) -> None:
    """skgemm_bf16 with the split-K workspace in the library's fixed per-GPU
    scratch: allocates nothing (SKGEMM_ESCRATCH when the call needs more)."""
    code = lib().skgemm_bf16_noalloc(_ptr(W, 2 * _n(N, K), "W"), _ptr(X, 2 * _n(T, K), "X"),
                                     _ptr(C, 2 * _n(T, N), "C"), T, N, K, split_k, _stream(stream))
    _check(code, "skgemm_bf16_noalloc")


def skgemm_mxfp4(Wq, Wscale, X, C, T: int, N: int, K: int, split_k: int, stream=None) -> None:
    """C = X . dequant(Wq, Wscale)^T with MXFP4 weights decoded in registers."""
    code = lib().skgemm_mxfp4(_ptr(Wq, _n(N, K) // 2, "Wq"), _ptr(Wscale, _n(N, K) // 32, "Wscale"),
                              _ptr(X, 2 * _n(T, K), "X"), _ptr(C, 2 * _n(T, N), "C"), T, N, K, split_k,
                              _stream(stream))
    _check(code, "skgemm_mxfp4")


def skgemm_bf16_batched(W, X, C, T: int, N: int, K: int, split_k: int, L: int, w_stride: int,
                        x_stride: int, c_stride: int, stream=None) -> None:
    """L problems of one shape in one launch; strides in bytes."""
    code = lib().skgemm_bf16_batched(_ptr(W, _batched(L, w_stride, 2 * _n(N, K)), "W"),
                                     _ptr(X, _batched(L, x_stride, 2 * _n(T, K)), "X"),
                                     _ptr(C, _batched(L, c_stride, 2 * _n(T, N)), "C"),
                                     T, N, K, split_k, L, w_stride, x_stride, c_stride, _stream(stream))
    _check(code, "skgemm_bf16_batched")


def skgemm_mxfp4_batched(Wq, Wscale, X, C, T: int, N: int, K: int, split_k: int, L: int, wq_stride: int,
                         wscale_stride: int, x_stride: int, c_stride: int, stream=None) -> None:
    """L MXFP4 problems of one shape in one launch; strides in bytes."""
    code = lib().skgemm_mxfp4_batched(_ptr(Wq, _batched(L, wq_stride, _n(N, K) // 2), "Wq"),
                                      _ptr(Wscale, _batched(L, wscale_stride, _n(N, K) // 32), "Wscale"),
                                      _ptr(X, _batched(L, x_stride, 2 * _n(T, K)), "X"),
                                      _ptr(C, _batched(L, c_stride, 2 * _n(T, N)), "C"),
                                      T, N, K, split_k, L, wq_stride, wscale_stride, x_stride, c_stride,
                                      _stream(stream))
    _check(code, "skgemm_mxfp4_batched")


def skgemm_mxfp8(Wq8, Wscale, X, C, T: int, N: int, K: int, split_k: int, stream=None) -> None:
    """C = X . dequant(Wq8, Wscale)^T with E4M3 weights and E8M0 block scales."""
    code = lib().skgemm_mxfp8(_ptr(Wq8, _n(N, K), "Wq8"), _ptr(Wscale, _n(N, K) // 32, "Wscale"),
                              _ptr(X, 2 * _n(T, K), "X"), _ptr(C, 2 * _n(T, N), "C"), T, N, K, split_k,
                              _stream(stream))
    _check(code, "skgemm_mxfp8")


def skgemm_mxfp8_batched(Wq8, Wscale, X, C, T: int, N: int, K: int, split_k: int, L: int, wq8_stride: int,
                         wscale_stride: int, x_stride: int, c_stride: int, stream=None) -> None:
    """L MXFP8 problems of one shape in one launch; strides in bytes."""
    code = lib().skgemm_mxfp8_batched(_ptr(Wq8, _batched(L, wq8_stride, _n(N, K)), "Wq8"),
                                      _ptr(Wscale, _batched(L, wscale_stride, _n(N, K) // 32), "Wscale"),
                                      _ptr(X, _batched(L, x_stride, 2 * _n(T, K)), "X"),
                                      _ptr(C, _batched(L, c_stride, 2 * _n(T, N)), "C"),
                                      T, N, K, split_k, L, wq8_stride, wscale_stride, x_stride, c_stride,
                                      _stream(stream))
    _check(code, "skgemm_mxfp8_batched")


def skgemm_mxfp8_dequant(Wq8, Wscale, W_out, N: int, K: int, stream=None) -> None:
    code = lib().skgemm_mxfp8_dequant(_ptr(Wq8, _n(N, K), "Wq8"), _ptr(Wscale, _n(N, K) // 32, "Wscale"),
                                      _ptr(W_out, 2 * _n(N, K), "W_out"), N, K, _stream(stream))
    _check(code, "skgemm_mxfp8_dequant")


def skgemm_reserve_batched(max_T: int, max_N: int, max_split_k: int, max_L: int, stream=None) -> None:
    _check(lib().skgemm_reserve_batched(max_T, max_N, max_split_k, max_L, _stream(stream)),
           "skgemm_reserve_batched")


def skgemm_reserve(max_T: int, max_N: int, max_split_k: int, stream=None) -> None:
    _check(lib().skgemm_reserve(max_T, max_N, max_split_k, _stream(stream)), "skgemm_reserve")


def skgemm_release() -> None:
    _check(lib().skgemm_release(), "skgemm_release")


def skgemm_mxfp4_dequant(Wq, Wscale, W_out, N: int, K: int, stream=None) -> None:
    code = lib().skgemm_mxfp4_dequant(_ptr(Wq, _n(N, K) // 2, "Wq"), _ptr(Wscale, _n(N, K) // 32, "Wscale"),
                                      _ptr(W_out, 2 * _n(N, K), "W_out"), N, K, _stream(stream))
    _check(code, "skgemm_mxfp4_dequant")


def skgemm_pack_bf16(inp, out, n_pairs: int, stream=None) -> None:
    _check(lib().skgemm_pack_bf16(_ptr(inp, 8 * n_pairs, "in"), _ptr(out, 4 * n_pairs, "out"), n_pairs,
                                  _stream(stream)), "skgemm_pack_bf16")


def skgemm_pack_e4m3(inp, out, n_quads: int, stream=None) -> None:
    _check(lib().skgemm_pack_e4m3(_ptr(inp, 16 * n_quads, "in"), _ptr(out, 4 * n_quads, "out"), n_quads,
                                  _stream(stream)), "skgemm_pack_e4m3")


def skgemm_wave_sum(inp, out, n_waves: int, stream=None) -> None:
    _check(lib().skgemm_wave_sum(_ptr(inp, 256 * n_waves, "in"), _ptr(out, 256 * n_waves, "out"), n_waves,
                                 _stream(stream)), "skgemm_wave_sum")


def skgemm_tactic_for(T: int, N: int, K: int, split_k: int, weight_format: int = 0) -> dict:
    """The launch configuration a call with these sizes uses (host only).
    weight_format: 0 bf16, 1 MXFP4 (True also means MXFP4), 2 MXFP8."""
    buf = ctypes.create_string_buffer(512)
    code = lib().skgemm_tactic_for(T, N, K, split_k, int(weight_format), buf, len(buf))
    _check(code, "skgemm_tactic_for")
    return json.loads(buf.value.decode())


def skgemm_set_timeline(buf, capacity: int) -> None:
    """Opt-in per-workgroup phase stamps of the stream kernel (None turns them off)."""
    _check(lib().skgemm_set_timeline(_ptr(buf, 8 * capacity if buf is not None else 0, "buf"),
                                     capacity if buf is not None else 0), "skgemm_set_timeline")


def skgemm_read_probe(src, nbytes: int, sink, stream=None) -> None:
    """Plain coalesced read of nbytes at src (the streaming-read reference)."""
    _check(lib().skgemm_read_probe(_ptr(src, nbytes, "src"), nbytes, _ptr(sink, 4 * 512, "sink"),
                                   _stream(stream)), "skgemm_read_probe")


def skgemm_health(stream=None) -> dict:
    """Owner time-outs of the stream's split-K hand-off since the last call
    (read and cleared): {"timeouts": n, "records": [(group, rank, problem, ticks), ...]}."""
    words = (ctypes.c_uint32 * 128)()
    _check(lib().skgemm_health(words, 128, _stream(stream)), "skgemm_health")
    recs = [tuple(words[8 + 8 * r + i] for i in range(1, 5))
            for r in range(min(words[0], 15)) if words[8 + 8 * r] == 1]
    return {"timeouts": int(words[0]), "records": recs}


def skgemm_strerror(code: int) -> str:
    return strerror(code)


def skgemm_last_hip_error() -> int:
    return lib().skgemm_last_hip_error()


def skgemm_set_override(knob, value: int) -> None:
    """Pin a choice the library otherwise makes itself (tests and tuning runs);
    knob is a name of ``KNOBS`` or its number, value -1 restores the default."""
    k = KNOBS[knob] if isinstance(knob, str) else int(knob)
    _check(lib().skgemm_set_override(k, int(value)), "skgemm_set_override")


def clear_overrides() -> None:
    """Restore the library's own choice for every knob."""
    for k in KNOBS.values():
        _check(lib().skgemm_set_override(k, -1), "skgemm_set_override")
