"""Oracle GEMM: the plain definition of what the split-K decode GEMM computes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): never imported by the
product path.

The split-K kernel on page
``vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.splitk`` (module
summary and ``SplitKGemm.kernel``) computes C = X . W^T with A = W (M, K) and
B = X (N, K) both K-major ("kernel-M carries public N"). Each split rank sums
one exact, contiguous K slice in FP32; the owner adds the peers' partials,
casts once and stores once. That reaches, up to the order of rounding, the
plain product

    C[t, n] = sum_{k < K} X[t, k] * W[n, k]

so the oracle is that product, evaluated in float64 on the bf16 operands
(products of two bf16 values are exact in float64, and the float64 sum error
is far below the acceptance bound). The result is *not* rounded to bf16: the
acceptance bound covers the kernel's final RNE cast.

The MXFP4 form decodes W first (``oracle.formats.mxfp4_dequant_f64``), as
``fp4x8_bf16`` on page ``vllm.models.muse_spark.amd.mono.kernels.dev`` does
before the bf16 MFMA.
"""

from __future__ import annotations

import math

import numpy as np

from .formats import E4M3_MAX, bf16_bits_to_f64, e4m3_rne_sat, e4m3_value, mxfp4_dequant_f64, mxfp8_dequant_f64


def gemm_decoded_ref(x_bits: np.ndarray, w: np.ndarray) -> np.ndarray:
    """C[T, N] float64 = X[T, K] . W[N, K]^T with X as bf16 bit patterns and W
    already holding exact float64 weight values (a decoded weight matrix, kept
    by a caller that multiplies several X by one large W)."""
    x = bf16_bits_to_f64(x_bits)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shape mismatch X{x.shape} W{w.shape}")
    return x @ w.T


def gemm_bf16_ref(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """C[T, N] float64 = X[T, K] . W[N, K]^T from bf16 bit patterns (uint16)."""
    return gemm_decoded_ref(x_bits, bf16_bits_to_f64(w_bits))


def gemm_mxfp4_ref(x_bits: np.ndarray, wq: np.ndarray, wscale: np.ndarray) -> np.ndarray:
    """C[T, N] float64 = X . dequant(Wq, Wscale)^T."""
    return gemm_decoded_ref(x_bits, mxfp4_dequant_f64(wq, wscale))


def gemm_mxfp8_ref(x_bits: np.ndarray, wq8: np.ndarray, wscale: np.ndarray) -> np.ndarray:
    """C[T, N] float64 = X . dequant(Wq8, Wscale)^T (E4M3 elements, E8M0 block scales)."""
    return gemm_decoded_ref(x_bits, mxfp8_dequant_f64(wq8, wscale))


def gemm_bruteforce(x_vals, w_vals) -> list:
    """Pure-Python triple loop over float64 values, for tiny shapes only.

    ``x_vals`` is a T x K and ``w_vals`` an N x K nested list (or array) of
    numbers; returns the T x N nested list of dot products summed in K order.
    """
    t_n = len(x_vals)
    n_n = len(w_vals)
    out = []
    for t in range(t_n):
        row = []
        for n in range(n_n):
            acc = 0.0
            for xv, wv in zip(x_vals[t], w_vals[n], strict=True):
                acc += float(xv) * float(wv)
            row.append(acc)
        out.append(row)
    return out


# ---------------------------------------------------------------------------
# Acceptance bound
# ---------------------------------------------------------------------------


def tolerance_bound(c_ref: np.ndarray, k: int, rms=None) -> np.ndarray:
    """Per-element bound 2**-7 * |ref| + 1e-3 * sqrt(K) * rms(ref).

    The bf16 RNE cast of the output contributes at most 2**-8 * |ref| (one
    half unit in the last place of an 8-bit significand); the FP32
    accumulation in an order the oracle does not fix contributes at most a
    few units of 2**-24 per addend, summed over K addends and bounded in the
    mean by sqrt(K) times the output scale. ``rms`` is the root mean square
    of the whole reference output; pass it when ``c_ref`` is a sample.
    """
    c_ref = np.asarray(c_ref, dtype=np.float64)
    if rms is None:
        rms = math.sqrt(float(np.mean(c_ref * c_ref))) if c_ref.size else 0.0
    return 2.0**-7 * np.abs(c_ref) + 1e-3 * math.sqrt(k) * rms


def violation_ratio(c_test: np.ndarray, c_ref: np.ndarray, k: int, rms=None) -> float:
    """max |test - ref| / bound (<= 1 passes). NaN anywhere counts as a failure."""
    c_test = np.asarray(c_test, dtype=np.float64)
    c_ref = np.asarray(c_ref, dtype=np.float64)
    if c_test.shape != c_ref.shape:
        raise ValueError(f"shape mismatch {c_test.shape} vs {c_ref.shape}")
    if c_ref.size == 0:
        return 0.0
    if np.any(np.isnan(c_test)):
        return math.inf
    bound = tolerance_bound(c_ref, k, rms)
    err = np.abs(c_test - c_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(err == 0, 0.0, err / bound)
    return float(np.max(r))


# ---------------------------------------------------------------------------
# Chained GEMMs
# ---------------------------------------------------------------------------


def gemm_chain_ref(x_bits: np.ndarray, w_bits_list) -> list:
    """The outputs C_0 .. C_(L-1) of a chain C_i = bf16(A_i . W_i^T) with
    A_0 = X and A_i = C_(i-1) (the pages' dependent launches: each step's
    activations are the previous step's stored bf16 output), as float64
    values of the bf16 outputs.

    Defined here for chains whose every output is exactly representable in
    bf16 (checked; a ValueError otherwise): the bf16 rounding between steps is
    then the identity and the chain is exact. Chains of general values are
    checked step by step instead, each step on the stored output of the one
    before it (gemm_bf16_ref)."""
    from .formats import f32_to_bf16_rne

    a_bits = np.asarray(x_bits, dtype=np.uint16)
    outs = []
    for w_bits in w_bits_list:
        c = gemm_bf16_ref(a_bits, w_bits)
        c32 = c.astype(np.float32)
        bits = f32_to_bf16_rne(c32)
        if not np.array_equal(bf16_bits_to_f64(bits), c):
            raise ValueError("a chain output is not exactly representable in bf16")
        outs.append(c)
        a_bits = bits
    return outs


# ---------------------------------------------------------------------------
# E4M3 output
# ---------------------------------------------------------------------------


def gemm_bf16_e4m3_ref(x_bits: np.ndarray, w_bits: np.ndarray, c_scale: float):
    """The E4M3-output GEMM: y = clamp(c_scale * X . W^T, -448, 448) in
    float64 (not rounded) and the codes of y, rounded to nearest even
    (``formats.e4m3_rne_sat``). Returns (y, codes)."""
    y = np.clip(gemm_bf16_ref(x_bits, w_bits) * float(c_scale), -E4M3_MAX, E4M3_MAX)
    return y, e4m3_rne_sat(y)


def e4m3_out_violation_ratio(codes: np.ndarray, ref: np.ndarray, k: int, c_scale: float, rms=None) -> float:
    """max |E4M3(code) - y| / bound over the output (<= 1 passes), with
    y = clamp(c_scale * ref, -448, 448) and

        bound = 2**-4 |y| + 2**-10 + (1 + 2**-4) * c_scale * 1e-3 * sqrt(K) * rms(ref).

    Where the kernel's FP32 value is v = c_scale * (ref + e) with |e| within
    the bf16 output's accumulation term 1e-3 sqrt(K) rms(ref) (the scale
    multiply adds one rounding of 2**-24 relative, far below it), saturation
    to [-448, 448] moves v and y by no more than |v - y|, and round to nearest
    E4M3 adds at most half a unit in the last place: 2**-4 of the magnitude
    for normal values (3 mantissa bits), 2**-10 below 2**-6 (subnormal step
    2**-9). Summed: |E4M3 - y| <= 2**-4 (|y| + |v - y|) + 2**-10 + |v - y|.
    NaN codes count as failures."""
    vals = e4m3_value(np.asarray(codes))
    ref = np.asarray(ref, dtype=np.float64)
    if vals.shape != ref.shape:
        raise ValueError(f"shape mismatch {vals.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    if np.any(np.isnan(vals)):
        return math.inf
    if rms is None:
        rms = math.sqrt(float(np.mean(ref * ref)))
    y = np.clip(ref * float(c_scale), -E4M3_MAX, E4M3_MAX)
    bound = 2.0**-4 * np.abs(y) + 2.0**-10 + (1 + 2.0**-4) * float(c_scale) * 1e-3 * math.sqrt(k) * rms
    return float(np.max(np.abs(vals - y) / bound))


# ---------------------------------------------------------------------------
# Fixed-order wave reduction
# ---------------------------------------------------------------------------


def butterfly_f32(v: np.ndarray, offsets=(32, 16, 8, 4, 2, 1)) -> np.ndarray:
    """Butterfly sum over the lanes of each 64-lane row of ``v`` in float32.

    Step by step, in the order given, every lane i replaces its value with
    value[i] + value[i ^ off], rounded to float32 (``butterfly`` / ``xred`` on
    page ``vllm.models.deepseek_v41.amd.mono.common.ops``: the order of the
    offsets is the numerical contract). ``v`` is float32 [rows, 64]; returns
    the float32 [rows, 64] lane values after the last step.
    """
    v = np.array(v, dtype=np.float32, copy=True)
    if v.ndim != 2 or v.shape[1] != 64:
        raise ValueError("expected [rows, 64] lanes")
    lanes = np.arange(64)
    for off in offsets:
        v = (v + v[:, lanes ^ off]).astype(np.float32)
    return v
