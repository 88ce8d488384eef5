"""Seeded synthetic workloads for the split-K decode GEMM.

This module only draws random inputs; it holds none of the GEMM's arithmetic.
Both the oracle-side tests and the HIP-side tests and benchmark read the same
bytes from here. Random values are drawn with numpy's PCG64 (``default_rng``)
in float32 and rounded to bf16 by torch's CPU conversion (a library routine,
round-to-nearest-even); MXFP4 weights are uniform random bytes (so every E2M1
nibble is uniform on 0..15) and uniform E8M0 codes.

Workloads (no public dataset is involved; these stand for the decode-time
shapes the pages' split-K GEMM serves):

=========================  ====  =====  =====  ===  ===========================
name                          T      K      N    S   distribution
=========================  ====  =====  =====  ===  ===========================
bf16_t1_k1024_n1024           1   1024   1024    4  W~N(0,0.02^2), X~N(0,1)
bf16_t8_k7168_n2048           8   7168   2048    4  W~N(0,0.02^2), X~N(0,1)
bf16_t32_k7168_n18432        32   7168  18432    8  as above, 1% outlier K
                                                    channels of X scaled x50
mxfp4_t16_k7168_n4096        16   7168   4096    4  nibbles U{0..15}, scale
                                                    codes U{118..130}, X~N(0,1)
mxfp8_t16_k7168_n4096        16   7168   4096    4  E4M3 codes U over the 254
                                                    non-NaN bytes, scales as above
bf16_sweep_k16384_n16384    T*  16384  16384   S*  W~N(0,0.01^2), X~N(0,1)
=========================  ====  =====  =====  ===  ===========================

T* in {1, 2, 4, 8, 16, 24, 32, 64, 128}; S* is picked per T (see ``SWEEP_SPLIT``).
The outlier reading: round(0.01 * K) distinct K indices drawn without
replacement; those columns of the float32 X are multiplied by 50 before the
single rounding to bf16.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20260

SWEEP_T = (1, 2, 4, 8, 16, 24, 32, 64, 128)
# split_k per T for the K = N = 16384 sweep (a tuning choice, not part of the
# method: every choice in {1, 2, 4, 8} gives results within the same bound).
SWEEP_SPLIT = {1: 8, 2: 8, 4: 8, 8: 8, 16: 8, 24: 8, 32: 8, 64: 4, 128: 4}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "bf16" or "mxfp4"
    T: int
    K: int
    N: int
    split_k: int
    seed: int
    w_sigma: float = 0.02
    x_sigma: float = 1.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    scale_lo: int = 118
    scale_hi: int = 130  # inclusive
    extra: dict = field(default_factory=dict)

    def weight_bytes(self) -> int:
        if self.kind == "mxfp4":
            return self.N * self.K // 2 + self.N * self.K // 32
        if self.kind == "mxfp8":
            return self.N * self.K + self.N * self.K // 32
        return self.N * self.K * 2

    def flops(self) -> int:
        return 2 * self.T * self.N * self.K


WORKLOADS = {
    "bf16_t1_k1024_n1024": Workload("bf16_t1_k1024_n1024", "bf16", 1, 1024, 1024, 4, SEED_BASE + 1),
    "bf16_t8_k7168_n2048": Workload("bf16_t8_k7168_n2048", "bf16", 8, 7168, 2048, 4, SEED_BASE + 2),
    "bf16_t32_k7168_n18432": Workload(
        "bf16_t32_k7168_n18432", "bf16", 32, 7168, 18432, 8, SEED_BASE + 3,
        outlier_frac=0.01, outlier_scale=50.0,
    ),
    "mxfp4_t16_k7168_n4096": Workload("mxfp4_t16_k7168_n4096", "mxfp4", 16, 7168, 4096, 4, SEED_BASE + 4),
    # the MXFP4 shape with eight-bit E4M3 elements (an extra, not one of the pages' workloads)
    "mxfp8_t16_k7168_n4096": Workload("mxfp8_t16_k7168_n4096", "mxfp8", 16, 7168, 4096, 4, SEED_BASE + 200),
}


def sweep_workload(T: int, split_k: int | None = None) -> Workload:
    """The K = N = 16384 bf16 sweep point at T tokens."""
    s = SWEEP_SPLIT.get(T, 4) if split_k is None else split_k
    return Workload(
        f"bf16_sweep_t{T}_k16384_n16384", "bf16", T, 16384, 16384, s, SEED_BASE + 5 + T,
        w_sigma=0.01,
    )


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name.startswith("bf16_sweep_t"):
        return sweep_workload(int(name[len("bf16_sweep_t"):].split("_")[0]))
    raise KeyError(name)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16) through torch's CPU conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, sigma: float, chunk_rows: int = 4096) -> np.ndarray:
    """N(0, sigma^2) draws rounded to bf16, generated in row chunks (bounded memory)."""
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            z *= np.float32(sigma)
        out[r0:r1] = to_bf16_bits(z)
    return out


def gen_x(w: Workload, T: int | None = None, seed_offset: int = 0) -> np.ndarray:
    """Activations X [T, K] as bf16 bits."""
    T = w.T if T is None else T
    rng = np.random.default_rng(w.seed * 1000 + 1 + seed_offset)
    z = rng.standard_normal((T, w.K), dtype=np.float32) * np.float32(w.x_sigma)
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * w.K))
        cols = rng.choice(w.K, size=n_out, replace=False)
        z[:, cols] *= np.float32(w.outlier_scale)
    return to_bf16_bits(z)


def gen_w_bf16(w: Workload, rows: int | None = None) -> np.ndarray:
    """Weights W [N, K] as bf16 bits (first ``rows`` rows only when given)."""
    rng = np.random.default_rng(w.seed * 1000 + 2)
    n = w.N if rows is None else rows
    return normal_bf16(rng, (n, w.K), w.w_sigma)


def gen_w_mxfp4(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 weights: (Wq uint8 [N, K/2], Wscale uint8 [N, K/32])."""
    rng = np.random.default_rng(w.seed * 1000 + 3)
    wq = rng.integers(0, 256, size=(w.N, w.K // 2), dtype=np.uint8)
    ws = rng.integers(w.scale_lo, w.scale_hi + 1, size=(w.N, w.K // 32), dtype=np.uint8)
    return wq, ws


def mxfp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform E4M3FN codes over the 254 non-NaN bytes (0x7F and 0xFF excluded)."""
    c = rng.integers(0, 254, size=shape, dtype=np.int32)
    c = c + (c >= 0x7F)  # skip 0x7F
    c = c + (c >= 0xFF)  # skip 0xFF (0xFE + 1 above lands on 0xFF)
    return np.minimum(c, 0xFE).astype(np.uint8)


def gen_w_mxfp8(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 weights: (Wq8 uint8 [N, K] E4M3 codes, Wscale uint8 [N, K/32])."""
    rng = np.random.default_rng(w.seed * 1000 + 4)
    wq8 = mxfp8_codes(rng, (w.N, w.K))
    ws = rng.integers(w.scale_lo, w.scale_hi + 1, size=(w.N, w.K // 32), dtype=np.uint8)
    return wq8, ws


def small_mxfp8_case(T: int, K: int, N: int, seed: int, lo: int = 118, hi: int = 130):
    """A small seeded (X, Wq8, Wscale) triple for parity tests."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    wq8 = mxfp8_codes(rng, (N, K))
    ws = rng.integers(lo, hi + 1, size=(N, K // 32), dtype=np.uint8)
    return x, wq8, ws


def small_bf16_case(T: int, K: int, N: int, seed: int, w_sigma: float = 0.02):
    """A small seeded (X, W) pair of bf16 bit arrays for parity tests."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    wv = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_sigma)
    return x, to_bf16_bits(wv)


def small_mxfp4_case(T: int, K: int, N: int, seed: int, lo: int = 118, hi: int = 130):
    """A small seeded (X, Wq, Wscale) triple for parity tests."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ws = rng.integers(lo, hi + 1, size=(N, K // 32), dtype=np.uint8)
    return x, wq, ws


def integer_bf16_case(T: int, K: int, N: int, seed: int, mag: int = 3):
    """Integer-valued operands in [-mag, mag] as bf16 bits (exactly representable)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-mag, mag + 1, size=(T, K)).astype(np.float32)
    wv = rng.integers(-mag, mag + 1, size=(N, K)).astype(np.float32)
    return to_bf16_bits(x), to_bf16_bits(wv)
