"""Helpers for the GPU tests: device upload/download and the parity check.

Inputs come from ``workloads`` (seeded, host-generated) and expected values
from ``oracle``; the device side is reached only through the C ABI binding.
"""

import sys

import numpy as np

DEV = "cuda:0"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch():
    import torch as _t

    return _t


def to_dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(t.bfloat16)


def to_dev_u8(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def to_dev_f32(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bf16_bits(t_dev) -> np.ndarray:
    t = torch()
    return t_dev.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def empty_bf16(T: int, N: int):
    t = torch()
    return t.empty((T, N), dtype=t.bfloat16, device=DEV)


# A quiet-NaN bf16 pattern no kernel produces from finite inputs. Outputs are
# filled with it before a call, so an element the call never wrote (a tile no
# workgroup finished) cannot pass on a value left in memory by an earlier call.
SENTINEL = 0x7FC1


def sentinel_bf16(T: int, N: int):
    t = torch()
    return t.full((T, N), SENTINEL, dtype=t.int16, device=DEV).view(t.bfloat16)


def checked_bits(C) -> np.ndarray:
    """C's bits after a call; fails if any element still holds the sentinel."""
    bits = bf16_bits(C)
    left = int(np.count_nonzero(bits == SENTINEL))
    assert left == 0, f"{left} output elements were never written"
    return bits


def run_bf16(x_bits, w_bits, split_k, W=None):
    """C bits from skgemm_bf16 on the given host operands."""
    import split_reduction_amd as sk

    T, K = x_bits.shape
    N = w_bits.shape[0] if W is None else W.shape[0]
    X = to_dev_bf16(x_bits)
    W = to_dev_bf16(w_bits) if W is None else W
    C = sentinel_bf16(T, N)
    sk.skgemm_bf16(W, X, C, T, N, K, split_k)
    torch().cuda.synchronize()
    return checked_bits(C)


def run_mxfp4(x_bits, wq, ws, split_k):
    import split_reduction_amd as sk

    T, K = x_bits.shape
    N = wq.shape[0]
    X = to_dev_bf16(x_bits)
    Wq = to_dev_u8(wq)
    Ws = to_dev_u8(ws)
    C = sentinel_bf16(T, N)
    sk.skgemm_mxfp4(Wq, Ws, X, C, T, N, K, split_k)
    torch().cuda.synchronize()
    return checked_bits(C)


def assert_parity(c_bits, c_ref, K, what, rms=None):
    """Element-wise |C - ref| <= 2^-7 |ref| + 1e-3 sqrt(K) rms(ref)."""
    from oracle import formats, gemm

    c = formats.bf16_bits_to_f64(c_bits)
    ratio = gemm.violation_ratio(c, c_ref, K, rms)
    log(f"  {what}: max |err|/bound = {ratio:.4f}")
    assert ratio <= 1.0, f"{what}: parity ratio {ratio}"
    return ratio


def run_mxfp8(x_bits, wq8, ws, split_k):
    import split_reduction_amd as sk

    T, K = x_bits.shape
    N = wq8.shape[0]
    X = to_dev_bf16(x_bits)
    Wq = to_dev_u8(wq8)
    Ws = to_dev_u8(ws)
    C = sentinel_bf16(T, N)
    sk.skgemm_mxfp8(Wq, Ws, X, C, T, N, K, split_k)
    torch().cuda.synchronize()
    return checked_bits(C)
