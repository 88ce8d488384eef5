"""Bit-exact GPU checks of the device helpers against the oracle: bf16 and
E4M3 packing, the fixed-order wave sum and the MXFP4 decode."""

import numpy as np
import pytest

import split_reduction_amd as sk
from oracle import formats as F
from oracle import gemm as G
from tests.gpu_util import DEV, bf16_bits, log, to_dev_f32, to_dev_u8, torch
import workloads

pytestmark = pytest.mark.gpu


def _u32_out(n):
    t = torch()
    return t.empty(n, dtype=t.int32, device=DEV)


def test_pack_bf16_bit_exact():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(21)
    pats = np.concatenate([pats, rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)])
    if len(pats) % 2:
        pats = pats[:-1]
    x = pats.view(np.float32)
    log(f"pack_bf16: {len(x)} values")
    out = _u32_out(len(x) // 2)
    sk.skgemm_pack_bf16(to_dev_f32(x), out, len(x) // 2)
    torch().cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    lo = (got & 0xFFFF).astype(np.uint16)
    hi_ = (got >> 16).astype(np.uint16)
    gb = np.empty(len(x), dtype=np.uint16)
    gb[0::2], gb[1::2] = lo, hi_
    ref = F.f32_to_bf16_rne(x)
    nan = np.isnan(x)
    assert np.array_equal(gb[~nan], ref[~nan])
    assert np.all(np.isnan(F.bf16_bits_to_f64(gb[nan])))


def test_pack_e4m3_bit_exact():
    mags = F.e4m3_value(np.arange(0x7F))
    mids = (mags[:-1] + mags[1:]) / 2
    vals = np.concatenate([mags, mids]).astype(np.float32)
    v = np.concatenate([vals, np.nextafter(vals, np.float32(np.inf)), np.nextafter(vals, np.float32(0))])
    rng = np.random.default_rng(22)
    v = np.concatenate([v, (rng.random(1 << 18) * 448).astype(np.float32)])
    v = v[np.abs(v) <= 448]
    v = np.concatenate([v, -v])
    v = v[: len(v) // 4 * 4]
    log(f"pack_e4m3: {len(v)} values")
    out = _u32_out(len(v) // 4)
    sk.skgemm_pack_e4m3(to_dev_f32(v), out, len(v) // 4)
    torch().cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    q = v.reshape(-1, 4)
    ref = F.e4m3_pack4_word(q[:, 0], q[:, 1], q[:, 2], q[:, 3])
    bad = np.nonzero(got != ref)[0]
    assert len(bad) == 0, [(q[i].tolist(), hex(got[i]), hex(ref[i])) for i in bad[:8]]


def test_wave_sum_bit_exact_and_ordered():
    rng = np.random.default_rng(23)
    v = rng.standard_normal((4096, 64)).astype(np.float32) * np.float32(1e3)
    crafted = np.zeros((1, 64), dtype=np.float32)
    crafted[0, 0], crafted[0, 1], crafted[0, 33] = 2.0**24, 1.0, 1.0
    ints = rng.integers(-1000, 1000, size=(64, 64)).astype(np.float32)
    v = np.concatenate([v, crafted, ints])
    log(f"wave_sum: {v.shape[0]} waves")
    t = torch()
    out = t.empty(v.size, dtype=t.float32, device=DEV)
    sk.skgemm_wave_sum(to_dev_f32(v.ravel()), out, v.shape[0])
    t.cuda.synchronize()
    got = out.cpu().numpy().reshape(v.shape)
    ref = G.butterfly_f32(v)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.all(got[4096] == 2.0**24 + 2)  # the order-sensitive case


def test_mxfp4_dequant_every_code_and_scale():
    codes = np.arange(16, dtype=np.uint8)
    scales = np.arange(2, 253, dtype=np.uint8)
    n = len(scales)
    nib = np.tile(codes, 2)
    row = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)  # 32 elements = 16 bytes
    wq = np.tile(row, (n, 1))
    ws = scales.reshape(n, 1)
    log(f"mxfp4_dequant: {n} scales x 16 codes")
    t = torch()
    out = t.empty((n, 32), dtype=t.bfloat16, device=DEV)
    sk.skgemm_mxfp4_dequant(to_dev_u8(wq), to_dev_u8(ws), out, n, 32)
    t.cuda.synchronize()
    got = bf16_bits(out)
    ref = F.mxfp4_dequant_bf16_bits(wq, ws)
    assert np.array_equal(got, ref)


def test_mxfp4_dequant_workload_tensor():
    w = workloads.WORKLOADS["mxfp4_t16_k7168_n4096"]
    wq, ws = workloads.gen_w_mxfp4(w)
    log(f"mxfp4_dequant: {w.name} weights")
    t = torch()
    out = t.empty((w.N, w.K), dtype=t.bfloat16, device=DEV)
    sk.skgemm_mxfp4_dequant(to_dev_u8(wq), to_dev_u8(ws), out, w.N, w.K)
    t.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), F.mxfp4_dequant_bf16_bits(wq, ws))


def test_read_probe_reads_and_writes_nothing():
    """The streaming-read reference runs over odd and large sizes and leaves
    its sink untouched (it stores only on an impossible fold value)."""
    t = torch()
    buf = t.randint(0, 2**31 - 1, (1 << 22,), dtype=t.int32, device=DEV)
    sink = t.zeros(512, dtype=t.int32, device=DEV)
    for nbytes in (16, 4096 + 16, 1 << 20, buf.numel() * 4):
        log(f"read probe {nbytes} bytes")
        sk.skgemm_read_probe(buf, nbytes, sink)
    t.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0
    with pytest.raises(sk.SkgemmError) as e:
        sk.skgemm_read_probe(buf, 24, sink)
    assert e.value.code == sk.SKGEMM_EINVAL


def test_mxfp8_dequant_every_code_and_scale():
    """The in-register E4M3 decode, bit for bit against the oracle: every
    code (NaN codes stay NaN) at every scale 10..246, and the byte order
    (element k of a row in byte k)."""
    t = torch()
    codes = np.arange(256, dtype=np.uint8)
    scales = np.arange(10, 247, dtype=np.uint8)
    n = len(scales)
    wq8 = np.tile(codes, (n, 1))
    ws = np.repeat(scales.reshape(n, 1), 256 // 32, axis=1)
    out = t.empty((n, 256), dtype=t.int16, device=DEV)
    log(f"mxfp8 dequant {n} scales x 256 codes")
    sk.skgemm_mxfp8_dequant(to_dev_u8(wq8), to_dev_u8(ws), out, n, 256)
    t.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = F.mxfp8_dequant_bf16_bits(wq8, ws)
    nan_g = np.isnan(F.bf16_bits_to_f64(got))
    nan_w = np.isnan(F.bf16_bits_to_f64(want))
    assert np.array_equal(nan_g, nan_w)
    assert np.array_equal(got[~nan_w], want[~nan_w])


def test_mxfp8_dequant_workload_tensor():
    w = workloads.WORKLOADS["mxfp8_t16_k7168_n4096"]
    wq8, ws = workloads.gen_w_mxfp8(w)
    t = torch()
    out = t.empty((w.N, w.K), dtype=t.int16, device=DEV)
    log("mxfp8 dequant of the whole T=16 K=7168 N=4096 weight tensor")
    sk.skgemm_mxfp8_dequant(to_dev_u8(wq8), to_dev_u8(ws), out, w.N, w.K)
    t.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), F.mxfp8_dequant_bf16_bits(wq8, ws))
