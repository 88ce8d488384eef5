"""Benchmark of the split-K decode GEMM on one MI355X.

Prints ONE JSON line. The headline workload is the largest single-GPU
configuration: bf16 T=32, K=16384, N=16384, split_k=8 (W ~ N(0, 0.01^2),
X ~ N(0, 1)), the largest token count of the K = N = 16384 sweep that the
70 %-of-peak target covers (T <= 32). One step is one skgemm_bf16 call (the
whole hot path: weight stream, X staging, MFMA, LDS and split-K reductions,
bf16 epilogue). The metric is the weight-stream rate: weight bytes per step /
step time, in TB/s, and its fraction of the 8 TB/s HBM3E peak.

Timing protocol:
* inputs are resident in HBM before the timed region; R copies of the weights
  (R * weight bytes >= 1 GiB, four times the 256 MiB last-level cache) are
  rotated so every step streams weights that are not cache-resident;
* W untimed warmup steps run eagerly, then exactly K steps are replayed from
  one HIP graph (no host launch gaps), bracketed by synchronisations and
  timed with HIP events recorded on the stream the kernels run on;
* the same protocol without rotation gives the labelled cache-resident rate.

The other workloads (bf16 T=1 K=1024 N=1024; bf16 T=8 K=7168 N=2048; bf16
T=32 K=7168 N=18432 with outlier channels; MXFP4 and MXFP8 T=16 K=7168
N=4096; the rest of the K = N = 16384 bf16 sweep over T) are timed the same
way and reported under "workloads", each with its own roofline block. The
cpu_baseline leg times the fp64 oracle's GEMM on the host on the headline
workload (the bf16 -> fp64 conversion of the weights done once, outside the
timing).

``--trace-summary DIR`` reads a rocprofv3 kernel trace written under DIR and
prints per-workload kernel durations (runs of dispatches in time order).

``--pmc-run [WORKLOAD ...|all]`` is the short program the HBM counters are
taken on: 10 eager launches of each named workload on rotated weights, then 5
plain device copies of 256 MiB (which read and write exactly 256 MiB each)
that calibrate the counters. ``--pmc-summary DIR [WORKLOAD ...|all]`` turns
the rocprofv3 counter CSVs under DIR into bytes per launch for each workload
and writes ``profiles/traffic_<workload>.json``.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
ROTATE_BYTES = 1 << 30
HEADLINE = "bf16_sweep_t32_k16384_n16384"
CSRC = os.path.join("split_reduction_amd", "csrc")


def kernel_sources() -> list:
    """Every kernel, launch and header source of the library (repo-relative)."""
    out = []
    for d, _, files in os.walk(os.path.join(ROOT, CSRC)):
        out += [os.path.relpath(os.path.join(d, f), ROOT) for f in files if f.endswith((".hip", ".h"))]
    return sorted(out)


def kernel_source_hash(read=None) -> str:
    """Hash of the library sources; HBM counters are used only while it matches."""
    h = hashlib.sha256()
    for rel in kernel_sources():
        if read is None:
            with open(os.path.join(ROOT, rel), "rb") as f:
                data = f.read()
        else:
            data = read(rel)
        h.update(rel.encode() + b"\0" + data)
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------


class Case:
    """Device-resident operands of one workload at one T, with rotated weights."""

    def __init__(self, wl: workloads.Workload, host_w=None):
        import torch

        self.wl = wl
        self.torch = torch
        dev = "cuda:0"
        x = workloads.gen_x(wl)
        self.x_bits = x
        self.X = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.C = torch.empty((wl.T, wl.N), dtype=torch.bfloat16, device=dev)
        if wl.kind in ("mxfp4", "mxfp8"):
            gen = workloads.gen_w_mxfp4 if wl.kind == "mxfp4" else workloads.gen_w_mxfp8
            wq, ws = host_w if host_w is not None else gen(wl)
            base = (torch.from_numpy(wq).to(dev), torch.from_numpy(ws).to(dev))
        else:
            wb = host_w if host_w is not None else workloads.gen_w_bf16(wl)
            base = (torch.from_numpy(wb.view(np.int16)).to(dev).view(torch.bfloat16),)
        self.copies = max(1, math.ceil(ROTATE_BYTES / wl.weight_bytes()))
        self.weights = [base] + [tuple(t.clone() for t in base) for _ in range(self.copies - 1)]

    def launch(self, i: int, stream):
        import split_reduction_amd as sk

        wl = self.wl
        w = self.weights[i % len(self.weights)]
        if wl.kind == "mxfp4":
            sk.skgemm_mxfp4(w[0], w[1], self.X, self.C, wl.T, wl.N, wl.K, wl.split_k, stream)
        elif wl.kind == "mxfp8":
            sk.skgemm_mxfp8(w[0], w[1], self.X, self.C, wl.T, wl.N, wl.K, wl.split_k, stream)
        else:
            sk.skgemm_bf16(w[0], self.X, self.C, wl.T, wl.N, wl.K, wl.split_k, stream)

    def time(self, steps: int, warmup: int, rotate: bool = True, probe: bool = False) -> dict:
        """Per-launch time of exactly `steps` launches replayed from one graph.
        probe=True times the streaming-read reference over the same rotated
        weight buffers instead of the GEMM."""
        torch = self.torch
        import split_reduction_amd as sk

        wl = self.wl
        stream = torch.cuda.Stream()
        sk.skgemm_reserve(wl.T, wl.N, wl.split_k, stream)
        if probe:
            sink = torch.zeros(512, dtype=torch.int32, device="cuda:0")

            def launch(i, st):
                w = self.weights[i % len(self.weights)][0]
                sk.skgemm_read_probe(w, w.numel() * w.element_size(), sink, st)
        else:
            launch = self.launch
        with torch.cuda.stream(stream):
            for i in range(warmup):
                launch(i if rotate else 0, stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                launch(i if rotate else 0, stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()  # the graph's own first replay (uploads it); untimed
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):  # replay() launches on the current stream
            start.record(stream)
            g.replay()
            end.record(stream)
        end.synchronize()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        del g
        t_s = ms * 1e-3 / steps
        return {
            "t_us": t_s * 1e6,
            "weight_TBps": wl.weight_bytes() / t_s / 1e12,
            "algo_GBps": self.algo_bytes() / t_s / 1e9,
            "TFLOPs": wl.flops() / t_s / 1e12,
        }

    def time_batched(self, L: int, steps: int, warmup: int) -> dict:
        """Per-launch time of batched launches of L independent problems
        (distinct weights and activations per problem), cold rotated weights."""
        torch = self.torch
        import split_reduction_amd as sk

        wl = self.wl
        dev = "cuda:0"
        R = max(2, math.ceil(ROTATE_BYTES / (L * wl.weight_bytes())))
        base = self.weights[0]
        wq = torch.empty((R, L) + tuple(base[0].shape), dtype=base[0].dtype, device=dev)
        wq.copy_(base[0].expand(R, L, *base[0].shape))
        ws = None
        if wl.kind in ("mxfp4", "mxfp8"):
            ws = torch.empty((R, L) + tuple(base[1].shape), dtype=base[1].dtype, device=dev)
            ws.copy_(base[1].expand(R, L, *base[1].shape))
        X = self.X.expand(L, *self.X.shape).contiguous()
        C = torch.empty((L, wl.T, wl.N), dtype=torch.bfloat16, device=dev)
        wstride = base[0].numel() * base[0].element_size()
        xstride = self.X.numel() * 2
        cstride = wl.T * wl.N * 2
        stream = torch.cuda.Stream()
        sk.skgemm_reserve_batched(wl.T, wl.N, wl.split_k, L, stream)

        def launch(i, st):
            r = i % R
            if wl.kind in ("mxfp4", "mxfp8"):
                fn = sk.skgemm_mxfp4_batched if wl.kind == "mxfp4" else sk.skgemm_mxfp8_batched
                fn(wq[r], ws[r], X, C, wl.T, wl.N, wl.K, wl.split_k, L, wstride, base[1].numel(), xstride,
                   cstride, st)
            else:
                sk.skgemm_bf16_batched(wq[r], X, C, wl.T, wl.N, wl.K, wl.split_k, L, wstride, xstride,
                                       cstride, st)

        with torch.cuda.stream(stream):
            for i in range(warmup):
                launch(i, stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                launch(i, stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            start.record(stream)
            g.replay()
            end.record(stream)
        end.synchronize()
        t_s = start.elapsed_time(end) * 1e-3 / steps
        del g, wq, ws, X, C
        return {"L": L, "t_us": round(t_s * 1e6, 3), "t_us_per_problem": round(t_s * 1e6 / L, 3),
                "weight_TBps": round(L * wl.weight_bytes() / t_s / 1e12, 4)}

    def algo_bytes(self) -> int:
        """Compulsory bytes of one call: weights + X + C."""
        wl = self.wl
        return wl.weight_bytes() + 2 * wl.T * wl.K + 2 * wl.T * wl.N


BATCH_L = 8  # problems per batched launch reported for the small workloads
BATCH_MAX_WEIGHT_BYTES = 64 << 20

# Every workload the benchmark reports, the headline first. The K = N = 16384
# sweep points share one weight matrix (generated once).
OTHERS = ("bf16_t1_k1024_n1024", "bf16_t8_k7168_n2048", "bf16_t32_k7168_n18432",
          "mxfp4_t16_k7168_n4096", "mxfp8_t16_k7168_n4096")


def all_workloads() -> list:
    sweep = [workloads.sweep_workload(T).name for T in workloads.SWEEP_T]
    return [HEADLINE] + list(OTHERS) + [n for n in sweep if n != HEADLINE]


def is_sweep(name: str) -> bool:
    return name.startswith("bf16_sweep_t")


def roofline_block(name: str, algo_bytes: int, t_us: float) -> dict:
    """HBM roofline of one workload's kernel: algorithmic bytes (weights + X +
    C) per launch over the measured launch time, against the 8 TB/s peak, and
    the HBM bytes the rocprofv3 counters saw per launch (None unless they were
    taken on the current kernel sources)."""
    achieved = algo_bytes / (t_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(name),
            "algorithmic_bytes": algo_bytes}


def run_workload(wl, steps, warmup, host_w=None) -> dict:
    import split_reduction_amd as sk

    case = Case(wl, host_w)
    cold = case.time(steps, warmup, rotate=True)
    hot = case.time(steps, warmup, rotate=False)
    probe = case.time(steps, warmup, rotate=True, probe=True)
    batched = None
    if wl.weight_bytes() <= BATCH_MAX_WEIGHT_BYTES:
        batched = case.time_batched(BATCH_L, steps, warmup)
    probe_bytes = case.weights[0][0].numel() * case.weights[0][0].element_size()
    probe_tbps = probe_bytes / (probe["t_us"] * 1e-6) / 1e12
    tac = sk.skgemm_tactic_for(wl.T, wl.N, wl.K, wl.split_k, {"bf16": 0, "mxfp4": 1, "mxfp8": 2}[wl.kind])
    out = {
        "workload": wl.name, "kind": wl.kind, "T": wl.T, "K": wl.K, "N": wl.N,
        "split_k": wl.split_k, "weight_bytes": wl.weight_bytes(), "flops": wl.flops(),
        "rotated_copies": case.copies,
        "t_us": round(cold["t_us"], 3),
        "weight_TBps": round(cold["weight_TBps"], 4),
        "frac_hbm_peak": round(cold["weight_TBps"] * 1000 / HBM_PEAK_GBS, 4),
        "TFLOPs": round(cold["TFLOPs"], 3),
        "frac_mfma_peak": round(cold["TFLOPs"] / BF16_MFMA_PEAK_TFLOPS, 5),
        "roofline": roofline_block(wl.name, case.algo_bytes(), cold["t_us"]),
        "hot_t_us": round(hot["t_us"], 3),
        "hot_weight_TBps": round(hot["weight_TBps"], 4),
        # The streaming-read reference over the same rotated buffers: what a
        # plain coalesced read of this many bytes reaches on this GPU.
        "read_probe": {"bytes": probe_bytes, "t_us": round(probe["t_us"], 3),
                       "TBps": round(probe_tbps, 4),
                       "gemm_frac": round(cold["weight_TBps"] / probe_tbps, 4)},
        "tactic": {k: tac[k] for k in ("kind", "nt", "wk", "wn", "d", "kc", "tile_n", "grid", "shape",
                                       "fold", "pdefer")},
    }
    if batched is not None:
        out["batched"] = batched
    del case
    import torch

    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# Chained launches (the pages' launch overlap)
# ---------------------------------------------------------------------------

CHAIN_DIMS = [7168, 2048] * 4 + [7168]  # eight steps: the T=8 K=7168 N=2048 shape and its transpose


def chain_bench(steps: int, warmup: int, T: int = 8, S: int = 4) -> dict:
    """Per-step time of eight dependent GEMMs (X of step i+1 is C of step i),
    alternating K=7168 -> N=2048 and K=2048 -> N=7168 (29.4 MB of bf16 weights
    each), T=8, split_k=4, cold weights (sets of the eight matrices rotated
    through >= 1 GiB): one skgemm_bf16_chain launch per chain, against the
    same eight steps as separate skgemm_bf16 launches replayed from a graph."""
    import torch

    import split_reduction_amd as sk

    dev = "cuda:0"
    L = len(CHAIN_DIMS) - 1
    rng = np.random.default_rng(SEED_CHAIN)
    base = [torch.from_numpy(workloads.normal_bf16(rng, (CHAIN_DIMS[i + 1], CHAIN_DIMS[i]), 0.02).view(np.int16))
            .to(dev).view(torch.bfloat16) for i in range(L)]
    set_bytes = sum(w.numel() * 2 for w in base)
    R = max(2, math.ceil(ROTATE_BYTES / set_bytes))
    sets = [base] + [[w.clone() for w in base] for _ in range(R - 1)]
    X = torch.from_numpy(workloads.normal_bf16(rng, (T, CHAIN_DIMS[0]), 1.0).view(np.int16)).to(dev).view(torch.bfloat16)
    Cs = [torch.empty((T, d), dtype=torch.bfloat16, device=dev) for d in CHAIN_DIMS[1:]]
    stream = torch.cuda.Stream()
    sk.skgemm_reserve(T, max(CHAIN_DIMS), S, stream)

    def chain(i):
        sk.skgemm_bf16_chain(sets[i % R], X, Cs, CHAIN_DIMS, T, S, stream)

    def separate(i):
        ws = sets[i % R]
        for j in range(L):
            sk.skgemm_bf16(ws[j], X if j == 0 else Cs[j - 1], Cs[j], T, CHAIN_DIMS[j + 1], CHAIN_DIMS[j], S, stream)

    def timed(fn, n, graph):
        with torch.cuda.stream(stream):
            for i in range(warmup):
                fn(i)
        stream.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    fn(i)
            with torch.cuda.stream(stream):
                g.replay()
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                start.record(stream)
                g.replay()
                end.record(stream)
        else:
            with torch.cuda.stream(stream):
                start.record(stream)
                for i in range(n):
                    fn(i)
                end.record(stream)
        end.synchronize()
        return start.elapsed_time(end) * 1e3 / (n * L)

    # a longer chain of the same steps: the launch's fixed cost spread wider
    L4 = 4 * L
    dims4 = CHAIN_DIMS + CHAIN_DIMS[1:] * 3
    Cs4 = [torch.empty((T, d), dtype=torch.bfloat16, device=dev) for d in dims4[1:]]

    def chain4(i):
        ws = sets[i % R] * 4
        sk.skgemm_bf16_chain(ws, X, Cs4, dims4, T, S, stream)

    n = max(10, steps // 4)
    t_chain = timed(chain, n, graph=False)
    t_chain4 = timed(chain4, max(4, n // 4), graph=False) * L / L4
    t_sep = timed(separate, n, graph=True)
    del sets, base
    torch.cuda.empty_cache()
    return {"steps": L, "T": T, "split_k": S, "dims": CHAIN_DIMS,
            "weight_bytes_per_step": set_bytes // L, "chains_timed": n,
            "t_us_per_step_chain_launch": round(t_chain, 3),
            "t_us_per_step_chain_launch_32_steps": round(t_chain4, 3),
            "t_us_per_step_separate_launches_graph": round(t_sep, 3),
            "weight_TBps_chain": round(set_bytes / L / (t_chain * 1e-6) / 1e12, 4),
            "timing": "chain: eager launches on one stream, HIP events; separate: one graph of all launches"}


SEED_CHAIN = workloads.SEED_BASE + 300


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host cores
# ---------------------------------------------------------------------------


def cpu_baseline(wl, wb=None, budget_s: float = 12.0) -> dict:
    """The oracle's fp64 GEMM on the host, timed alone: the weights are
    decoded to float64 once before the timing (as the oracle's
    gemm_decoded_ref takes them), then the GEMM is repeated for ``budget_s``."""
    from oracle import formats, gemm

    x = workloads.gen_x(wl)
    if wb is None:
        wb = workloads.gen_w_bf16(wl)
    w64 = formats.bf16_bits_to_f64(wb)
    try:
        from threadpoolctl import threadpool_info

        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: report the visible CPUs
        cores = os.cpu_count() or 1
    gemm.gemm_decoded_ref(x, w64)  # first call outside the timing
    n = 0
    t0 = time.perf_counter()
    while True:
        gemm.gemm_decoded_ref(x, w64)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / n
    del w64
    return {
        "value": round(wl.weight_bytes() / per / 1e12, 6),
        "unit": "TB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"the whole {wl.name} workload: the oracle's fp64 numpy GEMM on weights decoded "
                   f"to fp64 once beforehand, {n} calls in {el:.1f} s, {per * 1e3:.2f} ms per call "
                   f"({wl.flops() / per / 1e9:.1f} GFLOP/s)"),
    }


# ---------------------------------------------------------------------------
# rocprofv3 trace summary
# ---------------------------------------------------------------------------


def trace_summary(path: str, steps: int, warmup: int) -> None:
    """Per-kernel durations from a rocprofv3 kernel trace of this script.

    Dispatches are taken in time order and cut into runs of the same kernel
    and grid. The first run is the headline workload's single launches: per
    timing pass, W eager warmup launches, the graph's untimed first replay and
    its timed replay of K launches; one cold (rotated weights) pass, then one
    cache-resident pass.
    """
    import csv

    files = glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {path}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows = [r for r in rows if "splitk_" in r.get("Kernel_Name", "")]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    segs = []
    for r in rows:
        key = (r["Kernel_Name"], r.get("Grid_Size", r.get("Grid_Size_X", "?")))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        if segs and segs[-1][0] == key:
            segs[-1][1].append(dur)
        else:
            segs.append((key, [dur]))
    print("run  calls   avg(us)   med(us)   min(us)     grid  kernel")
    singles = {}  # one-dispatch runs (launches alternating between kernels), grouped by kernel
    for i, ((name, grid), durs) in enumerate(segs):
        d = np.array(durs)
        short = name.replace("void skg::", "").replace("(skg::GemmParams)", "").replace("(skg::ChainParams)", "")
        if len(d) == 1:
            singles.setdefault((short, grid), []).append(d[0])
            continue
        print(f"{i:3d} {len(d):6d} {d.mean():9.3f} {np.median(d):9.3f} {d.min():9.3f} {grid:>8}  {short}")
    for (short, grid), durs in singles.items():
        d = np.array(durs)
        print(f"  * {len(d):6d} {d.mean():9.3f} {np.median(d):9.3f} {d.min():9.3f} {grid:>8}  {short}"
              "  (one-dispatch runs, alternating kernels)")
    per_pass = warmup + 2 * steps
    head = [s for s in segs if len(s[1]) >= 2 * per_pass]
    if head:
        d = np.array(head[0][1])
        if len(d) >= 2 * per_pass:
            cold = d[warmup + steps:per_pass]
            hot = d[per_pass + warmup + steps:2 * per_pass]
            print(f"headline cold timed replay: {len(cold)} launches, avg {cold.mean():.3f} us, "
                  f"median {np.median(cold):.3f} us")
            print(f"headline cache-resident timed replay: {len(hot)} launches, avg {hot.mean():.3f} us")


# ---------------------------------------------------------------------------
# rocprofv3 counter passes
# ---------------------------------------------------------------------------

COPY_BYTES = 256 << 20
PMC_LAUNCHES = 10
PMC_COPIES = 5


def pmc_names(args: list) -> list:
    if not args or args == ["all"]:
        return all_workloads() if args == ["all"] else [HEADLINE]
    return list(args)


def pmc_run(names: list) -> None:
    """PMC_LAUNCHES eager launches of each workload in turn (rotated weights),
    then the calibration copies. Progress goes to stderr per workload."""
    import torch

    import split_reduction_amd as sk

    sweep_w = None
    stream = torch.cuda.current_stream()
    for name in names:
        wl = workloads.get(name)
        host_w = None
        if is_sweep(name):
            if sweep_w is None:
                sweep_w = workloads.gen_w_bf16(workloads.sweep_workload(1))
            host_w = sweep_w
        case = Case(wl, host_w)
        for i in range(PMC_LAUNCHES):
            case.launch(i, stream)
        torch.cuda.synchronize()
        del case
        torch.cuda.empty_cache()
        log(f"pmc-run {name}: {PMC_LAUNCHES} launches")
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0").random_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(PMC_COPIES):
        dst.copy_(src)
    torch.cuda.synchronize()
    del sk
    print(json.dumps({"pmc_run": names, "launches": PMC_LAUNCHES, "copies": PMC_COPIES,
                      "copy_bytes": COPY_BYTES}))


def _counter_rows(path: str, counter: str) -> list:
    import csv

    rows = []
    for f in sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r.get("Counter_Name") == counter]
    if not rows:
        raise SystemExit(f"no {counter} rows under {path}")
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _per_workload(rows: list, names: list) -> list:
    """The GEMM dispatches of a --pmc-run, cut into consecutive groups of
    PMC_LAUNCHES, one per workload in run order: [(kernel, [values])]."""
    gemm = [r for r in rows if "splitk_" in r["Kernel_Name"]]
    if len(gemm) != PMC_LAUNCHES * len(names):
        raise SystemExit(f"{len(gemm)} GEMM dispatches for {len(names)} workloads")
    out = []
    for i, _ in enumerate(names):
        grp = gemm[i * PMC_LAUNCHES:(i + 1) * PMC_LAUNCHES]
        kernels = {r["Kernel_Name"] for r in grp}
        if len(kernels) != 1:
            raise SystemExit(f"workload {names[i]}: kernels {kernels}")
        out.append((kernels.pop(), [float(r["Counter_Value"]) for r in grp]))
    return out


def pmc_summary(path: str, names: list) -> list:
    """HBM bytes per launch of each workload from the FETCH_SIZE and
    WRITE_SIZE passes of ``--pmc-run`` under ``path`` (KiB per dispatch, each
    scaled by what the same counter reads for the 256 MiB calibration copies:
    the last PMC_COPIES copyBuffer dispatches of the run). Writes
    profiles/traffic_<workload>.json per workload and profiles/traffic_summary.md."""
    per = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        rows = _counter_rows(os.path.join(path, counter.split("_")[0].lower()), counter)
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-PMC_COPIES:]
        if len(copies) != PMC_COPIES:
            raise SystemExit(f"{counter}: {len(copies)} calibration copies")
        per[counter] = (_per_workload(rows, names), float(np.mean(copies)))
    fetch_factor = per["FETCH_SIZE"][1] * 1024 / COPY_BYTES
    write_factor = per["WRITE_SIZE"][1] * 1024 / COPY_BYTES
    sha = kernel_source_hash()
    outs = []
    table = ["| workload | kernel | HBM read / launch | HBM write / launch | total | algorithmic (W+X+C) | ratio |",
             "|---|---|---|---|---|---|---|"]
    for i, name in enumerate(names):
        kname, fetch = per["FETCH_SIZE"][0][i]
        _, write = per["WRITE_SIZE"][0][i]
        fetch, write = float(np.mean(fetch)), float(np.mean(write))
        rd = fetch * 1024 / fetch_factor
        wr = write * 1024 / write_factor
        wl = workloads.get(name)
        algo = wl.weight_bytes() + wl.T * wl.K * 2 + wl.T * wl.N * 2
        kshort = kname.split("(")[0].replace("void ", "")
        out = {
            "workload": name,
            "kernel": kshort,
            "kernel_source_sha": sha,
            "fetch_size_kib_per_launch": round(fetch, 1),
            "write_size_kib_per_launch": round(write, 1),
            "copy_calibration": {
                "bytes_read_and_written": COPY_BYTES,
                "fetch_size_kib": round(per["FETCH_SIZE"][1], 1),
                "write_size_kib": round(per["WRITE_SIZE"][1], 1),
                "fetch_kib_x1024_per_byte": round(fetch_factor, 4),
                "write_kib_x1024_per_byte": round(write_factor, 4),
            },
            "hbm_read_bytes_per_launch": int(round(rd)),
            "hbm_write_bytes_per_launch": int(round(wr)),
            "hbm_bytes_per_launch": int(round(rd + wr)),
            "algorithmic_bytes_per_launch": algo,
            "commands": [
                "cd /tmp && timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv "
                "-d $OUT/pmc/fetch -o fetch -- python3 $R/bench.py --pmc-run all",
                "cd /tmp && timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv "
                "-d $OUT/pmc/write -o write -- python3 $R/bench.py --pmc-run all",
                "python bench.py --pmc-summary $OUT/pmc all",
            ],
            "note": (f"R is the repository root, OUT any output directory. Counters are per dispatch: {PMC_LAUNCHES} launches of each "
                     f"workload on rotated weights, then {PMC_COPIES} copies of {COPY_BYTES >> 20} MiB whose "
                     "counter readings calibrate KiB per byte moved."),
        }
        with open(os.path.join(ROOT, "profiles", f"traffic_{name}.json"), "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
        outs.append(out)
        table.append(f"| {name} | `{kshort}` | {rd / 1e6:.2f} MB | {wr / 1e6:.3f} MB | {(rd + wr) / 1e6:.2f} MB "
                     f"| {algo / 1e6:.2f} MB | {(rd + wr) / algo:.3f} |")
    with open(os.path.join(ROOT, "profiles", "traffic_summary.md"), "w") as f:
        f.write("# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)\n\n")
        f.write(f"Kernel sources: `{sha}`. Counters calibrated on {PMC_COPIES} plain device copies of "
                f"{COPY_BYTES >> 20} MiB: FETCH_SIZE reads {fetch_factor:.4f} KiB x 1024 per byte read, "
                f"WRITE_SIZE {write_factor:.4f} per byte written.\n\n")
        f.write("Commands (R = repository root, OUT any output directory):\n\n")
        for c in outs[0]["commands"]:
            f.write(f"    {c}\n")
        f.write("\n" + "\n".join(table) + "\n")
    print("\n".join(table))
    return outs


def mfma_summary(path: str, names: list) -> list:
    """Matrix-core use of each workload's kernel from one ``--pmc MfmaUtil
    MfmaFlopsBF16`` pass of ``--pmc-run`` under ``path`` (rocprofv3's derived
    counters: MFMA busy cycles over all SIMDs / (GPU active cycles x SIMDs),
    and BF16 MFMA operations x 512), per dispatch, averaged over the
    workload's launches. Writes profiles/mfma_summary.md."""
    sha = kernel_source_hash()
    util = _per_workload(_counter_rows(path, "MfmaUtil"), names)
    flops = _per_workload(_counter_rows(path, "MfmaFlopsBF16"), names)
    table = ["| workload | kernel | MfmaUtil % | MFMA bf16 flops / launch | 2TNK | executed / algorithmic |",
             "|---|---|---|---|---|---|"]
    outs = []
    for i, name in enumerate(names):
        wl = workloads.get(name)
        kname = util[i][0].split("(")[0].replace("void ", "")
        u = float(np.mean(util[i][1]))
        fl = float(np.mean(flops[i][1]))
        outs.append({"workload": name, "kernel": kname, "mfma_util_percent": round(u, 2),
                     "mfma_flops_bf16_per_launch": int(round(fl)), "algorithmic_flops_per_launch": wl.flops()})
        table.append(f"| {name} | `{kname}` | {u:.2f} | {fl:.4g} | {wl.flops():.4g} | {fl / wl.flops():.3f} |")
    with open(os.path.join(ROOT, "profiles", "mfma_summary.md"), "w") as f:
        f.write("# Matrix-core use per launch (rocprofv3 MfmaUtil, MfmaFlopsBF16)\n\n")
        f.write(f"Kernel sources: `{sha}`. Command (R = repository root, OUT any output directory):\n\n"
                "    cd /tmp && timeout -s KILL 300 rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv "
                "-d $OUT/mfma -o mfma -- python3 $R/bench.py --pmc-run all\n"
                "    python bench.py --mfma-summary $OUT/mfma all\n\n"
                "Executed MFMA flops exceed 2*T*N*K by the token padding to 16 and, in folded tiles, by "
                "the off-diagonal blocks that are computed and not read.\n\n")
        f.write("\n".join(table) + "\n")
    print("\n".join(table))
    return outs


# Phase names of the per-workgroup stamps each kernel kind writes
# (skgemm_set_timeline).
PHASES = {
    "stream": ["entry", "X staged", "stream done", "own partials stored", "exit", "arrivals done",
               "owned polls done"],
    "cluster": ["entry", "loads issued", "wave 0 stream done", "sums in LDS", "exit"],
    "wide": ["entry", "first X chunk staged", "stream done", "partial stored", "exit"],
}


def phases(names: list, overrides: list, out_dir: str, launches: int = 3) -> None:
    """Per-workgroup phase stamps of single cold launches (eager, one stream),
    pooled over `launches` launches, each relative to its earliest entry.
    `overrides` are NAME=VALUE library overrides (skgemm_set_override), e.g.
    kind=1 to run a workload on the persistent kernel. Writes
    phases_<workload>[_<overrides>].md with the command under out_dir
    (profiles/ by default)."""
    import torch

    import split_reduction_amd as sk

    sk.lib()
    pins = [o.split("=") for o in overrides]
    for k, v in pins:
        sk.skgemm_set_override(k, int(v))
    suffix = "".join(f"_{k}{v}" for k, v in pins)
    fmt = {"bf16": 0, "mxfp4": 1, "mxfp8": 2}
    wsweep = None
    try:
        for name in names:
            wl = workloads.get(name)
            host_w = None
            if is_sweep(name):
                if wsweep is None:
                    wsweep = workloads.gen_w_bf16(workloads.sweep_workload(1))
                host_w = wsweep
            case = Case(wl, host_w)
            tac = sk.skgemm_tactic_for(wl.T, wl.N, wl.K, wl.split_k, fmt[wl.kind])
            kind = tac["kind"]
            grid = tac["grid"]
            stream = torch.cuda.Stream()
            sk.skgemm_reserve(wl.T, wl.N, wl.split_k, stream)
            buf = torch.zeros(grid * 8, dtype=torch.int64, device="cuda:0")
            warm = 2 * case.copies
            with torch.cuda.stream(stream):
                for i in range(warm):
                    case.launch(i, stream)
            stream.synchronize()
            pooled, spans = [], []
            for r in range(launches):
                buf.zero_()
                torch.cuda.synchronize()
                sk.skgemm_set_timeline(buf, buf.numel())
                try:
                    with torch.cuda.stream(stream):
                        case.launch(warm + r, stream)  # the copy launched least recently
                    stream.synchronize()
                finally:
                    sk.skgemm_set_timeline(None, 0)
                st = buf.view(grid, 8).cpu().numpy().astype(np.float64)
                t0 = st[:, 0].min()
                rel = np.where(st > 0, (st - t0) * 0.01, np.nan)  # microseconds
                pooled.append(rel)
                spans.append(float(np.nanmax(rel[:, 4])))
            allst = np.concatenate(pooled)
            cmd = "python bench.py --phases " + name + "".join(f" --override {k}={v}" for k, v in pins)
            lines = [f"# Phase stamps: {name}{' (' + ', '.join(overrides) + ')' if overrides else ''}", "",
                     f"Kernel sources `{kernel_source_hash()}`; tactic {json.dumps(tac)}.", "",
                     f"Command: `{cmd}` (eager single launches on cold weights, device clock "
                     f"s_memrealtime at 100 MHz; {launches} launches pooled, each relative to its "
                     f"earliest workgroup entry; wave 0's view per workgroup).", "",
                     "Launch spans (first entry to last exit): "
                     + ", ".join(f"{v:.2f}" for v in spans) + " us", "",
                     "| phase | min | p10 | median | p90 | max |", "|---|---|---|---|---|---|"]
            names_k = PHASES.get(kind, [f"stamp {i}" for i in range(5)])
            order = [0, 1, 2, 3, 5, 6, 4] if len(names_k) == 7 else list(range(len(names_k)))
            for j in order:  # in time order
                ph = names_k[j]
                v = allst[:, j]
                v = v[~np.isnan(v)]
                if v.size == 0:
                    continue
                lines.append(f"| {ph} | {v.min():.2f} | {np.percentile(v, 10):.2f} | {np.median(v):.2f} | "
                             f"{np.percentile(v, 90):.2f} | {v.max():.2f} |")
            xcd = np.tile(np.arange(grid) % 8, launches)
            lines += ["", "Per XCD (block index mod 8): median and max of the stream-done stamp, max exit (us):", "",
                      "| XCD | median stream done | max stream done | max exit |", "|---|---|---|---|"]
            for x in range(8):
                m = xcd == x
                lines.append(f"| {x} | {np.nanmedian(allst[m, 2]):.2f} | {np.nanmax(allst[m, 2]):.2f} | "
                             f"{np.nanmax(allst[m, 4]):.2f} |")
            text = "\n".join(lines) + "\n"
            print(text, flush=True)
            os.makedirs(out_dir, exist_ok=True)
            with open(os.path.join(out_dir, f"phases_{name}{suffix}.md"), "w") as f:
                f.write(text)
            del case, buf
            torch.cuda.empty_cache()
    finally:
        if pins:
            sk.clear_overrides()


# ---------------------------------------------------------------------------


def load_traffic(name: str):
    """HBM bytes per launch measured by rocprofv3 counters for a workload, if
    they were taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-headline", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace-summary", metavar="DIR", help="summarise a rocprofv3 kernel trace and exit")
    ap.add_argument("--pmc-run", nargs="*", metavar="WORKLOAD",
                    help="the short run counters are taken on (default: the headline; 'all': every workload)")
    ap.add_argument("--mfma-summary", nargs="+", metavar=("DIR", "WORKLOAD"),
                    help="summarise an MfmaUtil / MfmaFlopsBF16 counter pass of --pmc-run and exit")
    ap.add_argument("--pmc-summary", nargs="+", metavar=("DIR", "WORKLOAD"),
                    help="summarise the FETCH_SIZE / WRITE_SIZE passes under DIR and exit")
    ap.add_argument("--phases", nargs="+", metavar="WORKLOAD",
                    help="per-workgroup phase stamps of single cold launches, written to profiles/; exit")
    ap.add_argument("--override", action="append", default=[], metavar="KNOB=VALUE",
                    help="with --phases: a library override (skgemm_set_override) for the run")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"), metavar="DIR",
                    help="with --phases: where the summaries go (default profiles/)")
    args = ap.parse_args()
    if args.phases:
        phases(pmc_names(args.phases), args.override, args.out)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], pmc_names(args.pmc_summary[1:]))
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary[0], pmc_names(args.mfma_summary[1:]))
        return
    if args.pmc_run is not None:
        pmc_run(pmc_names(args.pmc_run))
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps, args.warmup)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        raise SystemExit(2)

    import torch

    import split_reduction_amd as sk

    if not os.path.exists(sk.LIB_PATH):
        from split_reduction_amd import build

        build.build()
    sk.lib()
    torch.cuda.init()

    head = workloads.get(HEADLINE)
    log("sweep weights K = N = 16384")
    wsweep = workloads.gen_w_bf16(workloads.sweep_workload(1))
    log(f"headline {head.name}")
    h = run_workload(head, args.steps, args.warmup, host_w=wsweep)
    log(json.dumps(h))

    extra = []
    if not args.only_headline:
        steps = max(20, args.steps // 2)
        warm = max(3, args.warmup // 2)
        for name in all_workloads()[1:]:
            log(f"workload {name}")
            r = run_workload(workloads.get(name), steps, warm, host_w=wsweep if is_sweep(name) else None)
            log(json.dumps(r))
            extra.append(r)

    chain = None
    if not args.only_headline:
        log("chained launches")
        chain = chain_bench(args.steps, max(3, args.warmup // 2))
        log(json.dumps(chain))

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(head, wsweep)
    del wsweep

    line = {
        "metric": "weight-stream HBM TB/s (% of peak) + TFLOP/s, split-K decode GEMM, 1 GPU",
        "value": h["weight_TBps"],
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["t_us"] * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "frac_hbm_peak": h["frac_hbm_peak"],
        "TFLOPs": h["TFLOPs"],
        "config": {
            "workload": head.name, "T": head.T, "K": head.K, "N": head.N,
            "split_k": head.split_k, "weights": "bf16 N(0,0.01^2)", "activations": "bf16 N(0,1)",
            "cache": f"cold: {h['rotated_copies']} rotated weight copies (>= 1 GiB)",
            "timing": "HIP graph of exactly `steps` launches, HIP events on the launch stream",
            "parallelism": "single GPU",
        },
        "roofline": h["roofline"],
        "cpu_baseline": cpu,
        "hot_cache": {"t_us": h["hot_t_us"], "weight_TBps": h["hot_weight_TBps"]},
        "read_probe": h["read_probe"],
        "tactic": h["tactic"],
        "workloads": extra,
        "chain": chain,
        "kernel_source_sha": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
