#!/usr/bin/env python3
"""Throughput of the gfx950 GEMM library on one MI355X.

One step = one call of the library on one batch of seeded synthetic
operands already resident in HBM (the whole hot path: tile scheduler,
global->LDS loads, MFMA loop, tails, fp32 epilogue, all inside one kernel
launch).  The default workload is the square bf16 GEMM M=N=K=8192 with
row-major A and column-major B (NT), entries uniform[-1, 1] rounded to bf16,
seed 0, fp32 output.

Prints ONE JSON line: TFLOP/s (2 M N K per step / time), the roofline block
of the GEMM kernel (per-launch duration from HIP events on the launch
stream, against the MI355X dense MFMA peak) and the CPU oracle timed on a
bounded row sample of the same workload on this host.

Before the W warm-up steps the step runs untimed for --settle seconds: an
idle MI355X needs tens of milliseconds of load before its clocks leave the
idle state, and without this the timed steps measure the ramp.  The shader
clock and board power are sampled from sysfs during the timed steps and
reported under "clocks".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s at 8192³ bf16 + % of MI355X dense MFMA peak (1 GPU)"
HEADLINE = "square8192_nt"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--all", action="store_true", help="also print one line per other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="rows of A in the oracle's timed sample")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the warm-up, so the GPU's clocks "
                         "leave their idle state (reported as settle_s)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of COPY_BYTES (for scaling HBM counters)")
    ap.add_argument("--measure-build", action="store_true",
                    help="load libgemm_measure.so (built by `python -m dense_gemm_mxfp8_amd.build "
                         "--measure`), whose LIBGEMM_* variant switches are live")
    return ap.parse_args()


COPY_BYTES = 1 << 30  # 1 GiB read + 1 GiB written per copy launch


def copy_calibration(steps: int):
    """A plain elementwise copy kernel of known size: FETCH_SIZE / WRITE_SIZE of
    its launches give the scale from counter KiB to bytes."""
    import torch
    n = COPY_BYTES // 4
    src = torch.rand(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": True, "bytes_read": COPY_BYTES,
                      "bytes_written": COPY_BYTES, "launches": steps}), flush=True)


def operand_bytes(w) -> int:
    if w["kind"] == "mx":
        M, N, K = w["M"], w["N"], w["K"]
        return M * K + N * K + (M + N) * (K // 32) + 4 * M * N
    M, N, K = w["M"], w["N"], w["K"]
    return 2 * (M * K + K * N) + 4 * M * N


class ClockSampler:
    """Samples the GPU's shader clock and board power from sysfs (the amdgpu
    driver's pp_dpm_sclk and hwmon power1_input) on a background thread while
    the timed steps run.  Reports None where the files are not readable."""

    def __init__(self, period_s: float = 0.004):
        import threading
        self.period = period_s
        self.sclk, self.power = [], []
        self.dev = self._device_dir()
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _device_dir():
        try:
            import torch
            p = torch.cuda.get_device_properties(0)
            path = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (p.pci_domain_id, p.pci_bus_id, p.pci_device_id)
            return path if os.path.isdir(path) else None
        except Exception:
            return None

    def _read(self):
        try:
            with open(os.path.join(self.dev, "pp_dpm_sclk")) as fh:
                for ln in fh:
                    if ln.startswith("S:") or ln.rstrip().endswith("*"):
                        self.sclk.append(float(ln.split(":")[1].strip().split("Mhz")[0]))
                        break
        except Exception:
            pass
        try:
            import glob
            for h in glob.glob(os.path.join(self.dev, "hwmon", "hwmon*", "power1_input")):
                with open(h) as fh:
                    self.power.append(float(fh.read()) / 1e6)
                break
        except Exception:
            pass

    def _run(self):
        while not self._stop.is_set():
            self._read()
            time.sleep(self.period)

    def __enter__(self):
        if self.dev:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.sclk and not self.power:
            return None
        out = {"samples": max(len(self.sclk), len(self.power)),
               "source": "sysfs pp_dpm_sclk, hwmon power1_input"}
        if self.sclk:
            out["sclk_mhz"] = {"median": float(np.median(self.sclk)), "min": min(self.sclk),
                               "max": max(self.sclk)}
        if self.power:
            out["power_w"] = {"median": round(float(np.median(self.power)), 1),
                              "max": round(max(self.power), 1)}
        return out


def bench_workload(name: str, steps: int, warmup: int, settle: float = 0.0):
    import torch
    import dense_gemm_mxfp8_amd as dg
    from dense_gemm_mxfp8_amd import inputs

    dev = torch.device("cuda:0")
    if name in inputs.ATTN_WORKLOADS:
        return bench_attention(name, steps, warmup, settle)
    w = inputs.WORKLOADS[name]
    prob = inputs.workload(name, seed=0)
    M, N, K = prob.M, prob.N, prob.K
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    C = torch.empty((M, N), dtype=torch.float32, device=dev)
    # A memory-bound problem whose B fits in the 256 MiB Infinity Cache is
    # timed over rotating copies of its operands so that every step streams
    # from HBM.
    bytes_per_step = operand_bytes(w)
    copies = 4 if bytes_per_step < 512 * 2**20 and 2 * M * N * K / bytes_per_step < 300 else 1
    splits = 1
    if w["kind"] == "mx":
        ops = [(prob.A.to(dev), prob.B.to(dev), prob.SA.to(dev), prob.SB.to(dev))
               for _ in range(copies)]
        if w.get("splitk"):
            # split-K: the library's plan, with its workspace allocated once
            A0, B0, SA0, SB0 = ops[0]
            rc, splits, nbytes = dg.gemm_mxfp8_splitk_workspace(M, N, K, A0.data_ptr(), K, B0.data_ptr(), K,
                                                                SA0.data_ptr(), SB0.data_ptr(), C.data_ptr(), N,
                                                                dg.GEMM_OUT_F32, None, None, None, 0)
            if rc:
                raise RuntimeError(dg.gemm_strerror(rc))
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)

            def step(i):
                A, B, SA, SB = ops[i % copies]
                rc = dg.gemm_mxfp8_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(), SB.data_ptr(),
                                          C.data_ptr(), N, dg.GEMM_OUT_F32, None, None, None, 0, ws.data_ptr(),
                                          ws.numel(), s)
                if rc:
                    raise RuntimeError(dg.gemm_strerror(rc))
        else:
            def step(i):
                A, B, SA, SB = ops[i % copies]
                rc = dg.gemm_mxfp8(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(),
                                   SB.data_ptr(), C.data_ptr(), N, s)
                if rc:
                    raise RuntimeError(dg.gemm_strerror(rc))
        dtype, peak_key = "fp8(e4m3)+e8m0", "fp8"
    else:
        ops = [(prob.A.to(dev), prob.B.to(dev)) for _ in range(copies)]
        fn = dg.gemm_bf16_nt if prob.b_colmajor else dg.gemm_bf16
        ldb = K if prob.b_colmajor else N
        if w.get("splitk"):
            # split-K: the library's plan, with its workspace allocated once
            A0, B0 = ops[0]
            rc, splits, nbytes = dg.gemm_bf16_splitk_workspace(M, N, K, A0.data_ptr(), K, B0.data_ptr(), ldb,
                                                               prob.b_colmajor, C.data_ptr(), N, dg.GEMM_OUT_F32,
                                                               None, None, None, 0)
            if rc:
                raise RuntimeError(dg.gemm_strerror(rc))
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)

            def step(i):
                A, B = ops[i % copies]
                rc = dg.gemm_bf16_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, prob.b_colmajor,
                                         C.data_ptr(), N, dg.GEMM_OUT_F32, None, None, None, 0, ws.data_ptr(),
                                         ws.numel(), s)
                if rc:
                    raise RuntimeError(dg.gemm_strerror(rc))
        else:
            splits = 1

            def step(i):
                A, B = ops[i % copies]
                rc = fn(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, C.data_ptr(), N, s)
                if rc:
                    raise RuntimeError(dg.gemm_strerror(rc))
        dtype, peak_key = "bf16", "bf16"

    timing = time_steps(step, stream, steps, warmup, settle)
    flops = 2.0 * M * N * K
    config = {"workload": name, "M": M, "N": N, "K": K,
              "layout": ("NT" if getattr(prob, "b_colmajor", True) else "NN"), "dist": w.get("dist"),
              "seed": 0, "output": "fp32", "parallelism": "single-gpu",
              **({"splitk_ranges": splits} if splits > 1 else {})}
    res = {"workload": name, "dtype": dtype, "peak_key": peak_key, "flops": flops, "bytes": bytes_per_step,
           "operand_copies": copies, "config": config, **timing}
    res["tflops"] = flops / (res["ms_per_step"] * 1e-3) / 1e12
    return res, prob


def time_steps(step, stream, steps: int, warmup: int, settle: float):
    """Settle, warm up and time `steps` launches of step(i) on `stream`."""
    import torch
    # The clocks ramp up from idle over the first tens of milliseconds of
    # work; settle steps bring them to their loaded state before the warm-up.
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < settle:
        for _ in range(8):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: K back-to-back launches between two events on the launch
    # stream; the mean launch duration is their span over K.  Events between
    # the launches would add a marker's latency to every launch, which shows
    # on the short kernels.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    mean_ms = ev0.elapsed_time(ev1) / steps
    # Spread of single launches: a separate, untimed pass with events around
    # each launch (these include the marker latency).
    nd = min(steps, 50)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nd)]
    for i in range(nd):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])  # ms per launch
    ms_step = wall * 1e3 / steps
    return {"ms_per_step": ms_step, "kernel_ms_mean": float(mean_ms),
            "kernel_ms_median": float(np.median(per)), "single_launches": nd,
            "kernel_ms_p10": float(np.percentile(per, 10)), "kernel_ms_p90": float(np.percentile(per, 90)),
            "settle_s": round(settle, 3), "settle_steps": settle_steps, "clocks": clocks.summary()}


def attention_pairs(p) -> int:
    """(query, key) pairs the softmax covers, summed over batch and heads."""
    if not p.causal:
        return p.B * p.Hq * p.Sq * p.Sk
    off = p.Sk - p.Sq
    per_head = sum(min(p.Sk, max(0, i + off + 1)) for i in range(p.Sq))
    return p.B * p.Hq * per_head


def attention_flops(p) -> float:
    """Two products of 2 FLOPs per multiply-add over head_dim per visible pair."""
    return 4.0 * p.D * attention_pairs(p)


def attention_bytes(p) -> int:
    """Q, K, V read once (bf16), O (fp32) and lse written once."""
    return 2 * (p.B * p.Hq * p.Sq * p.D + 2 * p.B * p.Hkv * p.Sk * p.D) + 4 * p.B * p.Hq * p.Sq * (p.D + 1)


def bench_attention(name: str, steps: int, warmup: int, settle: float):
    import torch
    import dense_gemm_mxfp8_amd as dg
    from dense_gemm_mxfp8_amd import inputs

    dev = torch.device("cuda:0")
    p = inputs.workload(name, seed=0)
    stream = torch.cuda.current_stream(dev)
    s = stream.cuda_stream
    Q, K, V = p.Q.to(dev), p.K.to(dev), p.V.to(dev)
    O = torch.empty((p.B, p.Hq, p.Sq, p.D), dtype=torch.float32, device=dev)
    L = torch.empty((p.B, p.Hq, p.Sq), dtype=torch.float32, device=dev)

    def step(i):
        rc = dg.attn_fwd_bf16(p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.D, Q.data_ptr(), None, K.data_ptr(), None,
                              V.data_ptr(), None, O.data_ptr(), None, L.data_ptr(), p.scale, p.causal, s)
        if rc:
            raise RuntimeError(dg.gemm_strerror(rc))

    timing = time_steps(step, stream, steps, warmup, settle)
    flops = attention_flops(p)
    config = {"workload": name, "batch": p.B, "heads_q": p.Hq, "heads_kv": p.Hkv, "seq_q": p.Sq,
              "seq_k": p.Sk, "head_dim": p.D, "causal": p.causal, "layout": "BHSD", "dist": "normal",
              "seed": 0, "output": "fp32 O + fp32 lse", "parallelism": "single-gpu"}
    res = {"workload": name, "dtype": "bf16", "peak_key": "bf16", "flops": flops, "bytes": attention_bytes(p),
           "operand_copies": 1, "config": config, **timing}
    res["tflops"] = flops / (res["ms_per_step"] * 1e-3) / 1e12
    return res, p


def cpu_baseline(prob, rows: int, single_rows: int = 32):
    """The oracle, untouched, on rows [0, rows) of the same product with all
    the host threads it uses, and on rows [0, single_rows) with one thread."""
    import torch
    import oracle
    from dense_gemm_mxfp8_amd.inputs import MxProblem

    def run(nrows, nthreads):
        nrows = min(nrows, prob.M)
        if isinstance(prob, MxProblem):
            A = prob.A[:nrows].numpy()
            t0 = time.perf_counter()
            oracle.gemm_mxfp8(A, prob.B.numpy().T, prob.SA[:nrows].numpy(), prob.SB.numpy(), nthreads=nthreads)
        else:
            A = prob.A[:nrows].contiguous().view(torch.int16).numpy().view(np.uint16)
            B = prob.B.view(torch.int16).numpy().view(np.uint16)
            Bv = B.T if prob.b_colmajor else B
            t0 = time.perf_counter()
            oracle.gemm_bf16(A, Bv, nthreads=nthreads)
        dt = time.perf_counter() - t0
        return nrows, dt, 2.0 * nrows * prob.N * prob.K / dt / 1e12

    cores = oracle.default_threads()
    n, dt, tf = run(rows, cores)
    n1, dt1, tf1 = run(single_rows, 1)
    return {"value": tf, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"rows 0..{n - 1} of A against all of B ({n}x{prob.N}x{prob.K}), {dt:.2f} s wall",
            "single_core": {"value": tf1, "unit": "TFLOP/s", "cores": 1,
                            "sample": f"rows 0..{n1 - 1} ({n1}x{prob.N}x{prob.K}), {dt1:.2f} s wall"}}


ATTN_CPU_ROWS = 131072  # about 15 s of the oracle on 16 host threads at 4096 keys


def cpu_baseline_attention(p, rows: int = ATTN_CPU_ROWS):
    """The attention oracle, untouched, on the first `rows` query rows of head
    (0, 0) onward (all the host threads it uses), scaled by the rows' own
    algorithmic FLOPs."""
    import torch
    import oracle
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    n = min(rows, p.B * p.Hq * p.Sq)
    idx = np.arange(n)
    sel = np.stack([idx // (p.Hq * p.Sq), (idx // p.Sq) % p.Hq, idx % p.Sq], axis=1).astype(np.int64)
    Qb, Kb, Vb = bits(p.Q), bits(p.K), bits(p.V)
    t0 = time.perf_counter()
    oracle.attention_fwd_at(Qb, Kb, Vb, p.scale, p.causal, sel)
    dt = time.perf_counter() - t0
    off = p.Sk - p.Sq
    pairs = sum(min(p.Sk, max(0, int(i) + off + 1)) if p.causal else p.Sk for i in sel[:, 2])
    cores = oracle.default_threads()
    return {"value": 4.0 * p.D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"query rows 0..{n - 1} in (batch, head, row) order ({pairs} query-key pairs), "
                      f"{dt:.2f} s wall"}


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, or None if there is none or the kernels changed since."""
    from dense_gemm_mxfp8_amd import profiling
    return profiling.read_traffic(os.path.join(ROOT, "profiles", f"traffic_{workload}.md"),
                                  profiling.family_of(workload))


def line(res, steps, warmup, cpu=None, headline=True):
    peak = PEAK_TFLOPS[res["peak_key"]]
    traffic = measured_traffic(res["workload"])
    achieved = res["flops"] / (res["kernel_ms_mean"] * 1e-3) / 1e12
    ai = res["flops"] / res["bytes"]
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai < ridge:
        gbs = res["bytes"] / (res["kernel_ms_mean"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic}
    kind = "attention forward" if "heads_q" in res["config"] else "GEMM"
    out = {
        "metric": METRIC if headline else f"{kind} TFLOP/s ({res['workload']})",
        "value": round(res["tflops"], 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": res["dtype"], "data": "synthetic",
        "config": res["config"],
        "kernel_ms": {"mean": round(res["kernel_ms_mean"], 5),
                      "median": round(res["kernel_ms_median"], 5),
                      "p10": round(res["kernel_ms_p10"], 5), "p90": round(res["kernel_ms_p90"], 5),
                      "single_launches": res["single_launches"],
                      "method": "mean: events around the K timed launches / K; median, p10, p90: "
                                "events around single launches in a separate pass after them"},
        "pct_of_peak": round(100 * achieved / peak, 2),
        "roofline": roof,
        "settle_s": res["settle_s"],
        "clocks": res["clocks"],
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMM needs no collectives; multi-GPU sharding is a design note only).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.measure_build:
        import dense_gemm_mxfp8_amd as dg
        from dense_gemm_mxfp8_amd.build import MEASURE_LIBRARY
        dg.LIBRARY = MEASURE_LIBRARY
    names = [args.workload]
    if args.all:
        from dense_gemm_mxfp8_amd.inputs import WORKLOADS
        from dense_gemm_mxfp8_amd.inputs import ATTN_WORKLOADS
        names += [n for n in list(WORKLOADS) + list(ATTN_WORKLOADS) if n != args.workload]
    for i, name in enumerate(names):
        print(f"[bench] {name}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
              flush=True)
        res, prob = bench_workload(name, args.steps, args.warmup, args.settle)
        cpu = None
        if i == 0 and not args.no_cpu_baseline:
            if name.startswith("attn"):
                print(f"[bench] oracle on {ATTN_CPU_ROWS} query rows", file=sys.stderr, flush=True)
                cpu = cpu_baseline_attention(prob, ATTN_CPU_ROWS)
            else:
                print(f"[bench] oracle on {args.cpu_rows} rows", file=sys.stderr, flush=True)
                cpu = cpu_baseline(prob, args.cpu_rows)
        out = line(res, args.steps, args.warmup, cpu, headline=(name == HEADLINE))
        if args.measure_build:
            out["config"]["library"] = "measure build: " + " ".join(
                f"{k}={v}" for k, v in sorted(os.environ.items()) if k.startswith("LIBGEMM_"))
        print(json.dumps(out), flush=True)
        del prob
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
