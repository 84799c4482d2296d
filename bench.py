"""Benchmark of the exact-attention hot path on one MI355X.

One step = the whole path over one batch of seeded synthetic inputs already
resident in HBM: fa_fwd, then fa_bwd_preprocess, fa_bwd_dkdv and fa_bwd_dq
(the three steps of fa_bwd), all through the C ABI on one stream (called in
their grouped-K/V forms, which are the plain ones when every query head has its
own K/V head).  Throughput is counted with the method's FLOP formula: forward
4*B*H*N^2*d (halved under the causal mask), backward 2.5x the forward.

Prints ONE JSON line.  Besides the step throughput it reports:
  * per-kernel times from HIP events recorded on the launch stream around
    every launch inside the timed region;
  * "roofline" for the dominant (longest) kernel against the dense MFMA peak of
    the workload's dtype, with HBM traffic from committed rocprofv3 counter
    runs when they were taken on the current kernel source, and "per_kernel"
    entries for every kernel of the step (algorithmic and executed FLOPs);
  * the shader clock under the same load (sampled while the step runs again
    after the timed region) and the peak at that clock, and the run's
    conditions (device, ROCm, compiler, torch versions);
  * "secondary": with the default workload, the causal bf16 workload
    (B=4 H=32 N=4096 d=128), the other one the throughput target is stated
    on, timed the same way in the same process;
  * "cpu_baseline": the fp64 CPU oracle timed on a bounded sample (whole heads
    from head 0 on) of the same workload, plus the GPU-vs-oracle error on the
    first sampled head.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--no-secondary] [--mode step|copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

DEFAULT_WORKLOAD = workloads.PEAKED_BF16.name
METRIC = "attention fwd/bwd TFLOPS on 1 MI355X and % of bf16 MFMA peak"
# Published dense MFMA peaks of MI355X (TFLOP/s): bf16/fp16 2.5 PFLOP/s
# (2516.6 = 256 CUs x 4096 flop/clk x 2.4 GHz), fp32 157.3.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
DOMINANT = "bwd_dkdv16_kernel"
KERNEL_SOURCES = ("io_aware_exact_fa_amd/csrc/fa_bwd_kernels.hpp", "io_aware_exact_fa_amd/csrc/fa_common.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(workloads.BY_NAME) + sorted(workloads.VARLEN_BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", default="two-pass", choices=["two-pass", "one-pass"],
                    help="fa_bwd's two-pass backward (dQ by its own pass), or the one-pass "
                         "steps (dQ by atomic adds inside the dK/dV kernel; 16-bit types)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="time only --workload (not also the causal bf16 workload)")
    ap.add_argument("--mode", default="step", choices=["step", "copy"])
    return ap.parse_args()


def source_sha() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name: str):
    """HBM bytes per launch of the dominant kernel from committed counter runs, if they
    were taken on the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(DOMINANT, {}).get(workload_name)
    if not e or e.get("source_sha") != source_sha():
        return None
    return e.get("hbm_bytes_per_launch")


def copy_calibration(steps: int):
    """A plain 1 GiB device-to-device copy, for scaling the HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(max(steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "launches": max(steps, 1)}))


def cpu_baseline(w, inp, gpu_out, budget_s: float = 10.0):
    """Time the fp64 oracle (numpy, S and P materialized), forward then backward, on
    whole heads from head 0 on until about ``budget_s`` seconds of CPU work (at least
    one head); the GPU-vs-oracle error on the first sampled head (group).  `cores`
    is the BLAS thread count numpy's products ran on (the threads the oracle used;
    its elementwise steps run on one), `host_cpus` the host's CPU count."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:   # threadpoolctl missing: report the process's CPU affinity
        cores = len(os.sched_getaffinity(0))
    # One K/V head and its G query heads at a time (G = 1 without grouped K/V):
    # forward and backward of each query head, dK and dV summed over the group.
    G = w.H // w.kv_heads
    groups = [(b, j) for b in range(w.B) for j in range(w.kv_heads)]
    f64 = lambda t, b, h: t[b, h].to(dtype=torch.float64).numpy()
    rel = lambda a, r: float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-30))
    secs, done, check = 0.0, 0, None
    win = w.window if w.windowed else None
    bmask = workloads.block_mask(w).numpy() if w.sparse else None
    for b, j in groups:
        k, v = f64(inp["k"], b, j), f64(inp["v"], b, j)
        res = []
        for h in range(j * G, (j + 1) * G):
            q, do = f64(inp["q"], b, h), f64(inp["do"], b, h)
            t0 = time.perf_counter()
            drop = oracle.head_drop(w.dropout or None, b * w.H + h, w.N)
            blk = bmask[h] if bmask is not None else None
            o, lse = oracle.forward_head(q, k, v, w.scale, w.causal, win, drop, blk)
            res.append((h, o, lse,
                        oracle.backward_head(q, k, v, do, w.scale, w.causal, win, drop, blk)))
            secs += time.perf_counter() - t0
            done += 1
            if secs >= budget_s:
                break   # a long sequence: part of a group is sample enough
        if check is None:   # GPU-vs-oracle error on the first sampled group
            whole = len(res) == G   # dK and dV sum over the whole group
            oerr = max(float(np.max(np.abs(gpu_out["o"][b, h].double().numpy() - o))) for h, o, _, _ in res)
            lerr = max(float(np.max(np.abs(gpu_out["lse"][b, h].double().numpy() - l))) for h, _, l, _ in res)
            dqerr = max(rel(gpu_out["dq"][b, h].double().numpy(), g["dq"]) for h, _, _, g in res)
            check = {
                "head": [b, j * G] if G == 1 else {"batch": b, "kv_head": j, "query_heads": [j * G, j * G + len(res) - 1]},
                "o_maxabs": oerr,
                "lse_maxabs": lerr,
                "dq_rel": dqerr,
            }
            if whole:
                check["dk_rel"] = rel(gpu_out["dk"][b, j].double().numpy(), sum(r[3]["dk"] for r in res))
                check["dv_rel"] = rel(gpu_out["dv"][b, j].double().numpy(), sum(r[3]["dv"] for r in res))
        if secs >= budget_s:
            break
    head_flops = (w.fwd_flops() + w.bwd_flops()) / (w.B * w.H)
    return {
        "value": head_flops * done / secs / 1e12,
        "unit": "TFLOPS",
        "cores": int(cores),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} query heads (from head 0 on), forward + backward each, "
                  f"fp64 numpy oracle with S and P materialized (BLAS on {int(cores)} threads); "
                  f"{secs:.2f} s wall",
        "seconds": round(secs, 3),
        "parity_on_sample": check,
    }


class ClockSampler:
    """Samples the GPU's shader (GFX) clock in a background thread while the
    timed steps run: amdsmi's GPU metrics table (the mean of the per-XCC
    current_gfxclks; readings at the idle clock, below 500 MHz, are dropped:
    the table lags the start of the load).  Median and range in MHz, or None
    where the table cannot be read.  The published dense peak
    assumes 2.4 GHz; under sustained MFMA load the clock runs lower, so the
    peak at the sampled clock is reported beside it."""

    def __init__(self, period_s: float = 0.005):
        import threading
        self.period, self.samples, self.error = period_s, [], None
        self._stop = threading.Event()
        self._read = self._open()
        self._thread = threading.Thread(target=self._run, daemon=True) if self._read else None

    def _open(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]

            def read():
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                clks = [c for c in m.get("current_gfxclks") or []
                        if isinstance(c, (int, float)) and 0 < c < 10000]
                busy = m.get("average_gfx_activity")
                return (sum(clks) / len(clks) if clks else None,
                        busy if isinstance(busy, (int, float)) else None)
            if read()[0] is None:
                raise RuntimeError("no per-XCC gfx clocks in the GPU metrics table")
            return read
        except Exception as e:   # no amdsmi or no access: report no clock
            self.error = f"{type(e).__name__}: {e}"[:200]
            return None

    def _run(self):
        while not self._stop.is_set():
            try:
                clk, _ = self._read()
                if clk is not None and clk >= 500:
                    self.samples.append(float(clk))
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"[:200]
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self._thread:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join(timeout=2)

    def summary(self):
        if not self.samples:
            return {"sclk_mhz": None, "error": self.error}
        t = sorted(self.samples)
        return {"sclk_mhz": round(t[len(t) // 2], 1), "sclk_mhz_min": round(t[0], 1),
                "sclk_mhz_max": round(t[-1], 1), "samples": len(t),
                "source": "amdsmi gpu metrics, mean of current_gfxclks over the XCCs"}


def sustained_clock(step, seconds: float = 1.5) -> dict:
    """The shader clock under the step's load: after the timed steps (outside the
    timed region), the same step runs again for `seconds` while ClockSampler
    reads the metrics table, whose readings lag the load by a few hundred ms;
    the second half of the samples is reported."""
    import torch
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(5):
                step()
            torch.cuda.synchronize()
    s = clock.summary()
    if clock.samples:
        t = sorted(clock.samples[len(clock.samples) // 2:])
        s.update(sclk_mhz=round(t[len(t) // 2], 1), sclk_mhz_min=round(t[0], 1),
                 sclk_mhz_max=round(t[-1], 1), samples=len(t),
                 window_s=seconds / 2)
    return s


def run_conditions(dev_index: int = 0) -> dict:
    """Versions and device of the run (the conditions a throughput figure needs)."""
    import platform
    import torch
    cond = {"device": torch.cuda.get_device_name(dev_index),
            "arch": getattr(torch.cuda.get_device_properties(dev_index), "gcnArchName", None),
            "torch": torch.__version__, "hip_runtime": torch.version.hip,
            "python": platform.python_version(), "host_cpus": os.cpu_count()}
    try:
        with open("/opt/rocm/.info/version") as f:
            cond["rocm"] = f.read().strip()
    except OSError:
        cond["rocm"] = None
    # The compiler that built libfa.so, from the ident string it left in the
    # library (no child process: this process has initialised the GPU).
    try:
        import re
        import io_aware_exact_fa_amd as fa
        with open(fa.LIB_PATH, "rb") as f:
            m = re.search(rb"AMD clang version [^\x00)]*\)?", f.read())
        cond["compiler"] = m.group(0).decode() if m else None
    except OSError:
        cond["compiler"] = None
    return cond


# MFMA work each kernel executes per unit of its algorithmic share, by design
# (masked diagonal tiles aside): the two-pass backward's dQ pass recomputes S
# and dP to form dS, three products where its share of the backward count is
# one; the one-pass kernel computes each of the five products once.
EXECUTED_RATIO = {"fwd": 1.0, "dkdv": 1.0, "dq": 3.0, "dkdvq": 1.0}
KERNEL_NAMES = {"fwd": "fwd16_kernel", "pre": "bwd_pre_kernel", "dkdv": "bwd_dkdv16_kernel",
                "dq": "bwd_dq16_kernel", "dkdvq": "bwd_dkdv16_kernel (one pass, dQ by atomics)",
                "dqfin": "bwd_dqfin_kernel"}


def kernel_name(key: str, w) -> str:
    """The kernel the library launches for step `key` of workload w (its
    launchers choose by dtype, head dimension, mask, dropout and length)."""
    wide = w.dtype != "f32"
    drop = bool(getattr(w, "dropout", ())) and w.dropout[0] > 0.0
    if key == "fwd":
        if not wide:
            return "fwd_kernel"
        if w.d == 64:
            return "fwd16_kernel"
        n = w.max_s if hasattr(w, "max_s") else w.N   # a packed batch launches with its longest length
        return "fwd64_kernel" if not (w.causal or drop) and n >= 2048 else "fwd16_kernel"
    if key == "dkdv":
        return ("bwd_dkdv16p_kernel" if w.d == 64 or drop else "bwd_dkdv16_kernel") if wide else "bwd_dkdv_kernel"
    if key == "dq":
        return "bwd_dq16_kernel" if wide else "bwd_dq_kernel"
    return KERNEL_NAMES[key]


def time_dense(args, w, fa, steps=None):
    """Seeded inputs of a dense workload on the GPU, `args.warmup` untimed steps,
    then `steps` timed ones; one step = fa_fwd_gqa and the backward's launches
    called one by one on one stream, HIP events around each: fa_bwd's two-pass
    backward (fa_bwd_preprocess, fa_bwd_dkdv_gqa, fa_bwd_dq_gqa), or with
    --backward one-pass (16-bit types) fa_bwd_preprocess, fa_bwd_dkdv_dq,
    fa_bwd_dq_finalize.  Returns the timings and, for the oracle check, the
    inputs and outputs."""
    import torch
    steps = steps or args.steps
    dev = torch.device("cuda:0")
    inp = workloads.make_inputs(w)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    one_pass = args.backward == "one-pass" and w.dtype != "f32"
    ws = fa.workspace(B, H, N, d, dev, one_pass=one_pass)
    code = fa.dtype_code(q.dtype)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    P = lambda t: t.data_ptr()

    def check(st, where):
        if st != fa.FA_OK:
            raise fa.FaError(st, where)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        check(fa.fa_fwd_gqa(P(q), P(k), P(v), P(o), P(lse), B, H, Hkv, N, d, w.causal, w.scale, code,
                            sh), "fwd")
        if ev is not None:
            ev[1].record(stream)
        check(fa.fa_bwd_preprocess(P(o), P(do), P(lse), B, H, N, d, code, P(ws), ws.numel(), sh), "pre")
        if ev is not None:
            ev[2].record(stream)
        if one_pass:
            check(fa.fa_bwd_dkdv_dq(P(q), P(k), P(v), P(do), P(lse), P(dk), P(dv), B, H, Hkv, N, d,
                                    w.causal, w.scale, code, P(ws), ws.numel(), sh), "dkdv_dq")
        else:
            check(fa.fa_bwd_dkdv_gqa(P(q), P(k), P(v), P(do), P(lse), P(dk), P(dv), B, H, Hkv, N,
                                     d, w.causal, w.scale, code, P(ws), ws.numel(), sh), "dkdv")
        if ev is not None:
            ev[3].record(stream)
        if one_pass:
            check(fa.fa_bwd_dq_finalize(P(dq), B, H, N, d, w.scale, code, P(ws), ws.numel(), sh),
                  "dq_finalize")
        else:
            check(fa.fa_bwd_dq_gqa(P(q), P(k), P(v), P(do), P(lse), P(dq), B, H, Hkv, N, d,
                                   w.causal, w.scale, code, P(ws), ws.numel(), sh), "dq")
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock = sustained_clock(step)
    ms = lambda a, b_: sum(e[a].elapsed_time(e[b_]) for e in events) / steps
    if one_pass:
        kms = {"fwd": ms(0, 1), "pre": ms(1, 2), "dkdvq": ms(2, 3), "dqfin": ms(3, 4)}
    else:
        kms = {"fwd": ms(0, 1), "pre": ms(1, 2), "dkdv": ms(2, 3), "dq": ms(3, 4)}
    return {"w": w, "shape": (B, H, Hkv, N, d), "steps": steps, "wall": wall, "events": events,
            "kernel_ms": kms, "clock": clock, "inp": inp,
            "out": {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}}


def kernel_entries(w, kms, peak):
    """Per launch of each kernel: algorithmic FLOPs (the method's count split
    over the kernels: forward 4 B H N^2 d; two-pass backward: dK/dV 4/5 of the
    backward's 2.5x, dQ 1/5; one-pass: all of it), MFMA FLOPs executed by
    design, time and rate against the peak; the preprocess and the dQ finalize
    against HBM, at the bytes they move."""
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    alg = {"fwd": fwd_f, "dkdv": 0.8 * bwd_f, "dq": 0.2 * bwd_f, "dkdvq": bwd_f}
    e = 4 if w.dtype == "f32" else 2
    out = []
    for key in ("fwd", "dkdv", "dq", "dkdvq"):
        if key not in kms:
            continue
        t = kms[key] * 1e-3
        out.append({"kernel": kernel_name(key, w), "ms": round(kms[key], 4), "bound": "mfma",
                    "algorithmic_tflop": round(alg[key] / 1e12, 4),
                    "executed_tflop": round(alg[key] * EXECUTED_RATIO[key] / 1e12, 4),
                    "achieved": round(alg[key] / t / 1e12, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(alg[key] / t / 1e12 / peak, 4),
                    "executed_frac": round(alg[key] * EXECUTED_RATIO[key] / t / 1e12 / peak, 4)})
    rows = w.B * w.H * w.N
    prow = w.B * w.H * ((w.N + 63) // 64 * 64)
    hbm = {
        # O and dO read, LSE read, D and L2 written (+ the accumulator zeroed, one pass)
        "pre": 2 * rows * w.d * e + 4 * rows + 8 * prow + (4 * prow * w.d if "dkdvq" in kms else 0),
        # accumulator read, dq written
        "dqfin": 4 * rows * w.d + rows * w.d * e,
    }
    for key in ("pre", "dqfin"):
        if key not in kms:
            continue
        rate = hbm[key] / (kms[key] * 1e-3) / 1e9
        out.append({"kernel": kernel_name(key, w), "ms": round(kms[key], 4), "bound": "hbm",
                    "bytes": hbm[key], "achieved": round(rate, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(rate / HBM_PEAK_GBS, 4)})
    return out


def summary(res, peak):
    """fwd / bwd / step rates of one timed dense workload."""
    w, kms, steps = res["w"], res["kernel_ms"], res["steps"]
    fwd_ms = kms["fwd"]
    bwd_ms = sum(v for k_, v in kms.items() if k_ != "fwd")
    ms_per_step = res["wall"] * 1e3 / steps
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    value = (fwd_f + bwd_f) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = fwd_f / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_f / (bwd_ms * 1e-3) / 1e12
    clk = res["clock"]["sclk_mhz"]
    d = {
        "workload": w.name, "B": w.B, "H": w.H, "H_kv": w.kv_heads, "N": w.N, "d": w.d,
        "causal": w.causal,
        "step": ("fa_fwd + fa_bwd one pass (preprocess, dkdv_dq, dq_finalize)" if "dkdvq" in kms
                 else "fa_fwd + fa_bwd two pass (preprocess, dkdv, dq)"),
        "step_gpu_ms": step_spread(res["events"]),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        **{f"bwd_{k_}_ms": round(v, 4) for k_, v in kms.items() if k_ != "fwd"},
        "fwd_tflops": round(fwd_tf, 2), "bwd_tflops": round(bwd_tf, 2),
        "step_tflops": round(value, 2),
        "fwd_pct_of_peak": round(100 * fwd_tf / peak, 2),
        "bwd_pct_of_peak": round(100 * bwd_tf / peak, 2),
        "step_pct_of_peak": round(100 * value / peak, 2),
        "peak_tflops": peak,
        "sclk": res["clock"],
        # The same peak at the shader clock measured under the same load.
        "peak_tflops_at_sclk": round(peak * clk / 2400.0, 1) if clk else None,
        "fwd_pct_of_peak_at_sclk": round(100 * fwd_tf / (peak * clk / 2400.0), 2) if clk else None,
        "bwd_pct_of_peak_at_sclk": round(100 * bwd_tf / (peak * clk / 2400.0), 2) if clk else None,
    }
    return d, value, ms_per_step


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "every workload here is one GPU's share, see the sharding paragraph of the design "
              "notes", file=sys.stderr)
        sys.exit(2)

    import torch
    import io_aware_exact_fa_amd as fa

    if args.mode == "copy":
        copy_calibration(args.steps)
        return

    if args.workload in workloads.VARLEN_BY_NAME:
        bench_varlen(args, workloads.VARLEN_BY_NAME[args.workload])
        return
    w = workloads.BY_NAME[args.workload]
    if w.windowed or w.sparse or w.dropout:
        dev = torch.device("cuda:0")
        inp = workloads.make_inputs(w)
        q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
        B, H, N, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
        ws = fa.workspace(B, H, N, d, dev)
        bench_windowed(args, w, fa, inp, q, k, v, do, o, lse, dq, dk, dv, ws,
                       fa.dtype_code(q.dtype), torch.cuda.current_stream())
        return

    peak = PEAK_TFLOPS[w.dtype]
    res = time_dense(args, w, fa)
    config, value, ms_per_step = summary(res, peak)
    kernels = kernel_entries(w, res["kernel_ms"], peak)
    dominant = max(kernels, key=lambda e: e["ms"])
    traffic = load_traffic(w.name) if dominant["kernel"] == DOMINANT else None
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal Q/K/V/dO of the workload's shape and distribution)",
        "config": config,
        "roofline": {**{k_: dominant[k_] for k_ in ("kernel", "bound", "achieved", "peak", "unit",
                                                    "frac")},
                     "traffic": traffic, "per_kernel": kernels},
        "conditions": run_conditions(),
    }
    gpu_out = None
    if not args.no_cpu_baseline:
        o = res["out"]
        gpu_out = {n: o[n].cpu() for n in ("o", "lse", "dq", "dk", "dv")}
    inp = res["inp"]
    del res
    torch.cuda.empty_cache()
    # The other workload the throughput target is stated on (N >= 4096, d = 128,
    # bf16): the causal one, timed in the same process after the headline one.
    if not args.no_secondary and w is workloads.PEAKED_BF16:
        w2 = workloads.CAUSAL_BF16
        peak2 = PEAK_TFLOPS[w2.dtype]
        res2 = time_dense(args, w2, fa)
        c2, _, ms2 = summary(res2, peak2)
        c2["ms_per_step"] = round(ms2, 4)
        c2["per_kernel"] = kernel_entries(w2, res2["kernel_ms"], peak2)
        out["secondary"] = [c2]
        del res2
        torch.cuda.empty_cache()
    if gpu_out is not None:
        out["cpu_baseline"] = cpu_baseline(w, inp, gpu_out)
    print(json.dumps(out), flush=True)


def two_call_result(args, w, events, wall, peak_dtype, config, data, kernel_name):
    """The JSON line of a step made of one forward and one backward call, timed with
    HIP events around each call (the backward's launches timed as one)."""
    ms = lambda a, b_: sum(e[a].elapsed_time(e[b_]) for e in events) / args.steps
    fwd_ms, bwd_ms = ms(0, 1), ms(1, 2)
    ms_per_step = wall * 1e3 / args.steps
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    peak = PEAK_TFLOPS[peak_dtype]
    value = (fwd_f + bwd_f) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = fwd_f / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_f / (bwd_ms * 1e-3) / 1e12
    config = dict(config)
    config.update({
        "step_gpu_ms": step_spread(events),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_tflops": round(fwd_tf, 2), "bwd_tflops": round(bwd_tf, 2),
        "fwd_pct_of_peak": round(100 * fwd_tf / peak, 2),
        "bwd_pct_of_peak": round(100 * bwd_tf / peak, 2),
        "step_pct_of_peak": round(100 * value / peak, 2),
        "peak_tflops": peak,
    })
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": data,
        "config": config,
        # The backward call (three launches) timed as one, at the method's FLOP count.
        "roofline": {
            "kernel": kernel_name,
            "bound": "mfma",
            "achieved": round(bwd_tf, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(bwd_tf / peak, 4),
            "traffic": None,
        },
    }


def step_spread(events):
    """Median and 10th / 90th percentiles (ms) of the per-step GPU time, first to
    last event of each timed step."""
    t = sorted(e[0].elapsed_time(e[-1]) for e in events)
    q = lambda f: t[min(len(t) - 1, max(0, round(f * (len(t) - 1))))]
    return {"median": round(q(0.5), 4), "p10": round(q(0.1), 4), "p90": round(q(0.9), 4)}


def time_two_calls(args, step):
    import torch
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    return events, time.perf_counter() - t0


def bench_windowed(args, w, fa, inp, q, k, v, do, o, lse, dq, dk, dv, ws, code, stream):
    """A local-window, dropout or block-sparse workload: fa_fwd_ex then fa_bwd_ex per
    step."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    bm = workloads.block_mask(w).to(q.device) if w.sparse else None
    p = fa.attn(B, H, Hkv, N, d, w.causal, w.scale, code, w.window, dropout=w.dropout or None,
                block_mask=bm.data_ptr() if bm is not None else None,
                block_mask_heads=H if bm is not None else 1)
    sh = stream.cuda_stream
    P = lambda t: t.data_ptr()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        st = fa.fa_fwd_ex(p, P(q), P(k), P(v), P(o), P(lse), sh)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_fwd_ex")
        if ev is not None:
            ev[1].record(stream)
        st = fa.fa_bwd_ex(p, P(q), P(k), P(v), P(o), P(do), P(lse), P(dq), P(dk), P(dv), P(ws),
                          ws.numel(), sh)
        if st != fa.FA_OK:
            raise fa.FaError(st, "fa_bwd_ex")
        if ev is not None:
            ev[2].record(stream)

    events, wall = time_two_calls(args, step)
    config = {"workload": w.name, "B": B, "H": H, "H_kv": Hkv, "N": N, "d": d, "causal": w.causal,
              "window": list(w.window), "dropout": list(w.dropout),
              "block_density": w.block_density, "step": "fa_fwd_ex + fa_bwd_ex",
              "visible_pairs_per_head": workloads.visible_pairs(N, w.causal, w.window)}
    out = two_call_result(args, w, events, wall, w.dtype, config,
                          "synthetic (seeded normal Q/K/V/dO of the workload's shape and "
                          "distribution)", "fa_bwd_ex (preprocess, dK/dV, dQ)")
    if not args.no_cpu_baseline:
        gpu_out = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
        out["cpu_baseline"] = cpu_baseline(w, inp, gpu_out, budget_s=5.0)
    print(json.dumps(out), flush=True)


def cpu_baseline_varlen(w, inp, gpu_out, budget_s: float = 10.0):
    """The fp64 oracle on whole sequences (all heads), shortest first, until about
    ``budget_s`` seconds of CPU work; GPU-vs-oracle error on the first one."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    cu = inp["cu_seqlens"].tolist()
    order = sorted((b for b in range(w.B) if w.lens[b] > 0), key=lambda b: w.lens[b])
    f64 = lambda t: t.to(dtype=torch.float64).numpy()
    q, k, v, do = (f64(inp[n]) for n in ("q", "k", "v", "do"))
    secs, flops, done, check = 0.0, 0.0, 0, None
    for b in order:
        s0, s1 = cu[b], cu[b + 1]
        n = s1 - s0
        one = [0, n]   # the sequence alone, as a packed batch of one
        t0 = time.perf_counter()
        o, lse = oracle.forward_varlen(q[:, s0:s1], k[:, s0:s1], v[:, s0:s1], one, n, w.scale,
                                       w.causal)
        dq, dk, dv = oracle.backward_varlen(q[:, s0:s1], k[:, s0:s1], v[:, s0:s1], do[:, s0:s1],
                                            one, n, w.scale, w.causal)
        secs += time.perf_counter() - t0
        flops += 3.5 * 4.0 * w.H * n * n * w.d / (2 if w.causal else 1)
        done += 1
        if check is None:
            rel = lambda a, r: float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), 1e-30))
            check = {
                "sequence": b, "length": n,
                "o_maxabs": float(np.max(np.abs(f64(gpu_out["o"][:, s0:s1]) - o))),
                "lse_maxabs": float(np.max(np.abs(f64(gpu_out["lse"][b, :, :n]) - lse[0]))),
                "dq_rel": rel(f64(gpu_out["dq"][:, s0:s1]), dq),
                "dk_rel": rel(f64(gpu_out["dk"][:, s0:s1]), dk),
                "dv_rel": rel(f64(gpu_out["dv"][:, s0:s1]), dv),
            }
        if secs >= budget_s:
            break
    return {
        "value": flops / secs / 1e12,
        "unit": "TFLOPS",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{done} of {w.B} sequences (shortest first), all {w.H} query heads, forward + "
                  f"backward, fp64 numpy oracle; {secs:.2f} s wall",
        "seconds": round(secs, 3),
        "parity_on_sample": check,
    }


def bench_varlen(args, w):
    """A packed variable-length batch: fa_fwd_varlen then fa_bwd_varlen per step."""
    import torch
    import io_aware_exact_fa_amd as fa
    dev = torch.device("cuda:0")
    inp = workloads.make_varlen_inputs(w)
    q, k, v, do = (inp[n].to(dev) for n in ("q", "k", "v", "do"))
    cu = inp["cu_seqlens"].to(dev)
    H, total, d = q.shape
    Hkv = k.shape[0]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, H, w.max_s), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    ws = fa.workspace(w.B, H, w.max_s, d, dev)
    code = fa.dtype_code(q.dtype)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    P = lambda t: t.data_ptr()

    def check(st, where):
        if st != fa.FA_OK:
            raise fa.FaError(st, where)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        check(fa.fa_fwd_varlen(P(q), P(k), P(v), P(o), P(lse), P(cu), w.B, w.max_s, total, H, Hkv,
                               d, w.causal, w.scale, code, sh), "fwd_varlen")
        if ev is not None:
            ev[1].record(stream)
        check(fa.fa_bwd_varlen(P(q), P(k), P(v), P(o), P(do), P(lse), P(dq), P(dk), P(dv), P(cu),
                               w.B, w.max_s, total, H, Hkv, d, w.causal, w.scale, code, P(ws),
                               ws.numel(), sh), "bwd_varlen")
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = lambda a, b_: sum(e[a].elapsed_time(e[b_]) for e in events) / args.steps
    fwd_ms, bwd_ms = ms(0, 1), ms(1, 2)
    ms_per_step = wall * 1e3 / args.steps
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    peak = PEAK_TFLOPS[w.dtype]
    value = (fwd_f + bwd_f) / (ms_per_step * 1e-3) / 1e12
    fwd_tf = fwd_f / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_f / (bwd_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal Q/K/V/dO, packed sequences of the workload's lengths)",
        "config": {
            "workload": w.name, "B": w.B, "H": H, "H_kv": Hkv, "total": total, "max_s": w.max_s,
            "d": d, "causal": w.causal, "lens": list(w.lens),
            "step": "fa_fwd_varlen + fa_bwd_varlen", "step_gpu_ms": step_spread(events),
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "fwd_tflops": round(fwd_tf, 2), "bwd_tflops": round(bwd_tf, 2),
            "fwd_pct_of_peak": round(100 * fwd_tf / peak, 2),
            "bwd_pct_of_peak": round(100 * bwd_tf / peak, 2),
            "step_pct_of_peak": round(100 * value / peak, 2),
            "peak_tflops": peak,
        },
        # The backward call (three launches) timed as one, at the method's FLOP count.
        "roofline": {
            "kernel": "fa_bwd_varlen (preprocess, dK/dV, dQ)",
            "bound": "mfma",
            "achieved": round(bwd_tf, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(bwd_tf / peak, 4),
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        gpu_out = {"o": o.cpu(), "lse": lse.cpu(), "dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
        out["cpu_baseline"] = cpu_baseline_varlen(w, inp, gpu_out)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
