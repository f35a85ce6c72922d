"""Attention-forward benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

NAME is a key of gen.WORKLOADS (default: bf16 inputs, causal, 1 x 32 heads,
16384 x 16384 tokens, head dim 128), a backward workload (bwd_ + a forward key)
or a row-primitive workload.

A step is one attention forward (every kernel of the path) over the
workload's synthetic inputs, already resident in HBM. Prints one JSON line:
the headline TFLOP/s on the metric's FLOP formula (4*B*H*Sq*Skv*d, halved when
causal), the fraction of the dtype's dense MFMA peak, a roofline object for
the main attention kernel timed with HIP events inside the timed region, and
the CPU oracle timed on a bounded sample of the same workload on the host.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·Sq·Skv·d, causal halved) and % of MFMA peak"
# MI355X published dense MFMA peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0, "f16": 2500.0}
HBM_GBPS = 8000.0
# The largest workload that fits one GPU, and the one the >= 50 %-of-peak target is
# about: bf16 inputs, causal, 1 x 32 heads, 16384 x 16384 tokens, head dim 128.
DEFAULT_WORKLOAD = "bf16_causal_b1h32_s16384_d128"
PEAK_SCLK_MHZ = 2400.0  # the engine clock the published peaks assume


def metric_flops(w) -> float:
    f = 4.0 * w.batch * w.heads * w.seq_q * w.seq_kv * w.head_dim
    return f / 2 if w.causal else f


def allowed_pairs(w) -> int:
    """Admitted (query, key) pairs: all, or j <= i + Skv - Sq under the causal mask."""
    if not w.causal:
        return w.batch * w.heads * w.seq_q * w.seq_kv
    off = w.seq_kv - w.seq_q
    per = 0
    for i in range(w.seq_q):
        per += min(max(i + off + 1, 0), w.seq_kv)
    return per * w.batch * w.heads


def min_bytes(w, o_elem: int = 4) -> int:
    e = 4 if w.dtype == "f32" else 2
    bh = w.batch * w.heads
    return bh * ((w.seq_q + 2 * w.seq_kv) * w.head_dim * e + w.seq_q * w.head_dim * o_elem + w.seq_q * 4)


# Device function of each sma_kernel code (the name rocprofv3 reports); the 16-bit kernel
# code runs the role-split function at head dim 256.
KERNEL_FUNCTIONS = {0: "attn_fwd_f32_kernel", 1: "attn_fwd_f32_wsplit_kernel", 2: "attn_fwd_bf16_kernel"}


def kernel_function(plan_kernel: int, head_dim: int) -> str:
    if plan_kernel == 2 and head_dim == 256:
        return "attn_fwd_bf16_rs_kernel"
    if plan_kernel == 2 and head_dim == 128:
        return "attn_fwd_bf16_rb2_kernel"
    return KERNEL_FUNCTIONS[plan_kernel]


class HipEvents:
    """hipEvent_t handles through the HIP runtime (torch's events only see torch streams)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.hip.hipEventSynchronize(b) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """Engine (SCLK) and memory (MCLK) clocks of the GPU in use, from the amd-smi library's
    GPU metrics table, read by a host thread every few milliseconds. The firmware refreshes
    that table about once a second, so only reads that carry a new table (a new
    system_clock_counter) count as samples. Values are MHz; SCLK is the mean over the XCDs."""

    NA = 0xFFFF  # amd-smi's marker for a field the firmware does not report

    def __init__(self, period_s: float = 0.01):
        self.period_s = period_s
        self.samples, self.mclk = [], []
        self.error = None
        self.field = None
        self.handle = None
        self.last_stamp = None
        self._stop = None
        self._thread = None
        try:
            import amdsmi
            import torch

            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) == 1:
                self.handle = handles[0]
            else:  # match the PCI bus of torch's device 0
                props = torch.cuda.get_device_properties(0)
                bus = getattr(props, "pci_bus_id", None)
                for h in handles:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                    if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                        self.handle = h
                        break
            if self.handle is None:
                raise RuntimeError(f"no amd-smi handle matches the device ({len(handles)} found)")
            self._read(first=True)  # fail here, not in the thread, if the metrics are unreadable
        except Exception as e:  # noqa: BLE001 - report, never fail the bench for it
            self.error = f"{type(e).__name__}: {e}"

    def _read(self, first=False):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        stamp = m.get("system_clock_counter")
        if first or stamp == self.last_stamp:
            self.last_stamp = stamp  # the table on entry describes the time before the run
            return

        def ok(x):
            return isinstance(x, (int, float)) and 0 < x < self.NA

        self.last_stamp = stamp
        xs = [x for x in (m.get("current_gfxclks") or []) if ok(x)]
        if xs:
            self.field = "current_gfxclks (mean over XCDs)"
            self.samples.append(sum(xs) / len(xs))
        elif ok(m.get("current_gfxclk")):
            self.field = "current_gfxclk"
            self.samples.append(float(m["current_gfxclk"]))
        u = m.get("current_uclk")
        if ok(u):
            self.mclk.append(float(u))

    def start(self):
        import threading

        if self.error:
            return
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    self._read()
                except Exception as e:  # noqa: BLE001
                    self.error = f"{type(e).__name__}: {e}"
                    return
                self._stop.wait(self.period_s)

        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()

    def fresh(self) -> int:
        return len(self.samples)

    def stop(self) -> dict:
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        out = {"source": "amd-smi GPU metrics (refreshed about once a second), read while the "
                         "measured step runs"}
        # The first refreshed table can still average in time from before the run.
        xs = self.samples[1:] if len(self.samples) > 1 else self.samples
        if xs:
            out.update(sclk_mhz_mean=round(float(np.mean(xs)), 1),
                       sclk_mhz_min=round(float(np.min(xs)), 1),
                       sclk_mhz_max=round(float(np.max(xs)), 1),
                       sclk_field=self.field, samples=len(xs))
        if self.mclk:
            out["mclk_mhz_mean"] = round(float(np.mean(self.mclk[1:] or self.mclk)), 1)
        if self.error or not self.samples:
            out["error"] = self.error or "no refreshed metrics table during the run"
        return out


CLOCK_SECONDS = 3.0  # set from --clock-seconds


def clock_window(sampler, step, seconds: float = None, min_samples: int = 3) -> float:
    """After a timed loop too short for the metrics table to refresh a few times, keep
    running the same step, untimed, until `min_samples` refreshed tables have been read or
    `seconds` have passed; returns the wall seconds spent."""
    import torch

    seconds = CLOCK_SECONDS if seconds is None else seconds
    if sampler.error or seconds <= 0:
        return 0.0
    t0 = time.perf_counter()
    while sampler.fresh() < min_samples and time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    return round(time.perf_counter() - t0, 2)


def with_host(baseline: dict) -> dict:
    """The CPU baseline with the host's processor model beside its thread count."""
    baseline["cpu_model"] = host_cpu_model()
    return baseline


def clock_adjusted(frac: float, clocks: dict):
    """The roofline fraction against the peak at the sampled engine clock (the published
    peak assumes 2.4 GHz), or None without clock samples."""
    s = clocks.get("sclk_mhz_mean")
    return round(frac * PEAK_SCLK_MHZ / s, 4) if s else None


def step_stats(durations_ms):
    d = np.asarray(durations_ms, dtype=np.float64)
    return {"median": round(float(np.median(d)), 5), "min": round(float(d.min()), 5),
            "max": round(float(d.max()), 5), "n": int(d.size)}


def settle(step, ms: float) -> int:
    """Run the measured step, untimed, for about `ms` milliseconds of wall time before the
    warmup steps; returns how many steps that took. The GPU's clock settles to the running
    workload over tens of milliseconds: a short kernel timed right after an idle (or a
    differently loaded) period runs part of its timed steps on the ramp."""
    import torch

    if ms <= 0:
        return 0
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step()
        n += 8
        torch.cuda.synchronize()
    return n


def traffic_summary_path(kernel_function: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel_function}_{workload}_hbm_traffic.txt")


def read_traffic(kernel_function: str, workload: str, kernel_src_digest: str):
    """HBM bytes per launch from the committed counter summary, or None if absent or stale."""
    path = traffic_summary_path(kernel_function, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_src_digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# Source file of each kernel (with the shared device header, what its traffic depends on).
KERNEL_SOURCES = {"attn_fwd_f32_kernel": ["attn_fwd_f32.hip", "attn_common.h"],
                  "attn_bwd_dkdv_f32_kernel": ["attn_bwd_f32.hip", "attn_common.h"],
                  "attn_bwd_dkdv_bf16_kernel": ["attn_bwd_bf16.hip", "attn_common.h"],
                  "attn_bwd_dkdv_bf16_kb2_kernel": ["attn_bwd_bf16.hip", "attn_common.h"],
                  "attn_fwd_f32_wsplit_kernel": ["attn_fwd_f32_wsplit.hip", "attn_common.h"],
                  "attn_fwd_bf16_kernel": ["attn_fwd_bf16.hip", "attn_common.h"],
                  "attn_fwd_bf16_rs_kernel": ["attn_fwd_bf16.hip", "attn_common.h"],
                  "attn_fwd_bf16_rb2_kernel": ["attn_fwd_bf16.hip", "attn_common.h"],
                  "row_softmax": ["row_softmax.hip"]}


def kernel_source_digest(kernel_function: str) -> str:
    """SHA-256 of the device sources of one kernel: a committed traffic figure is used only
    while these are unchanged."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_masked_attention_amd", "csrc")
    for f in KERNEL_SOURCES[kernel_function]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def cpu_baseline(w, vals, target_s: float):
    """The oracle on a bounded sample of rows of the same workload, scaled to TFLOP/s."""
    import numpy as np

    import oracle

    B, H, sq, skv = w.batch, w.heads, w.seq_q, w.seq_kv
    total_rows = B * H * sq
    rng = np.random.default_rng(0)
    # Calibrate on a small row sample, then size the sample for ~target_s seconds.
    n0 = min(total_rows, 64)
    rows0 = np.sort(rng.choice(total_rows, size=n0, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attention_fwd(*vals, w.scale, w.causal, rows=rows0)
    dt0 = max(time.perf_counter() - t0, 1e-4)
    n = int(min(total_rows, max(n0, n0 * target_s / dt0)))
    rows = np.sort(rng.choice(total_rows, size=n, replace=False)).astype(np.int64)
    passes = 0
    t0 = time.perf_counter()
    while True:  # whole passes over the sample until the time target is reached
        oracle.attention_fwd(*vals, w.scale, w.causal, rows=rows)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s or passes >= 1000:
            break
    # metric FLOPs attributable to the sampled rows (each row's share of the formula)
    frac = n / total_rows
    flops = metric_flops(w) * frac * passes
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n} of {total_rows} query rows chosen at random (seed 0), all keys each, "
                      f"{passes} pass(es) in {dt:.1f} s; metric FLOPs scaled by the row fraction"}


BWD_PREFIX = "bwd_"


def gen_workloads():
    import gen

    # The backward runs head dims 32-128, and 256 with 16-bit inputs.
    bwd = [BWD_PREFIX + n for n, w in gen.WORKLOADS.items()
           if w.head_dim in (32, 64, 128) or (w.head_dim == 256 and w.dtype != "f32")]
    return list(gen.WORKLOADS) + bwd + list(gen.ROW_WORKLOADS)


def dkdv_min_bytes(w) -> int:
    """The dK/dV kernel reads Q, dO, K, V (in the input type; dO as the 16-bit copy for
    16-bit inputs) and each row's lse2 and D once, and writes dK, dV (fp32)."""
    bh = w.batch * w.heads
    e = 4 if w.dtype == "f32" else 2
    return bh * ((2 * w.seq_q + 2 * w.seq_kv) * w.head_dim * e + 2 * w.seq_kv * w.head_dim * 4 + 8 * w.seq_q)


BWD_METRIC = "attention bwd TFLOP/s (10·B·H·Sq·Skv·d, causal halved) and % of MFMA peak"


def bwd_cpu_baseline_last_rows(w, q, k, v, g, target_s: float):
    """The backward oracle on exact sub-problems of a square causal workload too large for
    whole heads: the last T query rows of a head with every key keep the bottom-right mask
    (row i' admits keys up to i' + S - T), one head per thread. T grows until a round takes
    a few seconds; FLOPs are the metric's per admitted pair times the pairs processed."""
    import oracle

    bh, S, d = w.batch * w.heads, w.seq_q, w.head_dim
    qf, kf, vf, gf = (x.reshape(bh, 1, x.shape[2], x.shape[3]) for x in (q, k, v, g))
    threads = max(1, oracle.num_threads())
    n = min(bh, threads)
    ids = np.sort(np.random.default_rng(0).permutation(bh)[:n])
    per_pair = 2.5 * metric_flops(w) / allowed_pairs(w)
    T = 8
    while True:
        t0 = time.perf_counter()
        oracle.attention_bwd(qf[ids, :, S - T:], kf[ids], vf[ids], gf[ids, :, S - T:], w.scale, True)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or 2 * T > S:
            break
        T *= 2
    passes, total = 0, 0.0
    while total < target_s and passes < 1000:
        t0 = time.perf_counter()
        oracle.attention_bwd(qf[ids, :, S - T:], kf[ids], vf[ids], gf[ids, :, S - T:], w.scale, True)
        total += time.perf_counter() - t0
        passes += 1
    pairs = n * sum(S - T + i + 1 for i in range(T)) * passes
    return {"value": per_pair * pairs / total / 1e12, "unit": "TFLOP/s", "cores": n, "kind": "oracle",
            "sample": f"the last {T} query rows (all {S} keys) of {n} of {bh} (batch, head) slices "
                      f"chosen at random (seed 0), {passes} pass(es) in {total:.1f} s; metric FLOPs "
                      f"per admitted pair times the pairs processed"}


def bwd_cpu_baseline(w, q, k, v, g, target_s: float):
    """The backward oracle on a bounded random sample of whole (batch, head) slices."""
    import oracle

    bh = w.batch * w.heads
    if w.causal and w.seq_q == w.seq_kv and w.seq_q * w.seq_kv * w.head_dim > (1 << 33):
        return bwd_cpu_baseline_last_rows(w, q, k, v, g, target_s)
    rng = np.random.default_rng(0)
    order = rng.permutation(bh)
    qf, kf, vf, gf = (x.reshape(bh, 1, x.shape[2], x.shape[3]) for x in (q, k, v, g))

    def run(ids):
        ids = np.sort(ids)
        oracle.attention_bwd(qf[ids], kf[ids], vf[ids], gf[ids], w.scale, w.causal)

    t0 = time.perf_counter()
    run(order[:1])
    dt1 = max(time.perf_counter() - t0, 1e-4)
    # one head per thread runs concurrently: size the sample in whole rounds of the threads,
    # then repeat whole passes over it until the time target is reached
    threads = max(1, oracle.num_threads())
    n = int(min(bh, max(1, threads * max(1, int(target_s / dt1)))))
    passes = 0
    t0 = time.perf_counter()
    while True:
        run(order[:n])
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s or passes >= 1000:
            break
    flops = 2.5 * metric_flops(w) * n / bh * passes
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(threads, n), "kind": "oracle",
            "sample": f"{n} of {bh} (batch, head) slices chosen at random (seed 0), every query and "
                      f"key of each, {passes} pass(es) in {dt:.1f} s; metric FLOPs scaled by the "
                      f"slice fraction"}


def to_device_inputs(vals, bits, dtype):
    """q, k, v on the device: fp32 values, or 16-bit tensors from the exact bit patterns."""
    import torch

    if dtype == "f32":
        return tuple(torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in vals)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return tuple(torch.from_numpy(b.view(np.int16)).to("cuda").view(tdt) for b in bits)


def bench_bwd(args, w, name):
    import torch

    import gen
    import scaled_masked_attention_amd as sma

    vals, bits = gen.make_inputs(w)
    g = gen.upstream_grad(w.seed, w.q_shape)
    tq, tk, tv = to_device_inputs(vals, bits, w.dtype)
    tg = torch.from_numpy(np.ascontiguousarray(g)).to("cuda")
    in_dt = {"f32": sma.SMA_DTYPE_F32, "bf16": sma.SMA_DTYPE_BF16, "f16": sma.SMA_DTYPE_F16}[w.dtype]
    B, H, sq, skv, d = w.batch, w.heads, w.seq_q, w.seq_kv, w.head_dim
    o, lse = sma.attention_fwd(tq, tk, tv, scale=w.scale, causal=w.causal, return_lse=True)
    dq, dk, dv = (torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in (tq, tk, tv))
    ws_n = sma.attention_bwd_workspace_bytes(in_dt, B, H, sq, skv, d, w.causal)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    call = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), o.data_ptr(), lse.data_ptr(), tg.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), in_dt, B, H, sq, skv, d, w.scale,
            w.causal, ws.data_ptr(), ws_n, sptr)
    settled = settle(lambda: sma.attention_bwd_raw(*call), args.settle_ms)
    for _ in range(args.warmup):
        sma.attention_bwd_raw(*call)
    torch.cuda.synchronize()
    ev = HipEvents()
    e_pre = [ev.create() for _ in range(args.steps)]
    e_kv = [ev.create() for _ in range(args.steps)]
    clocks = ClockSampler()
    clocks.start()
    t0 = time.perf_counter()
    for i in range(args.steps):
        sma.attention_bwd_raw(*call, e_pre[i], e_kv[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    window = clock_window(clocks, lambda: sma.attention_bwd_raw(*call))
    clock_info = clocks.stop()
    clock_info["untimed_seconds_after_the_timed_loop"] = window
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launches = [ev.elapsed_ms(e_pre[i], e_kv[i]) for i in range(args.steps)]
    k_avg = sum(launches) / args.steps
    for e in e_pre + e_kv:
        ev.destroy(e)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item(), "non-finite gradient"

    flops = 2.5 * metric_flops(w)
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    pairs = allowed_pairs(w)
    kernel_flops = 8.0 * d * pairs  # S, dP, dV and dK: four products over the admitted pairs
    achieved = kernel_flops / (k_avg * 1e-3) / 1e12
    kname = ("attn_bwd_dkdv_f32_kernel" if w.dtype == "f32" else
             "attn_bwd_dkdv_bf16_kb2_kernel" if d == 128 else "attn_bwd_dkdv_bf16_kernel")
    traffic = read_traffic(kname, name, kernel_source_digest(kname))
    line = {
        "metric": BWD_METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": settled, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded SplitMix64 + Box-Muller normals; dO on its own stream)",
        "clocks": clock_info, "gpu": torch.cuda.get_device_name(0),
        "config": {"workload": name, "batch": B, "heads": H, "seq_q": sq, "seq_kv": skv,
                   "head_dim": d, "causal": w.causal, "scale": w.scale, "input_dtype": w.dtype,
                   "o_and_dout": "f32", "gradients": "f32", "workspace_bytes": ws_n},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": (f"{kname}<{str(w.causal).lower()}" if kname.endswith("kb2_kernel")
                                else f"{kname}<{d},{str(w.causal).lower()}") + (",f16>" if w.dtype == "f16" else ">"),
                     "kernel_avg_ms": round(k_avg, 5), "kernel_ms": step_stats(launches),
                     "frac_at_sampled_sclk": clock_adjusted(achieved / peak, clock_info),
                     "kernel_timing": "HIP events recorded by the library around each dK/dV launch",
                     "flops_per_launch": kernel_flops,
                     "min_hbm_bytes_per_launch": dkdv_min_bytes(w)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = with_host(bwd_cpu_baseline(w, *vals, g, args.cpu_seconds))
    print(json.dumps(line), flush=True)


ROW_METRIC = "row-primitive GB/s (algorithmic bytes: inputs read once, outputs written once)"


def row_algorithmic_bytes(w) -> int:
    n = w.batch * w.rows * w.cols
    if w.op == "logsumexp_rows":
        return 4 * n + 4 * w.batch * w.rows
    if w.op in ("masked_softmax_rows", "softmax_rows_backward"):
        return 12 * n  # two inputs read, one output written
    return 8 * n


def row_oracle(w, x, mask, sample):
    """The oracle on a sample: row ids, or matrix ids for the scaled op (whole matrices)."""
    import oracle

    if w.op == "scaled_causal_softmax":
        return oracle.scaled_causal_softmax(x[sample], w.scale, w.causal)
    if w.op == "softmax_rows":
        return oracle.softmax_rows(x[sample])
    if w.op == "logsumexp_rows":
        return oracle.logsumexp_rows(x[sample])
    if w.op == "softmax_rows_backward":  # `mask` carries dy; y is the oracle's own forward
        y = oracle.softmax_rows(x[sample]).astype(np.float32)
        return oracle.softmax_rows_backward(y, mask[sample], w.scale)
    return oracle.masked_softmax_rows(x[sample], mask[sample])


def row_cpu_baseline(w, x, mask, target_s: float):
    """The oracle on a bounded random sample, scaled to GB/s of the same algorithmic bytes."""
    import oracle

    scaled = w.op == "scaled_causal_softmax"
    total = w.batch if scaled else w.batch * w.rows
    rng = np.random.default_rng(0)
    size = min(total, 1 if scaled else 256)
    sample = np.sort(rng.choice(total, size=size, replace=False)).astype(np.int64)
    passes = 0
    t0 = time.perf_counter()
    while True:
        row_oracle(w, x, mask, sample)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s or passes >= 100000:
            break
    frac = sample.size / total
    unit = "matrices" if scaled else "rows"
    return {"value": row_algorithmic_bytes(w) * frac * passes / dt / 1e9, "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{sample.size} of {total} {unit} chosen at random (seed 0), {passes} pass(es) "
                      f"in {dt:.1f} s; algorithmic bytes scaled by the sampled fraction"}


def bench_rows(args, w):
    import torch

    import gen
    import scaled_masked_attention_amd as sma

    x, mask = gen.make_row_inputs(w)
    if w.op == "softmax_rows_backward":
        mask = gen.make_row_grad(w)  # dy, passed where the masked op takes its mask
    tx = torch.from_numpy(x).to("cuda")
    tm = torch.from_numpy(mask).to("cuda") if mask is not None else None
    if w.op == "logsumexp_rows":
        out = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    else:
        out = torch.empty_like(tx)
    stream = torch.cuda.current_stream()
    lib = sma.library()
    s = stream.cuda_stream
    rows, cols = x.shape[0], x.shape[1]
    # One C call per step on an argument tuple built once (see the attention loop).
    if w.op == "softmax_rows":
        fn, call = lib.sma_softmax_rows, (tx.data_ptr(), out.data_ptr(), rows, cols, s)
    elif w.op == "logsumexp_rows":
        fn, call = lib.sma_logsumexp_rows, (tx.data_ptr(), out.data_ptr(), rows, cols, s)
    elif w.op == "masked_softmax_rows":
        fn, call = lib.sma_masked_softmax_rows, (tx.data_ptr(), tm.data_ptr(), out.data_ptr(), rows, cols, s)
    elif w.op == "softmax_rows_backward":
        ty = sma.softmax_rows(tx)  # the forward's output y, untimed
        fn, call = (lib.sma_softmax_rows_backward,
                    (ty.data_ptr(), tm.data_ptr(), out.data_ptr(), rows, cols, float(w.scale), s))
    else:
        fn, call = (lib.sma_scaled_causal_softmax,
                    (tx.data_ptr(), out.data_ptr(), w.batch, w.rows, w.cols, float(w.scale), int(w.causal), s))

    def step():
        st = fn(*call)
        if st != 0:
            raise RuntimeError(sma.status_string(st))

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents()
    e0, e1 = ev.create(), ev.create()
    clocks = ClockSampler()
    clocks.start()
    t0 = time.perf_counter()
    ev.record(e0, stream.cuda_stream)
    for _ in range(args.steps):
        step()
    ev.record(e1, stream.cuda_stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    window = clock_window(clocks, step)
    clock_info = clocks.stop()
    clock_info["untimed_seconds_after_the_timed_loop"] = window
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    k_avg = ev.elapsed_ms(e0, e1) / args.steps
    ev.destroy(e0)
    ev.destroy(e1)
    nbytes = row_algorithmic_bytes(w)
    kname = "row_softmax"
    traffic = read_traffic(kname, w.name, kernel_source_digest(kname))
    line = {
        "metric": ROW_METRIC, "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_steps": settled, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "clocks": clock_info, "gpu": torch.cuda.get_device_name(0),
        "data": ("synthetic (seeded SplitMix64 + Box-Muller normals; y = the GPU row softmax of the "
                 "scores, untimed)" if w.op == "softmax_rows_backward" else
                 "synthetic (seeded SplitMix64 + Box-Muller normals; Bernoulli mask)"),
        "config": {"workload": w.name, "op": w.op, "batch": w.batch, "rows": w.rows, "cols": w.cols,
                   "scale": w.scale, "causal": w.causal, "sigma": w.sigma, "mask_density": w.density},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (k_avg * 1e-3) / 1e9, 1),
                     "peak": HBM_GBPS, "unit": "GB/s",
                     "frac": round(nbytes / (k_avg * 1e-3) / 1e9 / HBM_GBPS, 4), "traffic": traffic,
                     "kernel": kname, "kernel_avg_ms": round(k_avg, 5),
                     "kernel_timing": "HIP events around the timed loop / steps",
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = with_host(row_cpu_baseline(w, x, mask, args.cpu_seconds))
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(gen_workloads()))
    ap.add_argument("--out-dtype", default="f32", choices=["f32", "bf16"],
                    help="element type of the attention output O (bf16: rounded to nearest even)")
    ap.add_argument("--mask-density", type=float, default=None,
                    help="apply a hard mask [1,1,Sq,Skv] admitting each pair with this probability")
    ap.add_argument("--layout", default="bhsd", choices=["bhsd", "bshd"],
                    help="memory layout of q, k, v and O: [B,H,S,d] or [B,S,H,d]")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="wall milliseconds of untimed steps before the warmup steps (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock-seconds", type=float, default=3.0,
                    help="untimed run of the step after the timed loop while engine-clock samples "
                         "are still missing (0: none; counter-collection runs use 0)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    global CLOCK_SECONDS
    CLOCK_SECONDS = args.clock_seconds
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding of the attention path is not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import scaled_masked_attention_amd as sma

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4}))
        return
    if args.workload in gen.ROW_WORKLOADS:
        bench_rows(args, gen.ROW_WORKLOADS[args.workload])
        return
    if args.workload.startswith(BWD_PREFIX):
        bench_bwd(args, gen.WORKLOADS[args.workload[len(BWD_PREFIX):]], args.workload)
        return
    w = gen.WORKLOADS[args.workload]
    vals, bits = gen.make_inputs(w)
    tq, tk, tv = to_device_inputs(vals, bits, w.dtype)
    in_dt = {"f32": sma.SMA_DTYPE_F32, "bf16": sma.SMA_DTYPE_BF16, "f16": sma.SMA_DTYPE_F16}[w.dtype]
    B, H, sq, skv, d = w.batch, w.heads, w.seq_q, w.seq_kv, w.head_dim
    lay = sma.LAYOUTS[args.layout]
    if args.layout == "bshd":  # the same data, heads of one position adjacent
        tq, tk, tv = (t.transpose(1, 2).contiguous() for t in (tq, tk, tv))
    o16 = args.out_dtype == "bf16"
    o_shape = (B, sq, H, d) if args.layout == "bshd" else (B, H, sq, d)
    out = torch.empty(o_shape, dtype=torch.bfloat16 if o16 else torch.float32, device="cuda")
    o_dt = sma.SMA_DTYPE_BF16 if o16 else sma.SMA_DTYPE_F32
    lse = torch.empty((B, H, sq), dtype=torch.float32, device="cuda")
    masked = args.mask_density is not None
    if masked:
        mask_np = gen.bernoulli_mask(w.seed, (1, 1, sq, skv), args.mask_density)
        tmask = torch.from_numpy(mask_np).to("cuda")
        ws_n = sma.library().sma_attention_fwd_masked_workspace_bytes(in_dt, B, H, sq, skv, d,
                                                                      int(w.causal), lay, 1, 1)
    else:
        ws_n = sma.workspace_bytes(in_dt, B, H, sq, skv, d, w.causal)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    plan = sma.plan(in_dt, B, H, sq, skv, d, w.causal)
    ev = HipEvents()
    call = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), lse.data_ptr(), in_dt,
            o_dt, B, H, sq, skv, d, w.scale, w.causal, ws.data_ptr(), ws_n)

    # One C call per step on argument tuples built once: the Python wrapper's own
    # per-call work would otherwise hold back the launches of a ~25 us kernel.
    lib = sma.library()
    if masked:
        fn = lib.sma_attention_fwd_masked
        base = (*call[:5], tmask.data_ptr(), 1, 1, *call[5:14], lay, *call[14:], None, sptr)
    else:
        fn = lib.sma_attention_fwd_ex
        base = (*call[:14], lay, *call[14:], None, sptr)
    no_events = base + (None, None)

    def run(events=no_events):
        st = fn(*events)
        if st != 0:
            raise RuntimeError(sma.status_string(st))

    settled = settle(run, args.settle_ms)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # Timed region. A one-kernel step gets one event between consecutive launches
    # (K + 1 events: the first before step 0), so each launch's duration is read
    # apart without bracketing it twice; a step with a split-combine kernel (or the
    # mask packing) records events around every main-kernel launch instead, so
    # that the main kernel is timed alone.
    per_launch = plan.nsplit > 1 or masked
    if per_launch:
        ev_a = [ev.create() for _ in range(args.steps)]
        ev_b = [ev.create() for _ in range(args.steps)]
        with_events = [base + (ev_a[i], ev_b[i]) for i in range(args.steps)]
    else:
        marks = [ev.create() for _ in range(args.steps + 1)]
    clocks = ClockSampler()
    clocks.start()
    t0 = time.perf_counter()
    if per_launch:
        for i in range(args.steps):
            run(with_events[i])
    else:
        ev.record(marks[0], sptr)
        for i in range(args.steps):
            run()
            ev.record(marks[i + 1], sptr)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    window = clock_window(clocks, run)
    clock_info = clocks.stop()
    clock_info["untimed_seconds_after_the_timed_loop"] = window
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    if per_launch:
        launches = [ev.elapsed_ms(ev_a[i], ev_b[i]) for i in range(args.steps)]
        events = ev_a + ev_b
    else:
        launches = [ev.elapsed_ms(marks[i], marks[i + 1]) for i in range(args.steps)]
        events = marks
    k_avg = sum(launches) / len(launches)
    for e in events:
        ev.destroy(e)
    assert torch.isfinite(out).all().item(), "non-finite output"

    value = metric_flops(w) / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    exact = 4.0 * d * allowed_pairs(w)
    achieved = exact / (k_avg * 1e-3) / 1e12
    # the committed counter passes were taken with fp32 output in [B,H,S,d]
    kfn = kernel_function(plan.kernel, d)
    traffic = None if (o16 or masked or args.layout != "bhsd") else read_traffic(kfn, w.name,
                                                                                 kernel_source_digest(kfn))
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "settle_steps": settled, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded SplitMix64 + Box-Muller normals)",
        "clocks": clock_info, "gpu": torch.cuda.get_device_name(0),
        "config": {"workload": w.name, "batch": B, "heads": H, "seq_q": sq, "seq_kv": skv,
                   "head_dim": d, "causal": w.causal, "scale": w.scale,
                   "input_dtype": w.dtype, "accumulate": "f32", "output": args.out_dtype, "lse": True,
                   "layout": args.layout, "mask_density": args.mask_density,
                   "key_splits_workspace_bytes": ws_n},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": (f"{kfn}<{d},{str(w.causal).lower()}"
                                + (",f16>" if w.dtype == "f16" else ">")),
                     "kernel_avg_ms": round(k_avg, 5),
                     "kernel_ms": step_stats(launches),
                     "frac_at_sampled_sclk": clock_adjusted(achieved / peak, clock_info),
                     "kernel_timing": ("HIP events around each main-kernel launch" if per_launch else
                                       "HIP events between consecutive launches in the timed loop"),
                     "plan": {"kernel": sma.KERNEL_NAMES[plan.kernel], "key_splits": plan.nsplit,
                              "workgroups": plan.workgroups},
                     "flops_per_launch": exact,
                     "min_hbm_bytes_per_launch": min_bytes(w, 2 if o16 else 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = with_host(masked_cpu_baseline(w, vals, mask_np, args.cpu_seconds)
                                         if masked else cpu_baseline(w, vals, args.cpu_seconds))
    print(json.dumps(line), flush=True)


def masked_cpu_baseline(w, vals, mask, target_s: float):
    """The masked oracle on a bounded random sample of whole (batch, head) slices."""
    import oracle

    bh = w.batch * w.heads
    q, k, v = (x.reshape(bh, 1, x.shape[2], x.shape[3]) for x in vals)
    order = np.random.default_rng(0).permutation(bh)
    threads = max(1, oracle.num_threads())
    n, passes = min(bh, threads), 0
    t0 = time.perf_counter()
    while True:
        ids = np.sort(order[:n])
        oracle.attention_fwd_masked(q[ids], k[ids], v[ids], mask, w.scale, w.causal)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= target_s or passes >= 1000:
            break
    return {"value": metric_flops(w) * n / bh * passes / dt / 1e12, "unit": "TFLOP/s",
            "cores": min(threads, n), "kind": "oracle",
            "sample": f"{n} of {bh} (batch, head) slices chosen at random (seed 0), every row of each, "
                      f"{passes} pass(es) in {dt:.1f} s; metric FLOPs scaled by the slice fraction"}


if __name__ == "__main__":
    main()
