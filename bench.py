"""Benchmark: attention forward TFLOP/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill8k]
                    [--no-cpu-baseline]

A step is one fa_fwd call (the whole forward: every query tile, head and
batch) over the workload's seeded synthetic bf16 inputs, which are resident
in device memory before timing starts. Timing uses HIP events recorded on the
stream the kernel runs on (torch's current stream), bracketed by device
synchronisations. Prints ONE JSON line.

Default workload: B=1, H=32, N=8192, d=128, causal (LLM-prefill shape), the
configuration the MFMA-utilisation target is quoted on. FLOPs per step are
4*N*N*d*H*B halved for causal; for a banded workload, 4*d*H*B times the
exact number of visible (query, key) pairs. The CPU baseline is the float64 oracle timed
on the host on a bounded sample of the same workload (whole heads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "attention fwd TFLOPS (bf16) and % of MFMA peak, N=1025..8192, d=128"
METRIC_BWD = "attention bwd TFLOPS (bf16) and % of MFMA peak"
METRIC_DECODE = "attention decode HBM GB/s (bf16, one query per head)"
METRIC_MX8 = "attention fwd TFLOPS (FP8 E4M3, MX block-scaled) and % of MFMA peak"
PEAK_FP8_TFLOPS = 5000.0           # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
PEAK_SCLK_MHZ = 2400.0             # the shader clock that peak is quoted at
KERNEL_SOURCES = [os.path.join(ROOT, "aware_attention_amd", "csrc", f)
                  for f in ("fa_fwd_kernel.hpp", "fa_api.hip")]
KERNEL_SOURCES_MX8 = [os.path.join(ROOT, "aware_attention_amd", "csrc", f)
                      for f in ("fa_mx8_kernel.hpp", "fa_mx8_api.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{workload}.txt")


class ClockSampler:
    """Samples the GPU's shader (GFX) clock through the amdsmi library in a
    background thread, with host timestamps. The SMU refreshes these metrics
    about once a second (measured on MI355X: the readings stay constant for
    ~1 s), so a reading is only meaningful once a refresh has happened under
    load; `sustained` reports the last refresh seen in a window. Silent (no
    samples) where amdsmi or the metric is unavailable."""

    def __init__(self, period_s: float = 0.005):
        import threading
        self.period_s = period_s
        self.samples = []          # (perf_counter, MHz)
        self.source = None
        self._stop = threading.Event()
        self._thread = None
        self._read = self._open()

    def _open(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
        except Exception:   # noqa: BLE001 - no SMI library or no access: no samples
            return None
        if not handles:
            return None
        handle = handles[0]
        if len(handles) > 1:   # the device torch uses, by PCI bus
            try:
                import torch
                bus = torch.cuda.get_device_properties(0).pci_bus_id
                for h in handles:
                    if int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                        handle = h
            except Exception:   # noqa: BLE001
                pass

        def from_metrics():
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            vals = m.get("current_gfxclks")
            if isinstance(vals, (list, tuple)):
                vals = [float(x) for x in vals if isinstance(x, (int, float)) and 0 < x < 10000]
                if vals:
                    return sum(vals) / len(vals)
            x = m.get("current_gfxclk")
            return float(x) if isinstance(x, (int, float)) and 0 < x < 10000 else None

        def from_clock_info():
            x = amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX).get("clk")
            return float(x) if isinstance(x, (int, float)) and 0 < x < 10000 else None

        for name, fn in (("amdsmi gpu_metrics current_gfxclks (mean over XCDs)", from_metrics),
                         ("amdsmi clock_info GFX", from_clock_info)):
            try:
                if fn() is not None:
                    self.source = name
                    return fn
            except Exception:   # noqa: BLE001
                continue
        return None

    def start(self):
        import threading
        if self._read is None:
            return self

        def run():
            while not self._stop.is_set():
                try:
                    mhz = self._read()
                except Exception:   # noqa: BLE001
                    mhz = None
                if mhz is not None:
                    self.samples.append((time.perf_counter(), mhz))
                self._stop.wait(self.period_s)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def sustained(self, t_load: float, t1: float):
        """The clock of the last metrics refresh observed in (t_load, t1]: a
        reading that differs from the one current when the load started at
        t_load. Returns (MHz, seconds before t1 it was first seen), or
        (None, None) if no refresh happened under load."""
        before = [mhz for t, mhz in self.samples if t <= t_load]
        prev = before[-1] if before else None
        last = None
        for t, mhz in self.samples:
            if t_load < t <= t1 and mhz != prev:
                last, prev = (mhz, t), mhz
        if last is None:
            return None, None
        return last[0], t1 - last[1]


def host_cores() -> dict:
    """Host CPU figures for the baseline: logical CPUs, the affinity set and the
    threads the BLAS library runs with."""
    info = {"cpu_count": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except AttributeError:
        info["affinity"] = None
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = max([i.get("num_threads", 1) for i in threadpool_info()
                                    if i.get("user_api") == "blas"] or [None])
    except Exception:   # noqa: BLE001
        info["blas_threads"] = None
    return info


def kernel_digest(fp8: bool = False) -> str:
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES_MX8 if fp8 else KERNEL_SOURCES):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, fp8: bool = False):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if current."""
    path = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    if kv.get("kernel_digest") != kernel_digest(fp8):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl: dict, budget_s: float = 12.0):
    """Time the float64 oracle on whole heads of the workload until budget_s is used."""
    from oracle import attention
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    spec = wl["spec"]
    flops, heads, t0 = 0.0, 0, time.perf_counter()
    if isinstance(spec, W.Dense):
        pairs = [(b, h) for b in range(spec.B) for h in range(spec.H)]
        per_head = spec.flops() / (spec.B * spec.H)
        for b, h in pairs:
            f64 = lambda x: W.bf16_bits_to_f32(x[b, :, h]).astype(np.float64)  # noqa: E731
            if "mask" in wl:   # padded batch: the valid tokens of row b (right padding)
                n = int(wl["mask"][b].sum())
                attention(f64(wl["q"])[:n], f64(wl["k"])[:n], f64(wl["v"])[:n], spec.scale,
                          spec.causal)
                flops += 4.0 * n * n * spec.d / (2 if spec.causal else 1)
            elif spec.local is not None:   # anchors + local window on the token map
                from oracle import attention_local
                attention_local(f64(wl["q"]), f64(wl["k"]), f64(wl["v"]), spec.scale,
                                *spec.local, spec.causal)
                flops += per_head
            else:
                attention(f64(wl["q"]), f64(wl["k"]), f64(wl["v"]), spec.scale, spec.causal,
                          window=spec.window)
                flops += per_head
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        sample = f"{heads} of {len(pairs)} (batch, head) pairs, all {spec.N} rows each"
    else:
        cu = wl["cu_seqlens"]
        for s in range(spec.num_seqs):
            a, b = int(cu[s]), int(cu[s + 1])
            for h in range(spec.H):
                f64 = lambda x: W.bf16_bits_to_f32(x[a:b, h]).astype(np.float64)  # noqa: E731
                attention(f64(wl["q"]), f64(wl["k"]), f64(wl["v"]), spec.scale, spec.causal)
                flops += W.varlen_flops([b - a], 1, spec.d, spec.causal)
                heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        sample = f"{heads} (sequence, head) pairs of {spec.num_seqs * spec.H}"
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": sample + f"; float64 numpy, {dt:.1f} s", **host_cores()}


def cpu_baseline_bwd(wl: dict, budget_s: float = 12.0):
    """Time the float64 backward oracle on whole heads of the workload until budget_s is used."""
    from oracle import attention_backward
    threads = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        pass
    spec = wl["spec"]
    do = W.make_dense(spec.B, spec.N, spec.H, spec.d, spec.seed + 1)[0]
    per_head = 2.5 * spec.flops() / (spec.B * spec.H)
    flops, heads, t0 = 0.0, 0, time.perf_counter()
    for b in range(spec.B):
        for h in range(spec.H):
            f64 = lambda x: W.bf16_bits_to_f32(x[b, :, h]).astype(np.float64)  # noqa: E731
            if "mask" in wl:   # padded batch: the valid tokens of row b (right padding)
                n = int(wl["mask"][b].sum())
                attention_backward(f64(wl["q"])[:n], f64(wl["k"])[:n], f64(wl["v"])[:n],
                                   f64(do)[:n], spec.scale, spec.causal)
                flops += 2.5 * 4.0 * n * n * spec.d / (2 if spec.causal else 1)
            elif spec.local is not None:   # anchors + local window on the token map
                from oracle import attention_local_backward
                attention_local_backward(f64(wl["q"]), f64(wl["k"]), f64(wl["v"]), f64(do),
                                         spec.scale, *spec.local, spec.causal)
                flops += per_head
            else:
                attention_backward(f64(wl["q"]), f64(wl["k"]), f64(wl["v"]), f64(do), spec.scale,
                                   spec.causal, window=spec.window)
                flops += per_head
            heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": f"{heads} of {spec.B * spec.H} (batch, head) pairs, "
                                        f"backward, float64 numpy, {dt:.1f} s", **host_cores()}


def cpu_baseline_decode(wl: dict, budget_s: float = 12.0):
    """Time the float64 oracle on whole (batch, head) decode rows until budget_s is used;
    reported in GB/s of the same compulsory bytes."""
    from oracle import attention
    spec = wl["spec"]
    per_head = spec.bytes_compulsory() / (spec.B * spec.H)
    done, t0 = 0, time.perf_counter()
    for b in range(spec.B):
        for h in range(spec.H):
            f64 = lambda x: W.bf16_bits_to_f32(x[b, :, h]).astype(np.float64)  # noqa: E731
            attention(f64(wl["q"]), f64(wl["k"]), f64(wl["v"]), spec.scale)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    hc = host_cores()
    return {"value": done * per_head / dt / 1e9, "unit": "GB/s",
            "cores": int(hc["blas_threads"] or hc["cpu_count"] or 1),
            "kind": "oracle", "sample": f"{done} of {spec.B * spec.H} (batch, head) rows, "
                                        f"float64 numpy, {dt:.1f} s", **hc}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--min-warmup-s", type=float, default=1.2,
                    help="after the --warmup steps, keep running untimed steps until the "
                         "warm-up has lasted this long: the shader clock settles under load "
                         "over tens of milliseconds (the first launches run up to 15%% slower), "
                         "and the SMU's clock reading refreshes about once a second")
    ap.add_argument("--workload", default="prefill8k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (fa_bwd: dQ, dK, dV from a seeded dO) instead of "
                         "the forward; FLOPs counted as 2.5x the forward's (five products)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the FP8 forward (fa_fwd_mx8) on the workload's operands quantised "
                         "to the MX block-scaled format beforehand (d = 128 dense workloads)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device-to-device copy of 1 GiB (3 times), to "
                         "calibrate HBM byte counters against a known size")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the attention "
              f"forward shards over batch and heads with no exchange, so per-GPU throughput is "
              f"the one-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch
    import aware_attention_amd as aa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = 1 << 30
        src_t = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n,
                          "launches": 3}), flush=True)
        return
    wl = W.make_workload(args.workload)
    spec = wl["spec"]
    to_dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    q, k, v = to_dev(wl["q"]), to_dev(wl["k"]), to_dev(wl["v"])
    o = torch.empty_like(q)
    decode = isinstance(spec, W.Decode)
    if decode:
        if args.backward:
            print("--backward is measured on equal-length workloads", file=sys.stderr)
            sys.exit(2)
        lse = torch.empty((spec.B, spec.H), dtype=torch.float32, device="cuda")
        flops = spec.flops()
        config = {"workload": args.workload, "B": spec.B, "H": spec.H, "Nk": spec.Nk, "d": spec.d,
                  "queries_per_head": 1}
        ws = torch.empty(aa._lib.decode_workspace_bytes(spec.B, spec.Nk, spec.H, spec.d),
                         dtype=torch.uint8, device="cuda")

        def step():
            aa.fa_decode(q, k, v, softmax_scale=spec.scale, out=o, lse=lse, workspace=ws)
    elif isinstance(spec, W.Dense):
        lse = torch.empty((spec.B, spec.H, spec.N), dtype=torch.float32, device="cuda")
        flops = spec.flops()
        config = {"workload": args.workload, "B": spec.B, "H": spec.H, "N": spec.N, "d": spec.d,
                  "causal": spec.causal}
        if spec.window is not None:
            config["window"] = list(spec.window)
        kpm = None
        if "mask" in wl:
            kpm = torch.from_numpy(wl["mask"]).cuda()
            config["key_padding_mask"] = "right padding, lengths U{256..N}"
            config["valid_tokens"] = int(wl["mask"].sum())

        def step():
            aa.fa_fwd(q, k, v, softmax_scale=spec.scale, causal=spec.causal, out=o, lse=lse,
                      window=spec.window, key_padding_mask=kpm)

        if spec.local is not None:
            G, map_w, wr, wc = spec.local
            config["local"] = {"n_global": G, "map_w": map_w, "window": [wr, wc]}

            def step():  # noqa: F811 - the local-window entry point
                aa.fa_fwd_local(q, k, v, G, map_w, (wr, wc), softmax_scale=spec.scale,
                                causal=spec.causal, out=o, lse=lse)

        if args.fp8:
            if spec.d != 128 or spec.window is not None or spec.local is not None or "mask" in wl:
                print("--fp8 runs dense d = 128 workloads (causal or not)", file=sys.stderr)
                sys.exit(2)
            qq, qe = aa.mx8_quantize_qk(q)
            kq, ke = aa.mx8_quantize_qk(k)
            vt, vte = aa.mx8_quantize_v(v)
            torch.cuda.synchronize()
            tq0 = time.perf_counter()
            for _ in range(10):
                aa.mx8_quantize_qk(q, out=qq, exponents=qe)
                aa.mx8_quantize_qk(k, out=kq, exponents=ke)
                aa.mx8_quantize_v(v)
            torch.cuda.synchronize()
            quant_ms = (time.perf_counter() - tq0) / 10 * 1e3
            config["operands"] = "MX FP8: E4M3 elements, one E8M0 exponent per 32 (V transposed)"

            def step():  # noqa: F811 - the timed step is the FP8 forward
                aa.fa_fwd_mx8(qq, qe, kq, ke, vt, vte, softmax_scale=spec.scale,
                              causal=spec.causal, out=o, lse=lse)
        if args.backward:
            step()
            do = to_dev(W.make_dense(spec.B, spec.N, spec.H, spec.d, spec.seed + 1)[0])
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            delta = torch.empty_like(lse)
            flops = 2.5 * flops

            def step():  # noqa: F811 - the timed step is the backward
                aa.fa_bwd(q, k, v, o, lse, do, softmax_scale=spec.scale, causal=spec.causal,
                          dq=dq, dk=dk, dv=dv, delta=delta, window=spec.window,
                          key_padding_mask=kpm, local=spec.local)
    else:
        if args.backward:
            print("--backward is measured on equal-length workloads", file=sys.stderr)
            sys.exit(2)
        cu = torch.from_numpy(wl["cu_seqlens"]).cuda()
        total = q.shape[0]
        lse = torch.empty((spec.H, total), dtype=torch.float32, device="cuda")
        flops = W.varlen_flops(wl["lengths"], spec.H, spec.d, spec.causal)
        config = {"workload": args.workload, "num_seqs": spec.num_seqs, "total": int(total),
                  "max_seqlen": wl["max_seqlen"], "H": spec.H, "d": spec.d, "causal": spec.causal}

        def step():
            aa.fa_fwd_varlen(q, k, v, cu, wl["max_seqlen"], softmax_scale=spec.scale,
                             causal=spec.causal, out=o, lse=lse)

    clock = ClockSampler().start()
    tw = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    warm_launches = args.warmup
    while time.perf_counter() - tw < args.min_warmup_s:
        for _ in range(8):
            step()
        warm_launches += 8
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - tw
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    clock.stop()
    sclk, sclk_age = clock.sustained(tw + 0.05, t1)
    sclk_info = {"sclk_mhz": None if sclk is None else round(sclk, 1),
                 "sclk_age_s": None if sclk_age is None else round(sclk_age, 3),
                 "sclk_source": clock.source}
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    # rows that see no key (padding positions, empty band rows) have L = -inf
    assert not torch.isnan(lse).any() and not torch.isposinf(lse).any(), \
        "NaN or +inf log-sum-exp in the timed output"

    traffic = read_traffic(args.workload + ("_bwd" if args.backward else "")
                           + ("_fp8" if args.fp8 else ""), args.fp8)
    if decode:
        gbs = spec.bytes_compulsory() / (ms_per_step * 1e-3) / 1e9
        out = {
            "metric": METRIC_DECODE, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16, shapes of the workload)", "config": config,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic},
            "tflops": round(tflops, 2), "wall_s_timed": round(wall, 4),
            "warmup_launches": warm_launches, "warmup_s": round(warm_s, 3), **sclk_info,
        }
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_decode(wl)
        print(json.dumps(out), flush=True)
        return
    fp8 = getattr(args, "fp8", False)
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    out = {
        "metric": METRIC_BWD if args.backward else (METRIC_MX8 if fp8 else METRIC),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3-mx" if fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) bf16, shapes of the workload)",
        "config": config,
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic,
        },
        "kernel_digest": kernel_digest(fp8),
        "wall_s_timed": round(wall, 4),
        "warmup_launches": warm_launches,
        "warmup_s": round(warm_s, 3),
        **sclk_info,
    }
    if fp8:
        out["quantize_ms"] = round(quant_ms, 4)
    if sclk is not None:   # the dense MFMA peak scales with the shader clock (quoted at 2.4 GHz)
        peak_at = peak * sclk / PEAK_SCLK_MHZ
        out["peak_at_sclk_tflops"] = round(peak_at, 1)
        out["frac_at_sclk"] = round(tflops / peak_at, 4)
    if args.backward:
        config["pass"] = "backward"
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_bwd(wl) if args.backward else cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
