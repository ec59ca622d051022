"""Benchmark of the relative-position attention hot path on one MI355X.

One step = relpos_build (rel_h/rel_w from q and the tables) followed by
relpos_attn_fwd, on the DeepEncoder global-attention workload (B=1, 12 heads,
64x64 grid, D=64, bf16), inputs resident in HBM.  The fused call
relpos_attn_fused (the same step in one launch, bias computed in the attention
kernel) is timed beside it.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps 50] [--warmup 20] [--settle-ms 300] [--workload deepencoder]
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/call + TFLOP/s (% bf16 MFMA peak), rel-pos attn B=1 12h 64x64 D=64"
PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")


def kernel_source_hash():
    csrc = os.path.join(ROOT, "relative_position_bias_relpos_amd", "csrc")
    h = hashlib.sha256()
    for name in ("relpos_attn_fwd.hip", "relpos_attn16.hip", "relpos_attn12.hip", "relpos_attn_common.hpp",
                 "relpos_device.hpp", "relpos_kernels.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def roofline(flops, nbytes, ms, traffic):
    """The attention call against the roof that bounds it: MFMA when its
    arithmetic intensity (FLOP per algorithmic byte) is above the ridge
    PEAK_TFLOPS / PEAK_HBM_GBS (about 313 FLOP/B), else HBM."""
    intensity = flops / nbytes
    common = {"kernel": "relpos_attn_fwd", "traffic": traffic, "algorithmic_bytes": nbytes,
              "flop_per_byte": round(intensity, 1)}
    if intensity >= PEAK_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS, 4), **common}
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), **common}


def load_traffic(workload):
    """HBM bytes per attention launch from committed rocprofv3 counter runs,
    only if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, d, budget_s):
    """Time the float64 oracle on whole heads of the same workload (host cores)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import relpos_oracle as O

    f64 = lambda t: t.float().numpy().astype(np.float64)
    q, k, v = d["q"], d["k"], d["v"]
    th, tw = f64(d["rel_pos_h"]), f64(d["rel_pos_w"])
    heads_total = w.B * w.heads
    done = 0
    t0 = time.perf_counter()
    while done < heads_total:
        b, h = divmod(done, w.heads)
        O.relpos_attention(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]), f64(v[b:b + 1, h:h + 1]),
                           th, tw, w.H, w.W, w.scale)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    per_call_ms = el / done * heads_total * 1e3
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": round(per_call_ms, 1), "unit": "ms/call", "cores": int(threads), "kind": "oracle",
        "sample": f"{done} of {heads_total} (batch, head) pairs of the same workload, full rows, "
                  f"float64 numpy, {el:.1f} s measured, scaled to one call",
        "cpu_model": _cpu_model(),
    }


def dense_sdpa_context(w, q, k, v, rel_h, rel_w, ours, out, rounds=3):
    """Context only: the unfused path the fused kernel replaces, on this GPU.

    Materialises the dense bias (rel_h + rel_w) as a [B, heads, N, N] tensor in
    the input dtype and runs torch's scaled_dot_product_attention pinned to the
    memory-efficient backend (no fallback to other backends).  Rounds alternate
    with librelpos's attention call; the medians are reported.
    """
    import statistics

    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    def bias():
        return (rel_h[..., :, None] + rel_w[..., None, :]).reshape(w.B, w.heads, w.N, w.N).to(q.dtype)

    def t(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    try:
        with sdpa_kernel([SDPBackend.EFFICIENT_ATTENTION]):
            mask = bias()
            sd = lambda m: F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=w.scale)
            o = sd(mask)
            torch.cuda.synchronize()
            ours_ms, sdpa_ms, full_ms = [], [], []
            for _ in range(rounds):
                ours_ms.append(t(ours, 10))
                sdpa_ms.append(t(lambda: sd(mask), 5))
                full_ms.append(t(lambda: sd(bias()), 5))
            ours()
            torch.cuda.synchronize()
            diff = (o.float() - out.float()).abs().max().item()
        del mask
        torch.cuda.empty_cache()
        med = statistics.median
        return {
            "kind": "context: dense bias + torch SDPA (memory-efficient backend), same GPU, same inputs",
            "sdpa_with_dense_mask_ms": round(med(sdpa_ms), 5),
            "bias_materialise_plus_sdpa_ms": round(med(full_ms), 5),
            "librelpos_attn_ms_same_rounds": round(med(ours_ms), 5),
            "dense_mask_bytes": w.B * w.heads * w.N * w.N * q.element_size(),
            "max_abs_diff_vs_librelpos": diff,
        }
    except Exception as e:  # backend missing on this build: report, do not fall back
        return {"kind": "context: dense bias + torch SDPA", "unavailable": f"{type(e).__name__}: {e}"[:200]}


class Clocks:
    """Graphics/memory clock and socket power of the GPU torch uses, read from
    the SMU metrics table through amdsmi.  The table is refreshed about once a
    second, so a reading reflects the last second or so: readings are taken
    after at least a second of sustained load.  Best effort: where amdsmi is
    missing or not permitted, the reason is reported and the bench goes on."""

    def __init__(self, dev_index=0):
        self.handle = None
        self.error = None
        self.readings = {}
        try:
            import amdsmi
            import torch

            self.amdsmi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self.handle = handles[0] if handles else None
            want = getattr(torch.cuda.get_device_properties(dev_index), "pci_bus_id", None)
            for h in handles:
                try:
                    if want is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == int(want):
                        self.handle = h
                        break
                except Exception:
                    pass
        except Exception as e:
            self.error = f"{type(e).__name__}: {e}"[:120]
            self.handle = None

    def read(self, label):
        if self.handle is None:
            return
        try:
            m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
            per_xcd = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and c > 0]
            num = lambda x: x if isinstance(x, (int, float)) else None
            self.readings[label] = {
                "gfxclk_mhz": num(m.get("current_gfxclk")),
                "gfxclk_per_xcd_mhz": per_xcd or None,
                "uclk_mhz": num(m.get("current_uclk")),
                "socket_power_w": num(m.get("current_socket_power")),
            }
        except Exception as e:
            self.error = f"{type(e).__name__}: {e}"[:120]

    def report(self):
        try:
            if self.handle is not None:
                self.amdsmi.amdsmi_shut_down()
        except Exception:
            pass
        if self.handle is None:
            return {"unavailable": self.error}
        out = {"source": "amdsmi SMU metrics table (refreshed about once a second)", "gfxclk_max_mhz": 2400}
        out.update(self.readings)
        if self.error:
            out["error"] = self.error
        return out


def rocm_version():
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return None


def stats_ms(xs):
    import statistics
    return {"mean": round(sum(xs) / len(xs), 5), "median": round(statistics.median(xs), 5),
            "min": round(min(xs), 5), "max": round(max(xs), 5)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before the timed ones")
    ap.add_argument("--attn-config", type=int, default=-1,
                    help="force this launch configuration of relpos_attn_fwd (relpos_attn_fwd_cfg; -1: the "
                         "library's own choice, the default) to measure the configurations against each other")
    ap.add_argument("--rounds", type=int, default=5, help="rounds of the per-call measurements")
    ap.add_argument("--calls-per-round", type=int, default=20, help="back-to-back calls per round and kind")
    ap.add_argument("--settle-ms", type=float, default=1200.0,
                    help="untimed back-to-back steps for this long (wall clock) before the warm-up, so the "
                         "GPU clock has ramped up; recorded in the output line")
    ap.add_argument("--workload", default="deepencoder")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-baseline", action="store_true",
                    help="skip the dense-bias torch SDPA context measurement")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of this many MiB (scales HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every (batch, head) is independent; see DESIGN.md for how it would shard).",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.rounds < 1 or args.calls_per_round < 1:
        print("--steps, --rounds and --calls-per-round must be >= 1, --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from relative_position_bias_relpos_amd import binding as rp
    from relative_position_bias_relpos_amd import inputs

    w = inputs.workload(args.workload)
    d = inputs.make(w, seed=0)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (d[n].to(dev) for n in ("q", "k", "v"))
    th, tw = d["rel_pos_h"].to(dev), d["rel_pos_w"].to(dev)
    H, W, scale = w.H, w.W, w.scale
    rel_h = torch.empty((w.B, w.heads, w.N, H), dtype=torch.float32, device=dev)
    rel_w = torch.empty((w.B, w.heads, w.N, W), dtype=torch.float32, device=dev)
    out = torch.empty((w.B, w.heads, w.N, w.D), dtype=torch.float32, device=dev)

    def build():
        rp.relpos_build(q, th, tw, H, W, rel_h=rel_h, rel_w=rel_w)

    cfg = None if args.attn_config < 0 else args.attn_config

    def attn():
        rp.relpos_attn_fwd(q, k, v, rel_h, rel_w, H, W, scale, out=out, config=cfg)

    def step():
        build()
        attn()

    out_fused = torch.empty_like(out)
    ws_fused = torch.empty(rp.fused_workspace_bytes(w.B, w.heads, H, W, q.dtype,
                                                    torch.cuda.get_device_properties(dev).multi_processor_count),
                           dtype=torch.uint8, device=dev)

    def fused():
        rp.relpos_attn_fused(q, k, v, th, tw, H, W, scale, out=out_fused, workspace=ws_fused)

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # C calls with their arguments marshalled once, for the per-call loops
    # (the Python binding's own cost, about 8-11 us a call, would otherwise bound
    # the shorter calls); they run the same C entry points as the binding.
    lib = rp._load()
    stream = rp._stream(q)
    common = (w.B, w.heads, H, W, w.D)
    c_build = (rp._ptr(q), rp._ptr(th), rp._ptr(tw), rp._ptr(rel_h), rp._ptr(rel_w), *common,
               rp._DT[q.dtype], stream)
    c_attn = (rp._ptr(q), rp._ptr(k), rp._ptr(v), rp._ptr(rel_h), rp._ptr(rel_w), rp._ptr(out), *common,
              float(scale), rp._DT[q.dtype], rp._DT[out.dtype])
    c_attn = (c_attn + (stream,) if cfg is None
              else c_attn + (ctypes.c_int(cfg), ctypes.c_void_p(0), 0, stream))
    attn_c = lib.relpos_attn_fwd if cfg is None else lib.relpos_attn_fwd_cfg
    c_fused = (rp._ptr(q), rp._ptr(k), rp._ptr(v), rp._ptr(th), rp._ptr(tw), rp._ptr(out_fused), *common,
               float(scale), rp._DT[q.dtype], rp._DT[out_fused.dtype], rp._ptr(ws_fused), ws_fused.numel(), stream)
    per_call = {
        "attn": lambda: attn_c(*c_attn),
        "build": lambda: lib.relpos_build(*c_build),
        "fused": lambda: lib.relpos_attn_fused(*c_fused),
    }

    def region(fn, n):
        """n back-to-back calls between two HIP events on the launch stream
        (torch's current stream, which every call here is given): ms per call."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    clk = Clocks(dev.index or 0)
    clk.read("idle")
    # Clock settle: back-to-back steps (and fused calls) for --settle-ms of wall
    # time, synchronised every 20 so the queue stays short.
    settle_calls = 0
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
            fused()
        settle_calls += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
        fused()
    torch.cuda.synchronize()
    clk.read("end_of_settle")
    mem_before = torch.cuda.memory_allocated()

    # Timed region: exactly K steps through the Python binding, back to back,
    # bracketed by synchronisations and one HIP event on each side.
    K = args.steps
    ms_step = region(step, K)

    # Per-call figures: R rounds, each with `n` back-to-back calls of every
    # kind in turn (attention, build, fused); a round's time / n is one sample.
    R, n = args.rounds, args.calls_per_round
    samples = {name: [] for name in per_call}
    for _ in range(R):
        for name, fn in per_call.items():
            samples[name].append(region(fn, n))
    clk.read("after_timed")
    attn_calls, build_calls, fused_calls = samples["attn"], samples["build"], samples["fused"]
    for name, fn in per_call.items():
        if fn() != 0:
            raise RuntimeError(f"{name} call failed")
    torch.cuda.synchronize()
    mem_after = torch.cuda.memory_allocated()

    # Host cost of one attention call (binding + argument checks + launch),
    # enqueued back to back without synchronising; and of the C call alone
    # with the arguments already marshalled.
    n_host = 200
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_host):
        attn()
    host_us = (time.perf_counter() - t0) / n_host * 1e6
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_host):
        per_call["attn"]()
    c_us = (time.perf_counter() - t0) / n_host * 1e6
    torch.cuda.synchronize()

    attn_ms = sum(attn_calls) / R
    build_ms = sum(build_calls) / R
    fused_ms = sum(fused_calls) / R

    # Output check on sampled rows of the last call (two heads) against the oracle
    # is left to the test-suite; here only finiteness is asserted.
    finite = bool(torch.isfinite(out).all().item())
    fused_diff = (out_fused - out).abs().max().item()

    flops = w.flops
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    step_tflops = flops / (ms_step * 1e-3) / 1e12
    isz = 2
    build_bytes = (w.B * w.heads * w.N * w.D * isz + ((2 * H - 1) + (2 * W - 1)) * w.D * isz
                   + w.B * w.heads * w.N * (H + W) * 4)
    attn_bytes = (3 * w.B * w.heads * w.N * w.D * isz + w.B * w.heads * w.N * (H + W) * 4
                  + w.B * w.heads * w.N * w.D * 4)
    traffic = load_traffic(w.name)

    rec = {
        "metric": METRIC,
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal draws, bf16-rounded; no trained weights)",
        "config": {
            "workload": f"{w.name}: B={w.B} heads={w.heads} H={H} W={W} D={w.D} {w.dtype}, "
                        f"step = relpos_build + relpos_attn_fwd",
            "B": w.B, "heads": w.heads, "H": H, "W": W, "D": w.D, "seq_len": w.N,
            "global_batch": w.B, "parallelism": "none (1 GPU)",
        },
        "attn_launch_config": (cfg if cfg is not None else
                               rp.attn_config(w.B, w.heads, H, W, q.dtype,
                                              torch.cuda.get_device_properties(dev).multi_processor_count)),
        "attn_ms_per_call": round(attn_ms, 5),
        "attn_ms_per_call_stats": stats_ms(attn_calls),
        "attn_tflops": round(attn_tflops, 2),
        "attn_tflops_at_median": round(flops / (stats_ms(attn_calls)["median"] * 1e-3) / 1e12, 2),
        "attn_pct_bf16_peak": round(100.0 * attn_tflops / PEAK_TFLOPS, 2),
        "build_ms_per_call": round(build_ms, 5),
        "build_ms_per_call_stats": stats_ms(build_calls),
        "build_gbs": round(build_bytes / (build_ms * 1e-3) / 1e9, 1),
        "timing": "ms_per_step: the K steps back to back through the Python binding, one HIP event on "
                  "each side (launch stream); *_ms_per_call: R rounds of n back-to-back C calls of each "
                  "kind in turn, one event pair per round, a sample = round time / n; mean over all calls, "
                  "median/min/max over the rounds",
        "rounds": {"R": R, "calls_per_round": n},
        "settle": {"ms": args.settle_ms, "calls": settle_calls,
                   "what": "untimed back-to-back steps and fused calls before the warm-up (clock ramp)"},
        "clocks": clk.report(),
        "rocm": rocm_version(),
        "torch_hip": torch.version.hip,
        "host_us_per_attn_call": {"python_binding": round(host_us, 2), "c_call_only": round(c_us, 2)},
        "roofline": roofline(flops, attn_bytes, attn_ms, traffic),
        "fused": {
            "call": "relpos_attn_fused (bias rows computed in the attention kernel; no rel_h/rel_w tensors)",
            "ms_per_call": round(fused_ms, 5),
            "ms_per_call_stats": stats_ms(fused_calls),
            "tflops": round(flops / (fused_ms * 1e-3) / 1e12, 2),
            "pct_bf16_peak": round(100.0 * flops / (fused_ms * 1e-3) / 1e12 / PEAK_TFLOPS, 2),
            "workspace_bytes": ws_fused.numel(),
            "max_abs_diff_vs_step": fused_diff,
        },
        "output_finite": finite,
        "allocated_delta_bytes": mem_after - mem_before,
        "gpu": torch.cuda.get_device_name(dev),
    }
    if not args.no_dense_baseline:
        rec["dense_bias_sdpa"] = dense_sdpa_context(w, q, k, v, rel_h, rel_w, attn, out)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, d, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
