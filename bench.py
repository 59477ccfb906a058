"""Benchmark: one fwd+bwd step of the routed MoE SwiGLU layer on one MI355X.

A step is one pass of the whole path over one synthetic batch: route, permute,
expert FFN (grouped GEMMs), combine, backward (all gradients) and the
balancing statistic -- the six C-ABI calls, back to back on one stream.
Inputs are resident in HBM before the timed region starts.

The default workload is the largest single-GPU one: 32768 tokens, d_model
1536, 4 routed experts top-2 plus one shared expert, SwiGLU width 3072, f16.

Prints ONE JSON line (rank 0, N = 1).  The timed region is K steps, each after
a 1 GiB scratch write that evicts the 256 MB last-level cache and the L2s (so
no operand is left on chip), with hipEvents on the stream around every step;
``value`` = T / the median of those per-step times (tokens/s) and
``ms_per_step`` that median.  Plus
  roofline      -- the dominant kernel's algorithmic FLOPs per launch over its
                   average launch time (hipEvents recorded around that kernel
                   inside the timed region), against the MFMA peak of its
                   dtype, and its measured HBM bytes per launch ("traffic")
                   when a counter summary of the current kernel sources exists
                   under profiles/ (else null);
  cpu_baseline  -- the fp64 numpy oracle timed on the host on a bounded
                   sample of the same workload, with the BLAS library, its
                   threads and a single-thread pass of the tiny workload;
  step_ms       -- the flushed per-step distribution (median / p10 / p90) and,
                   after the timed region, the same with the caches warm.
Per-kernel times go to stderr.

--traffic-calibration runs only a plain streaming kernel of known size (an
elementwise negation over 1 GiB of float32: 1 GiB read, 1 GiB written), the
reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import moe_inputs as MI  # noqa: E402

METRIC = "MoE FFN layer tokens/s fwd+bwd; grouped-GEMM TFLOP/s as % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3, "mxfp8": 5000.0}
HBM_PEAK_GBS = 8000.0


def kernel_flops(wl):
    """Algorithmic FLOPs per launch of each GEMM kernel (real rows only)."""
    A = wl.T * wl.k
    d, I = wl.d, wl.I
    f = {
        "gemm_gate_up_swiglu": 2.0 * A * d * 2 * I,
        "gemm_down": 2.0 * A * I * d,
        "gemm_down_dgrad_swiglu": 2.0 * A * d * I,
        "gemm_wgrad_down": 2.0 * A * d * I,
        "gemm_gate_up_dgrad": 2.0 * A * 2 * I * d,
        "gemm_wgrad_gate_up": 2.0 * A * 2 * I * d,
        "gemm_router_dx": 2.0 * wl.T * wl.E * d,
        "gemm_wgrad_router": 2.0 * wl.T * wl.E * d,
    }
    if wl.n_shared:
        NI = wl.n_shared * wl.I_shared
        f.update({
            "gemm_gate_up_swiglu_shared": 2.0 * wl.T * d * 2 * NI,
            "gemm_down_shared": 2.0 * wl.T * NI * d,
            "gemm_down_dgrad_swiglu_shared": 2.0 * wl.T * d * NI,
            "gemm_wgrad_down_shared": 2.0 * wl.T * d * NI,
            "gemm_gate_up_dgrad_shared": 2.0 * wl.T * 2 * NI * d,
            "gemm_wgrad_gate_up_shared": 2.0 * wl.T * 2 * NI * d,
        })
    return f


def expert_flops(wl):
    return 18.0 * wl.d * (wl.T * wl.k * wl.I + wl.T * wl.n_shared * wl.I_shared)


def make_layer(wl, device="cuda", mx_path="fused"):
    """mx_path (MX-fp8 experts): "fused" = a fused-only plan (x gathered on
    load, the forward's saved codes, H and the backward's [dG | dU] and
    dY_perm kept only as codes, the smaller workspace); "unfused" = x_perm
    formed and quantised, every act-dtype intermediate stored, the backward
    quantising the weights and H itself."""
    from mixture_experts_ffn_wave_amd import MoELayer, Plan
    inp = MI.make_inputs(wl)
    dev = {k: (v.to(device) if v is not None else None) for k, v in inp.items()}
    mx = wl.expert_dtype == "mxfp8"
    plan = Plan(wl.T, wl.d, wl.E, wl.k, wl.I, n_shared=wl.n_shared, d_ff_shared=wl.I_shared,
                renorm=wl.renorm, has_router_bias=dev["bias"] is not None, dtype=wl.torch_dtype,
                aux_coef=wl.aux_coef, expert_dtype=wl.expert_dtype or None,
                mx_fused=mx and mx_path == "fused")
    layer = MoELayer(plan, device)
    if mx and mx_path == "unfused":
        layer.mx_gather = False
        layer.mx_save = False
        layer.store_h = True
        layer.keep_intermediates()
    layer.set_params(dev["x"], dev["w_router"], dev["w_gate_up"], dev["w_down"], bias=dev["bias"],
                     ws_gate_up=dev.get("ws_gate_up"), ws_down=dev.get("ws_down"))
    return layer, dev


# probe name of a GEMM launch -> prefix of its kernel symbol (dtype and tile follow)
KERNEL_SYMBOL = {
    "gemm_gate_up_swiglu": "moe_gemm_gate_up_swiglu",
    "gemm_down": "moe_gemm_down",
    "gemm_down_dgrad_swiglu": "moe_gemm_down_dgrad_swiglu",
    "gemm_gate_up_dgrad": "moe_gemm_gate_up_dgrad",
    "gemm_wgrad_down": "moe_wgrad_down",
    "gemm_wgrad_gate_up": "moe_wgrad_gate_up",
    "gemm_router_dx": "moe_gemm_router_dx_f32out",
    "gemm_wgrad_router": "moe_wgrad_router_f32out",
}
CALIBRATION_BYTES = 1 << 30


def kernel_source_hash():
    """sha256 over the HIP/C++ sources, in name order: counter summaries taken
    from other sources do not describe the kernels that run now."""
    d = os.path.join(ROOT, "mixture_experts_ffn_wave_amd", "csrc")
    h = hashlib.sha256()
    for n in sorted(os.listdir(d)):
        if n.endswith((".hip", ".cpp", ".h")):
            h.update(n.encode())
            with open(os.path.join(d, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def traffic_per_launch(wl, probe_name):
    """HBM bytes per launch of one kernel from profiles/traffic_<workload>.md,
    or None (no summary, other sources, or no unique kernel row)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl.name}.md")
    sym = KERNEL_SYMBOL.get(probe_name[:-len("_shared")] if probe_name.endswith("_shared") else probe_name)
    if sym is None or not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source sha256: `([0-9a-f]{64})`", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    # a row is a call site: the kernel symbol (dtype, tile, "pp" for the
    # ping-pong tiles), and "(routed)" / "(shared)" where one symbol ran with
    # both the routed and the shared experts' grids
    pat = re.compile(r"^\| `" + re.escape(sym) + r"(?:_f32out)?_" + wl.dtype + r"_\d+x\d+(?:pp)?(?: \((\w+)\))?` \|"
                     r"[^|]*\|[^|]*\|[^|]*\| *([0-9.]+) *\|", re.M)
    rows = pat.findall(text)
    site = "shared" if probe_name.endswith("_shared") else "routed"
    labelled = [v for lab, v in rows if lab == site]
    plain = [v for lab, v in rows if not lab]
    pick = labelled if labelled else plain
    return float(pick[0]) if len(pick) == 1 else None


def traffic_calibration():
    n = CALIBRATION_BYTES // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "neg", "bytes_read": CALIBRATION_BYTES, "bytes_written": CALIBRATION_BYTES}),
          flush=True)


def per_kernel_times(layer, dy, names, steps=3):
    """Average launch time (ms) of every kernel, one probe pass per name."""
    from mixture_experts_ffn_wave_amd import probe_enable, probe_read
    out = {}
    for n in names:
        probe_enable(layer.plan, n, 64)
        for _ in range(steps):
            layer.step(dy)
        ms, cnt = probe_read(layer.plan)
        probe_enable(layer.plan, n, 0)
        if cnt:
            out[n] = (ms / cnt, cnt // steps)
    return out


def step_distribution(layer, dy, steps, flush_bytes=0):
    """Per-step times in ms (hipEvents on the current stream around each step);
    with flush_bytes, a scratch buffer of that size is written before every
    step (outside the events) to evict the caches."""
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda") if flush_bytes else None
    times = []
    for i in range(steps):
        if scratch is not None:
            scratch.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.step(dy)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    times.sort()
    q = lambda f: times[min(len(times) - 1, int(round(f * (len(times) - 1))))]
    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9), "steps": len(times)}


def _oracle_pass(O, wl, f):
    fwd = O.layer_forward(f["x"], f["w_router"], f["w_gate_up"], f["w_down"], top_k=wl.k, renorm=wl.renorm,
                          bias=f["bias"], ws_gate_up=f.get("ws_gate_up"), ws_down=f.get("ws_down"))
    O.layer_backward(fwd, f["dy"], aux_coef=wl.aux_coef)
    O.aux_statistics(fwd["p"], fwd["counts"], wl.k)


def cpu_baseline(wl, budget_s=12.0, sample_tokens=2048):
    """The fp64 oracle, untuned, on the host cores, on a bounded sample of the
    workload: whole fwd+bwd+aux passes over the first ``sample_tokens`` tokens
    of the same synthetic batch (same d, experts, k, inner widths, shared
    experts and router bias; the routing is the sample's own) until ~budget_s
    have run, reported as tokens/s.  Also the BLAS library and its thread
    count, and one pass of the tiny f32 workload on one BLAS thread."""
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    inp = MI.make_inputs(wl)
    Ts = min(wl.T, sample_tokens)
    f = {k: (MI.to_f64(v[:Ts]) if k in ("x", "dy") else MI.to_f64(v)) for k, v in inp.items()}
    swl = wl.with_(T=Ts)
    runs, t0 = 0, time.perf_counter()
    while True:
        _oracle_pass(O, swl, f)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 50:
            break
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = blas[0]["num_threads"] if blas else 1
    vendor = f"{blas[0]['internal_api']} {blas[0].get('version', '')}".strip() if blas else "none"
    tiny = MI.WORKLOADS[MI.TINY]
    ft = {k: MI.to_f64(v) for k, v in MI.make_inputs(tiny).items()}
    with threadpool_limits(limits=1, user_api="blas"):
        t1 = time.perf_counter()
        _oracle_pass(O, tiny, ft)
        tiny_s = time.perf_counter() - t1
    return {"value": Ts * runs / el, "unit": "tokens/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"{runs} fwd+bwd+aux pass(es) of the first {Ts} of {wl.T} tokens of the {wl.name} "
                      f"workload in float64 numpy ({el:.1f} s wall)",
            "blas": vendor, "blas_threads": threads, "host_cores": cores,
            "single_core_tiny_s": tiny_s, "single_core_tiny_workload": tiny.name}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=MI.LARGEST)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--traffic-calibration", action="store_true")
    ap.add_argument("--balance-gamma", type=float, default=0.0,
                    help="route with aux-loss-free balancing, the selection bias updated by this step "
                         "size at the end of every step (0 = the plain router)")
    ap.add_argument("--mx-path", choices=("fused", "unfused"), default="fused",
                    help="MX-fp8 workloads: the fused path (default) or every intermediate formed, for comparison")
    ap.add_argument("--filler-frac", type=float, default=0.0,
                    help="mark about this share of the tokens as fillers (seeded runs) and take the balancing "
                         "statistic over the real tokens only (0 = every token real)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the MoE layer path runs on one GPU only (no collectives, no sharding); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.traffic_calibration:
        traffic_calibration()
        return
    wl = MI.WORKLOADS[args.workload]
    torch.cuda.init()
    layer, dev = make_layer(wl, mx_path=args.mx_path)
    if args.balance_gamma > 0:
        layer.enable_balancing(gamma=args.balance_gamma)
    if args.filler_frac > 0:
        layer.set_real_mask(torch.from_numpy(MI.real_token_mask(wl.T, args.filler_frac)).to(dev["x"].device))
    dy = dev["dy"]
    print(f"[bench] workload {wl.name}: {MI.describe(wl)}", file=sys.stderr, flush=True)

    flops = kernel_flops(wl)
    for _ in range(max(args.warmup, 1)):
        layer.step(dy)
    torch.cuda.synchronize()
    # device memory the inputs, the layer's buffers and its workspace took at
    # their peak (torch's allocator), before the cache-flush buffer below
    peak_alloc = torch.cuda.max_memory_allocated()

    from mixture_experts_ffn_wave_amd import kernel_names, probe_enable, probe_read
    breakdown = {}
    if not args.no_breakdown:
        breakdown = per_kernel_times(layer, dy, kernel_names())
        for n, (ms, per) in sorted(breakdown.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
            extra = ""
            if n in flops:
                extra = f"  {flops[n] / (ms * 1e-3) / 1e12:8.1f} TFLOP/s"
            print(f"[bench] {n:34s} {ms * 1e3:9.1f} us x{per}{extra}", file=sys.stderr, flush=True)
    gemms = {n: v for n, v in breakdown.items() if n in flops}
    expert_gemms = {n: v for n, v in gemms.items() if "router" not in n}
    dominant = max(gemms, key=lambda n: gemms[n][0] * gemms[n][1]) if gemms else "gemm_gate_up_swiglu"

    # ---- timed region: K steps, each after a 1 GiB scratch write that evicts
    # the 256 MB last-level cache and the L2s, so no operand is left on chip;
    # per-step hipEvents on the stream around each step, and the dominant
    # kernel's launches bracketed by hipEvents on the stream it runs on
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    probe_enable(layer.plan, dominant, args.steps * 4)
    torch.cuda.synchronize()
    times = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        scratch.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.step(dy)
        e1.record()
        times.append((e0, e1))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_total, launches = probe_read(layer.plan)
    probe_enable(layer.plan, dominant, 0)
    del scratch
    step_ms = sorted(a.elapsed_time(b) for a, b in times)
    q = lambda f: step_ms[min(len(step_ms) - 1, int(round(f * (len(step_ms) - 1))))]
    flushed = {"median": q(0.5), "p10": q(0.1), "p90": q(0.9), "steps": len(step_ms)}

    ms_step = flushed["median"]
    avg_ms = ms_total / max(launches, 1)
    achieved = flops[dominant] / (avg_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.expert_dtype or wl.dtype]
    gemm_ms = sum(ms * per for ms, per in expert_gemms.values())
    result = {
        "metric": METRIC,
        "value": wl.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # expert GEMMs in MX-fp8 (e4m3 payload, f32 accumulate), the rest in the layer dtype
        "dtype": "mxfp8_e4m3+" + wl.dtype if wl.expert_dtype == "mxfp8" else wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "d_model": wl.d, "experts": wl.E, "top_k": wl.k,
                   "d_ff": wl.I, "shared": f"{wl.n_shared}x{wl.I_shared}", "renorm": wl.renorm,
                   "parallelism": "none (1 GPU)",
                   **({"balance_gamma": args.balance_gamma} if args.balance_gamma > 0 else {}),
                   **({"filler_frac": args.filler_frac} if args.filler_frac > 0 else {})},
        "roofline": {"bound": "mfma", "kernel": dominant, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic_per_launch(wl, dominant),
                     "avg_launch_us": avg_ms * 1e3, "launches": launches},
    }
    if gemms:
        result["grouped_gemm"] = {"tflops": expert_flops(wl) / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None,
                                  "frac_of_peak": (expert_flops(wl) / (gemm_ms * 1e-3) / 1e12) / peak
                                  if gemm_ms else None,
                                  "gemm_ms_per_step": gemm_ms}
    result["memory"] = {"peak_alloc_gb": peak_alloc / 2 ** 30,
                        "workspace_gb": layer.plan.workspace_bytes() / 2 ** 30,
                        **({"mx_path": args.mx_path} if wl.expert_dtype == "mxfp8" else {})}
    warm = step_distribution(layer, dy, args.steps)
    result["step_ms"] = {"flushed": flushed, "warm": warm, "timed_region_s": el,
                         "warm_tokens_per_s": wl.T / (warm["median"] * 1e-3)}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
