#!/usr/bin/env python3
"""Benchmark: MoE-layer forward tokens/s at the DeepSeek-V3 shape on one MI355X.

One step = one moe_layer_forward (router, top-k, permutation, grouped gate/up,
grouped down, combine) over T tokens already resident in HBM.  Prints ONE JSON
line.  Per-stage times come from HIP events the library records on the launch
stream; the roofline block reports the dominant kernel (grouped gate/up GEMM)
against the bf16 dense matrix-core peak.  A decode-size measurement (T = 64,
same weights) reports achieved HBM bandwidth over the touched experts'
weights.  The CPU oracle is timed on a bounded token slice as a baseline.

Other lines (one JSON line each, same fields):
  --workload dsv3_dense_prefill   the dense prefix layer FFN (width 18432), and
                                  its T = 64 decode size;
  --block                         the pre-norm block x + layer(RMSNorm(x));
  --capacity-factor CF            the layer with ceil(CF * T * k / N_r) seats per expert;
  --groups NG,TG                  the layer with group-limited top-k (NG groups, TG kept).
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

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12  # 2516.6: 256 CUs x 4096 FLOP/clk x 2.4 GHz (dense)
PEAK_HBM_GBS = 8000.0
STAGES = ["router_logits", "topk", "permute", "gate_up", "down", "combine"]
CSRC = os.path.join(ROOT, "fine_grained_routed_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")


def source_sha256(name: str) -> str:
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()


def measured_traffic(key: str, source: str):
    """HBM bytes per dispatch from the committed counter summary, or None when the
    kernel source has changed since the counters were taken (or none were)."""
    try:
        kv = dict(l.strip().split("=", 1) for l in open(TRAFFIC_FILE) if "=" in l and not l.startswith("#"))
    except OSError:
        return None
    if kv.get(f"{key}_source_sha256") != source_sha256(source) or not kv.get(f"{key}_bytes"):
        return None
    return float(kv[f"{key}_bytes"])


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            evs.append(e.value)
        return evs

    def ms(self, a, b) -> float:
        out = ctypes.c_float()
        self.hip.hipEventSynchronize(b)
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return out.value


def timed_steps(step, steps, warmup, hev, stages=STAGES, between=None, per_step=None):
    """Time `steps` calls of step(events) after `warmup` untimed ones; the library
    records len(stages) + 1 events per call at its stage boundaries.  between()
    (if given) runs after every call, outside the events; per_step (a list, if
    given) receives each call's event-measured total."""
    import torch
    for _ in range(warmup):
        step(None)
        if between:
            between()
    evs = [hev.create(len(stages) + 1) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(evs[s])
        if between:
            between()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    stage = {name: sum(hev.ms(e[i], e[i + 1]) for e in evs) / steps for i, name in enumerate(stages)}
    totals = [hev.ms(e[0], e[len(stages)]) for e in evs]
    if per_step is not None:
        per_step.extend(totals)
    return wall_ms, sum(totals) / steps, stage


def graph_ms_per_step(fn, steps, warmup):
    """Wall time per call of fn() replayed from one captured HIP graph: the same
    kernels as the eager calls, without the host's launch cost between them
    (the way a serving loop would run small batches)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


class _TimedWidening:
    """Expert stack view for the oracle that widens expert e's bf16/fp32 matrix to
    fp64 when the oracle asks for it and adds the time spent widening to a
    shared clock, so that the baseline can leave the conversion out: only the
    oracle's own arithmetic is timed.  Holding every expert widened at once
    would take about 93 GB of host memory at the DeepSeek-V3 shape."""

    def __init__(self, t, clock):
        self.t, self.clock = t, clock

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, e):
        import torch
        t0 = time.perf_counter()
        m = self.t[e].to(torch.float64).numpy()
        self.clock[0] += time.perf_counter() - t0
        return m


def host_description():
    """CPU model, usable cores and the BLAS library numpy calls."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    blas, blas_threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        for p in threadpool_info():
            if p.get("user_api") == "blas":
                blas = f"{p.get('internal_api')} {p.get('version')} ({os.path.basename(p.get('filepath', ''))})"
                blas_threads = p.get("num_threads")
                break
    except Exception:
        pass
    return {"cpu_model": model, "affinity_cores": cores, "blas": blas, "blas_threads": blas_threads}


def cpu_baseline(wl, inp, n_tokens, block=False):
    """The oracle as it stands, on the first n_tokens tokens.  The inputs are
    copied to the host untimed; the routed experts' weights are widened to fp64
    one expert at a time as the oracle walks them, and that widening is left
    out of the timed figure (its duration is reported beside it)."""
    import torch
    import oracle
    import workloads
    host = {k: (None if v is None else v.to("cpu")) for k, v in inp.items()}
    widen = [0.0]
    args = dict(w_router=workloads.to_f64(host["w_router"]), w1=_TimedWidening(host["w1"], widen),
                w3=_TimedWidening(host["w3"], widen), w2=_TimedWidening(host["w2"], widen), k=wl.top_k,
                bias=workloads.to_f64(host["router_bias"]), w1s=workloads.to_f64(host["w1s"]),
                w3s=workloads.to_f64(host["w3s"]), w2s=workloads.to_f64(host["w2s"]))
    hd = host_description()
    what = "fp64 numpy oracle (route, permute, per-expert SwiGLU, shared MLP, combine)"
    if block:
        x64 = host["x"][:n_tokens].to(torch.float64).numpy()
        g64 = host["gamma"].to(torch.float64).numpy()
        t0 = time.perf_counter()
        oracle.block_forward(x64, g64, workloads.NORM_EPS, wl.dtype, **args)
        what = "fp64 numpy oracle of the pre-norm block (RMSNorm, layer, residual)"
    elif wl.top_k == 0:
        u64 = host["u"][:n_tokens].to(torch.float64).numpy()
        t0 = time.perf_counter()
        oracle.dense_ffn(u64, args["w1s"], args["w3s"], args["w2s"])
        what = "fp64 numpy oracle of the dense SwiGLU"
    else:
        u64 = host["u"][:n_tokens].to(torch.float64).numpy()
        t0 = time.perf_counter()
        oracle.forward(u64, **args)
    total = time.perf_counter() - t0
    dt = total - widen[0]
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": hd["blas_threads"] or hd["affinity_cores"],
            "kind": "oracle", "cpu_model": hd["cpu_model"], "affinity_cores": hd["affinity_cores"],
            "blas": hd["blas"], "seconds": dt, "weight_widening_seconds_excluded": widen[0],
            "sample": f"first {n_tokens} of {wl.T} tokens of {wl.name} (a contiguous slice; tokens are independent, "
                      f"so tokens/s carries over to the whole batch); {what}; {dt:.1f} s timed, plus "
                      f"{widen[0]:.1f} s of bf16 -> fp64 weight widening left out"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--block", action="store_true", help="time the pre-norm block instead of the bare layer")
    ap.add_argument("--capacity-factor", type=float, default=0.0,
                    help="seat limit ceil(CF * T * k / N_r) per expert (0: no limit)")
    ap.add_argument("--groups", default="", metavar="NG,TG",
                    help="group-limited routing: NG expert groups, TG kept per token (e.g. 8,4)")
    ap.add_argument("--flush-mb", type=int, default=0, metavar="MB",
                    help="write an MB-sized scratch buffer between timed steps (outside the events), so that "
                         "small layers are timed without their weights in the 256 MB last-level cache")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens the oracle baseline runs on (default: 2048 for the MoE layer, 16384 dense)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times): the reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the layer runs on a single "
              "MI355X (how it would shard across GPUs is described in the design document)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    from fine_grained_routed_amd import PATH_AUTO, PATH_DECODE, MoELayer, capacity_seats

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": n * 4, "dispatches": 3}), flush=True)
        return
    wl = workloads.get(args.workload)
    dense = wl.top_k == 0
    print(f"[bench] drawing inputs for {wl.name}", file=sys.stderr, flush=True)
    inp = (workloads.make_block_inputs if args.block else workloads.make_inputs)(wl, seed=args.seed, device="cuda")
    cap = capacity_seats(args.capacity_factor, wl.T, wl.top_k, wl.n_routed) if args.capacity_factor > 0 else 0
    weights = {k: v for k, v in inp.items() if k not in ("u", "x", "gamma")}
    ng, tg = (int(v) for v in args.groups.split(",")) if args.groups else (0, 0)
    layer = MoELayer(weights, wl.top_k, capacity=cap, n_group=ng, topk_group=tg)
    hev = HipEvents()
    if args.block:
        x, gamma = inp["x"], inp["gamma"]
        T = x.shape[0]
        stages = ["rmsnorm"] + STAGES
        step = lambda ev: layer.block_forward(x, gamma, workloads.NORM_EPS, path=PATH_AUTO, events=ev)
    else:
        u = inp["u"]
        T = u.shape[0]
        stages = STAGES
        step = lambda ev: layer.forward(u, path=PATH_AUTO, events=ev)
    between = None
    if args.flush_mb:
        scratch = torch.empty(args.flush_mb << 18, dtype=torch.float32, device="cuda")
        between = lambda: scratch.fill_(1.0)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    per_step = []
    wall_ms, ev_ms, stage = timed_steps(step, args.steps, args.warmup, hev, stages, between, per_step)
    per_step.sort()
    graph_ms = None
    if not between:
        print("[bench] timing the same step replayed from a HIP graph", file=sys.stderr, flush=True)
        graph_ms = graph_ms_per_step(lambda: step(None), args.steps, args.warmup)

    R = T * wl.top_k
    gu_flop = 4.0 * wl.d * (R * wl.d_ff + T * wl.d_ff_shared)
    dn_flop = gu_flop / 2.0
    total_flop = wl.flops(T)
    gu_tflops = gu_flop / (stage["gate_up"] * 1e-3) / 1e12
    if dense:
        metric = "dense prefix FFN tokens/s at DeepSeek-V3 shape (d=7168, width 18432); % bf16 MFMA peak"
    elif args.block:
        metric = "pre-norm MoE block tokens/s at DeepSeek-V3 shape (RMSNorm + layer + residual)"
    elif ng:
        metric = "MoE-layer tokens/s at DeepSeek-V3 shape with group-limited top-k"
    else:
        metric = "MoE-layer tokens/s at DeepSeek-V3 shape; % bf16 MFMA peak (prefill), % HBM (decode)"
    config = {"workload": wl.name, "T": T, "d_model": wl.d, "n_routed": wl.n_routed, "d_ff": wl.d_ff,
              "n_shared": wl.n_shared, "top_k": wl.top_k}
    if dense:
        config = {"workload": wl.name, "T": T, "d_model": wl.d, "width": wl.d_ff_shared}
    if args.block:
        config["block"] = "x + layer(RMSNorm(x))"
    if cap:
        config["capacity_factor"] = args.capacity_factor
        config["capacity_seats"] = cap
    if ng:
        config["n_group"], config["topk_group"] = ng, tg
    result = {
        "metric": metric,
        "value": T / (wall_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded RMS-normalised N(0,1) tokens, N(0,0.02) weights"
                + ("; block input: per-token scaled N(0,1) stream, gain 1+N(0,0.1)" if args.block else ""),
        "config": config,
        "roofline": {"bound": "mfma", "kernel": "grouped_gemm_bf16_kernel<gate_up>",
                     "achieved": gu_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu_tflops / PEAK_BF16_TFLOPS,
                     # the committed counters were taken on the two DeepSeek-V3 prefill workloads only
                     "traffic": measured_traffic("dense_gate_up_prefill" if dense else "gate_up_prefill",
                                                 "ffn_prefill.hip")
                     if wl.name in ("dsv3_prefill", "dsv3_dense_prefill") and not (args.block or cap or ng)
                     else None,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"},
        "layer_tflops": total_flop / (wall_ms * 1e-3) / 1e12,
        "layer_frac_of_peak": total_flop / (wall_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stage_ms": stage,
        "event_ms_per_step": ev_ms,
        "event_ms_median": per_step[len(per_step) // 2],
        "event_ms_min": per_step[0],
        "flush_mb_between_steps": args.flush_mb,
        "down_tflops": dn_flop / (stage["down"] * 1e-3) / 1e12,
        "graph": None if graph_ms is None else {"ms_per_step": graph_ms, "tokens_per_s": T / (graph_ms * 1e-3)},
    }
    if args.block:
        eb = 2 if wl.dtype == "bf16" else 4
        nb = 2 * T * wl.d * eb + 4 * wl.d  # read x, write u, read the gain
        result["rmsnorm"] = {"bound": "hbm", "bytes": nb, "achieved": nb / (stage["rmsnorm"] * 1e-3) / 1e9,
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": nb / (stage["rmsnorm"] * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if cap:
        idx, _ = layer.router_topk(inp["u"])
        kept = int(layer.permute(idx)[1][-1].item())
        result["capacity_dropped_pairs"] = R - kept

    dec_name = {"dsv3_prefill": "dsv3_decode", "dsv3_dense_prefill": "dsv3_dense_decode"}.get(wl.name)
    if not args.no_decode and not args.block and not cap and not ng and dec_name:
        dec = workloads.get(dec_name)
        ud = inp["u"][:dec.T].contiguous()
        d_wall, d_ev, d_stage = timed_steps(lambda ev: layer.forward(ud, path=PATH_DECODE, events=ev),
                                            max(args.steps, 20), args.warmup, hev)
        if dense:
            touched = 0
        else:
            idx, _ = layer.router_topk(ud)
            counts = layer.permute(idx)[0].cpu()
            touched = int((counts > 0).sum())
        eb = 2  # bf16
        gu_bytes = eb * (touched * 2 * wl.d_ff * wl.d + 2 * wl.d_ff_shared * wl.d)
        dn_bytes = eb * (touched * wl.d * wl.d_ff + wl.d * wl.d_ff_shared)
        layer_bytes = gu_bytes + dn_bytes + eb * (wl.n_routed * wl.d + dec.T * wl.d) + 4 * dec.T * wl.d
        d_graph = graph_ms_per_step(lambda: layer.forward(ud, path=PATH_DECODE), max(args.steps, 20), args.warmup)
        result["decode"] = {
            "workload": dec.name, "T": dec.T, "tokens_per_s": dec.T / (d_wall * 1e-3), "ms_per_step": d_wall,
            "graph": {"ms_per_step": d_graph, "tokens_per_s": dec.T / (d_graph * 1e-3)},
            "touched_experts": touched, "stage_ms": d_stage,
            "layer_GBps": layer_bytes / (d_wall * 1e-3) / 1e9,
            "layer_frac_hbm": layer_bytes / (d_wall * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "roofline": {"bound": "hbm", "kernel": "gate_up (decode path)",
                         "achieved": gu_bytes / (d_stage["gate_up"] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": gu_bytes / (d_stage["gate_up"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "traffic": measured_traffic("dense_gate_up_decode" if dense else "gate_up_decode",
                                                     "ffn_decode.hip"),
                         "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"},
        }

    if not args.no_cpu_baseline:
        n_cpu = min(args.cpu_tokens or (16384 if dense else 2048), T)
        print(f"[bench] timing the oracle on {n_cpu} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, inp, n_cpu, block=args.block)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
