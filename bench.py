"""Benchmark: one MoE layer, forward + backward, at the DeepSeek-V3 shape on one
MI355X, through the C ABI of libmoe_gfx950.

    python bench.py [--steps K] [--warmup W] [--workload deepseek_v3] [--no-cpu-baseline]

A step is one full pass of the layer over one batch: route -> permute ->
grouped SwiGLU experts (+ shared expert) -> combine, then the backward in
reverse (combine, experts, router, permute).  Inputs are seeded synthetic
tensors already resident in HBM when the timed region starts.  Prints ONE JSON
line.  Per-kernel durations come from HIP events that the library records
around each kernel on its own stream during the timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the MXFP8 GEMMs)
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense fp4 MFMA (the MXFP4 GEMMs)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

# HBM bytes per launch of a kernel as read from rocprofv3 counters: FETCH_SIZE
# and WRITE_SIZE (KiB per dispatch) of one layer pass at the bench workload,
# each times the factor that makes the same counter match a plain 1 GiB copy
# (FETCH_SIZE reads 512 MiB for it: x2; WRITE_SIZE reads 1 GiB: x1).  A figure
# only holds for the kernel sources it was taken with: `src_sha` is the sha256
# of the GEMM sources at that time, and a mismatch reports traffic as null.
GEMM_SOURCES = ("gemm.hpp", "gemm_regs.hpp", "gemm_mfma.hpp", "gemm_band.hpp", "gemm.hip")
TRAFFIC_MEASURED = {
    # profiles/gemm_wgrad_gateup_deepseek_v3_hbm_bytes.md
    "gemm_wgrad_gateup": {"src_sha": "8935f744abd01638b1a2386a905cfc0a480871e1ce46a6c95d1be94ad414a7d8",
                          "fetch_bytes": 879678693, "write_bytes": 15032457952},
}


def gemm_src_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_limited_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    t = TRAFFIC_MEASURED.get(kernel)
    if not t or t["src_sha"] != gemm_src_sha():
        return None
    return t["fetch_bytes"] + t["write_bytes"]


def step_flops(cfg: mi.MoEConfig, backward: bool = True) -> float:
    """Algorithmic FLOPs of one layer pass: router 2TdE, routed experts 6Tk d f,
    shared expert 6 T d f_s; the backward costs twice the forward.  Elementwise
    work is not counted, nor padded tile rows."""
    fwd = 2.0 * cfg.T * cfg.d * cfg.E + 6.0 * cfg.T * cfg.k * cfg.d * cfg.f + 6.0 * cfg.T * cfg.d * cfg.f_shared
    return fwd * (3.0 if backward else 1.0)


def kernel_work_mx(cfg: mi.MoEConfig, counts) -> dict:
    """Algorithmic (flops, HBM bytes) per launch of each MXFP8 / MXFP4 expert
    GEMM: quantised operands cost 1 + 1/32 bytes per value for fp8 and
    1/2 + 1/32 for fp4 (codes + one scale per 32), bf16 outputs 2; the
    weight gradients' operands count as read once in their quantised size
    (the kernels read them widened to bf16, see mx_qdq_rows)."""
    fp4 = cfg.dtype == "mxfp4"
    q, B = (0.5 if fp4 else 1.0) + 1.0 / 32.0, 2
    rows, d, f, fs, T, E = cfg.T * cfg.k, cfg.d, cfg.f, cfg.f_shared, cfg.T, cfg.E
    ne = int((counts > 0).sum())
    out = {
        "gemm_mx_swiglu_fwd": (2.0 * rows * d * 2 * f, q * (ne * 2 * f * d + rows * d) + B * rows * 3 * f),
        "gemm_mx_down_fwd": (2.0 * rows * f * d, q * (ne * d * f + rows * f) + B * rows * d),
        "gemm_mx_down_dgrad_swiglu_bwd": (2.0 * rows * d * f, q * (ne * f * d + rows * d) + B * rows * 4 * f),
        "gemm_mx_wgrad_down": (2.0 * rows * d * f, q * rows * (d + f) + B * E * d * f),
        "gemm_mx_gateup_dgrad": (2.0 * rows * 2 * f * d, q * (ne * d * 2 * f + rows * 2 * f) + B * rows * d),
        "gemm_mx_wgrad_gateup": (2.0 * rows * 2 * f * d, q * rows * (2 * f + d) + B * E * 2 * f * d),
    }
    if fs:
        out.update({
            "gemm_mx_swiglu_fwd_shared": (2.0 * T * d * 2 * fs, q * (2 * fs * d + T * d) + B * T * 3 * fs),
            "gemm_mx_down_fwd_shared": (2.0 * T * fs * d, q * (d * fs + T * fs) + B * T * d),
            "gemm_mx_down_dgrad_swiglu_bwd_shared": (2.0 * T * d * fs, q * (fs * d + T * d) + B * T * 4 * fs),
            "gemm_mx_wgrad_down_shared": (2.0 * T * d * fs, q * T * (d + fs) + B * d * fs),
            "gemm_mx_gateup_dgrad_shared": (2.0 * T * 2 * fs * d, q * (d * 2 * fs + T * 2 * fs) + 4 * T * d),
            "gemm_mx_wgrad_gateup_shared": (2.0 * T * 2 * fs * d, q * T * (2 * fs + d) + B * 2 * fs * d),
        })
    return out


def kernel_work(cfg: mi.MoEConfig, counts) -> dict:
    """Algorithmic (flops, HBM bytes) per launch of each expert GEMM kernel:
    every non-empty expert's weights read once, activations read and written
    once, weight gradients written for every expert (bf16 = 2 bytes)."""
    B = 2
    rows, d, f, fs, T, E = cfg.T * cfg.k, cfg.d, cfg.f, cfg.f_shared, cfg.T, cfg.E
    ne = int((counts > 0).sum())
    w13, w2 = ne * 2 * f * d * B, ne * d * f * B
    out = {
        "gemm_swiglu_fwd": (2.0 * rows * d * 2 * f, w13 + rows * d * B + rows * f * B + rows * 2 * f * B),
        "gemm_down_fwd": (2.0 * rows * f * d, w2 + rows * f * B + rows * d * B),
        "gemm_down_dgrad_swiglu_bwd": (2.0 * rows * d * f, w2 + rows * d * B + 2 * rows * 2 * f * B),
        "gemm_wgrad_down": (2.0 * rows * d * f, rows * d * B + rows * f * B + E * d * f * B),
        "gemm_gateup_dgrad": (2.0 * rows * 2 * f * d, w13 + rows * 2 * f * B + rows * d * B),
        "gemm_wgrad_gateup": (2.0 * rows * 2 * f * d, rows * 2 * f * B + rows * d * B + E * 2 * f * d * B),
    }
    if fs:
        out.update({
            "gemm_swiglu_fwd_shared": (2.0 * T * d * 2 * fs, 2 * fs * d * B + T * d * B + T * fs * B + T * 2 * fs * B),
            "gemm_down_fwd_shared": (2.0 * T * fs * d, d * fs * B + T * fs * B + T * d * B),
            "gemm_down_dgrad_swiglu_bwd_shared": (2.0 * T * d * fs, d * fs * B + T * d * B + 2 * T * 2 * fs * B),
            "gemm_wgrad_down_shared": (2.0 * T * d * fs, T * d * B + T * fs * B + d * fs * B),
            "gemm_gateup_dgrad_shared": (2.0 * T * 2 * fs * d, 2 * fs * d * B + T * 2 * fs * B + T * d * 4),
            "gemm_wgrad_gateup_shared": (2.0 * T * 2 * fs * d, T * 2 * fs * B + T * d * B + 2 * fs * d * B),
        })
    return out


def bandwidth_work(cfg: mi.MoEConfig) -> dict:
    """Algorithmic HBM bytes per launch of the row-moving kernels (bf16 rows;
    routing tables of T*k entries counted too): the permute reads each token row
    once and writes its k copies; the combine reads the k rows (and the shared
    output) and writes y; its backward reads dy and the k rows and writes the k
    gradient rows and the gate gradients; the unpermute-sum reads the k rows and
    the fp32 partial dx and writes dx."""
    B = 4 if cfg.dtype == "f32" else 2
    T, k, d = cfg.T, cfg.k, cfg.d
    tab = T * k * 4
    sh = T * d * B if cfg.f_shared else 0
    return {
        "scatter_rows": T * d * B + T * k * d * B + tab,
        "combine": T * k * d * B + sh + T * d * B + 2 * tab,
        "combine_bwd": T * d * B + 2 * T * k * d * B + 3 * tab,
        "unpermute_sum": T * k * d * B + T * d * 4 + T * d * B + tab,
    }


def _threads() -> int:
    try:
        import threadpoolctl
        return max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(cfg, dev_inp, backward: bool, flop_budget: float) -> dict:
    """Time the CPU oracle (as it stands: numpy float64) on a bounded sample of
    the same workload, as an algorithmic-FLOP rate in the metric's unit:

    * the router (logits, scores, selection, gates) and the permutation of all
      T tokens;
    * the SwiGLU forward (+ backward) of a sample of experts with all of their
      rows, experts taken evenly over the id range until the sample's FLOPs
      pass `flop_budget`; each expert's bf16 weights and rows are converted to
      float64 before its timed calls (the conversion is not timed);
    * the shared expert on the same fraction of the tokens.
    """
    from oracle import moe_oracle as O
    import numpy as np

    f64 = lambda t: t.float().cpu().double().numpy()
    T, d, E, k, f, fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.f_shared
    x, wr = f64(dev_inp["x"]), f64(dev_inp["w_router"])
    bias = None if dev_inp["bias"] is None else dev_inp["bias"].cpu().numpy()
    dy = f64(dev_inp["dy"]) if backward else None
    ffn_fwd, ffn_bwd = O._ffn_fns(cfg.dtype)

    t0 = time.perf_counter()
    r = O.route(x, wr, bias, cfg)
    p = O.permutation(r["idx"], E)
    t_router = time.perf_counter() - t0
    flops = 2.0 * T * d * E
    timed = t_router

    counts = np.asarray(p["counts"])
    order = [e for e in np.argsort(np.arange(E) * 7919 % E) if counts[e] > 0]   # spread over the ids
    used, rows_done = [], 0
    for e in order:
        if flops >= flop_budget:
            break
        lo, hi = int(p["offsets"][e]), int(p["offsets"][e + 1])
        src = p["src_token"][lo:hi].astype(np.int64)
        xe = x[src]
        w13, w2 = f64(dev_inp["w13"][int(e)]), f64(dev_inp["w2"][int(e)])
        if backward:
            g = np.zeros(hi - lo)
            for j in range(k):                         # the gate of each of the expert's rows
                hit = r["idx"][src, j] == e
                g[hit] = np.asarray(r["gates"], np.float64)[src[hit], j]
            dye = O.store(g[:, None] * dy[src], "bf16")
        t0 = time.perf_counter()
        o = ffn_fwd(xe, w13, w2, "bf16")
        if backward:
            ffn_bwd(xe, o["H"], o["U"], o["A"], dye, w13, w2, "bf16")
        timed += time.perf_counter() - t0
        flops += (18.0 if backward else 6.0) * (hi - lo) * d * f
        used.append(int(e))
        rows_done += hi - lo
        print(f"# cpu baseline: expert {int(e)} ({hi - lo} rows) done, {timed:.1f} s", file=sys.stderr, flush=True)
    ts = 0
    if fs:
        ts = max(1, round(T * len(used) / E))
        ws13, ws2 = f64(dev_inp["ws13"]), f64(dev_inp["ws2"])
        t0 = time.perf_counter()
        o = ffn_fwd(x[:ts], ws13, ws2, "bf16")
        if backward:
            ffn_bwd(x[:ts], o["H"], o["U"], o["A"], dy[:ts], ws13, ws2, "bf16")
        timed += time.perf_counter() - t0
        flops += (18.0 if backward else 6.0) * ts * d * fs
    return {"value": round(flops / timed / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(), "kind": "oracle",
            "seconds": round(timed, 2),
            "sample": f"{cfg.name} {'fwd+bwd' if backward else 'fwd'}: router + permutation of all {T} tokens "
                      f"({t_router:.1f} s), the experts' SwiGLU {'fwd+bwd' if backward else 'fwd'} for "
                      f"{len(used)} of {E} experts with all their rows ({rows_done} of {T * k} rows)"
                      + (f", the shared expert on {ts} tokens" if fs else "")
                      + "; numpy float64, bf16->float64 weight conversion outside the timed region"}


def cpu_baseline_tiny() -> dict:
    """The oracle on the whole tiny workload (T=128, d=64, E=8, k=2, f=128,
    fp32, forward): median of three runs."""
    from oracle import moe_oracle as O
    cfg = mi.TINY
    inp = mi.make_inputs(cfg, seed=0)
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        O.layer_forward(inp, cfg)
        ts.append(time.perf_counter() - t0)
    t = sorted(ts)[1]
    return {"workload": "tiny fwd, whole", "seconds": round(t, 4), "tokens_per_s": round(cfg.T / t, 1),
            "tflops": round(step_flops(cfg, backward=False) / t / 1e12, 6), "cores": _threads()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="deepseek_v3", choices=sorted(mi.CONFIGS))
    ap.add_argument("--pass", dest="passes", default="auto", choices=["auto", "fwd", "fwd+bwd"],
                    help="auto: the workload's own pass (forward only for the Mixtral shape)")
    ap.add_argument("--fold-gates", action="store_true", help="gates applied to act before the down projection")
    ap.add_argument("--recompute-act", action="store_true", help="the backward forms act again from H, U")
    ap.add_argument("--force-balanced", action="store_true", help="round-robin expert assignment")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-flop-budget", type=float, default=0.0,
                    help="algorithmic FLOPs of the oracle's expert sample (default 2e12 for bf16 layers, "
                         "1.5e11 for MXFP8, whose oracle quantises every operand in numpy: about 10-60 s "
                         "on 16 cores)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cold-steps", type=int, default=3,
                    help="extra steps after the timed ones, each after a 512 MiB write that evicts "
                         "L2 and MALL (reported apart as cold_ms_per_step)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer 3 times (scale reference for HBM byte counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                          "launches": 3}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this layer runs on one GPU; sharding it over several GPUs (expert "
                                   "parallelism with all-to-all exchanges) is not built", "n_gpus": args.gpus}))
        sys.exit(2)

    from mixture_experts_layer_limited_amd import LayerShape, MoELayer, _abi as abi

    cfg = mi.CONFIGS[args.workload].with_(fold_gates=args.fold_gates, recompute_act=args.recompute_act,
                                           force_balanced=args.force_balanced)
    backward = cfg.backward if args.passes == "auto" else args.passes == "fwd+bwd"
    mx = cfg.dtype in ("mxfp8", "mxfp4")
    torch.cuda.set_device(0)
    print(f"# generating {cfg.name} inputs on the GPU", file=sys.stderr, flush=True)
    inp = mi.make_inputs(cfg, seed=args.seed, device="cuda", with_grad_inputs=True)
    shape = LayerShape(T=cfg.T, d=cfg.d, E=cfg.E, k=cfg.k, f=cfg.f, f_shared=cfg.f_shared, score=cfg.score,
                       n_group=cfg.n_group, topk_group=cfg.topk_group, renorm=cfg.renorm, scale=cfg.scale,
                       aux_coeff=cfg.aux_coeff, dtype=cfg.dtype, force_balanced=cfg.force_balanced,
                       fold_gates=cfg.fold_gates, recompute_act=cfg.recompute_act)
    layer = MoELayer(shape, "cuda", backward=backward)
    a = inp
    quant_ms = None
    if mx:
        # expert weights are quantised once per weight update, outside the layer (timed apart).
        # The first pass allocates the quantised copies; the timed second pass gets the same
        # buffers back from torch's cache, so it times the quantisation kernels alone.
        layer.prepare_mx_weights(a["w13"], a["w2"], a["ws13"], a["ws2"])
        layer.mx_tensors, layer.mx_weights, layer.mx_key, layer.mx_sources = None, None, None, None
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.prepare_mx_weights(a["w13"], a["w2"], a["ws13"], a["ws2"])
        e1.record()
        torch.cuda.synchronize()
        quant_ms = e0.elapsed_time(e1)

    def step():
        layer.forward(a["x"], a["w_router"], a["bias"], a["w13"], a["w2"], a["ws13"], a["ws2"])
        if backward:
            layer.backward(a["dy"], a["x"], a["w_router"], a["w13"], a["w2"], a["ws13"], a["ws2"], d_aux=1.0)

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    cap = 64 * max(args.steps, 1)
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # one event per step boundary (on the compute stream) gives the per-step
    # spread without adding work to the timed steps
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    abi.moe_trace_begin(cap)
    t_start.record(stream)
    for i in range(args.steps):
        marks[i].record(stream)
        step()
    marks[args.steps].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    trace = abi.moe_trace_end(cap)
    ms = t_start.elapsed_time(t_end) / max(args.steps, 1)
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    print("# timed steps done", file=sys.stderr, flush=True)

    def pct(v, q):
        return v[min(len(v) - 1, int(round(q * (len(v) - 1))))] if v else None

    cold = []
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        for _ in range(args.cold_steps):
            flush.zero_()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            step()
            c1.record(stream)
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        del flush
        cold.sort()

    flops = step_flops(cfg, backward)
    tflops = flops / (ms * 1e-3) / 1e12
    per_kernel = {}
    for name, t in trace:
        s = per_kernel.setdefault(name, [0.0, 0])
        s[0] += t
        s[1] += 1
    kern = {n: {"avg_ms": round(v[0] / v[1], 4), "launches_per_step": round(v[1] / max(args.steps, 1), 2)}
            for n, v in per_kernel.items()}
    counts = layer.buf["counts"].cpu()
    work = kernel_work_mx(cfg, counts) if mx else kernel_work(cfg, counts)
    peak_mfma = {"mxfp8": PEAK_FP8_TFLOPS, "mxfp4": PEAK_FP4_TFLOPS}.get(cfg.dtype, PEAK_BF16_TFLOPS)
    # dominant kernel: largest total time among the expert GEMMs (which carry
    # algorithmic work figures); every other kernel is far smaller at these shapes
    gemms = {n: v for n, v in per_kernel.items() if n in work} or per_kernel
    dom = max(gemms.items(), key=lambda kv: kv[1][0])[0]
    roof = None
    if dom in work:
        fl, by = work[dom]
        t = per_kernel[dom][0] / per_kernel[dom][1] * 1e-3
        ridge = peak_mfma * 1e12 / (PEAK_HBM_GBS * 1e9)
        if fl / by < ridge:
            ach = by / t / 1e9
            roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(dom),
                    "algorithmic_bytes": by, "algorithmic_flops": fl,
                    "achieved_tflops": round(fl / t / 1e12, 1)}
        else:
            ach = fl / t / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": peak_mfma,
                    "unit": "TFLOP/s", "frac": round(ach / peak_mfma, 4), "traffic": measured_traffic(dom),
                    "algorithmic_bytes": by, "algorithmic_flops": fl}
        for n, (fl2, by2) in work.items():
            if n in kern:
                tt = kern[n]["avg_ms"] * 1e-3
                if tt > 0:
                    kern[n]["tflops"] = round(fl2 / tt / 1e12, 1)
                    kern[n]["gbs"] = round(by2 / tt / 1e9, 1)
                    # fraction of the roofline that bounds this kernel (MFMA peak
                    # above the ridge, HBM peak below), and of both peaks
                    kern[n]["mfma_frac"] = round(fl2 / tt / 1e12 / peak_mfma, 4)
                    kern[n]["hbm_frac"] = round(by2 / tt / 1e9 / PEAK_HBM_GBS, 4)
                    kern[n]["bound"] = "hbm" if fl2 / by2 < ridge else "mfma"
                    kern[n]["roofline_frac"] = kern[n]["hbm_frac"] if kern[n]["bound"] == "hbm" else kern[n]["mfma_frac"]

    for n, by2 in bandwidth_work(cfg).items():
        if n in kern and kern[n]["avg_ms"] > 0:
            kern[n]["gbs"] = round(by2 / (kern[n]["avg_ms"] * 1e-3) / 1e9, 1)
            kern[n]["bound"] = "hbm"
            kern[n]["hbm_frac"] = kern[n]["roofline_frac"] = round(kern[n]["gbs"] / PEAK_HBM_GBS, 4)

    out = {
        "metric": "MoE layer fwd+bwd TFLOPS & tokens/s at DSv3 shape, 1 MI355X; % MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype if mx else "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name} MoE layer {'fwd+bwd' if backward else 'fwd'}", "T": cfg.T, "d": cfg.d, "E": cfg.E,
                   "k": cfg.k, "f": cfg.f, "f_shared": cfg.f_shared, "score": cfg.score,
                   "n_group": cfg.n_group, "topk_group": cfg.topk_group, "parallelism": "none (1 GPU)",
                   "pass": "fwd+bwd" if backward else "fwd", "fold_gates": cfg.fold_gates,
                   "recompute_act": cfg.recompute_act, "force_balanced": cfg.force_balanced},
        "step_ms": {"median": round(pct(per_step, 0.5), 4), "p10": round(pct(per_step, 0.1), 4),
                    "p90": round(pct(per_step, 0.9), 4)} if per_step else None,
        "cold_ms_per_step": round(pct(cold, 0.5), 4) if cold else None,
        "tokens_per_s": round(cfg.T / (ms * 1e-3), 1),
        "mfma_peak_frac": round(tflops / peak_mfma, 4),
        "roofline": roof,
        "kernels": kern,
        "expert_rows": {"min": int(counts.min()), "max": int(counts.max()), "empty": int((counts == 0).sum())},
    }
    if quant_ms is not None:
        out["weight_quant_ms"] = round(quant_ms, 3)
    if not args.no_cpu_baseline:
        print("# cpu baseline (the oracle on a bounded sample of the workload)", file=sys.stderr, flush=True)
        budget = args.cpu_flop_budget or (1.5e11 if mx else 2e12)
        out["cpu_baseline"] = cpu_baseline(cfg, inp, backward, budget)
        out["cpu_baseline"]["tiny_whole"] = cpu_baseline_tiny()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
