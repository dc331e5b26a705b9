#!/usr/bin/env python3
"""Benchmark of the MoE layer hot path on one MI355X (gfx950).

One step = one full forward and backward of the DeepSeek-V3-shaped layer in
MXFP8 (T=16384 tokens, d=7168, 256 routed experts top-8, I=2048, one bf16
shared expert I=2048, Zipf(1.2)-skewed router, dY ~ N(0,1)): routing, schedule,
quantized dispatch, shared and routed SwiGLU FFNs, weighted combine, then the
backward (dgrads with the fused SwiGLU backward and router-weight gradients
from the G/U the forward kept, dX, deferred weight gradients, router
gradient).
Inputs are seeded synthetic tensors already resident in HBM.

Also measured in the same run: the bf16 DeepSeek-V3 layer (T=8192) forward and
backward, standalone permute and combine bandwidth, and the CPU oracle on a
bounded sample of the headline workload.

Prints ONE JSON line.  Stage times come from HIP events that the library
records on its stream at fixed stage boundaries during the timed steps; the
roofline object describes the dominant kernel of the step.

--workloads NAME[,NAME...] (or "n3") instead measures the forward and the
backward of other layer shapes (gen/configs.py: the Kimi K2.7 Code, GLM-5.2,
Qwen3.5 and DeepSeek-V4-Pro layers whole on one GPU, and one GPU's share of
an EP-64 run) and prints one JSON line with a result per workload.

--workloads n2 instead measures, at the DSV3 MXFP8 shape, the backward with the
gate/up projections kept by the forward against the backward that replays
them, and a token-granularity sweep: 32,768 tokens run as layer calls of 512 to
32,768 tokens each (one JSON line).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd/bwd tokens/sec + MFMA TFLOPS (% peak), DSV3 shape, bf16 & MXFP8"
PEAK = {"bf16": 2500.0, "mxfp8": 5000.0}   # MI355X dense MFMA TFLOP/s
PEAK_HBM_GBS = 8000.0
# Parity of this workload against the float64 oracle at the stated MXFP8 bound
# (max|d|/max|ref| <= 6e-2), as the GPU parity tests measure it: y on every
# token (tests/test_gpu_forward.py::test_full_size_forward_every_token), the
# backward on sampled tokens and every expert's weight-gradient columns
# (tests/test_gpu_mxfp8_backward.py::test_c4_backward_sampled).  Reported, not
# measured here: "over_bound" tensors are expected failures of those tests
# because the quantization-aware model (exact arithmetic on the MX-rounded
# operands) is itself over the bound by the same margin.
MXFP8_BOUND_STATUS = {
    "bound": 6e-2, "source": "pytest -m gpu -rx (tests/test_gpu_mxfp8*.py)",
    "within_bound": {"y": 4.4e-2, "dx": 3.7e-2, "dw_router": 5.4e-2},
    "over_bound": {"dtopk_w": {"gpu": 7.0e-2, "quantized_operands_alone": 7.0e-2},
                   "dw_gate": {"gpu": 9.0e-2, "quantized_operands_alone": 9.1e-2},
                   "dw_up": {"gpu": 6.4e-2, "quantized_operands_alone": 6.4e-2},
                   "dw_down": {"gpu": 6.3e-2, "quantized_operands_alone": 6.2e-2}},
    "kernels_vs_quantized_model_max": 8.0e-3,
}

WORKLOAD = ("DSV3-shaped MoE layer forward+backward, MXFP8 routed experts (E4M3, E8M0 per 32 along K) with bf16 "
            "shared expert and router: T=16384 tokens, d=7168, 256 routed experts top-8, I=2048, 1 shared expert "
            "I=2048, router logits biased by Zipf(1.2) over a seeded expert permutation, dY ~ N(0,1)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_flops(D):
    """Algorithmic FLOPs of each single-kernel GEMM stage (routed rows R)."""
    r = 2.0 * D.R * D.d * D.I
    return {"gate_up": 2 * r, "down": r, "replay_gate_up": 2 * r, "down_dgrad_swiglu": r, "gate_up_dgrad": 2 * r,
            "wgrad_down": r, "wgrad_gate_up": 2 * r}


def gemm_bytes(D, eb, active):
    """Algorithmic HBM bytes of each GEMM stage: every operand read once and
    every output written once (eb: bytes per operand element, 1 + 1/32 for
    E4M3 with its E8M0 scales, 2 for bf16; weights of the `active` experts
    that have rows; outputs bf16; the forward also keeps G|U in bf16)."""
    R, d, I, E = float(D.R), float(D.d), float(D.I), float(D.E)
    w = active * I * d * eb  # one projection matrix of every active expert
    return {"gate_up": R * d * eb + 2 * w + R * I * eb + R * 2 * I * 2,
            "down": R * I * eb + w + R * d * 2,
            "replay_gate_up": R * d * eb + 2 * w + R * 2 * I * 2,
            "down_dgrad_swiglu": R * d * eb + w + R * 2 * I * 2 + R * 2 * I * (2 + (eb if eb < 2 else 0))
            + R * I * 2 + R * I / 8,
            "gate_up_dgrad": R * 2 * I * eb + 2 * w + R * d * 2,
            "wgrad_down": (d + I) * R * eb + E * d * I * 2,
            "wgrad_gate_up": (d + 2 * I) * R * eb + 2 * E * d * I * 2}


def measured_traffic(kernel, stage):
    """HBM bytes of one launch of `stage` (run by `kernel`) from the committed
    counter passes, or None when the kernel's source has changed since they
    were taken or the stage was not measured."""
    import hashlib
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))[kernel]
        src = open(os.path.join(ROOT, "mixture_experts_layer_prefix_amd", "csrc", "gemm_mxfp8.hip"), "rb").read()
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != t.get("source_sha256"):
        return None
    return t.get("bytes_per_launch", {}).get(stage) if isinstance(t.get("bytes_per_launch"), dict) else None


def split_flops(D):
    """(routed, bf16-side) FLOPs of one forward+backward step."""
    routed = 18.0 * D.R * D.d * D.I
    other = 18.0 * D.T * D.S * D.d * D.Is + 6.0 * D.T * D.d * D.E
    return routed, other


def timed_steps(run, steps, torch):
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        run(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return max(wall, ev0.elapsed_time(ev1) / 1e3)


# GEMM stage -> kernel (template instantiation) that runs it
KERNEL_OF = {"gate_up": "gate/up with SwiGLU epilogue", "down": "down projection",
             "replay_gate_up": "G|U replay", "down_dgrad_swiglu": "down dgrad with SwiGLU backward epilogue",
             "gate_up_dgrad": "gate/up dgrad (two matrices along K)",
             "wgrad_down": "K-grouped weight gradient dW_down",
             "wgrad_gate_up": "K-grouped weight gradient dW_gate and dW_up (one launch, M = 2I)"}


def roofline_of(stages, flops, nbytes, peak, label, traffic_key=None):
    """Roofline of the launch with the largest time in the step (every GEMM
    stage is one launch).  Its bound is MFMA or HBM, whichever its
    algorithmic FLOPs or bytes take longer on at the peak rate; achieved =
    that work over the launch's event-timed duration."""
    cand = {n: ms for n, ms in stages.items() if n in flops and ms >= 0.01}
    name = max(cand, key=cand.get)
    t_launch = cand[name] / 1e3
    fl, by = flops[name], nbytes[name]
    if by / (PEAK_HBM_GBS * 1e9) > fl / (peak * 1e12):
        achieved, pk, unit, bound = by / t_launch / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    else:
        achieved, pk, unit, bound = fl / t_launch / 1e12, peak, "TFLOP/s", "mfma"
    stage = name.split("_", 1)[1]
    traffic = measured_traffic(traffic_key, stage) if traffic_key else None
    return dict(bound=bound, achieved=round(achieved, 2), peak=pk, unit=unit, frac=round(achieved / pk, 4),
                traffic=traffic, kernel="%s: %s" % (label, KERNEL_OF[stage]), flops_per_launch=fl,
                bytes_per_launch=by, mfma_frac=round(fl / t_launch / 1e12 / peak, 4), launches_per_step=1,
                launch_ms=round(t_launch * 1e3, 4))


def cpu_baseline(D, rows_hot=8192, tokens=2048):
    """The oracle, as it stands, on a bounded sample of the headline workload,
    scaled to tokens/s.  A token's forward+backward costs its router
    projection and softmax top-k, k routed-expert FFN forward+backward
    evaluations on one row each, and one shared-expert forward+backward.  Timed
    on the host (input regeneration untimed): the oracle FFN forward and
    backward on `rows_hot` rows of the hottest expert plus every row of a
    median-load expert (per-row cost), the shared expert and the router on
    `tokens` tokens (per-token cost)."""
    import numpy as np
    import gen
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    p = gen.Problem(D)
    rng = np.random.default_rng(7)
    sample = np.sort(rng.choice(D.T, size=tokens, replace=False))
    x = p.host_rows("x", sample)
    dy = p.host_rows("dy", sample)
    t0 = time.perf_counter()
    logits = O.router_logits(x, p.host("w_router"), p.logit_bias())
    idx = O.topk_route(logits, D.k)
    g = O.renormalized_weights(logits, idx)
    t_router = (time.perf_counter() - t0) / tokens
    # expert loads of the sample's routing stand in for the full histogram shape
    counts = np.bincount(idx.reshape(-1), minlength=D.E)
    hot = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    med = int(nz[np.argsort(counts[nz])[len(nz) // 2]])
    spent_rows, nrows = 0.0, 0
    for e, n in ((hot, rows_hot), (med, max(int(counts[med]), 1))):
        wg, wu, wd = (p.host_expert(nm, e) for nm in ("w_gate", "w_up", "w_down"))
        xr = p.host_rows("x", rng.choice(D.T, size=n, replace=n > D.T))
        dyr = p.host_rows("dy", rng.choice(D.T, size=n, replace=n > D.T))
        t0 = time.perf_counter()
        O.swiglu_ffn(xr, wg, wu, wd)
        O.ffn_backward(xr, wg, wu, wd, 0.3 * dyr)
        spent_rows += time.perf_counter() - t0
        nrows += n
    t_row = spent_rows / nrows
    ws = [p.host(n)[0] for n in ("ws_gate", "ws_up", "ws_down")]
    t0 = time.perf_counter()
    O.swiglu_ffn(x, *ws)
    O.ffn_backward(x, *ws, dy)
    t_shared = (time.perf_counter() - t0) / tokens
    per_token = t_router + D.k * t_row + t_shared
    return dict(value=round(1.0 / per_token, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample="float64 numpy oracle: router + top-k on %d seeded tokens, routed-expert FFN forward+backward "
                       "on %d rows (hottest expert %d rows, median expert %d rows), shared-expert forward+backward on "
                       "the %d tokens; tokens/s = 1 / (router + k x per-row + shared) per-token cost; %.1f s of "
                       "oracle compute, input regeneration untimed"
                       % (tokens, nrows, rows_hot, nrows - rows_hot, tokens,
                          t_router * tokens + spent_rows + t_shared * tokens))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-sample", type=int, default=12288, help="tokens of the CPU oracle sample (0: skip)")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16 DeepSeek-V3 (T=8192) measurements")
    ap.add_argument("--only-bf16", action="store_true",
                    help="run only the bf16 DeepSeek-V3 (T=8192) measurements (for per-part profiles)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the forward throughput of c0-c3b and the full CPU oracle on c0-c2")
    ap.add_argument("--workloads", default="",
                    help='comma-separated config names, or "n3": measure these workloads instead')
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gen
    import mixture_experts_layer_prefix_amd as M

    if args.workloads == "n2":
        res = n2_part(args, torch, gen, M)
        print(json.dumps({"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "data": "synthetic", "n2": res}), flush=True)
        return
    if args.workloads:
        names = gen.configs.N3 if args.workloads == "n3" else args.workloads.split(",")
        res = {}
        for n in names:
            res[n] = workload_part(args, gen.get_config(n), torch, gen, M)
            torch.cuda.empty_cache()
        print(json.dumps({"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "data": "synthetic", "workloads": res}), flush=True)
        return

    D = gen.get_config("c4")
    log("[bench] workload", D)
    p = gen.Problem(D)
    names = ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
    w = M.Weights(**{n: p.device(n) for n in names})
    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "data": "synthetic"}
    if not args.only_bf16:
        headline(args, D, p, w, out, torch, M)
    if not args.no_bf16:
        bf16_part(args, D, w, out, torch, gen, M)
    if not args.only_bf16:
        out["vendor_dense_gemm"] = vendor_reference(D, torch)
        log("[bench] vendor dense GEMM reference:", out["vendor_dense_gemm"])
    if not args.only_bf16 and not args.no_configs:
        out["forward_configs"] = forward_configs_part(args, w, torch, gen, M)
    del w
    torch.cuda.empty_cache()
    if args.cpu_sample > 0 and not args.only_bf16:
        log("[bench] cpu baseline")
        out["cpu_baseline"] = cpu_baseline(D, rows_hot=4 * args.cpu_sample, tokens=args.cpu_sample)
        model, aff = host_info()
        out["cpu_baseline"].update({"cpu_model": model, "affinity_cores": aff})
        log("[bench] cpu baseline %.2f tokens/s on %d threads" % (out["cpu_baseline"]["value"],
                                                                  out["cpu_baseline"]["cores"]))
        if not args.no_configs:
            out["cpu_baseline"]["configs"] = cpu_oracle_configs()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def headline(args, D, p, w, out, torch, M):
    """The MXFP8 forward+backward step: value, roofline, stage times."""
    x, dy, bias = p.device("x"), p.device("dy"), p.device_bias()
    md = M.Dims(D.T, D.d, D.E, D.k, D.I, D.S, D.Is)
    wq = M.prepare_mxfp8(w, md)
    wb = M.prepare_backward(wq, mxfp8=True)
    fplan = M.ForwardPlan(md, "mxfp8", keep_gu=True)
    bplan = M.BackwardPlan(md, "mxfp8")
    for _ in range(args.warmup):
        fplan.run(x, wq, bias)
        bplan.run(dy, x, wb, fplan.routing)
    torch.cuda.synchronize()
    log("[bench] warmup done")
    tf, tb = M.StageTimer(0, args.steps), M.StageTimer(1, args.steps)

    def step(i):
        tf.arm(i)
        fplan.run(x, wq, bias)
        tb.arm(i)
        bplan.run(dy, x, wb, fplan.routing)

    elapsed = timed_steps(step, args.steps, torch)
    tf.disarm()
    tb.disarm()
    ms = elapsed / args.steps * 1e3
    tokens_s = D.T * args.steps / elapsed
    fwd_st, bwd_st = tf.mean_ms(), tb.mean_ms()
    routed, other = split_flops(D)
    tflops = (routed + other) / (ms / 1e3) / 1e12
    t_roof = routed / (PEAK["mxfp8"] * 1e12) + other / (PEAK["bf16"] * 1e12)
    stages = {"fwd_" + k: v for k, v in fwd_st.items()}
    stages.update({"bwd_" + k: v for k, v in bwd_st.items()})
    pre = lambda n: ("fwd_" if n in ("gate_up", "down") else "bwd_") + n
    flops = {pre(n): f for n, f in gemm_flops(D).items()}
    active = int((fplan.routing["expert_counts"] > 0).sum().item())
    nbytes = {pre(n): b for n, b in gemm_bytes(D, 1 + 1 / 32, active).items()}
    roofline = roofline_of(stages, flops, nbytes, PEAK["mxfp8"], "MXFP8 grouped GEMM (gemm_mxfp8_kernel)",
                           "gemm_mxfp8_kernel<6>")
    log("[bench] timed %d steps: %.3f ms/step (fwd %.3f, bwd %.3f), %.0f tokens/s, %.1f TFLOP/s"
        % (args.steps, ms, sum(fwd_st.values()), sum(bwd_st.values()), tokens_s, tflops))
    log("[bench] stages ms:", {k: round(v, 3) for k, v in stages.items()})
    del fplan, bplan, wb, wq
    torch.cuda.empty_cache()
    out.update({
        "value": round(tokens_s, 1), "ms_per_step": round(ms, 4), "dtype": "mxfp8",
        "config": {"workload": WORKLOAD, "T": D.T, "d": D.d, "E": D.E, "k": D.k, "I": D.I, "n_shared": D.S,
                   "I_shared": D.Is, "precision": "mxfp8 routed experts, bf16 shared expert and router",
                   "pass": "forward+backward", "parallelism": "1 GPU"},
        "tflops": round(tflops, 2), "roofline_step_frac": round(t_roof / (ms / 1e3), 4),
        "roofline": roofline, "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "mxfp8_bound_status": MXFP8_BOUND_STATUS,
    })


def vendor_reference(D, torch, M_rows=16384):
    """Context, not the product path: the vendor GEMM library (torch.matmul and
    torch._scaled_mm, i.e. hipBLASLt) on one dense GEMM of the gate/up shape
    (M_rows x 2I x d), bf16 and per-tensor-scaled E4M3, on this GPU."""
    N, K = 2 * D.I, D.d
    a = torch.randn(M_rows, K, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
    res = {"shape": "%d x %d x %d (M x N x K)" % (M_rows, N, K), "library": "hipBLASLt via torch"}

    def rate(fn):
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(20):
            fn()
        e.record()
        e.synchronize()
        return round(2.0 * M_rows * N * K / (s.elapsed_time(e) / 20 / 1e3) / 1e12, 1)

    res["bf16_tflops"] = rate(lambda: a @ b.t())
    try:
        a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
        one = torch.ones((), device="cuda")
        res["fp8_tflops"] = rate(lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one,
                                                          out_dtype=torch.bfloat16))
    except Exception as ex:  # the fp8 path of the library may be missing
        res["fp8_tflops"] = None
        res["fp8_error"] = str(ex)[:120]
    return res


def workload_part(args, D, torch, gen, M):
    """Forward and backward of one workload (weights and inputs from the
    seeded generator, MXFP8 weights quantized once outside the timing)."""
    log("[bench] workload", D)
    p = gen.Problem(D)
    names = ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
    w = M.Weights(**{n: (p.device(n) if (D.S or not n.startswith("ws_")) else None) for n in names})
    x, dy, bias = p.device("x"), p.device("dy"), p.device_bias()
    md = M.Dims(D.T, D.d, D.E, D.k, D.I, D.S, D.Is)
    mx = D.prec == "mxfp8"
    if mx:
        w = M.prepare_mxfp8(w, md)
    wb = M.prepare_backward(w, mxfp8=mx)
    f, b = M.ForwardPlan(md, D.prec, keep_gu=True), M.BackwardPlan(md, D.prec)
    for _ in range(args.warmup):
        f.run(x, w, bias)
        b.run(dy, x, wb, f.routing)
    ef = timed_steps(lambda i: f.run(x, w, bias), args.steps, torch)
    eb = timed_steps(lambda i: b.run(dy, x, wb, f.routing), args.steps, torch)
    fms, bms = ef / args.steps * 1e3, eb / args.steps * 1e3
    peak = PEAK["mxfp8"] if mx else PEAK["bf16"]
    hc = f.routing["expert_counts"].cpu()
    res = {"T": D.T, "d": D.d, "E": D.E, "k": D.k, "I": D.I, "n_shared": D.S, "I_shared": D.Is,
           "precision": D.prec, "router_skew": "Zipf(%g)" % D.zipf if D.zipf else "none",
           "fwd_ms": round(fms, 4), "fwd_tokens_s": round(D.T / (fms / 1e3), 1),
           "fwd_tflops": round(D.fwd_flops() / (fms / 1e3) / 1e12, 2),
           "bwd_ms": round(bms, 4), "bwd_tokens_s": round(D.T / (bms / 1e3), 1),
           "bwd_tflops": round(D.bwd_flops() / (bms / 1e3) / 1e12, 2),
           "step_tokens_s": round(D.T / ((fms + bms) / 1e3), 1),
           "mfma_peak_frac_step": round((D.fwd_flops() + D.bwd_flops()) / ((fms + bms) / 1e3) / 1e12 / peak, 4),
           "max_rows": int(hc.max()), "empty_experts": int((hc == 0).sum())}
    log("[bench]   fwd %.3f ms (%.1f TFLOP/s), bwd %.3f ms (%.1f TFLOP/s)"
        % (fms, res["fwd_tflops"], bms, res["bwd_tflops"]))
    del f, b, wb, w
    return res


WGRAD_SIDE = ("transposes", "wgrad_down", "wgrad_gate_up", "shared_wgrad", "router_grad")


def n2_part(args, torch, gen, M, total=32768, chunks=(512, 1024, 2048, 4096, 8192, 16384, 32768)):
    """Replay against kept G|U, and the token-granularity sweep, at the DSV3
    MXFP8 shape (the weights and router skew of the headline workload).

    Replay: the forward keeps the gate/up projections G|U (routed R x 2I and
    shared T x 2I_s, bf16) for the backward, or the backward recomputes them
    (the blog post's "Reversed ring order" replays the forward up to the
    SwiGLU); both give the same bits, and the replay trades one gate/up GEMM
    for the memory of G|U.

    Granularity: `total` tokens are run as layer calls of c tokens each
    (forward, then backward with the forward's G|U, call after call).  Per c:
    the forward time, the backward's input-gradient side and its
    weight-gradient side (the token-axis transposes, the deferred weight
    gradients and the router weight gradient), each summed over the calls.
    Per-token results do not depend on c (tested); the weight gradients of a
    call cover its own tokens, so a chunked pipeline defers them to one pass
    over the whole token axis, as the blog post's backward does: the sweep
    reports that step as forward + input-gradient side at c + the
    weight-gradient side of the single whole-axis call."""
    res = {}
    D = gen.get_config("c4", T=total)
    log("[bench] n2 workload", D)
    p = gen.Problem(D)
    names = ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
    w = M.Weights(**{n: p.device(n) for n in names})
    x, dy, bias = p.device("x"), p.device("dy"), p.device_bias()
    md0 = M.Dims(D.T, D.d, D.E, D.k, D.I, D.S, D.Is)
    wq = M.prepare_mxfp8(w, md0)
    wb = M.prepare_backward(wq, mxfp8=True)
    del w
    torch.cuda.empty_cache()
    # (a) kept G|U against replay, at the headline token count
    T1 = 16384
    md1 = M.Dims(T1, D.d, D.E, D.k, D.I, D.S, D.Is)
    x1, dy1 = x[:T1], dy[:T1]
    rep = {}
    for keep in (True, False):
        f, b = M.ForwardPlan(md1, "mxfp8", keep_gu=keep), M.BackwardPlan(md1, "mxfp8")
        for _ in range(args.warmup):
            f.run(x1, wq, bias)
            b.run(dy1, x1, wb, f.routing)
        tb = M.StageTimer(1, args.steps)
        ef = timed_steps(lambda i: f.run(x1, wq, bias), args.steps, torch)

        def bstep(i):
            tb.arm(i)
            b.run(dy1, x1, wb, f.routing)

        eb = timed_steps(bstep, args.steps, torch)
        tb.disarm()
        fms, bms = ef / args.steps * 1e3, eb / args.steps * 1e3
        kept = sum(t.numel() * t.element_size() for n, t in f.routing.items() if n.startswith("gu"))
        rep["kept" if keep else "replayed"] = {
            "fwd_ms": round(fms, 4), "bwd_ms": round(bms, 4), "step_ms": round(fms + bms, 4),
            "step_tokens_s": round(T1 / ((fms + bms) / 1e3), 1),
            "replay_gate_up_ms": round(tb.mean_ms()["replay_gate_up"], 4),
            "gu_bytes_kept": kept, "fwd_workspace_bytes": f.ws_bytes, "bwd_workspace_bytes": b.ws_bytes}
        log("[bench] n2 G|U %s: fwd %.3f ms, bwd %.3f ms" % ("kept" if keep else "replayed", fms, bms))
        del f, b
        torch.cuda.empty_cache()
    rep["workload"] = "T=%d, d=%d, E=%d, k=%d, I=%d, 1 bf16 shared expert, MXFP8 routed experts" % (
        T1, D.d, D.E, D.k, D.I)
    res["replay_vs_kept"] = rep
    # (b) granularity sweep
    sweep = {}
    steps = max(1, min(args.steps, 3))
    for c in chunks:
        n = total // c
        mdc = M.Dims(c, D.d, D.E, D.k, D.I, D.S, D.Is)
        f, b = M.ForwardPlan(mdc, "mxfp8", keep_gu=True), M.BackwardPlan(mdc, "mxfp8")

        def one_pass(i, tf=None, tb=None):
            for j in range(n):
                xs, ds = x[j * c:(j + 1) * c], dy[j * c:(j + 1) * c]
                if tf is not None:
                    tf.arm(i * n + j)
                f.run(xs, wq, bias)
                if tb is not None:
                    tb.arm(i * n + j)
                b.run(ds, xs, wb, f.routing)

        one_pass(0)
        tf, tb = M.StageTimer(0, steps * n), M.StageTimer(1, steps * n)
        el = timed_steps(lambda i: one_pass(i, tf, tb), steps, torch)
        tf.disarm()
        tb.disarm()
        fst, bst = tf.mean_ms(), tb.mean_ms()
        fwd = sum(fst.values()) * n
        wside = sum(bst[k] for k in WGRAD_SIDE) * n
        dside = sum(bst.values()) * n - wside
        sweep[c] = {"calls": n, "pass_ms": round(el / steps * 1e3, 3), "fwd_ms": round(fwd, 3),
                    "bwd_input_grad_side_ms": round(dside, 3), "bwd_weight_grad_side_ms": round(wside, 3),
                    "tokens_s_per_call_wgrads": round(total / (el / steps), 1),
                    "fwd_tokens_s": round(total / (fwd / 1e3), 1),
                    "workspace_bytes": f.ws_bytes + b.ws_bytes}
        log("[bench] n2 chunk %d: pass %.2f ms (fwd %.2f, input-grad side %.2f, weight-grad side %.2f)"
            % (c, el / steps * 1e3, fwd, dside, wside))
        del f, b, tf, tb
        torch.cuda.empty_cache()
    whole = sweep[chunks[-1]]["bwd_weight_grad_side_ms"]
    for c, r in sweep.items():
        r["tokens_s_deferred_wgrads"] = round(total / ((r["fwd_ms"] + r["bwd_input_grad_side_ms"] + whole) / 1e3), 1)
    res["granularity"] = {"total_tokens": total, "steps": steps, "per_chunk_tokens": sweep,
                          "workload": "T=%d tokens as layer calls of 512..%d tokens, d=%d, E=%d, k=%d, I=%d, "
                                      "1 bf16 shared expert, MXFP8 routed experts, Zipf(1.2) router skew"
                                      % (total, chunks[-1], D.d, D.E, D.k, D.I)}
    return res


def bf16_part(args, D, w, out, torch, gen, M):
    """The bf16 DeepSeek-V3 layer at T=8192: forward, backward, permute/combine."""
    D3 = gen.get_config("c3a")
    assert (D3.d, D3.E, D3.I, D3.S, D3.Is, D3.seed) == (D.d, D.E, D.I, D.S, D.Is, D.seed)  # same weights
    p3 = gen.Problem(D3)
    x3, dy3, bias3 = p3.device("x"), p3.device("dy"), p3.device_bias()
    md3 = M.Dims(D3.T, D3.d, D3.E, D3.k, D3.I, D3.S, D3.Is)
    wb3 = M.prepare_backward(w)
    f3, b3 = M.ForwardPlan(md3, "bf16", keep_gu=True), M.BackwardPlan(md3, "bf16")
    for _ in range(args.warmup):
        f3.run(x3, w, bias3)
        b3.run(dy3, x3, wb3, f3.routing)
    t3f, t3b = M.StageTimer(0, args.steps), M.StageTimer(1, args.steps)

    def fstep(i):
        t3f.arm(i)
        f3.run(x3, w, bias3)

    def bstep(i):
        t3b.arm(i)
        b3.run(dy3, x3, wb3, f3.routing)

    ef = timed_steps(fstep, args.steps, torch)
    eb = timed_steps(bstep, args.steps, torch)
    t3f.disarm()
    t3b.disarm()
    fms, bms = ef / args.steps * 1e3, eb / args.steps * 1e3
    fst, bst = t3f.mean_ms(), t3b.mean_ms()
    ffl, bfl = D3.fwd_flops(), D3.bwd_flops()
    st3 = {"fwd_" + k: v for k, v in fst.items()}
    st3.update({"bwd_" + k: v for k, v in bst.items()})
    pre = lambda n: ("fwd_" if n in ("gate_up", "down") else "bwd_") + n
    fl3 = {pre(n): f for n, f in gemm_flops(D3).items()}
    active3 = int((f3.routing["expert_counts"] > 0).sum().item())
    by3 = {pre(n): b for n, b in gemm_bytes(D3, 2, active3).items()}
    out["bf16_dsv3_t8192"] = {
        "forward": {"ms": round(fms, 4), "tokens_s": round(D3.T / (fms / 1e3), 1),
                    "tflops": round(ffl / (fms / 1e3) / 1e12, 2),
                    "mfma_peak_frac": round(ffl / (fms / 1e3) / 1e12 / PEAK["bf16"], 4),
                    "roofline": roofline_of({k: v for k, v in st3.items() if k.startswith("fwd_")},
                                            {k: v for k, v in fl3.items() if k.startswith("fwd_")}, by3,
                                            PEAK["bf16"], "bf16 grouped GEMM (gemm_bf16_kernel)")},
        "backward": {"ms": round(bms, 4), "tokens_s": round(D3.T / (bms / 1e3), 1),
                     "tflops": round(bfl / (bms / 1e3) / 1e12, 2),
                     "mfma_peak_frac": round(bfl / (bms / 1e3) / 1e12 / PEAK["bf16"], 4),
                     "roofline": roofline_of({k: v for k, v in st3.items() if k.startswith("bwd_")},
                                             {k: v for k, v in fl3.items() if k.startswith("bwd_")}, by3,
                                             PEAK["bf16"], "bf16 grouped GEMM (gemm_bf16_kernel)")},
        "stages_ms": {k: round(v, 4) for k, v in st3.items()},
    }
    log("[bench] bf16 T=8192: fwd %.3f ms (%.1f TFLOP/s), bwd %.3f ms (%.1f TFLOP/s)"
        % (fms, ffl / (fms / 1e3) / 1e12, bms, bfl / (bms / 1e3) / 1e12))
    r = f3.routing
    out["hbm"] = hbm_part(D3, r, x3, md3, torch, M)
    hc = r["expert_counts"].cpu()
    out["routing_skew_t8192"] = dict(max_rows=int(hc.max()), empty_experts=int((hc == 0).sum()),
                                     under_32=int((hc < 32).sum()))
    del f3, b3, wb3


def flushed_times(fn, torch, reps=7, flush_bytes=1 << 30):
    """Device time of fn() per call with the last-level cache (the 256 MB
    Infinity Cache) flushed first: a 1 GiB fill runs before every timed call,
    outside its events; the median of reps calls."""
    junk = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        junk.fill_(1)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) / 1e3 for a, b in evs)
    del junk
    return t[len(t) // 2]


def hbm_part(D3, r, x3, md3, torch, M):
    """Standalone dispatch and weighted sum against HBM (algorithmic bytes
    over the flushed device time): the permute (schedule, then the row copy,
    pushed from token order; moe_permute's kernels through its no-allocation
    entry point into preallocated outputs), the schedule alone, the MXFP8
    quantizing dispatch of the same routing, moe_combine, and a plain device
    copy of 1 GiB as the attainable-bandwidth reference."""
    R, T, d, k = D3.R, D3.T, D3.d, D3.k
    perm = M.permute(r["topk_idx"], x3, md3, "bf16")
    o_perm = torch.empty(R, d, dtype=torch.bfloat16, device="cuda").normal_()
    y_sh = torch.empty(T, d, dtype=torch.bfloat16, device="cuda").normal_()
    out_bufs = tuple(None if v is None else torch.empty_like(v) for v in perm)
    t_perm = flushed_times(lambda: M.permute_noalloc(r["topk_idx"], x3, md3, "bf16", out_bufs), torch)
    sched_bufs = out_bufs[:4] + (None, None)
    t_sched = flushed_times(lambda: M.permute_noalloc(r["topk_idx"], x3, md3, "bf16", sched_bufs), torch)
    y_out = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    t_comb = flushed_times(lambda: M.combine_into(o_perm, perm[3], r["topk_w"], y_sh, md3, "bf16", y_out), torch)
    xq = torch.empty(R, d, dtype=torch.uint8, device="cuda")
    xs = torch.empty(R, d // 32, dtype=torch.uint8, device="cuda")
    mx_bufs = out_bufs[:4] + (xq, xs)
    t_perm_mx = flushed_times(lambda: M.permute_noalloc(r["topk_idx"], x3, md3, "mxfp8", mx_bufs), torch)
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    t_copy = flushed_times(lambda: dst.copy_(src), torch)
    perm_bytes = T * d * 2 + R * d * 2 + T * k * 4 * 3      # x, x_perm, ids in, rows out
    disp_bytes = T * d * 2 + R * d * 2 + T * k * 4          # the row copy: x once, every routed row, token_row
    disp_mx_bytes = T * d * 2 + R * d * (1 + 1 / 32) + T * k * 4   # quantizing copy: E4M3 codes + E8M0 scales
    comb_bytes = R * d * 2 + 2 * T * d * 2 + R * 8
    gbs = lambda b, t: b / t / 1e9
    res = {"permute_GBs": round(gbs(perm_bytes, t_perm), 1), "permute_frac": round(gbs(perm_bytes, t_perm) / PEAK_HBM_GBS, 4),
           "permute_ms": round(t_perm * 1e3, 4), "schedule_ms": round(t_sched * 1e3, 4),
           "dispatch_GBs": round(gbs(disp_bytes, t_perm - t_sched), 1),
           "dispatch_frac": round(gbs(disp_bytes, t_perm - t_sched) / PEAK_HBM_GBS, 4),
           "combine_GBs": round(gbs(comb_bytes, t_comb), 1), "combine_frac": round(gbs(comb_bytes, t_comb) / PEAK_HBM_GBS, 4),
           "combine_ms": round(t_comb * 1e3, 4),
           "dispatch_mx_GBs": round(gbs(disp_mx_bytes, t_perm_mx - t_sched), 1),
           "dispatch_mx_frac": round(gbs(disp_mx_bytes, t_perm_mx - t_sched) / PEAK_HBM_GBS, 4),
           "copy_GBs": round(gbs(2 * src.numel() * 2, t_copy), 1),
           "workload": "bf16, T=%d, d=%d, k=%d: moe_permute (schedule + row copy; dispatch = permute minus the "
                       "schedule alone) and moe_combine, each timed with the 256 MB last-level cache flushed by a "
                       "1 GiB fill before every call (median of 7); copy = torch copy of 1 GiB, same protocol" % (T, d, k)}
    log("[bench] hbm:", res)
    return res


def forward_configs_part(args, w_dsv3, torch, gen, M, names=("c0", "c1", "c2", "c3a", "c3b")):
    """Forward throughput of the other forward configurations on one GPU:
    tokens/s, TFLOP/s and the fraction of the precision's dense MFMA peak
    (c0 runs in fp32 and is launch-bound, reported only).  The DeepSeek-V3
    shapes reuse the headline's weights (same generator streams)."""
    res = {}
    for n in names:
        D = gen.get_config(n)
        p = gen.Problem(D)
        md = M.Dims(D.T, D.d, D.E, D.k, D.I, D.S, D.Is)
        wn = ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
        if (D.d, D.E, D.I) == (7168, 256, 2048):
            w = w_dsv3
        else:
            w = M.Weights(**{k: (p.device(k) if (D.S or not k.startswith("ws_")) else None) for k in wn})
        x, bias = p.device("x"), p.device_bias()
        plan = M.ForwardPlan(md, D.prec, keep_routing=True)
        for _ in range(max(args.warmup, 1)):
            plan.run(x, w, bias)
        el = timed_steps(lambda i: plan.run(x, w, bias), args.steps, torch)
        ms = el / args.steps * 1e3
        fl = D.fwd_flops()
        peak = PEAK["bf16"] if D.prec == "bf16" else 157.3
        res[n] = {"T": D.T, "d": D.d, "E": D.E, "k": D.k, "I": D.I, "S": D.S, "prec": D.prec, "ms": round(ms, 4),
                  "tokens_s": round(D.T / (ms / 1e3), 1), "tflops": round(fl / (ms / 1e3) / 1e12, 2),
                  "peak_frac": round(fl / (ms / 1e3) / 1e12 / peak, 4),
                  "peak": "bf16 dense MFMA 2.5 PF" if D.prec == "bf16" else "fp32 vector 157.3 TF (launch-bound)"}
        log("[bench] forward %s: %.3f ms, %.0f tokens/s, %.1f TFLOP/s (%.1f%% of peak)"
            % (n, ms, res[n]["tokens_s"], res[n]["tflops"], 100 * res[n]["peak_frac"]))
        del plan, x
        if w is not w_dsv3:
            del w
        torch.cuda.empty_cache()
    return res


def host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_oracle_configs(names=("c0", "c1", "c2"), one_thread=("c0", "c1")):
    """The oracle, as it stands, on the full forward of the small
    configurations (inputs regenerated on the host, untimed), with all the
    threads its BLAS uses and, for c0 and c1, with one thread."""
    import numpy as np
    import gen
    from oracle import moe_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    res = {}
    for n in names:
        D = gen.get_config(n)
        p = gen.Problem(D)
        get = lambda nm: p.host(nm) if (D.S or not nm.startswith("ws_")) else None
        a = [p.host("x"), p.host("w_router"), p.logit_bias()] + [get(nm) for nm in (
            "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]

        def run():
            t0 = time.perf_counter()
            O.layer_forward(*a, D.k)
            return time.perf_counter() - t0

        t_all = run()
        r = {"tokens_s": round(D.T / t_all, 1), "seconds": round(t_all, 3), "threads": threads}
        if n in one_thread:
            with threadpool_limits(limits=1):
                t1 = run()
            r.update({"tokens_s_1thread": round(D.T / t1, 1), "seconds_1thread": round(t1, 3)})
        res[n] = r
        log("[bench] oracle forward %s: %s" % (n, r))
        del a
    return res



if __name__ == "__main__":
    main()
