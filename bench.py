#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X (gfx950).

One step = one full forward of the layer (router, top-k, schedule and
dispatch, shared and routed SwiGLU expert FFNs, weighted sum) over one batch
of seeded synthetic tokens already resident in HBM.  Default workload: the
DeepSeek-V3-shaped layer (T=8192, d=7168, 256 routed experts top-8, I=2048,
one shared expert, Zipf(1.2)-skewed router) in bf16.

Prints ONE JSON line with the whole-job throughput, the roofline of the
dominant kernel (the grouped gate/up GEMM with its SwiGLU epilogue) measured
with HIP events on the stream it runs on, per-stage timings, and the CPU
oracle timed on a bounded token sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd/bwd tokens/sec + MFMA TFLOPS (% peak), DSV3 shape, bf16 & MXFP8"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

WORKLOAD_NAMES = {
    "c3a": "DSV3-shaped MoE layer forward, bf16, T=8192 tokens, d=7168, 256 routed experts top-8, I=2048, "
           "1 shared expert I=2048, router logits biased by Zipf(1.2) over a seeded expert permutation",
    "c3b": "DSV3-shaped MoE layer forward, bf16, T=32768 tokens, d=7168, 256 routed experts top-8, I=2048, "
           "1 shared expert I=2048, router logits biased by Zipf(1.2) over a seeded expert permutation",
    "c2": "Qwen3-235B-shaped MoE layer forward, bf16, T=8192 tokens, d=4096, 128 routed experts top-8, I=1536, "
          "no shared expert",
    "c1": "Mid MoE layer forward, bf16, T=4096 tokens, d=2048, 64 routed experts top-6, I=768, 1 shared expert",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_stream(fn, reps, torch):
    """Average duration (s) of fn() over reps calls, HIP events on the current stream."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / 1e3 / reps


def cpu_baseline(D, n_tokens):
    """The oracle, as it stands, on a seeded sample of the workload's tokens:
    routing of the sampled tokens plus their expert and shared FFNs and the
    weighted sum.  Only the oracle's own arithmetic is timed; regenerating
    the inputs on the host is not."""
    import numpy as np
    import gen
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: report the affinity mask
        threads = len(os.sched_getaffinity(0))
    p = gen.Problem(D)
    rng = np.random.default_rng(7)
    tokens = np.sort(rng.choice(D.T, size=min(n_tokens, D.T), replace=False))
    x = p.host_rows("x", tokens)
    wr = p.host("w_router")
    bias = p.logit_bias()
    spent = 0.0
    t0 = time.perf_counter()
    logits = O.router_logits(x, wr, bias)
    idx = O.topk_route(logits, D.k)
    g = O.renormalized_weights(logits, idx)
    spent += time.perf_counter() - t0
    y = np.zeros((len(tokens), D.d))
    for e in range(D.E):
        rows = np.nonzero(np.any(idx == e, axis=1))[0]
        if len(rows) == 0:
            continue
        wg, wu, wd = (p.host_expert(n, e) for n in ("w_gate", "w_up", "w_down"))
        t0 = time.perf_counter()
        out = O.swiglu_ffn(x[rows], wg, wu, wd)[0]
        gw = g[rows][idx[rows] == e].astype(np.float64)
        y[rows] += gw[:, None] * out
        spent += time.perf_counter() - t0
    if D.S:
        ws = [p.host(n)[0] for n in ("ws_gate", "ws_up", "ws_down")]
        t0 = time.perf_counter()
        y += O.swiglu_ffn(x, *ws)[0]
        spent += time.perf_counter() - t0
    return dict(value=len(tokens) / spent, unit="tokens/s", cores=threads, kind="oracle",
                sample="%d seeded tokens of the same workload (routing, all their routed and shared expert FFNs and "
                       "the weighted sum, float64 numpy); %.1f s of oracle compute, input regeneration untimed"
                       % (len(tokens), spent))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3a", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--cpu-sample", type=int, default=8192, help="tokens for the CPU oracle baseline (0: skip)")
    ap.add_argument("--stage-reps", type=int, default=5, help="repetitions per stage timing (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gen
    import mixture_experts_layer_prefix_amd as M
    D = gen.get_config(args.config)
    log("[bench] workload", D)
    p = gen.Problem(D)
    names = ("w_router", "w_gate", "w_up", "w_down") + (("ws_gate", "ws_up", "ws_down") if D.S else ())
    w = M.Weights(**{n: p.device(n) for n in names})
    x, bias = p.device("x"), p.device_bias()
    md = M.Dims(D.T, D.d, D.E, D.k, D.I, D.S, D.Is)
    plan = M.ForwardPlan(md, D.prec, keep_routing=True)
    for _ in range(args.warmup):
        plan.run(x, w, bias)
    torch.cuda.synchronize()
    log("[bench] warmup done")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        plan.run(x, w, bias)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    elapsed = max(wall, gpu_s)
    ms = elapsed / args.steps * 1e3
    tokens_s = D.T * args.steps / elapsed
    tflops = D.fwd_flops() * args.steps / elapsed / 1e12
    log("[bench] timed %d steps: %.3f ms/step, %.0f tokens/s, %.1f TFLOP/s" % (args.steps, ms, tokens_s, tflops))

    # ---- stages, each through its own entry point, on the current stream ----
    stages = {}
    roofline = None
    if args.stage_reps > 0:
        r = plan.routing
        reps = args.stage_reps
        counts = r["expert_counts"]
        stages["route"] = time_stream(lambda: M.route(x, w.w_router, md, D.prec, bias=bias), reps, torch)
        perm = M.permute(r["topk_idx"], x, md, D.prec)
        stages["permute"] = time_stream(lambda: M.permute(r["topk_idx"], x, md, D.prec), reps, torch)
        x_perm, offsets, token_row = perm[4], perm[1], perm[3]
        if D.S:
            stages["shared_ffn"] = time_stream(lambda: M.shared_ffn(x, w, md, D.prec), reps, torch)
        ws = torch.empty(max(M.workspace_bytes(md, D.prec, 2), 16), dtype=torch.uint8, device="cuda")
        h, _ = M.expert_gate_up(x_perm, None, offsets, w, md, D.prec, ws=ws)
        stages["gate_up"] = time_stream(lambda: M.expert_gate_up(x_perm, None, offsets, w, md, D.prec, ws=ws),
                                        reps, torch)
        o_perm = M.expert_down(h, None, offsets, w, md, D.prec, ws=ws)
        stages["down"] = time_stream(lambda: M.expert_down(h, None, offsets, w, md, D.prec, ws=ws), reps, torch)
        y_sh = M.shared_ffn(x, w, md, D.prec) if D.S else None
        stages["combine"] = time_stream(lambda: M.combine(o_perm, token_row, r["topk_w"], y_sh, md, D.prec), reps,
                                        torch)
        R = D.T * D.k
        gu_flops = 4.0 * R * D.d * D.I
        achieved = gu_flops / stages["gate_up"] / 1e12
        roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                        frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=None,
                        kernel="grouped gate/up GEMM + SwiGLU epilogue (gemm_bf16_kernel, gate/up mode)",
                        flops_per_launch=gu_flops)
        eb = 2
        perm_bytes = D.T * D.d * eb + R * D.d * eb + R * 4
        comb_bytes = R * D.d * eb + 2 * D.T * D.d * eb * (1 if D.S else 0.5) + R * 8
        hbm = dict(permute_GBs=round(perm_bytes / stages["permute"] / 1e9, 1),
                   combine_GBs=round(comb_bytes / stages["combine"] / 1e9, 1))
        hbm["permute_frac"] = round(hbm["permute_GBs"] / PEAK_HBM_GBS, 4)
        hbm["combine_frac"] = round(hbm["combine_GBs"] / PEAK_HBM_GBS, 4)
        hc = counts.cpu()
        skew = dict(max_rows=int(hc.max()), empty_experts=int((hc == 0).sum()), under_32=int((hc < 32).sum()))
        log("[bench] stages ms:", {k: round(v * 1e3, 3) for k, v in stages.items()})
    cpu = None
    if args.cpu_sample > 0:
        log("[bench] cpu baseline on %d tokens" % args.cpu_sample)
        cpu = cpu_baseline(D, args.cpu_sample)
        log("[bench] cpu baseline %.1f tokens/s on %d threads" % (cpu["value"], cpu["cores"]))

    out = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": D.prec, "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.config], "T": D.T, "d": D.d, "E": D.E, "k": D.k, "I": D.I,
                   "n_shared": D.S, "I_shared": D.Is, "precision": D.prec, "parallelism": "1 GPU"},
        "tflops": round(tflops, 2), "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline, "cpu_baseline": cpu,
    }
    if stages:
        out["stages_ms"] = {k: round(v * 1e3, 4) for k, v in stages.items()}
        out["hbm"] = hbm
        out["routing_skew"] = skew
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
