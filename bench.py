"""Benchmark: forward pass of one sparse MoE FFN layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral_bf16]
                    [--no-cpu-baseline] [--cpu-sample TOKENS]

One step = one moe_layer_forward (RMSNorm statistic + router + top-k,
capacity + dispatch, tile plans, expert GEMM 1 + 2 with their epilogues,
combine) over one batch of T tokens already resident in HBM.  Prints ONE
JSON line with tokens/s, the per-stage times from hipEvents recorded by the
library on its own stream, the roofline of the dominant kernel (the first
expert GEMM) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s + expert-GEMM TFLOP/s (% bf16 MFMA peak), 1 MI355X"
# MI355X dense peaks: MFMA bf16, MFMA fp8 (the MXFP8 GEMMs), fp32 vector
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "f32": 157.3}
PEAK_HBM_GBPS = 8000.0

# HBM bytes per launch of the first expert GEMM, per workload, from two
# rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) scaled by
# what the same counters read for a plain 1 GiB device copy
# (bench.py --copy-calibration: FETCH_SIZE 524302.2 KiB, WRITE_SIZE 1048576 KiB).
# The mean over the first 18 launches of the run (warm-up, stage-timer and
# timed forwards on the workload's own routing; the router-extras pass after
# them routes with noise and is left out).  Valid only for the kernel sources
# they were taken on: any change to those files reports null.
COPY_SCALE = {"fetch": 1048576.0 / 524302.2, "write": 1048576.0 / 1048576.0}
TRAFFIC = {
    "mixtral_bf16": {
        "kernel": "k_gemm_bf16_dma", "sources": ("gemm.hip", "gemm_args.h", "gemm_common.h",
                                                 "common.h"),
        "source_sha256": "ce5c4f874d5a9d58f02235c7bc1837e814967bee547c97cc86894d7cf28d43dc",
        "fetch_kib": 1980109.6, "write_kib": 229436.5},
    "variable_bcsr_bf16": {
        "kernel": "k_gemm_bf16_dma", "sources": ("gemm.hip", "gemm_args.h", "gemm_common.h",
                                                 "common.h"),
        "source_sha256": "ce5c4f874d5a9d58f02235c7bc1837e814967bee547c97cc86894d7cf28d43dc",
        "fetch_kib": 30436.4, "write_kib": 45981.9},
    # the routed first GEMM only (the shared experts' first GEMM is the same
    # kernel; the dispatches alternate, routed first)
    "finegrained_bf16": {
        "kernel": "k_gemm_bf16_dma", "sources": ("gemm.hip", "gemm_args.h", "gemm_common.h",
                                                 "common.h"),
        "source_sha256": "ce5c4f874d5a9d58f02235c7bc1837e814967bee547c97cc86894d7cf28d43dc",
        "fetch_kib": 774602.6, "write_kib": 113961.4},
    "atomic_bf16": {
        "kernel": "k_atomic_token", "sources": ("atomic.hip", "common.h"),
        "source_sha256": "7020a44046cfa9c4bc2ee1d7087ff80709367bd331479c1dadda27f72bc9993a",
        "fetch_kib": 535664.1, "write_kib": 16384.0},
    "mixtral_mxfp8": {
        "kernel": "k_gemm_mx", "sources": ("gemm_mx.hip", "gemm_args.h", "gemm_common.h",
                                           "common.h"),
        "source_sha256": "53018a0e8943184f34489804a04727993c74fdc252bc922f7112adc20271ab4a",
        "fetch_kib": 905508.5, "write_kib": 118332.6},
}


def source_sha256(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_mixture_experts_rmsnorm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    t = TRAFFIC.get(workload)
    if t is None or source_sha256(t["sources"]) != t["source_sha256"]:
        return None
    return (t["fetch_kib"] * COPY_SCALE["fetch"] + t["write_kib"] * COPY_SCALE["write"]) * 1024.0


def say(msg):
    """One progress line on stderr per finished leg of the run."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training step (forward + backward) measurement")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the MXFP8 variant of a grouped bf16 workload")
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens whose expert FFNs the CPU oracle computes")
    ap.add_argument("--cpu-baseline-mx", action="store_true",
                    help="also time the CPU oracle on an MXFP8 workload (its quantiser "
                         "re-quantises every expert weight on each call: minutes per run)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time torch.bmm (hipBLASLt) on per-expert GEMMs of the same "
                         "shapes, for context (outside the headline figure)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device copy of known size: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def flops_gemm1(wl, kept):
    mult = 2 if wl.act == "swiglu" else 1
    return sum(2.0 * wl.d * f * mult * m for f, m in zip(wl.sizes, kept))


def flops_gemm2(wl, kept):
    return sum(2.0 * wl.d * f * m for f, m in zip(wl.sizes, kept))


def vendor_gemm(wl, kept, stages, steps):
    """torch.bmm (hipBLASLt) on the uniform-routing form of the two expert
    linears: every expert takes the mean kept row count, one weight matrix per
    expert, bf16 in and out, no epilogue.  Context for the expert GEMMs' rate on
    the same chip; best of three timed runs of `steps` calls each."""
    import torch
    dev = "cuda"
    E, F = wl.E, wl.sizes[0]
    R = max(32, int(round(sum(kept) / E / 32)) * 32)
    n1 = F * (2 if wl.act == "swiglu" else 1)
    out = {"rows_per_expert": R}
    g = torch.Generator(device=dev).manual_seed(1)
    for name, k, n, ours in (("gemm1", wl.d, n1, stages["gemm1"]), ("gemm2", F, wl.d, stages["gemm2"])):
        a = torch.randn((E, R, k), generator=g, device=dev).to(torch.bfloat16)
        b = torch.randn((E, k, n), generator=g, device=dev).to(torch.bfloat16).contiguous()
        c = torch.bmm(a, b)
        best = min(_time_calls(lambda: torch.bmm(a, b, out=c), steps) for _ in range(3))
        fl = 2.0 * E * R * k * n
        ours_fl = (flops_gemm1 if name == "gemm1" else flops_gemm2)(wl, kept)
        out[name] = {"ms": best, "tflops": fl / (best * 1e-3) / 1e12,
                     "ours_tflops": ours_fl / (ours * 1e-3) / 1e12}
        out[name]["ours_over_vendor"] = out[name]["ours_tflops"] / out[name]["tflops"]
        del a, b, c
    torch.cuda.empty_cache()
    out["note"] = ("torch.bmm over E experts x the mean kept rows, uniform (no ragged rows, "
                   "no SwiGLU / gate / r-scale epilogue, no K pieces); the expert GEMMs "
                   "compared here run on the layer's real routing")
    return out


def time_dispatch_gather(B, wl, layer, ws, x, steps):
    """moe_dispatch with the token-row permutation, on the layer's own routing."""
    import torch
    rt = layer.routing(wl.T, ws)
    E, R = rt["counts"].numel(), rt["rows_max"]
    dev = x.device
    i32 = torch.int32
    out = dict(counts=torch.empty(E, dtype=i32, device=dev),
               offsets=torch.empty(E + 1, dtype=i32, device=dev),
               pos=torch.empty((wl.T, wl.k), dtype=i32, device=dev),
               row_token=torch.empty(R, dtype=i32, device=dev),
               row_r=torch.empty(R, device=dev), row_w=torch.empty(R, device=dev),
               row_expert=torch.empty(R, dtype=i32, device=dev))
    x_perm = torch.empty((R, wl.d), dtype=x.dtype, device=dev)
    dws = torch.empty(B.dispatch_workspace_size(wl.T, wl.k, E), dtype=torch.uint8, device=dev)
    cap = B.capacity(wl.T, wl.k, E, wl.cf)
    ids, w, r = rt["ids"].clone(), rt["w"].clone(), rt["r"].clone()
    run = lambda: B.dispatch(ids, w, r, E, cap, rt["pad"], R, out, x=x, x_perm=x_perm, ws=dws)  # noqa: E731
    for _ in range(2):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _time_calls(run, steps):
    """Average ms of run() over back-to-back calls between two events."""
    import torch
    for _ in range(2):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_combine_standalone(B, wl, layer, ws, x, steps):
    """moe_combine (one expert-output plane, residual) on the layer's slot positions."""
    import torch
    rt = layer.routing(wl.T, ws)
    y = torch.randn((rt["rows_max"], wl.d), device=x.device).to(x.dtype)
    out = torch.empty_like(x)
    pos = rt["pos"].clone()
    return _time_calls(lambda: B.combine(y, pos, x, None, wl.T, wl.d, wl.k, out), steps)


def time_router_standalone(B, wl, layer, ws, x, steps):
    """moe_router_topk alone (RMSNorm statistic, router GEMM, top-k) on x."""
    import torch
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=dev)
    w, r = torch.empty((wl.T, wl.k), **f32), torch.empty(wl.T, **f32)
    R = layer.desc.router
    rws = torch.empty(max(B.router_workspace_size(R, wl.T), 1), dtype=torch.uint8, device=dev)
    return _time_calls(lambda: B.router_topk(R, x, wl.k, wl.renorm, ids, w, r_out=r, ws=rws), steps)


def time_router_extras(B, wl, layer, x, out, ws, steps):
    """The layer with noise top-k and the routing statistics switched on
    (outside the headline figure): router stage and whole-step times."""
    import torch
    dev = x.device
    g = torch.Generator(device=dev).manual_seed(0)
    noise = torch.randn((wl.T, wl.E), generator=g, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    ex = B.router_extras(noise=noise, noise_std=1.0, prob_sum=torch.empty(wl.E, **f32),
                         gate_sum=torch.empty(wl.E, **f32), aux=torch.empty(3, **f32))
    for _ in range(2):
        layer.forward(x, out=out, ws=ws, router_extras=ex)
    timer = B.StageTimer(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, out=out, ws=ws, timer=timer, router_extras=ex)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    tot, n = timer.stage_ms("router")
    timer.close()
    return {"router_ms": tot / max(n, 1), "ms_per_step": ms,
            "note": "noise top-k (N(0,1) draws x 1.0) plus per-expert probability / gate sums "
                    "and the three squared-CV statistics"}


def time_layer(B, layer, x, out, ws, stats, steps, warmup):
    """W untimed forwards; then K forwards with the library's stage timer, whose
    hipEvents between the stages give the per-stage times (kept out of the
    headline pass, since each event adds a marker to the stream; running this
    pass first also lets the clock settle after the set-up's idle time); then
    the K timed forwards, bracketed by device syncs, with an event between
    consecutive steps on the stream the layer runs on (median and minimum)."""
    import torch
    for _ in range(warmup):
        layer.forward(x, out=out, ws=ws, stats=stats)
    torch.cuda.synchronize()
    timer = B.StageTimer(steps)
    t2 = time.perf_counter()
    for i in range(steps):
        layer.forward(x, out=out, ws=ws, stats=stats, timer=timer)
    torch.cuda.synchronize()
    with_timer = (time.perf_counter() - t2) * 1e3 / steps
    stages = {}
    for s in B.STAGES:
        tot, n = timer.stage_ms(s)
        stages[s] = tot / max(n, 1)
    timer.close()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        layer.forward(x, out=out, ws=ws, stats=stats)
        ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    step_ms = {"median": per[len(per) // 2] if len(per) % 2 else
               0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2]),
               "min": per[0], "max": per[-1], "mean_events": sum(per) / len(per),
               "mean_with_stage_timer": with_timer}
    return (t1 - t0) * 1e3 / steps, stages, step_ms


def time_layer_graph(layer, x, out, ws, stats, steps):
    """The same forward captured once in a HIP graph and replayed K times
    (no host launch work inside the timed region)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x, out=out, ws=ws, stats=stats)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, out=out, ws=ws, stats=stats)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del g
    return ms


def expert_kept(wl, layer, ws):
    """Rows each expert computes, without padding rows."""
    rt = layer.routing(wl.T, ws)
    counts = rt["counts"].cpu().numpy()
    offsets = rt["offsets"].cpu().numpy()
    kept = [int(offsets[e + 1] - offsets[e]) for e in range(wl.E)]
    if wl.pad > 1:
        kept = [int(min(c, offsets[e + 1] - offsets[e])) for e, c in enumerate(counts)]
    return kept, offsets


def train_step(B, wl, params, x, steps, warmup):
    """Forward (keeping what the backward needs) + backward of the same
    layer for a seeded upstream gradient: the training step of the layer."""
    import torch
    from sparse_mixture_experts_rmsnorm_amd.layer import MoELayer
    layer = MoELayer(wl, params, x.device, train=True)
    ws = layer.alloc_workspace(wl.T)
    bws = torch.empty(layer.backward_workspace_size(wl.T), dtype=torch.uint8, device=x.device)
    out = torch.empty_like(x)
    gen = torch.Generator(device=x.device).manual_seed(wl.seed + 7)
    dout = torch.randn(x.shape, generator=gen, device=x.device).to(x.dtype)
    grads = None
    for _ in range(warmup):
        layer.forward(x, out=out, ws=ws)
        grads = layer.backward(x, dout, ws, bws=bws, grads=grads)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd = bwd = 0.0
    t0 = time.perf_counter()
    for _ in range(steps):
        ev[0].record()
        layer.forward(x, out=out, ws=ws)
        ev[1].record()
        layer.backward(x, dout, ws, bws=bws, grads=grads)
        ev[2].record()
        ev[2].synchronize()
        fwd += ev[0].elapsed_time(ev[1])
        bwd += ev[1].elapsed_time(ev[2])
    wall = (time.perf_counter() - t0) * 1e3 / steps
    kept, _ = expert_kept(wl, layer, ws)
    f_fwd = flops_gemm1(wl, kept) + flops_gemm2(wl, kept)
    bwd_ms = bwd / steps
    res = {"fwd_ms": fwd / steps, "bwd_ms": bwd_ms, "step_ms": wall,
           "tokens_per_s": wl.T / (wall * 1e-3),
           "bwd_expert_tflop": 2 * f_fwd / 1e12,
           "bwd_tflops_incl_all": 2 * f_fwd / (bwd_ms * 1e-3) / 1e12,
           "note": ("fwd with save_for_backward, then moe_layer_backward for a seeded dout; "
                    "bwd_tflops_incl_all = the four expert GEMMs' algorithmic FLOP (twice the "
                    "forward's, kept rows only) over the whole backward time, router, "
                    "transposes and token pass included")}
    del layer, ws, bws, grads
    torch.cuda.empty_cache()
    return res


def mx_variant(B, wl, params, x, steps, warmup):
    """The same layer and weights with MXFP8 routed experts (E4M3 operands,
    E8M0 block scales, fp32 accumulation on the scaled MFMA)."""
    import torch
    from sparse_mixture_experts_rmsnorm_amd.layer import MoELayer
    wq = wl.scaled(name=wl.name.replace("bf16", "mxfp8"), quant="mxfp8")
    layer = MoELayer(wq, params, x.device)
    ws = layer.alloc_workspace(wq.T)
    out = torch.empty_like(x)
    stats = torch.zeros(4, dtype=torch.int32, device=x.device)
    ms, stages, step_ms = time_layer(B, layer, x, out, ws, stats, steps, warmup)
    kept, _ = expert_kept(wq, layer, ws)
    f1, f2 = flops_gemm1(wq, kept), flops_gemm2(wq, kept)
    g1, g2 = stages["gemm1"], stages["gemm2"]
    res = {"workload": wq.name, "ms_per_step": ms, "tokens_per_s": wq.T / (ms * 1e-3),
           "step_ms": step_ms, "stages_ms": stages, "gemm1_tflops": f1 / (g1 * 1e-3) / 1e12,
           "gemm2_tflops": f2 / (g2 * 1e-3) / 1e12,
           "frac_fp8_peak": (f1 + f2) / ((g1 + g2) * 1e-3) / 1e12 / PEAK_TFLOPS["mxfp8"],
           "note": "dispatch includes the per-slot MXFP8 quantisation of the gathered rows"}
    del layer, ws
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, params, sample_tokens):
    """The oracle, as it stands, on a bounded sample of the same workload, in
    its float32 work precision (BLAS sgemm with the library's thread pool):
    one untimed warm-up run, then the median of three timed runs."""
    import numpy as np
    import oracle as O
    from sparse_mixture_experts_rmsnorm_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [os.cpu_count() or 1])
    except Exception:
        threads = os.cpu_count() or 1
    host = {k: synth.to_host(v) for k, v in params.items()}
    p = dict(k=wl.k, eps=wl.eps, renorm=wl.renorm, cf=wl.cf, act=wl.act, residual=True,
             gamma=host.get("gamma"), pad=wl.pad)
    if wl.router == "cartesian":
        p.update(router="cartesian", k_rows=host["k_rows"], k_cols=host["k_cols"], W=host["W"],
                 V=host["V"])
    else:
        p.update(w_router=host["w_router"], bias=host.get("bias"), w1=host["w1"],
                 w3=host.get("w3"), w2=host["w2"], f_offsets=wl.f_offsets)
    if wl.shared_ffn:
        p.update(ws1=host["ws1"], ws3=host.get("ws3"), ws2=host["ws2"], shared_act=wl.shared_act)
    if wl.quant != "none":
        p.update(quant=wl.quant)
    rng = np.random.default_rng(0)
    tok = np.sort(rng.choice(wl.T, size=min(sample_tokens, wl.T), replace=False))
    runs = []
    with O.work_precision(np.float32):
        for i in range(4):
            t0 = time.perf_counter()
            O.layer_forward(p, host["x"], tokens=tok)
            dt = time.perf_counter() - t0
            say(f"cpu baseline {'warm-up' if i == 0 else f'run {i}'}: {dt:.2f} s")
            if i:
                runs.append(dt)
    dt = sorted(runs)[1]
    return {"value": len(tok) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "precision": "float32 (BLAS sgemm)",
            "seconds": dt, "runs_s": runs,
            "sample": (f"{len(tok)} of {wl.T} tokens through the oracle in its float32 work "
                       f"precision (routing, capacity and dispatch over all {wl.T} tokens; "
                       f"expert FFNs, shared FFN and combine for the sample; bf16 weights "
                       f"widened inside the timed call); one warm-up, median of three runs")}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the MoE layer here runs on a single MI355X "
              f"(--gpus {args.gpus} is not supported; sharding the layer over several GPUs "
              f"is a design note of this repository, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_mixture_experts_rmsnorm_amd import binding as B, synth
    from sparse_mixture_experts_rmsnorm_amd.layer import MoELayer
    from sparse_mixture_experts_rmsnorm_amd.workloads import WORKLOADS

    B.lib()
    wl = WORKLOADS[args.workload]
    dev = "cuda"
    torch.manual_seed(0)
    params = synth.make_torch(wl, dev)
    layer = MoELayer(wl, params, dev)
    x = params["x"]
    ws = layer.alloc_workspace(wl.T)
    out = torch.empty_like(x)
    stats = torch.zeros(4, dtype=torch.int32, device=dev)
    say(f"{wl.name}: layer built, timing {args.steps} steps")
    ms_per_step, stages, step_ms = time_layer(B, layer, x, out, ws, stats, args.steps,
                                              args.warmup)
    say(f"layer timed: {ms_per_step:.4f} ms per step")
    st = stats.cpu().numpy().tolist()
    tokens_per_s = wl.T / (ms_per_step / 1e3)
    dtype = "f32" if wl.dtype == "f32" else ("mxfp8" if wl.quant == "mxfp8" else "bf16")

    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic: seeded x ~ N(0,1), weights ~ N(0, 0.02^2), device generator",
        "config": {"workload": wl.name, "tokens": wl.T, "d_model": wl.d, "experts": wl.E,
                   "top_k": wl.k, "d_ffn": wl.sizes[0] if wl.sizes else 1, "act": wl.act,
                   "capacity_factor": wl.cf, "expert_kind": wl.expert_kind,
                   "router": wl.router, "shared_ffn": wl.shared_ffn, "quant": wl.quant},
        "step_ms": step_ms,
        "stages_ms": stages,
        "routing": {"rows": st[0], "dropped": st[1], "max_load": st[2], "errors": st[3]},
    }
    if wl.expert_kind != "atomic":
        kept, offsets = expert_kept(wl, layer, ws)
        f1, f2 = flops_gemm1(wl, kept), flops_gemm2(wl, kept)
        g1, g2 = stages["gemm1"], stages["gemm2"]
        a1 = f1 / (g1 * 1e-3) / 1e12
        result["expert_gemm"] = {
            "tflop": (f1 + f2) / 1e12, "ms": g1 + g2,
            "tflops": (f1 + f2) / ((g1 + g2) * 1e-3) / 1e12,
            "frac_peak": (f1 + f2) / ((g1 + g2) * 1e-3) / 1e12 / PEAK_TFLOPS[dtype],
            "gemm1_tflops": a1, "gemm2_tflops": f2 / (g2 * 1e-3) / 1e12}
        es = 4 if dtype == "f32" else 2
        epi = "SwiGLU" if wl.act == "swiglu" else "GELU"
        result["roofline"] = {"bound": "mfma", "achieved": a1, "peak": PEAK_TFLOPS[dtype],
                              "unit": "TFLOP/s", "frac": a1 / PEAK_TFLOPS[dtype],
                              "traffic": measured_traffic(wl.name),
                              "traffic_unit": "bytes per launch (HBM, from PMC counters)",
                              "kernel": (f"k_gemm_mx (first expert linear, {epi} epilogue, "
                                         "MXFP8 h)"
                                         if dtype == "mxfp8" else
                                         f"k_gemm_bf16_dma (first expert linear, {epi} epilogue"
                                         + (", BCSR tile list)" if wl.expert_kind == "bcsr"
                                            else ")")),
                              "algorithmic_flop_per_launch": f1}
        # the same launch's HBM floor: each expert's weight tile read once, its
        # rows read once, h written once (kept rows only); MXFP8 operands are one
        # code byte per element plus one scale byte per 32
        mult = 2 if wl.act == "swiglu" else 1
        eg = 33.0 / 32.0 if dtype == "mxfp8" else es
        g1_bytes = sum(mult * wl.d * f * eg + m * (wl.d + f) * eg for f, m in zip(wl.sizes, kept)
                       if m > 0)
        floor_ms = max(f1 / (PEAK_TFLOPS[dtype] * 1e12), g1_bytes / (PEAK_HBM_GBPS * 1e9)) * 1e3
        result["roofline"].update({
            "hbm_bytes_algorithmic": g1_bytes,
            "hbm_floor_ms": g1_bytes / (PEAK_HBM_GBPS * 1e9) * 1e3,
            "mfma_floor_ms": f1 / (PEAK_TFLOPS[dtype] * 1e12) * 1e3,
            "frac_of_floor": floor_ms / g1})
        rows = int(offsets[-1])
        # Algorithmic bytes.  combine: every kept expert row, x read, out written.
        # dispatch: each token row
        # read once and each kept row written once (moe_dispatch with x_perm; the
        # layer's dispatch moves indices only, the first GEMM gathers the rows).
        # router: x and the router weights read once.
        comb_bytes = (rows + 2 * wl.T) * wl.d * es
        disp_bytes = (wl.T + rows) * wl.d * es
        router_bytes = (wl.T + wl.E) * wl.d * es
        gather_ms = time_dispatch_gather(B, wl, layer, ws, x, args.steps)
        comb_ms = time_combine_standalone(B, wl, layer, ws, x, args.steps)
        router_ms = time_router_standalone(B, wl, layer, ws, x, args.steps)
        result["memory_bound"] = {
            "combine_ms": comb_ms, "combine_GBps": comb_bytes / (comb_ms * 1e-3) / 1e9,
            "combine_layer_stage_ms": stages["combine"],
            "dispatch_gather_ms": gather_ms,
            "dispatch_gather_GBps": disp_bytes / (gather_ms * 1e-3) / 1e9,
            "router_ms": router_ms, "router_GBps": router_bytes / (router_ms * 1e-3) / 1e9,
            "peak_GBps": PEAK_HBM_GBPS,
            "note": ("algorithmic bytes over back-to-back calls of the public entry points "
                     "on the layer's routing: moe_combine (one kept bf16 row per slot + x + "
                     "out), moe_dispatch with x_perm (token rows read once, kept rows written "
                     "once; its time includes the count / scan / rank index kernels), "
                     "moe_router_topk (x + router weights)")}
    if wl.expert_kind == "atomic":
        # the dominant kernel is the atomic experts' row gather (k_atomic_token):
        # HBM-bound on the W and V rows of the distinct experts the batch draws,
        # plus the token rows read and the routed rows written
        es = 2
        ids = layer.routing(wl.T, ws)["ids"]
        distinct = int(torch.unique(ids).numel())
        a_bytes = (2 * distinct + 2 * wl.T) * wl.d * es
        g1 = stages["gemm1"]
        ach = a_bytes / (g1 * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS,
                              "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS,
                              "traffic": measured_traffic(wl.name),
                              "traffic_unit": "bytes per launch (HBM, from PMC counters)",
                              "kernel": "k_atomic_token (atomic experts, W / V row gathers)",
                              "algorithmic_bytes_per_launch": a_bytes,
                              "distinct_experts": distinct,
                              "slot_row_bytes": 2 * wl.T * wl.k * wl.d * es}
        cf = 2.0 * wl.T * wl.d * (wl.Nr + wl.Nc)
        result["router_gemm"] = {"tflop": cf / 1e12, "stage_ms": stages["router"],
                                 "note": "Cartesian score GEMM plus the three top-32 selections"}
    if wl.shared_ffn:
        sf = 2.0 * wl.T * wl.d * wl.shared_ffn * (3 if wl.shared_act == "swiglu" else 2)
        result["shared_gemm"] = {"tflop": sf / 1e12, "ms": stages["shared"],
                                 "tflops": sf / (stages["shared"] * 1e-3) / 1e12,
                                 "frac_peak": sf / (stages["shared"] * 1e-3) / 1e12
                                 / PEAK_TFLOPS["bf16"]}
    if (args.vendor_gemm and wl.expert_kind == "grouped" and wl.dtype == "bf16"
            and wl.quant == "none" and len(set(wl.sizes)) == 1):
        result["vendor_gemm"] = vendor_gemm(wl, kept, stages, args.steps)
    say("standalone entry points timed")
    gms = time_layer_graph(layer, x, out, ws, stats, args.steps)
    say("graph replay timed")
    result["graph_replay"] = {"ms_per_step": gms, "tokens_per_s": wl.T / (gms * 1e-3),
                              "note": "the same forward captured in one HIP graph and replayed"}
    if wl.router == "dense":
        result["router_extras"] = time_router_extras(B, wl, layer, x, out, ws, args.steps)
    if (not args.no_backward and wl.router == "dense" and wl.dtype == "bf16"
            and wl.quant == "none" and wl.expert_kind in ("grouped", "bcsr")):
        del layer, ws
        torch.cuda.empty_cache()
        layer = ws = None
        result["train_step"] = train_step(B, wl, params, x, args.steps, args.warmup)
        say("training step timed")
    if (not args.no_mx and wl.expert_kind == "grouped" and wl.dtype == "bf16"
            and wl.quant == "none" and all(f % 128 == 0 for f in wl.sizes)):
        del layer, ws
        torch.cuda.empty_cache()
        result["mxfp8_variant"] = mx_variant(B, wl, params, x, args.steps, args.warmup)
        say("MXFP8 variant timed")
    if args.no_cpu_baseline:
        pass
    elif wl.quant != "none" and not args.cpu_baseline_mx:
        result["cpu_baseline"] = {
            "value": None, "unit": "tokens/s", "kind": "oracle",
            "skipped": ("the oracle's MX quantiser re-quantises all expert weights on every "
                        "call (about 4 minutes per run at any sample size on a 8-core host), "
                        "so this workload's CPU leg runs only with --cpu-baseline-mx; the "
                        "bf16 layer of the same shape carries the CPU baseline")}
    else:
        result["cpu_baseline"] = cpu_baseline(wl, params, args.cpu_sample)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
