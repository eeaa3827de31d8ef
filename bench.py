"""Benchmark of the Grok-1 MoE feed-forward layer on one MI355X.

One step = one full layer call (router, permutation, gate/up grouped GEMM with
GELU*up, down grouped GEMM, gate-weighted combine) over one batch of seeded
synthetic tokens already resident in HBM, through grok_moe_forward_ex with a
preallocated workspace. Default workload: the Grok-1-shape decode step (T=8,
d=6144, f=32768, E=8, k=2, bf16), whose layer is bound by streaming the hit
experts' weights from HBM.

Prints one JSON line with the whole-job throughput (tokens/s), the roofline of
the dominant kernel measured live with HIP events on the launch stream, and
the CPU oracle timed on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

WORKLOAD_NAMES = {
    "decode": "grok1_moe_layer_decode_T8",
    "prefill": "grok1_moe_layer_prefill_T8192",
    "int8": "grok1_moe_layer_int8w_T256",
    "skew": "grok1_moe_layer_skewed_T2048",
    "tiny_f32": "tiny_moe_layer_f32_T64",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="tokens the oracle times (0 = default per workload)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the FETCH/WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration(torch, steps):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes": n, "steps": steps, "ms_per_copy": dt * 1e3,
                      "GBps_read_plus_write": 2 * n / dt / 1e9}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the layer's sharding is a design "
              "note only); run with --gpus 1", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    import mixture_experts_transformer_gemm_amd as gm
    import synthetic
    from mixture_experts_transformer_gemm_amd import HipEvents

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch, max(args.steps, 1))
        return

    name = args.workload
    t0 = time.perf_counter()
    w = synthetic.make(name)
    log(f"generated {name} (T={w.T} d={w.d} f={w.f} E={w.E} k={w.k} weights {w.w_dtype}) in "
        f"{time.perf_counter() - t0:.1f}s")

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, rw, wg, wu, wd, sc = (dev(getattr(w, n)) for n in ("x", "router_w", "w_gate", "w_up", "w_down", "scales"))
    torch.cuda.synchronize()
    log("inputs resident in HBM")
    out = torch.empty_like(x)
    need = gm.grok_moe_workspace_bytes(w.T, w.d, w.f, w.E, w.k, gm._dtype_code(x), gm._dtype_code(wg))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    # routing of this batch (for the algorithmic byte count: only hit experts are read)
    _, dbg = gm.grok_moe_forward_ex(x, rw, wg, wu, wd, k=w.k, scales=sc, out=out, workspace=ws, debug=True)
    torch.cuda.synchronize()
    counts = dbg["counts"].cpu().numpy()
    n_hit = int(np.sum(counts > 0))
    rows = int(counts.sum())

    def step(events=None):
        gm.grok_moe_forward_ex(x, rw, wg, wu, wd, k=w.k, scales=sc, out=out, workspace=ws, events=events,
                               stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly K steps, no per-stage events
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = w.T * args.steps / elapsed

    # per-stage kernel durations: HIP events recorded by the library on the launch stream
    ev = HipEvents(6 * args.steps)
    for s in range(args.steps):
        step(events=ev.handles[6 * s:6 * s + 6])
    torch.cuda.synchronize()
    stage_ms = {n: 0.0 for n in gm.STAGES}
    for s in range(args.steps):
        for i, n in enumerate(gm.STAGES):
            stage_ms[n] += ev.elapsed_ms(6 * s + i, 6 * s + i + 1) / args.steps
    ev.close()
    log("stage ms: " + ", ".join(f"{n}={v:.4f}" for n, v in stage_ms.items()))

    # algorithmic work of the dominant kernel (gate/up grouped GEMM + GELU*up)
    wbytes = 1 if w.w_dtype == "i8" else (4 if w.w_dtype == "f32" else 2)
    abytes = 4 if w.act_dtype == "f32" else 2
    gu_bytes = n_hit * 2 * w.d * w.f * wbytes + rows * w.d * abytes + rows * w.f * abytes
    if w.w_dtype == "i8":
        gu_bytes += n_hit * 2 * w.f * 4
    gu_flops = 4.0 * rows * w.d * w.f
    layer_bytes = (n_hit * 3 * w.d * w.f * wbytes + 2 * w.T * w.d * abytes + w.E * w.d * abytes)
    layer_flops = 6.0 * rows * w.d * w.f + 2.0 * w.T * w.d * w.E
    gu_s = stage_ms["gate_up"] / 1e3
    hbm_bound = name in ("decode", "int8") or gu_flops / gu_bytes < (MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS) * 1e3
    if hbm_bound:
        achieved = gu_bytes / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = gu_flops / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof.update({"kernel": "gate_up grouped GEMM (+GELU*up)", "algorithmic_per_launch":
                 gu_bytes if hbm_bound else gu_flops, "avg_launch_ms": round(stage_ms["gate_up"], 5),
                 "traffic": None})

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n = args.cpu_sample or {"decode": 8, "tiny_f32": 64, "int8": 8, "skew": 8, "prefill": 8}[name]
        n = min(n, w.T)
        cores = oracle.threads()
        log(f"timing the CPU oracle on {n} tokens with {cores} threads")
        t0 = time.perf_counter()
        oracle.forward(w.x[:n], w.router_w, w.w_gate, w.w_up, w.w_down, w.k, scales=w.scales, nthreads=cores)
        dt = time.perf_counter() - t0
        cpu = {"value": round(n / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
               "sample": f"first {n} of the {w.T} tokens, whole layer (routing, {w.k} experts each, combine), "
                         f"fp64, {dt:.2f}s"}

    result = {
        "metric": "MoE-layer tokens/s + % roofline (HBM GB/s @T<=64, MFMA util @T=8192)",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "i8": "int8w-bf16", "f32": "f32"}[w.w_dtype],
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[name], "T": w.T, "d": w.d, "f": w.f, "E": w.E, "k": w.k,
                   "weights": w.w_dtype, "experts_hit": n_hit},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer": {"ms": round(ms_per_step, 5), "GBps": round(layer_bytes / (ms_per_step / 1e3) / 1e9, 1),
                  "TFLOPs": round(layer_flops / (ms_per_step / 1e3) / 1e12, 2),
                  "stage_ms": {k2: round(v, 5) for k2, v in stage_ms.items()}},
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
