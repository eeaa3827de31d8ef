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

The metric has two halves: HBM bandwidth at decode (T <= 64) and MFMA
utilisation at one full 8192-token context. The default run measures both in
one invocation: the decode step gives `value`, and the same resident weights
(the prefill workload draws identical weights from the same seed) then run the
8192-token prefill, reported under the "prefill" key with its own tokens/s,
MFMA roofline and sampled CPU baseline. --no-prefill skips that half.

Variants (not the headline): --workload mixtral_decode / mixtral_prefill (Mixtral
8x22B expert shapes, SiLU experts, renormalised gates), dsv3_decode /
dsv3_prefill (DeepSeek-V3-shape fine-grained layer: 256 routed experts of
width 2048, top-8, one shared expert, a selection bias), --sandwich (RMSNorm
before and after the MoE plus the residual), --capacity c (capacity factor).
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

METRIC = "MoE-layer tokens/s + % roofline (HBM GB/s @T\u226464, MFMA util @T=8192)"

WORKLOAD_NAMES = {
    "decode": "grok1_moe_layer_decode_T8",
    "prefill": "grok1_moe_layer_prefill_T8192",
    "int8": "grok1_moe_layer_int8w_T256",
    "skew": "grok1_moe_layer_skewed_T2048",
    "tiny_f32": "tiny_moe_layer_f32_T64",
    "mixtral_decode": "mixtral8x22b_moe_layer_decode_T8",
    "mixtral_prefill": "mixtral8x22b_moe_layer_prefill_T8192",
    "dsv3_decode": "dsv3_moe_layer_decode_T8",
    "dsv3_prefill": "dsv3_moe_layer_prefill_T8192",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the token count T (decode-shape sweep over T <= 64)")
    ap.add_argument("--shard", choices=("tp8", "ep8"), default=None,
                    help="tp8: one GPU's share of the layer split 8 ways over the expert width (f/8); "
                         "ep8: one GPU's share under expert parallelism (the busiest expert with its routed rows)")
    ap.add_argument("--sandwich", action="store_true",
                    help="the sandwich sub-layer: out = x + RMSNorm(MoE(RMSNorm(x)))")
    ap.add_argument("--capacity", type=float, default=0.0,
                    help="capacity factor c > 0: each expert runs at most floor(c*k*T/E) assignments")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="default decode run only: skip the 8192-token prefill half of the metric")
    ap.add_argument("--cpu-sample", type=int, default=0, help="tokens the oracle times (0 = default per workload)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the oracle repeats its sample until this much wall time has passed")
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
    f_override = None
    if args.shard == "tp8":
        f_override = synthetic.WORKLOADS[name][2] // 8
    w = synthetic.make(name, T=args.tokens or None, f=f_override, sandwich=args.sandwich,
                       capacity_factor=args.capacity or None)
    log(f"generated {name} (T={w.T} d={w.d} f={w.f} E={w.E} k={w.k} weights {w.w_dtype} act {w.activation} "
        f"renorm {w.renormalize} capacity {w.capacity_factor} sandwich {args.sandwich}) in "
        f"{time.perf_counter() - t0:.1f}s")
    workload = WORKLOAD_NAMES[name]
    if args.tokens:
        workload = f"{workload.rsplit('_T', 1)[0]}_T{w.T}"
    if args.shard == "tp8":
        workload += f"_{args.shard}_f{w.f}"
    if args.sandwich:
        workload += "_sandwich"
    if w.capacity_factor:
        workload += f"_cap{w.capacity_factor:g}"

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, rw, wg, wu, wd, sc, npre, npost, rbias = (
        dev(getattr(w, n)) for n in ("x", "router_w", "w_gate", "w_up", "w_down", "scales", "norm_pre", "norm_post",
                                     "router_bias"))
    variant = dict(activation=gm.ACT_SILU if w.activation == "silu" else gm.ACT_GELU, renormalize=w.renormalize,
                   capacity_factor=w.capacity_factor, norm_pre=npre, norm_post=npost, norm_eps=w.norm_eps,
                   n_shared=w.n_shared, router_bias=rbias)
    torch.cuda.synchronize()
    log("inputs resident in HBM")
    out = torch.empty_like(x)
    need = gm.grok_moe_workspace_bytes_ex(x, rw, wg, wu, wd, k=w.k, **variant)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    # routing of this batch (for the algorithmic byte count: only hit experts are read)
    _, dbg = gm.grok_moe_forward_ex(x, rw, wg, wu, wd, k=w.k, scales=sc, out=out, workspace=ws, debug=True, **variant)
    torch.cuda.synchronize()
    counts = dbg["counts"].cpu().numpy()
    if args.shard == "ep8" and w.n_shared:
        raise SystemExit("--shard ep8 models layers without shared experts")
    if args.shard == "ep8":
        # one expert per GPU: the busiest expert's GPU runs that expert on its routed rows
        # (gate 1 with E = 1, k = 1); the all-to-all that brings the rows is not modelled
        import dataclasses
        e = int(np.argmax(counts))
        offs, perm = dbg["offsets"].cpu().numpy(), dbg["perm"].cpu().numpy()
        tok = perm[offs[e]:offs[e + 1]].astype(np.int64)
        E0, f0, d0 = w.E, w.f, w.d
        sc_e = None
        if w.scales is not None:   # per-channel scales of expert e: [gate f | up f | down d]
            sc_e = np.concatenate([w.scales[e * f0:(e + 1) * f0], w.scales[E0 * f0 + e * f0:E0 * f0 + (e + 1) * f0],
                                   w.scales[2 * E0 * f0 + e * d0:2 * E0 * f0 + (e + 1) * d0]])
            sc = torch.from_numpy(sc_e).cuda()
        w = dataclasses.replace(w, T=len(tok), E=1, k=1, x=w.x[tok], router_w=w.router_w[e:e + 1],
                                w_gate=w.w_gate[e:e + 1], w_up=w.w_up[e:e + 1], w_down=w.w_down[e:e + 1],
                                scales=sc_e, renormalize=False, capacity_factor=0.0, router_bias=None)
        ti = torch.from_numpy(tok).cuda()
        x, rw, wg, wu, wd = x[ti].contiguous(), rw[e:e + 1], wg[e:e + 1], wu[e:e + 1], wd[e:e + 1]
        variant.update(renormalize=False, capacity_factor=0.0, router_bias=None)
        workload += f"_ep8_expert{e}_M{w.T}"
        log(f"expert-parallel share: expert {e}, {w.T} rows")
        out = torch.empty_like(x)
        need = gm.grok_moe_workspace_bytes(w.T, w.d, w.f, 1, 1, gm._dtype_code(x), gm._dtype_code(wg))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        _, dbg = gm.grok_moe_forward_ex(x, rw, wg, wu, wd, k=1, scales=sc, out=out, workspace=ws, debug=True,
                                        **variant)
        torch.cuda.synchronize()
        counts = dbg["counts"].cpu().numpy()
    result = measure(torch, gm, HipEvents, w, (x, rw, wg, wu, wd, sc), variant, out, ws, stream, counts, workload,
                     args)
    result["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(w, name, args)
    if name == "decode" and not (args.no_prefill or args.tokens or args.shard or args.sandwich or args.capacity):
        # The MFMA half of the metric: one full 8192-token context through the same resident weights.
        del ws, out, dbg
        torch.cuda.empty_cache()
        t0 = time.perf_counter()
        wp = synthetic.make("prefill", with_weights=False)
        assert wp.d == w.d and wp.f == w.f and wp.E == w.E and wp.k == w.k and np.array_equal(wp.router_w, w.router_w)
        import dataclasses
        wp = dataclasses.replace(wp, w_gate=w.w_gate, w_up=w.w_up, w_down=w.w_down, scales=w.scales)
        xp = dev(wp.x)
        outp = torch.empty_like(xp)
        need = gm.grok_moe_workspace_bytes_ex(xp, rw, wg, wu, wd, k=wp.k, **variant)
        wsp = torch.empty(need, dtype=torch.uint8, device="cuda")
        _, dbgp = gm.grok_moe_forward_ex(xp, rw, wg, wu, wd, k=wp.k, scales=sc, out=outp, workspace=wsp, debug=True,
                                         **variant)
        torch.cuda.synchronize()
        countsp = dbgp["counts"].cpu().numpy()
        del dbgp
        log(f"prefill: {wp.T} tokens resident in HBM ({time.perf_counter() - t0:.1f}s), rows per expert "
            f"{countsp.tolist()}")
        pre = measure(torch, gm, HipEvents, wp, (xp, rw, wg, wu, wd, sc), variant, outp, wsp, stream, countsp,
                      WORKLOAD_NAMES["prefill"], args)
        pre["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wp, "prefill", args)
        for key in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data"):
            pre.pop(key, None)
        result["prefill"] = pre
    print(json.dumps(result), flush=True)


def measure(torch, gm, HipEvents, w, tensors, variant, out, ws, stream, counts, workload, args):
    """Times exactly args.steps layer calls after args.warmup untimed ones; returns the bench record of one
    workload (throughput, the dominant kernel's roofline from HIP events on the launch stream, stage times)."""
    x, rw, wg, wu, wd, sc = tensors
    n_hit = int(np.sum(counts > 0))
    rows = int(counts.sum())

    def step(events=None):
        gm.grok_moe_forward_ex(x, rw, wg, wu, wd, k=w.k, scales=sc, out=out, workspace=ws, events=events,
                               stream=stream, **variant)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: exactly K steps. The library records a HIP event before and
    # after the gate/up GEMM on the launch stream (asynchronous, no host sync),
    # which gives the dominant kernel's duration over the same steps; the other
    # stages are left unmarked here (each event between two kernels adds a few
    # microseconds to a decode step).
    ev = HipEvents(2 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events=[None, None, ev.handles[2 * s], ev.handles[2 * s + 1]])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = w.T * args.steps / elapsed
    gate_up_ms = sum(ev.elapsed_ms(2 * s, 2 * s + 1) for s in range(args.steps)) / args.steps
    ev.close()
    # Stage breakdown: a separate, untimed pass of the same steps with an event
    # before each stage and after the last one.
    nb = min(args.steps, 20)
    ev = HipEvents(6 * nb)
    torch.cuda.synchronize()
    for s in range(nb):
        step(events=ev.handles[6 * s:6 * s + 6])
    torch.cuda.synchronize()
    stage_ms = {n: 0.0 for n in gm.STAGES}
    step_ms = []
    for s in range(nb):
        for i, n in enumerate(gm.STAGES):
            stage_ms[n] += ev.elapsed_ms(6 * s + i, 6 * s + i + 1) / nb
        step_ms.append(ev.elapsed_ms(6 * s, 6 * s + 5))
    ev.close()
    # per-step device time (first stage event to last) over the breakdown pass
    q = np.percentile(np.array(step_ms), [10, 50, 90])
    step_dist = {"p10": round(float(q[0]), 5), "median": round(float(q[1]), 5), "p90": round(float(q[2]), 5)}
    log(f"{workload}: {ms_per_step:.4f} ms/step; stage ms: " +
        ", ".join(f"{n}={v:.4f}" for n, v in stage_ms.items()))

    # algorithmic work of the dominant kernel (gate/up grouped GEMM + GELU*up):
    # per hit expert its two d x f weight matrices, plus the routed rows of x
    # read and the H rows written; 4*d*f FLOPs per routed row
    wbytes = 1 if w.w_dtype == "i8" else (4 if w.w_dtype == "f32" else 2)
    abytes = 4 if w.act_dtype == "f32" else 2
    gu_bytes = n_hit * 2 * w.d * w.f * wbytes + rows * w.d * abytes + rows * w.f * abytes
    if w.w_dtype == "i8":
        gu_bytes += n_hit * 2 * w.f * 4
    gu_flops = 4.0 * rows * w.d * w.f
    layer_bytes = (n_hit * 3 * w.d * w.f * wbytes + 2 * w.T * w.d * abytes + w.E * w.d * abytes)
    # rows counts every (token, expert) pair that runs, shared experts included
    layer_flops = 6.0 * rows * w.d * w.f + 2.0 * w.T * w.d * w.E
    gu_s = gate_up_ms / 1e3
    hbm_bound = gu_flops / gu_bytes < (MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS) * 1e3
    if hbm_bound:
        achieved = gu_bytes / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = gu_flops / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["traffic"], traffic_note = measured_traffic(workload)
    roof.update({"kernel": "gate_up grouped GEMM (+" + ("SiLU" if w.activation == "silu" else "GELU") + "*up)",
                 "algorithmic_per_launch": gu_bytes if hbm_bound else gu_flops,
                 "avg_launch_ms": round(gate_up_ms, 5), "traffic_source": traffic_note})
    layer_s = ms_per_step / 1e3
    # Per-expert split of the two grouped GEMMs' time (a model, stated as such): every row tile of an
    # expert reads that expert's weights for its output channels and runs tile_rows rows of matrix-core
    # work whatever its fill, so the GEMM time divides by tile count, not by rows.
    tile_rows = gm.grok_moe_tile_rows(x, rw, wg, wu, wd, k=w.k, **variant)
    split = expert_split(counts, tile_rows, stage_ms["gate_up"] + stage_ms["down"]) if len(counts) <= 16 else None
    return {
        "metric": METRIC,
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
        "config": {"workload": workload, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "k": w.k,
                   "weights": w.w_dtype, "experts_hit": n_hit, "activation": w.activation,
                   "renormalize": w.renormalize, "capacity_factor": w.capacity_factor,
                   "sandwich": w.norm_pre is not None,
                   "n_shared": w.n_shared, "router_bias": w.router_bias is not None, "rows_run": rows,
                   "rows_per_expert": counts.tolist() if len(counts) <= 16 else None},
        "roofline": roof,
        "layer": {"ms": round(ms_per_step, 5), "GBps": round(layer_bytes / layer_s / 1e9, 1),
                  "TFLOPs": round(layer_flops / layer_s / 1e12, 2),
                  "mfma_frac": round(layer_flops / layer_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                  "hbm_frac": round(layer_bytes / layer_s / 1e9 / HBM_PEAK_GBS, 4),
                  "stage_ms": {k2: round(v, 5) for k2, v in stage_ms.items()},
                  "device_step_ms": step_dist, "breakdown_steps": nb, "expert_split": split},
    }


def expert_split(counts, tile_rows, gemm_ms):
    """Per-expert share of the two grouped GEMMs' time, modelled by row tiles: an expert with c rows runs
    ceil(c / tile_rows) tiles, each reading the expert's weights for its channels and doing tile_rows rows
    of matrix-core work whatever its fill. None when the shape has no row tiles (tile_rows 0)."""
    if not tile_rows:
        return None
    tiles = [-(-int(c) // tile_rows) for c in counts]
    total = max(sum(tiles), 1)
    return {"model": "gate_up+down time x (expert's row tiles / all row tiles)", "tile_rows": int(tile_rows),
            "experts": [{"expert": e, "rows": int(c), "row_tiles": n, "empty_rows": n * tile_rows - int(c),
                         "gemm_ms": round(gemm_ms * n / total, 4)} for e, (c, n) in enumerate(zip(counts, tiles))]}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_sample(perm, offsets, T, n=256, per_expert=8, seed=0):
    """Seeded sample of n distinct tokens holding at least `per_expert` tokens of every expert that has
    rows (fewer where an expert has fewer), the rest drawn uniformly from the remaining tokens."""
    rng = np.random.default_rng(seed)
    pick = set()
    for e in range(len(offsets) - 1):
        toks = np.unique(perm[offsets[e]:offsets[e + 1]])
        if len(toks):
            pick.update(int(t) for t in rng.choice(toks, size=min(per_expert, len(toks)), replace=False))
    rest = np.setdiff1d(np.arange(T), np.fromiter(pick, dtype=np.int64, count=len(pick)))
    extra = max(0, min(n, T) - len(pick))
    pick.update(int(t) for t in rng.choice(rest, size=min(extra, len(rest)), replace=False))
    return np.array(sorted(pick), dtype=np.int64)


def cpu_baseline(w, name, args):
    """Times the CPU oracle on the host cores over a bounded sample of the same batch.

    Up to 256 tokens: the whole batch, whole layer, repeated until about ``--cpu-seconds`` of wall time
    has passed. Larger batches: routing and permutation of every token, then the expert outputs of a
    seeded sample of 256 tokens with at least 8 per expert that has rows; the rate is T over (routing and
    permutation time + sample time x T / 256)."""
    import oracle
    cores = oracle.threads()
    act = oracle.SILU if w.activation == "silu" else oracle.GELU
    sampled = w.T > 256 and not (w.n_shared or w.norm_pre is not None or w.capacity_factor or w.renormalize
                                 or w.router_bias is not None)
    if not sampled:
        n = min(args.cpu_sample or {"tiny_f32": 64}.get(name, w.T if w.T <= 256 else 8), w.T)
        log(f"timing the CPU oracle on {n} tokens with {cores} threads (at least {args.cpu_seconds:.0f} s)")
        passes, dt = 0, 0.0
        t0 = time.perf_counter()
        while passes == 0 or (dt < args.cpu_seconds and passes < 100000):
            oracle.layer(w.x[:n], w.router_w, w.w_gate, w.w_up, w.w_down, w.k, scales=w.scales, activation=act,
                         renormalize=w.renormalize, capacity_factor=w.capacity_factor, norm_pre=w.norm_pre,
                         norm_post=w.norm_post, norm_eps=w.norm_eps, n_shared=w.n_shared,
                         router_bias=w.router_bias, nthreads=cores)
            passes += 1
            dt = time.perf_counter() - t0
        return {"value": round(n * passes / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
                "sample": f"{'all' if n == w.T else f'first {n} of the'} {w.T} tokens as one batch, {passes} "
                          f"pass(es), whole layer (routing, {w.k} experts per token, combine) in fp64: {dt:.2f} s"}
    n = args.cpu_sample or 256
    log(f"timing the CPU oracle: routing + permutation of {w.T} tokens, expert outputs of a {n}-token sample, "
        f"{cores} threads")
    t0 = time.perf_counter()
    _, idx, gate = oracle.route(w.x, w.router_w, w.k, nthreads=cores)
    _, offsets, perm, _ = oracle.permute(idx, w.E)
    t_route = time.perf_counter() - t0
    tokens = oracle_sample(perm, offsets, w.T, n=n)
    t0 = time.perf_counter()
    oracle.forward_given_routing(w.x, w.w_gate, w.w_up, w.w_down, idx, gate, scales=w.scales, tokens=tokens,
                                 nthreads=cores)
    t_exp = time.perf_counter() - t0
    projected = t_route + t_exp * w.T / len(tokens)
    return {"value": round(w.T / projected, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"routing + permutation of all {w.T} tokens in fp64 ({t_route:.2f} s), then the {w.k} expert "
                      f"outputs and combine of a seeded {len(tokens)}-token sample with >= 8 tokens per expert "
                      f"({t_exp:.2f} s); value = {w.T} / (routing time + sample time x {w.T}/{len(tokens)})"}


def _source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for fn in files:
        with open(os.path.join(ROOT, "mixture_experts_transformer_gemm_amd", "csrc", fn), "rb") as fh:
            h.update(fn.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, each scaled by the factor a
    plain device copy of known size gives. None when no summary covers the
    workload or the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
    if not os.path.exists(path):
        return None, "no counter summary"
    for line in open(path):
        if not line.startswith("workload="):
            continue
        kv = dict(item.split("=", 1) for item in line.split())
        if kv["workload"] != workload:
            continue
        if _source_digest(kv["sources"].split(",")) != kv["sha256"]:
            return None, "kernel sources changed since the counters were taken"
        traffic = (float(kv["fetch_kib"]) * float(kv["fetch_factor"]) +
                   float(kv["write_kib"]) * float(kv["write_factor"])) * 1024.0
        return round(traffic), "profiles/hbm_traffic.txt"
    return None, "no counter summary for this workload"


if __name__ == "__main__":
    main()
