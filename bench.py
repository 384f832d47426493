#!/usr/bin/env python3
"""Benchmark: exact causal GQA attention, forward + backward, on one MI355X.

One step = attn_fwd + attn_bwd (the whole path: chunk packing, flash forward,
Delta preprocessing, dK/dV and dQ kernels, trunk copies and merges when the
workload is trunked) over one batch of seeded synthetic bf16 inputs already
resident in HBM.  Throughput counts the causal FLOPs 2*S^2*D*Hq for the
forward and 2.5x that for the backward (7*S^2*D*Hq per step).

Default workload: Llama3-8B heads at S=262144 (Hq=32, Hkv=8, D=128) with one
GQA group per chunk (head_chunk 4), the configuration whose head_chunk sweep
reports throughput and peak workspace bytes per setting.

Prints one JSON line.  Extra fields: the per-kernel roofline of the dominant
kernel (HIP events around every launch, on the stream it runs on), the
head_chunk sweep (TFLOP/s and workspace / peak intermediate bytes per
setting), a forward-only (prefill, no LSE kept) line, the 32B-class shape with
K/V trunks in pinned host memory (PCIe-inclusive, so never the headline), and
the fp64 CPU oracle timed on a bounded sample of the same workload on the
host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "causal attn fwd+bwd TFLOP/s & % bf16 MFMA peak; peak HBM bytes vs head_chunk"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 bf16 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5],
                    help="attention workload id (3 = Llama3-8B heads at S=262144)")
    ap.add_argument("--head-chunk", type=int, default=0,
                    help="query heads per chunk (default: one GQA group for workload 2/3)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the other head_chunk settings of the workload")
    ap.add_argument("--sweep-steps", type=int, default=2,
                    help="timed steps per other head_chunk setting")
    ap.add_argument("--no-forward-only", action="store_true",
                    help="skip the forward-only (no LSE) line")
    ap.add_argument("--no-host-trunks", action="store_true",
                    help="skip the pinned-host-trunk line (workload 4)")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the attention-layer line (projections around attention)")
    ap.add_argument("--group-loop-min-s", type=int, default=0,
                    help="sequence length from which dK/dV takes the group-loop schedule "
                         "(0 = the library default, 65536)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=12288,
                    help="tokens of the CPU-oracle sample (one GQA group)")
    ap.add_argument("--kv-trunk", default="-1",
                    help="key/value trunk length in tokens (default: the workload's; 0 = "
                         "untrunked; 'auto' = attn_pick_kv_trunk for --budget-gib)")
    ap.add_argument("--budget-gib", type=float, default=0.0,
                    help="workspace budget for --kv-trunk auto (GiB; 0 = no limit)")
    ap.add_argument("--trunk-merge", action="store_true",
                    help="trunked forward by per-trunk log-sum-exp merge (default: carried state)")
    ap.add_argument("--h2d-probe", action="store_true",
                    help="also time one pinned-host to device copy of the K/V trunk size")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the steps, run one plain device-to-device copy of MIB MiB "
                         "(the known-size reference for HBM byte counters)")
    return ap.parse_args()


def algorithmic_flops(family: str, S: int, Hq: int, D: int, causal: bool) -> float:
    """MFMA work the algorithm asks of one kernel family for one full pass over
    the workload: per visible (query, key) pair and head, QK^T and PV are 2*D
    each (forward 4*D); dK/dV needs S, dP, dV, dK (8*D); dQ needs S, dP, dQ
    (6*D).  Pairs per head = S^2/2 when causal (the counted convention)."""
    pairs = S * S / 2.0 if causal else float(S) * S
    per_pair = {"fwd": 4 * D, "dkdv": 8 * D, "dq": 6 * D}.get(family)
    return 0.0 if per_pair is None else per_pair * pairs * Hq


# the sources each kernel family is compiled from, with their code-generation
# options (traffic figures taken with the profiler are only used while these
# are unchanged)
FAMILY_SOURCES = {"fwd": ["fwd.hip"], "dkdv": ["bwd.hip"], "dq": ["bwd.hip"]}
COMMON_SOURCES = ["device_common.h", "kernels.h"]


ROOT_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC_DIR = os.path.join(ROOT_DIR, "head_chunked_context_amd", "csrc")
PROFILES_DIR = os.path.join(ROOT_DIR, "profiles")


def kernel_source_hash(family: str) -> str:
    import hashlib
    h = hashlib.sha256()
    from head_chunked_context_amd.build import FLAGS
    for name in FAMILY_SOURCES.get(family, []) + COMMON_SOURCES:
        with open(os.path.join(CSRC_DIR, name), "rb") as f:
            h.update(f.read())
        h.update(repr(FLAGS.get(name, [])).encode())
    return h.hexdigest()


def measured_traffic(family: str, shape: str, hc: int):
    """HBM bytes per launch of `family` on this shape from the committed
    counter summary (profiles/traffic_<family>_<shape>_hc<hc>.md, line
    `traffic_json: {...}`), or None when there is none or the kernel's sources
    changed since the counters were taken."""
    path = os.path.join(PROFILES_DIR, f"traffic_{family}_{shape}_hc{hc}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic_json:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("source_sha256") != kernel_source_hash(family):
                    return None
                return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    return None


def cpu_oracle_baseline(D: int, g: int, tokens: int) -> dict:
    """Time the fp64 oracle's forward + backward on one GQA group (g query
    heads, 1 kv head) over the first `tokens` positions, seeded like the
    workload; report its throughput in counted TFLOP/s."""
    import torch

    from head_chunked_context_amd.inputs import attention_inputs
    from oracle import oracle as orc
    inp = attention_inputs(tokens, g, 1, D, 900, device="cpu")
    cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    t0 = time.perf_counter()
    orc.attn_fwd(inp["q"], inp["k"], inp["v"], True)
    orc.attn_bwd(inp["q"], inp["k"], inp["v"], inp["dout"], True)
    dt = time.perf_counter() - t0
    counted = 7.0 * tokens * tokens * D * g
    del torch
    return {"value": counted / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu": cpu_model,
            "sample": f"fp64 oracle forward+backward of one GQA group ({g} query heads, 1 kv "
                      f"head, D={D}) over the first {tokens} tokens; {dt:.1f} s wall, counted "
                      f"FLOPs 7*S^2*D*heads"}


def group_loop_min_s(hcm) -> int:
    """The library's current group-loop threshold (read without changing it)."""
    prev = hcm.set_group_loop_min_s(0)
    hcm.set_group_loop_min_s(prev)
    return prev


def run_workload(hcm, torch, w, hc, T, dev, steps, warmup, timing, kv_on_host, trunk_merge=False,
                 forward_only=False):
    """Seeded inputs of workload w, then W warm-up and K timed steps at one
    head_chunk.  Returns the timings, workspace bytes and peak intermediate
    device memory (torch's peak-allocation delta over the user tensors)."""
    from head_chunked_context_amd.inputs import attention_inputs
    S, Hq, Hkv, D = w.S, w.Hq, w.Hkv, w.D
    causal = True
    inp = attention_inputs(S, Hq, Hkv, D, w.wid, device=dev, with_dout=not forward_only)
    if kv_on_host:
        for n in ("k", "v"):
            inp[n] = inp[n].cpu().pin_memory()
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp.get("dout")
    o = torch.empty_like(q)
    lse = None if forward_only else torch.empty((Hq, S), dtype=torch.float32, device=dev)
    if not forward_only:
        dq = torch.empty_like(q)
        pin = k.device.type == "cpu"
        dk = torch.empty(k.shape, dtype=k.dtype, device=k.device, pin_memory=pin)
        dv = torch.empty(v.shape, dtype=v.dtype, device=v.device, pin_memory=pin)
    fb = hcm.fwd_workspace_bytes(S, Hq, Hkv, D, causal, hc, T)
    bb = 0 if forward_only else hcm.bwd_workspace_bytes(S, Hq, Hkv, D, causal, hc, T)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)

    def step():
        hcm.attn_fwd(q, k, v, head_chunk=hc, kv_trunk=T, causal=causal, out=o, lse=lse,
                     workspace=ws, with_lse=not forward_only)
        mid = torch.cuda.Event(enable_timing=True)
        mid.record()
        if not forward_only:
            hcm.attn_bwd(q, k, v, o, do, lse, head_chunk=hc, kv_trunk=T, causal=causal, dq=dq,
                         dk=dk, dv=dv, workspace=ws)
        return mid

    prev_merge = hcm.set_trunk_merge(trunk_merge)
    try:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        print(f"{w.name}: head_chunk={hc}{' forward only' if forward_only else ''}: {warmup} "
              f"warm-up step(s) done, timing {steps}", file=sys.stderr, flush=True)
        if timing:
            hcm.timing_reset()
            hcm.timing_enable(True)
        starts, mids = [], []
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t_start.record()
        for _ in range(steps):
            s = torch.cuda.Event(enable_timing=True)
            s.record()
            starts.append(s)
            mids.append(step())
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    finally:
        hcm.set_trunk_merge(prev_merge)
    kern = moved = None
    if timing:
        hcm.timing_enable(False)
        kern = hcm.timing_read()
        moved = hcm.timing_bytes()
        hcm.timing_reset()
    total_ms = t_start.elapsed_time(t_end)
    fwd_ms = sum(a.elapsed_time(b) for a, b in zip(starts, mids))
    peak = torch.cuda.max_memory_allocated(dev) - base
    del ws
    print(f"{w.name}: head_chunk={hc}: {total_ms / steps:.1f} ms per step", file=sys.stderr,
          flush=True)
    return {"ms": total_ms / steps, "fwd_ms": fwd_ms / steps,
            "bwd_ms": (total_ms - fwd_ms) / steps, "wall_s": wall, "kern": kern, "moved": moved,
            "ws_fwd": fb, "ws_bwd": bb, "peak_intermediate": peak}


def run_layer(hcm, torch, w, hc, dev, steps, warmup, keep_o=False):
    """The attention layer around the attention at workload w's shape with
    d_model = Hq * D: forward + backward, head chunk by head chunk.  Returns
    timings, workspace bytes and the peak intermediate device memory (torch's
    peak-allocation delta over inputs, weights and outputs).  keep_o: the
    forward keeps the attention output and LSE for the backward, which then
    skips recomputing them (kept_bytes: that activation)."""
    from head_chunked_context_amd.inputs import layer_inputs
    S, Hq, Hkv, D = w.S, w.Hq, w.Hkv, w.D
    dm = Hq * D
    inp = layer_inputs(S, dm, Hq, Hkv, D, w.wid, device=dev)
    y = torch.empty((S, dm), dtype=torch.float32, device=dev)
    grads = [torch.empty(sh, dtype=torch.float32, device=dev)
             for sh in ((S, dm), (Hq * D, dm), (Hkv * D, dm), (Hkv * D, dm), (dm, Hq * D))]
    fb = hcm.layer_fwd_workspace_bytes(S, dm, Hq, Hkv, D, True, hc)
    bb = hcm.layer_bwd_workspace_bytes(S, dm, Hq, Hkv, D, True, hc)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)
    a = (inp["x"], inp["wq"], inp["wk"], inp["wv"], inp["wo"])
    kept = None
    if keep_o:
        kept = (torch.empty((Hq, S, D), dtype=torch.bfloat16, device=dev),
                torch.empty((Hq, S), dtype=torch.float32, device=dev))

    def step():
        if keep_o:
            hcm.attn_layer_fwd(*a, Hq=Hq, Hkv=Hkv, D=D, head_chunk=hc, out=y, keep_o=True,
                               o_keep=kept[0], lse=kept[1], workspace=ws)
            hcm.attn_layer_bwd(*a, inp["dy"], Hq=Hq, Hkv=Hkv, D=D, head_chunk=hc, o_kept=kept[0],
                               lse_kept=kept[1], grads=grads, workspace=ws)
        else:
            hcm.attn_layer_fwd(*a, Hq=Hq, Hkv=Hkv, D=D, head_chunk=hc, out=y, workspace=ws)
            hcm.attn_layer_bwd(*a, inp["dy"], Hq=Hq, Hkv=Hkv, D=D, head_chunk=hc, grads=grads,
                               workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    hcm.timing_reset()
    hcm.timing_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    hcm.timing_enable(False)
    kern = hcm.timing_read()
    hcm.timing_reset()
    ms = e0.elapsed_time(e1) / steps
    peak = torch.cuda.max_memory_allocated(dev) - base
    print(f"layer {w.name}: head_chunk={hc}{', kept O' if keep_o else ''}: {ms:.1f} ms per step",
          file=sys.stderr, flush=True)
    # counted work: attention 7*S^2*D*Hq, projections 2*S*dm*D*(2 Hq + 2 Hkv) forward and
    # twice that backward (the backward's recomputation is not counted)
    proj = 2.0 * S * dm * D * (2 * Hq + 2 * Hkv)
    flops = 7.0 * S * S * D * Hq + 3 * proj
    # products executed per step: forward projections + output projection,
    # backward recomputed projections, dO, dWo, dx and the weight gradients
    gemm_flops = 4 * proj - 2.0 * S * dm * D * Hq
    gemm_ms = kern["gemm"][1] / steps
    extra = {"keep_o": True, "kept_bytes": Hq * S * D * 2 + Hq * S * 4} if keep_o else {}
    return {"head_chunk": hc, **extra, "ms_per_step": round(ms, 1),
            "tflops": round(flops / (ms / 1e3) / 1e12, 2),
            "kernel_ms_per_step": {f: round(kern[f][1] / steps, 2) for f in kern if kern[f][0]},
            "gemm_tflops": round(gemm_flops / (gemm_ms / 1e3) / 1e12, 1) if gemm_ms > 0 else None,
            "workspace_bytes": {"fwd": fb, "bwd": bb}, "peak_intermediate": peak}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this attention path has no multi-GPU mode here "
              "(the head-sharded all-to-all design is documented, not built). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import head_chunked_context_amd as hcm
    from head_chunked_context_amd.inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    hc = args.head_chunk or (w.Hq // w.Hkv if w.Hq // w.Hkv in w.head_chunks else w.head_chunks[0])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    S, Hq, Hkv, D, T = w.S, w.Hq, w.Hkv, w.D, w.kv_trunk
    if args.kv_trunk == "auto":
        T = hcm.pick_kv_trunk(S, Hq, Hkv, D, True, hc, kv_on_host=w.kv_on_host,
                              budget_bytes=int(args.budget_gib * 2**30))
    elif int(args.kv_trunk) >= 0:
        T = int(args.kv_trunk)
    causal = True

    if args.group_loop_min_s > 0:
        hcm.set_group_loop_min_s(args.group_loop_min_s)
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    r = run_workload(hcm, torch, w, hc, T, dev, args.steps, args.warmup, True, w.kv_on_host,
                     args.trunk_merge)
    flops = 7.0 * S * S * D * Hq
    tflops = flops / (r["ms"] / 1e3) / 1e12

    # roofline of the dominant kernel family in the timed region
    kern = r["kern"]
    dom = max((f for f in kern if kern[f][0] > 0), key=lambda f: kern[f][1])
    n_launch, dom_ms = kern[dom]
    alg = algorithmic_flops(dom, S, Hq, D, causal) * args.steps
    if alg > 0:
        achieved = alg / (dom_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, f"S{S}_Hq{Hq}_Hkv{Hkv}_D{D}", hc),
                "launches": n_launch, "avg_launch_ms": round(dom_ms / n_launch, 4),
                "flops_per_launch": alg / n_launch}
    else:
        roof = {"bound": "hbm", "kernel": dom, "achieved": None, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": None, "traffic": None}

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "S": S, "Hq": Hq, "Hkv": Hkv, "D": D,
                   "head_chunk": hc, "kv_trunk": T, "kv_on_host": w.kv_on_host,
                   "trunk_schedule": ("merge" if args.trunk_merge else "carry") if T else None,
                   "kv_trunk_choice": ("auto" if args.kv_trunk == "auto"
                                       else "given" if int(args.kv_trunk) >= 0 else "workload"),
                   "causal": causal, "batch": 1},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "dkdv_schedule": "group loop" if S >= group_loop_min_s(hcm) else "per head",
        "fwd_tflops": round(2.0 * S * S * D * Hq / (r["fwd_ms"] / 1e3) / 1e12, 2),
        "bwd_tflops": round(5.0 * S * S * D * Hq / (r["bwd_ms"] / 1e3) / 1e12, 2),
        "workspace_bytes": {str(hc): {"fwd": r["ws_fwd"], "bwd": r["ws_bwd"],
                                      "peak_intermediate": r["peak_intermediate"]}},
        "kernel_ms_per_step": {f: round(kern[f][1] / args.steps, 3) for f in kern if kern[f][0]},
        "roofline": roof,
        # the HBM-bound passes: algorithmic bytes (fixed by each launch's
        # parameters) over their HIP-event time, against the 8 TB/s peak
        "hbm_passes": {f: {"ms_per_step": round(kern[f][1] / args.steps, 4),
                           "bytes_per_step": r["moved"][f] / args.steps,
                           "gbs": round(r["moved"][f] / (kern[f][1] / 1e3) / 1e9, 1),
                           "frac": round(r["moved"][f] / (kern[f][1] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}
                       for f in ("pack", "prep", "merge", "reduce") if kern[f][0] and kern[f][1] > 0},
    }
    # throughput and peak workspace per head_chunk setting of the workload
    others = [h for h in w.head_chunks if h != hc]
    if not args.no_compare and others:
        sweep = {str(hc): {"value": line["value"], "ms_per_step": line["ms_per_step"]}}
        for other in others:
            r2 = run_workload(hcm, torch, w, other, T, dev, max(1, args.sweep_steps), 1, False,
                              w.kv_on_host, args.trunk_merge)
            line["workspace_bytes"][str(other)] = {"fwd": r2["ws_fwd"], "bwd": r2["ws_bwd"],
                                                   "peak_intermediate": r2["peak_intermediate"]}
            sweep[str(other)] = {"value": round(flops / (r2["ms"] / 1e3) / 1e12, 2),
                                 "ms_per_step": round(r2["ms"], 3)}
        full = str(Hq) if str(Hq) in line["workspace_bytes"] else None
        if full is not None:
            wb = line["workspace_bytes"]
            for h in sweep:
                sweep[h]["workspace_ratio_vs_unchunked"] = round(
                    max(wb[h]["fwd"], wb[h]["bwd"]) / max(wb[full]["fwd"], wb[full]["bwd"]), 4)
        line["head_chunk_sweep"] = sweep
    # forward-only (prefill) mode: no LSE kept, no backward workspace
    if not args.no_forward_only:
        rf = run_workload(hcm, torch, w, hc, T, dev, 3, 1, False, w.kv_on_host, args.trunk_merge,
                          forward_only=True)
        line["forward_only"] = {"tflops": round(2.0 * S * S * D * Hq / (rf["ms"] / 1e3) / 1e12, 2),
                                "ms": round(rf["ms"], 3), "workspace_bytes": rf["ws_fwd"],
                                "peak_intermediate": rf["peak_intermediate"]}
    # the 32B-class shape with 65536-token K/V trunks in pinned host memory:
    # the trunk copies cross PCIe inside the step (PCIe-inclusive rate)
    if not args.no_host_trunks and args.workload != 4:
        torch.cuda.empty_cache()
        w4 = WORKLOADS[4]
        r4 = run_workload(hcm, torch, w4, w4.head_chunks[0], w4.kv_trunk, dev, 1, 1, False, True)
        f4 = 7.0 * w4.S * w4.S * w4.D * w4.Hq
        line["pinned_host_trunks"] = {
            "workload": w4.name, "head_chunk": w4.head_chunks[0], "kv_trunk": w4.kv_trunk,
            "tflops": round(f4 / (r4["ms"] / 1e3) / 1e12, 2), "ms_per_step": round(r4["ms"], 1),
            "pct_bf16_peak": round(100.0 * f4 / (r4["ms"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "workspace_bytes": {"fwd": r4["ws_fwd"], "bwd": r4["ws_bwd"]},
            "peak_intermediate": r4["peak_intermediate"], "pcie_inclusive": True}
    # the attention layer around it (d_model = Hq * D): memory vs head_chunk
    if not args.no_layer and args.workload in (2, 3):
        torch.cuda.empty_cache()
        rows = [run_layer(hcm, torch, w, h, dev, 1, 1) for h in (hc, Hq)]
        rows.append(run_layer(hcm, torch, w, hc, dev, 1, 1, keep_o=True))
        line["layer"] = {"d_model": Hq * D, "settings": rows,
                         "workspace_ratio": round(max(rows[0]["workspace_bytes"].values()) /
                                                  max(rows[1]["workspace_bytes"].values()), 4)}
    if args.h2d_probe and T > 0:
        # host-to-device rate of one trunk's K and V (the per-trunk copy)
        hb = torch.empty(2 * T * Hkv * D, dtype=torch.bfloat16, pin_memory=True)
        db = torch.empty(hb.shape, dtype=hb.dtype, device=dev)
        db.copy_(hb, non_blocking=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            db.copy_(hb, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        line["h2d_probe"] = {"bytes": hb.numel() * 2, "ms": round(ms, 4),
                             "gbs": round(hb.numel() * 2 / (ms / 1e3) / 1e9, 2)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_oracle_baseline(D, Hq // Hkv, args.cpu_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
