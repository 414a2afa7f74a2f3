"""Benchmark of the SpargeAttention2 hot path on one MI355X.

One step = the whole path over one synthetic layer already resident in HBM:
hybrid block mask (sa2_build_mask) -> sparse forward (sa2_attn_fwd) ->
backward (sa2_attn_bwd_dq then sa2_attn_bwd_dkdv, which is sa2_attn_bwd split
at its kernel boundary so that each kernel can be timed with HIP events).

Default workload: the Wan2.1-1.3B-shaped self-attention layer, B=1, H=12,
N=32760 (21x30x52 latent grid), d=128, bf16, q-block 128, k-block 64,
k = 3% plus Top-p tuned to 5% density (95% sparsity), forward + backward.

Prints one JSON line (stdout).  Effective FLOPs follow the FlashAttention
convention: forward 4 N^2 d H density, forward+backward 3.5x that.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# HBM bytes per launch of the attention kernels, from rocprofv3 FETCH_SIZE /
# WRITE_SIZE runs (scaled by a copy of known size), recorded with a digest of
# the kernel sources they were taken on; used only while the sources match.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "wan13_layer_hbm_traffic.md")
KERNEL_SOURCES = ("block_sparse_attention_sa2_amd/csrc/sa2_attn.hip",
                  "block_sparse_attention_sa2_amd/csrc/sa2_common.h")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str):
    """Measured HBM bytes per launch of `kernel` on `workload`, or None if the
    record is missing or was taken on another workload or other sources."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            line = next(l for l in fh if l.startswith("traffic-record "))
        rec = json.loads(line[len("traffic-record "):])
    except (OSError, StopIteration, ValueError):
        return None
    if (rec.get("source_digest") != kernel_source_digest() or rec.get("workload") != workload
            or kernel not in rec.get("kernels", {})):
        return None
    k = rec["kernels"][kernel]
    return float(k["fetch_bytes"] + k["write_bytes"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2", help="workload key (default: 1.3B layer fwd+bwd)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads the oracle times (default: the whole layer)")
    ap.add_argument("--no-work-order", action="store_true",
                    help="schedule the attention kernels in their fixed order")
    ap.add_argument("--no-dense-baseline", action="store_true",
                    help="skip the dense (all blocks kept) run of the same kernels")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only copy BYTES once on the GPU (calibrates the HBM byte counters)")
    return ap.parse_args()


def copy_probe(nbytes: int) -> None:
    """One device-to-device copy of a known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": src.numel() * 4}), flush=True)


def cpu_baseline(w, k_frac, p, ref, heads, eff_flops_layer):
    """The fp64 oracle on `heads` heads of the same inputs (mask, forward, backward)."""
    import numpy as np
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    for h in range(heads):
        Q, K, V, dO = (ref[t][0, h] for t in ("q", "k", "v", "do"))
        hm = O.build_mask_head(Q, K, w.bq, w.bk, k_frac, p)
        O.attention_gathered(Q, K, V, hm.row_lists(), w.bq, w.bk, dO=dO)
    dt = time.perf_counter() - t0
    flops = eff_flops_layer * heads / w.H
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of {w.H} heads of the same layer (mask + forward + backward, "
                      f"numpy fp64, gathered over kept blocks); {dt:.2f} s; "
                      f"ms/layer extrapolated x{w.H // heads if w.H % heads == 0 else w.H / heads:.3g}",
            "ms_per_layer": dt * 1e3 * w.H / heads, "seconds": dt,
            "cpu": platform.processor() or platform.machine()}


def dense_baseline(sa2, q, k, v, do, w, sparse_attn_ms, args):
    """The same attention kernels with every block kept (k_frac = 1): the dense
    attention this path replaces, for the sparse/dense speedup at this shape
    (the pages report 97 s -> 6 s of attention at 95% sparsity on Wan2.1-1.3B)."""
    import numpy as np
    import torch
    B, H, N, d = q.shape
    dev = q.device
    mask = sa2.BlockMask(B, H, N, w.bq, w.bk, dev, work_order=True)
    mws = torch.empty(sa2.mask_workspace_bytes(B, H, N, d, w.bq, w.bk), dtype=torch.uint8, device=dev)
    sa2.build_mask(q, k, w.bq, w.bk, 1.0, 0.0, mask=mask, workspace=mws)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(sa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    times = []
    for it in range(2 + 5):
        ev[0].record()
        sa2.attn_fwd(q, k, v, mask, o=o, lse=lse)
        ev[1].record()
        sa2.attn_bwd_dq(q, k, v, o, lse, do, mask, bws, dq=dq)
        ev[2].record()
        sa2.attn_bwd_dkdv(q, k, v, lse, do, mask, bws, dk=dk, dv=dv)
        ev[3].record()
        torch.cuda.synchronize()
        if it >= 2:
            times.append([ev[i].elapsed_time(ev[i + 1]) for i in range(3)])
    t = np.mean(np.array(times), axis=0)
    dense_ms = float(t.sum())
    dense_flops = 14.0 * N * N * d * H * B     # forward + backward, every block kept
    return {"density": round(mask.density(), 5), "attention_ms": round(dense_ms, 4),
            "stages_ms": {"fwd": round(float(t[0]), 4), "bwd_dq": round(float(t[1]), 4),
                          "bwd_dkdv": round(float(t[2]), 4)},
            "effective_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 1),
            "speedup_attention": round(dense_ms / sparse_attn_ms, 2),
            "note": "same kernels and shape, all blocks kept; speedup = dense / sparse "
                    "attention time (forward + backward, mask excluded)"}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the hot path is measured per GPU (heads shard "
              "with no exchange); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_sa2_amd as sa2
    import workloads as W

    w = W.WORKLOADS[args.workload]
    k_frac, p = W.tuned_params(args.workload)
    dev = torch.device("cuda:0")
    log(f"[bench] {w.name}: B{w.B} H{w.H} N{w.N} d{w.d} bq{w.bq} bk{w.bk} {w.dtype} "
        f"k_frac={k_frac} p={p:.6f}")
    x = W.make_inputs(w)
    ref = {}
    t = {}
    for name, arr in x.items():
        tt = W.to_device_dtype(arr, w.dtype)
        if not args.no_cpu_baseline:
            ref[name] = tt.to(torch.float64).numpy()[:, :args.cpu_heads].copy()
        t[name] = tt.to(dev)
    del x
    q, k, v = t["q"], t["k"], t["v"]
    do = t.get("do")
    B, H, N, d = q.shape

    # everything the step touches is allocated once, outside the timed region
    mask = sa2.BlockMask(B, H, N, w.bq, w.bk, dev, work_order=not args.no_work_order)
    mws = torch.empty(sa2.mask_workspace_bytes(B, H, N, d, w.bq, w.bk), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(sa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    backward = w.backward and do is not None
    stages = ["mask", "fwd"] + (["bwd_dq", "bwd_dkdv"] if backward else [])

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        sa2.build_mask(q, k, w.bq, w.bk, k_frac, p, mask=mask, workspace=mws)
        mark(1)
        sa2.attn_fwd(q, k, v, mask, o=o, lse=lse)
        mark(2)
        if backward:
            sa2.attn_bwd_dq(q, k, v, o, lse, do, mask, bws, dq=dq)
            mark(3)
            sa2.attn_bwd_dkdv(q, k, v, lse, do, mask, bws, dk=dk, dv=dv)
            mark(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    density = mask.density()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    per = {st: float(np.mean([events[s][i].elapsed_time(events[s][i + 1])
                              for s in range(args.steps)])) for i, st in enumerate(stages)}

    fwd_flops = 4.0 * N * N * d * H * B * density
    eff_flops = fwd_flops * (3.5 if backward else 1.0)
    value = eff_flops / (ms_step * 1e-3) / 1e12

    # per-kernel algorithmic work (each attention stage is exactly one kernel)
    unit = 2.0 * N * N * d * H * B * density          # one GEMM over the kept pairs
    # (the bf16, d = 128 kernels each stage launches)
    kernels = {"fwd": ("fwd_async_kernel", 2 * unit, 2 * unit)}
    if backward:
        kernels["bwd_dq"] = ("dq_async_kernel", 1 * unit, 3 * unit)     # S, dP recomputed
        kernels["bwd_dkdv"] = ("dkdv_pair_kernel", 4 * unit, 4 * unit)
    dom = max(kernels, key=lambda st: per[st])
    name, alg, exe = kernels[dom]
    achieved = alg / (per[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": name, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(name, args.workload),
                "per_launch": {"algorithmic_flop": alg, "executed_flop": exe, "ms": round(per[dom], 4)}}
    qk_bytes = 2.0 * B * H * N * d * q.element_size()
    mask_gbps = qk_bytes / (per["mask"] * 1e-3) / 1e9
    executed = sum(kernels[st][2] for st in kernels)
    attn_ms = sum(per[st] for st in kernels)

    out = {
        "metric": "effective TFLOPS + ms/layer fwd+bwd, 95% sparse, H=12 N=32760 d=128 bf16",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (smooth 3D-grid signal + noise, seeded)",
        "config": {"workload": "Wan2.1-1.3B-shaped self-attention layer, fwd+bwd" if args.workload == "c2" else w.name,
                   "B": B, "H": H, "N": N, "d": d, "bq": w.bq, "bk": w.bk, "k_frac": k_frac,
                   "p": p, "density": round(density, 5), "sparsity": round(1 - density, 5),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "stages_ms": {k_: round(v_, 4) for k_, v_ in per.items()},
        "mfma_util_executed": round(executed / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "mask_builder": {"ms": round(per["mask"], 4), "qk_read_bytes": qk_bytes,
                         "GBps_whole_call": round(mask_gbps, 1), "peak_GBps": PEAK_HBM_GBPS},
    }
    if not args.no_dense_baseline and backward:
        out["dense_baseline"] = dense_baseline(sa2, q, k, v, do, w, attn_ms, args)
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on {args.cpu_heads} head(s)")
        ref1 = {k_: v_ for k_, v_ in ref.items()}
        out["cpu_baseline"] = cpu_baseline(w, k_frac, p, ref1, args.cpu_heads, eff_flops)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
