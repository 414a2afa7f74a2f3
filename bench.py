"""Benchmark of the SpargeAttention2 hot path on one MI355X.

One step = the whole path over one synthetic layer already resident in HBM:
hybrid block mask (sa2_build_mask) -> sparse forward (sa2_attn_fwd) ->
backward (sa2_attn_bwd_dq then sa2_attn_bwd_dkdv, which is sa2_attn_bwd split
at its kernel boundary so that each kernel can be timed with HIP events).

Default workload: the Wan2.1-1.3B-shaped self-attention layer, B=1, H=12,
N=32760 (21x30x52 latent grid), d=128, bf16, q-block 128, k-block 64,
k = 3% plus Top-p tuned to 5% density (95% sparsity), forward + backward.

The timed step is that sequence captured once as a HIP graph and replayed K
times after W warm-up replays (--no-graph: K eager steps).  Per-stage times
and the roofline figure come from an eager run of the same K steps with HIP
events between the stages; its step time is reported beside the headline.

Prints one JSON line (stdout).  Effective FLOPs follow the FlashAttention
convention: forward 4 N^2 d H density, forward+backward 3.5x that.  Beside
the headline figures the line carries the dense baseline (the same kernels
with every block kept), the same layer with 64 x 64 blocks, and the fp64
oracle timed on the host.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline] [--no-graph]
    python bench.py --sweep variants   # mask rules at equal density, one line per case
    python bench.py --sweep sparsity   # the layer at densities 1 .. 0.01 (Top-k only)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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
                  "block_sparse_attention_sa2_amd/csrc/sa2_common.h",
                  "block_sparse_attention_sa2_amd/csrc/sa2_plan.h",
                  "block_sparse_attention_sa2_amd/build.py")   # compiler flags


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
    ap.add_argument("--sweep", choices=["variants", "sparsity"], default=None,
                    help="instead of the benchmark line: the mask-rule sweep (one JSON line "
                         "per regime, density and Top-k share) or the sparsity sweep of the "
                         "benchmark layer (one line per density); --steps timed steps each")
    ap.add_argument("--regimes", default=None, help="comma-separated subset of the sweep's "
                    "score regimes (sink, uniform, smooth)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager launches instead of the replayed HIP graph")
    ap.add_argument("--no-second-geometry", action="store_true",
                    help="skip the 64 x 64-block run of the same layer")
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
            "ms_per_layer": dt * 1e3 * w.H / heads, "seconds": dt, "cpu": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def dense_baseline(sa2, q, k, v, do, w, sparse_attn_ms, args):
    """The same attention kernels with every block kept (k_frac = 1): the dense
    attention this path replaces, for the sparse/dense speedup at this shape
    (the pages report 97 s -> 6 s of attention at 95% sparsity on Wan2.1-1.3B)."""
    import numpy as np
    import torch
    B, H, N, d = q.shape
    dev = q.device
    mask = sa2.BlockMask(B, H, N, w.bq, w.bk, dev)
    mws = torch.empty(sa2.mask_workspace_bytes(B, H, N, d, w.bq, w.bk), dtype=torch.uint8, device=dev)
    sa2.build_mask(q, k, w.bq, w.bk, 1.0, 0.0, mask=mask, workspace=mws)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(sa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(1, sa2.fwd_workspace_bytes(B, H, N, d)), dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    times = []
    for it in range(2 + 5):
        ev[0].record()
        sa2.attn_fwd(q, k, v, mask, o=o, lse=lse, workspace=fws)
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


def atomic_dq_backward(sa2, q, k, v, o, lse, do, mask, det_bwd_ms, steps, warmup):
    """The alternative backward: dQ formed inside the dK/dV pass and added to
    an fp32 accumulator with atomics (sa2_attn_bwd_atomic_dq), timed beside
    the deterministic dQ + dK/dV passes on the same inputs and mask."""
    import torch
    B, H, N, d = q.shape
    ws = torch.empty(sa2.bwd_atomic_workspace_bytes(B, H, N, d), dtype=torch.uint8,
                     device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    times = []
    for it in range(warmup + steps):
        ev[0].record()
        sa2.attn_bwd_atomic_dq(q, k, v, o, lse, do, mask, dq=dq, dk=dk, dv=dv, workspace=ws)
        ev[1].record()
        torch.cuda.synchronize()
        if it >= warmup:
            times.append(ev[0].elapsed_time(ev[1]))
    ms = sum(times) / len(times)
    return {"ms": round(ms, 4), "deterministic_ms": round(det_bwd_ms, 4),
            "speedup_vs_deterministic": round(det_bwd_ms / ms, 3),
            "note": "dQ by fp32 atomic adds inside the dK/dV pass (prep + fused pass + "
                    "rounding); not bitwise reproducible; the default backward is the "
                    "deterministic one"}


def graph_replay(step, steps, warmup):
    """ms per step of the same step captured once in a HIP graph (the library
    allocates nothing and records no memset) and replayed back to back: the
    kernels without host launch overhead or inter-kernel gaps."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def second_geometry(sa2, W, q, k, v, do, name="c2_b64", warmup=3, steps=10):
    """The same layer and inputs with square 64 x 64 blocks (its own tuned p for
    the same 5% density): mask + forward + backward, per-stage times."""
    import numpy as np
    import torch
    w = W.WORKLOADS[name]
    k_frac, p = W.tuned_params(name)
    B, H, N, d = q.shape
    dev = q.device
    mask = sa2.BlockMask(B, H, N, w.bq, w.bk, dev)
    mws = torch.empty(sa2.mask_workspace_bytes(B, H, N, d, w.bq, w.bk), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(sa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(1, sa2.fwd_workspace_bytes(B, H, N, d)), dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    times = []
    for it in range(warmup + steps):
        ev[0].record()
        sa2.build_mask(q, k, w.bq, w.bk, k_frac, p, mask=mask, workspace=mws)
        ev[1].record()
        sa2.attn_fwd(q, k, v, mask, o=o, lse=lse, workspace=fws)
        ev[2].record()
        sa2.attn_bwd_dq(q, k, v, o, lse, do, mask, bws, dq=dq)
        ev[3].record()
        sa2.attn_bwd_dkdv(q, k, v, lse, do, mask, bws, dk=dk, dv=dv)
        ev[4].record()
        torch.cuda.synchronize()
        if it >= warmup:
            times.append([ev[i].elapsed_time(ev[i + 1]) for i in range(4)])
    t = np.mean(np.array(times), axis=0)
    density = mask.density()
    ms = float(t.sum())
    eff = 14.0 * N * N * d * H * B * density
    return {"bq": w.bq, "bk": w.bk, "k_frac": k_frac, "p": p, "density": round(density, 5),
            "ms_per_step": round(ms, 4), "effective_tflops": round(eff / (ms * 1e-3) / 1e12, 1),
            "stages_ms": {st: round(float(x), 4) for st, x in
                          zip(("mask", "fwd", "bwd_dq", "bwd_dkdv"), t)},
            "note": "same inputs, 64 x 64 blocks, p tuned for the same density; "
                    "sum of per-stage event times"}


def _density_for(sa2, q, k, bq, bk, k_frac, target, mask, mws, steps=30):
    """p for which the hybrid mask with this k_frac has `target` density (the
    library's own masks, bisected on the host); (p, density, reached)."""
    def dens(p):
        sa2.build_mask(q, k, bq, bk, k_frac, p, mask=mask, workspace=mws)
        return mask.density()
    if k_frac > 0 and dens(0.0) >= target:
        return 0.0, dens(0.0), True
    top = dens(0.999)
    if top < target:
        return 0.999, top, False
    lo, hi, best = 0.0, 0.999, (0.999, top)
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        dm = dens(mid)
        if abs(dm - target) < abs(best[1] - target):
            best = (mid, dm)
        if abs(dm - target) <= 0.02 * target:
            break
        lo, hi = (mid, hi) if dm < target else (lo, mid)
    return best[0], best[1], True


def variant_sweep(args):
    """Mask rules at equal density over the three score regimes of the
    mask-rule stress workloads (H=8, N=16384, d=128, bf16; attention sink,
    near-uniform, smooth): Top-k only, Top-p only and hybrids whose Top-k
    share r = k_frac / density runs from 0 (Top-p only) to 1 (Top-k only),
    p tuned on the library's own masks to the target density.  Per case: the
    density reached, mask + forward + backward time, effective TFLOPS, and how
    far the sparse output is from the dense one (the layer-level distillation
    loss, mean squared difference, and the relative Frobenius error).
    One JSON line per case on stdout."""
    import numpy as np
    import torch

    import block_sparse_attention_sa2_amd as sa2
    import workloads as W

    dev = torch.device("cuda:0")
    ratios = (0.0, 0.25, 0.5, 0.6, 0.75, 1.0)
    for regime in (args.regimes.split(",") if args.regimes else W.C4_REGIMES):
        w = W.WORKLOADS[f"c4_{regime}_05"]
        log(f"[sweep] generating {regime} inputs")
        x = W.make_inputs(w)
        q, k, v, do = (W.to_device_dtype(x[t], w.dtype).to(dev) for t in ("q", "k", "v", "do"))
        del x
        B, H, N, d = q.shape
        mask = sa2.BlockMask(B, H, N, w.bq, w.bk, dev)
        mws = torch.empty(sa2.mask_workspace_bytes(B, H, N, d, w.bq, w.bk), dtype=torch.uint8,
                          device=dev)
        bws = torch.empty(sa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        fws = torch.empty(max(1, sa2.fwd_workspace_bytes(B, H, N, d)), dtype=torch.uint8,
                          device=dev)
        o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dense = sa2.BlockMask(B, H, N, w.bq, w.bk, dev)
        sa2.build_mask(q, k, w.bq, w.bk, 1.0, 0.0, mask=dense, workspace=mws)
        o_dense, _ = sa2.attn_fwd(q, k, v, dense, workspace=fws)
        ref_norm = float(o_dense.float().norm())
        for D in W.C4_DENSITIES:
            for r in ratios:
                k_frac = round(r * D, 6)
                if r >= 1.0:
                    p, dens, reached = 0.0, None, True
                else:
                    p, dens, reached = _density_for(sa2, q, k, w.bq, w.bk, k_frac, D, mask, mws)
                # steps queued back to back, one synchronisation at the end; the
                # median per stage is robust to a stalled host thread
                evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
                       for _ in range(2 + args.steps)]
                for ev in evs:
                    ev[0].record()
                    sa2.build_mask(q, k, w.bq, w.bk, k_frac, p, mask=mask, workspace=mws)
                    ev[1].record()
                    sa2.attn_fwd(q, k, v, mask, o=o, lse=lse, workspace=fws)
                    ev[2].record()
                    sa2.attn_bwd_dq(q, k, v, o, lse, do, mask, bws, dq=dq)
                    ev[3].record()
                    sa2.attn_bwd_dkdv(q, k, v, lse, do, mask, bws, dk=dk, dv=dv)
                    ev[4].record()
                torch.cuda.synchronize()
                times = [[ev[i].elapsed_time(ev[i + 1]) for i in range(4)] for ev in evs[2:]]
                stage = np.median(np.array(times), axis=0)
                ms = float(stage.sum())
                ccnt = mask.col_cnt.reshape(-1).float()
                rcnt = mask.row_cnt.reshape(-1).float()
                dens = mask.density()
                loss, _ = sa2.distill_loss_grad(o, o_dense)
                loss = float(loss.item())
                rule = "top-p only" if r == 0 else "top-k only" if r >= 1 else "hybrid"
                print(json.dumps({
                    "regime": regime, "target_density": D, "rule": rule, "topk_share": r,
                    "k_frac": k_frac, "p": round(p, 6), "density": round(dens, 5),
                    "target_reached": reached and abs(dens - D) <= 0.05 * D,
                    "ms_mask_fwd_bwd": round(ms, 4),
                    "stages_ms": {st: round(float(x), 4) for st, x in
                                  zip(("mask", "fwd", "bwd_dq", "bwd_dkdv"), stage)},
                    "row_cnt_max": int(rcnt.max()), "col_cnt_max": int(ccnt.max()),
                    "pairs_per_block_mean": round(float(rcnt.mean()), 2),
                    "effective_tflops": round(14.0 * N * N * d * H * B * dens / (ms * 1e-3) / 1e12, 1),
                    "distill_loss": loss,
                    "rel_err_vs_dense": math.sqrt(loss * o.numel()) / ref_norm}), flush=True)
        del q, k, v, do, o, dq, dk, dv, o_dense
        torch.cuda.empty_cache()


SWEEP_DENSITIES = (1.0, 0.5, 0.25, 0.1, 0.05, 0.025, 0.01)


def sparsity_sweep(args):
    """The benchmark layer (same inputs) at a ladder of densities, Top-k only
    (k_frac = density, so every row keeps the same number of key blocks):
    mask + forward + backward time per stage (medians of --steps queued
    steps), effective TFLOPS, and the attention speedup over the dense run of
    the same kernels.  One JSON line per density on stdout."""
    import numpy as np
    import torch

    import block_sparse_attention_sa2_amd as sa2
    import workloads as W

    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    log(f"[sweep] generating {w.name} inputs")
    x = W.make_inputs(w)
    q, k, v, do = (W.to_device_dtype(x[t], w.dtype).to(dev) for t in ("q", "k", "v", "do"))
    del x
    B, H, N, d = q.shape
    mask = sa2.BlockMask(B, H, N, w.bq, w.bk, dev)
    mws = torch.empty(sa2.mask_workspace_bytes(B, H, N, d, w.bq, w.bk), dtype=torch.uint8,
                      device=dev)
    bws = torch.empty(sa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(1, sa2.fwd_workspace_bytes(B, H, N, d)), dtype=torch.uint8, device=dev)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dense_attn = None
    for D in SWEEP_DENSITIES:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
               for _ in range(2 + args.steps)]
        for ev in evs:
            ev[0].record()
            sa2.build_mask(q, k, w.bq, w.bk, D, 0.0, mask=mask, workspace=mws)
            ev[1].record()
            sa2.attn_fwd(q, k, v, mask, o=o, lse=lse, workspace=fws)
            ev[2].record()
            sa2.attn_bwd_dq(q, k, v, o, lse, do, mask, bws, dq=dq)
            ev[3].record()
            sa2.attn_bwd_dkdv(q, k, v, lse, do, mask, bws, dk=dk, dv=dv)
            ev[4].record()
        torch.cuda.synchronize()
        stage = np.median(np.array([[ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
                                    for ev in evs[2:]]), axis=0)
        dens = mask.density()
        attn_ms = float(stage[1:].sum())
        if dense_attn is None:
            dense_attn = attn_ms
        flops = 14.0 * N * N * d * H * B * dens
        print(json.dumps({
            "workload": w.name, "k_frac": D, "density": round(dens, 5),
            "sparsity": round(1 - dens, 5),
            "stages_ms": dict(zip(("mask", "fwd", "bwd_dq", "bwd_dkdv"),
                                  (round(float(t), 4) for t in stage))),
            "ms_per_step": round(float(stage.sum()), 4),
            "effective_tflops": round(flops / (float(stage.sum()) * 1e-3) / 1e12, 1),
            "attention_effective_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 1),
            "speedup_attention_vs_dense": round(dense_attn / attn_ms, 2)}), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the hot path is measured per GPU (heads shard "
              "with no exchange); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.sweep == "variants":
        variant_sweep(args)
        return
    if args.sweep == "sparsity":
        sparsity_sweep(args)
        return

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
    mask = sa2.BlockMask(B, H, N, w.bq, w.bk, dev)
    mws = torch.empty(sa2.mask_workspace_bytes(B, H, N, d, w.bq, w.bk), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(sa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(1, sa2.fwd_workspace_bytes(B, H, N, d)), dtype=torch.uint8, device=dev)
    backward = w.backward and do is not None
    stages = ["mask", "fwd"] + (["bwd_dq", "bwd_dkdv"] if backward else [])

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        sa2.build_mask(q, k, w.bq, w.bk, k_frac, p, mask=mask, workspace=mws)
        mark(1)
        sa2.attn_fwd(q, k, v, mask, o=o, lse=lse, workspace=fws)
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
    eager_ms = wall * 1e3 / args.steps
    per = {st: float(np.mean([events[s][i].elapsed_time(events[s][i + 1])
                              for s in range(args.steps)])) for i, st in enumerate(stages)}
    # the timed step: the same step captured once as a HIP graph and replayed
    # (K replays after W, synchronised on both sides), unless --no-graph
    graph_ms, graph_error = None, None
    if not args.no_graph:
        try:
            graph_ms = graph_replay(step, args.steps, args.warmup)
        except RuntimeError as e:   # capture refused by the runtime: report eager timing
            graph_error = str(e).splitlines()[0][:200]
            log(f"[bench] graph capture failed ({graph_error}); timing eager launches")
            torch.cuda.synchronize()
    ms_step = graph_ms if graph_ms is not None else eager_ms

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
    traffic = recorded_traffic(name, args.workload)
    roofline = {"bound": "mfma", "kernel": name, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic,
                "per_launch": {"algorithmic_flop": alg, "executed_flop": exe, "ms": round(per[dom], 4)}}
    if traffic is not None:
        # the memory side of the same launch: measured HBM bytes over its live duration
        gbps = traffic / (per[dom] * 1e-3) / 1e9
        roofline["traffic_GBps"] = round(gbps, 1)
        roofline["traffic_frac_of_hbm_peak"] = round(gbps / PEAK_HBM_GBPS, 4)
    qk_bytes = 2.0 * B * H * N * d * q.element_size()
    mask_gbps = qk_bytes / (per["mask"] * 1e-3) / 1e9
    executed = sum(kernels[st][2] for st in kernels)
    attn_ms = sum(per[st] for st in kernels)

    out = {
        "metric": (f"effective TFLOPS + ms/layer {'fwd+bwd' if backward else 'fwd'}, "
                   f"{round(100 * (1 - (w.target_density or density)))}% sparse, "
                   f"H={H} N={N} d={d} {w.dtype}"),
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
    out["timing"] = {
        "ms_per_step": round(ms_step, 4),
        "mode": ("HIP graph replay of the captured step" if graph_ms is not None else
                 "eager launches" + (f" (graph capture failed: {graph_error})" if graph_error else "")),
        "eager_ms_per_step": round(eager_ms, 4),
        "note": "stages_ms and the roofline come from the eager run, with HIP events between "
                "the stages"}
    if backward:
        out["atomic_dq_backward"] = atomic_dq_backward(
            sa2, q, k, v, o, lse, do, mask, per["bwd_dq"] + per["bwd_dkdv"], args.steps,
            args.warmup)
    if not args.no_dense_baseline and backward:
        out["dense_baseline"] = dense_baseline(sa2, q, k, v, do, w, attn_ms, args)
    if args.workload == "c2" and not args.no_second_geometry:
        out["second_geometry"] = second_geometry(sa2, W, q, k, v, do)
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on {args.cpu_heads} head(s)")
        ref1 = {k_: v_ for k_, v_ in ref.items()}
        out["cpu_baseline"] = cpu_baseline(w, k_frac, p, ref1, args.cpu_heads, eff_flops)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
