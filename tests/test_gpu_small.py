"""GPU parity on small shapes: every output element against the fp64 oracle.

Covers the tiny CPU-checkable workload (B=1, H=2, N=1024, d=64, 64x64 blocks,
k = 2 blocks, p = 0.9; plus its two variants that make Top-k, and both rules,
active), ragged shapes spanning several tiles in both block geometries and
both element types, and the degenerate cases: one partial block, dense masks
(k = 100% or p = 1), a single rule, and reproducibility.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_sa2_amd as sa2
import oracle as O
import workloads as W

from parity import (check_forward, check_grad, check_lists, check_plans, compare_mask,
                    device_inputs, f64, log_parity)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()


def run_case(w: W.Workload, k_frac: float, p: float, backward: bool = True,
             attn_on_bf16_operands: bool = False):
    """Mask from the inputs as given; attention against the oracle.

    attn_on_bf16_operands: the attention multiplies bf16-rounded operands by
    contract (fp32 inputs are rounded to bf16 as they are loaded); set it for
    fp32 inputs whose logits are so large that the input rounding alone
    exceeds the tolerance, so that the oracle sees the same Q, K, V and dO
    (the mask is still compared on the unrounded inputs).
    """
    _say(f"[case] {w.name} B{w.B} H{w.H} N{w.N} d{w.d} bq{w.bq} bk{w.bk} {w.dtype} k{k_frac} p{p}")
    dev, ref = device_inputs(w) if w.B == 1 else _multi_batch(w)
    q, k, v = dev["q"], dev["k"], dev["v"]
    mask = sa2.build_mask(q, k, w.bq, w.bk, k_frac, p)
    o, lse = sa2.attn_fwd(q, k, v, mask)
    if backward:
        dq, dk, dv = sa2.attn_bwd(q, k, v, o, lse, dev["do"], mask)
    torch.cuda.synchronize()
    bm = mask.bitmap.cpu().numpy()
    rc, ri = mask.row_cnt.cpu().numpy(), mask.row_idx.cpu().numpy()
    cc, ci = mask.col_cnt.cpu().numpy(), mask.col_idx.cpu().numpy()
    check_plans(mask)   # after the attention calls, which leave the counters zeroed
    stats = []
    worst = dict(o_max=0.0, o_mean=0.0, dq=0.0, dk=0.0, dv=0.0)
    for b in range(w.B):
        for h in range(w.H):
            Q, K, V = (ref[t][b, h] for t in ("q", "k", "v"))
            dO = ref["do"][b, h]
            hm = O.build_mask_head(Q, K, w.bq, w.bk, k_frac, p)
            compare_mask(hm, bm[b, h], p)
            check_lists(bm[b, h], rc[b, h], ri[b, h], cc[b, h], ci[b, h])
            if attn_on_bf16_operands:
                Q, K, V, dO = _bf16(Q), _bf16(K), _bf16(V), _bf16(dO)
            Oo, L, P = O.attention_dense(Q, K, V, bm[b, h], w.bq, w.bk)
            st = check_forward(f64(o[b, h]), f64(lse[b, h]), Oo, L, f"{w.name} b{b}h{h}")
            stats.append(st)
            worst["o_max"] = max(worst["o_max"], st[0])
            worst["o_mean"] = max(worst["o_mean"], st[1])
            if backward:
                rq, rk, rv = O.attention_dense_bwd(Q, K, V, dO, P)
                for name, mine, want in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
                    r = check_grad(f64(mine[b, h]), want, f"{w.name} b{b}h{h} {name}")
                    worst[name] = max(worst[name], r)
    _say(f"[case] {w.name} worst: " + ", ".join(f"{k_} {v_:.2e}" for k_, v_ in worst.items()))
    log_parity("small", w.name, **worst)
    return mask, stats


def _multi_batch(w):
    """B > 1: batch entries drawn as independent heads of a one-batch workload."""
    from dataclasses import replace
    w1 = replace(w, B=1, H=w.B * w.H)
    dev, ref = device_inputs(w1)
    shape = lambda t: t.reshape(w.B, w.H, w.N, w.d)
    return ({k_: shape(t).contiguous() for k_, t in dev.items()},
            {k_: a.reshape(w.B, w.H, w.N, w.d) for k_, a in ref.items()})


def test_tiny_workload():
    w = W.WORKLOADS["c0"]
    mask, _ = run_case(w, *W.tuned_params("c0"))
    assert np.all(mask.row_cnt.cpu().numpy() >= 2)


def test_tiny_workload_topk_active():
    # shared Q/K signal at amplitude 2: logits near 150, nearly one-hot
    # attention rows and |O| up to 15; every output against the oracle on the
    # bf16-rounded operands (see run_case)
    w = W.WORKLOADS["c0b"]
    mask, _ = run_case(w, *W.tuned_params("c0b"), attn_on_bf16_operands=True)
    assert (mask.row_cnt.cpu().numpy() == 2).mean() > 0.5     # Top-k decides most rows


def test_tiny_workload_both_rules_active():
    w = W.WORKLOADS["c0c"]
    run_case(w, *W.tuned_params("c0c"))


SMALL = [
    W.Workload("r128_bf16", 1, 2, 1000, 128, 128, 64, "normal", 11, "bf16", 0.1, 0.5),
    W.Workload("r64_f32", 1, 2, 777, 64, 64, 64, "normal", 12, "f32", 0.1, 0.6),
    W.Workload("r128_f32", 1, 1, 1111, 128, 128, 64, "normal", 13, "f32", 0.05, 0.7),
    W.Workload("r64_bf16_d128", 1, 2, 900, 128, 64, 64, "normal", 14, "bf16", 0.2, 0.3),
    W.Workload("r128_bf16_d64", 1, 1, 1300, 64, 128, 64, "normal", 15, "bf16", 0.08, 0.8),
    W.Workload("smooth_4k", 1, 1, 4096, 128, 128, 64, "smooth", 16, "bf16", 0.05, 0.5,
               grid=(4, 32, 32)),
    W.Workload("batch2", 2, 2, 640, 64, 64, 64, "normal", 17, "bf16", 0.2, 0.5),
    W.Workload("batch2_d128", 2, 3, 900, 128, 128, 64, "normal", 18, "bf16", 0.1, 0.5),
    W.Workload("batch3_d128_q64", 3, 1, 700, 128, 64, 64, "normal", 19, "bf16", 0.15, 0.4),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_ragged_shapes(w):
    run_case(w, w.k_frac, w.p)


@pytest.mark.parametrize("N", [50, 1])
def test_single_partial_block(N):
    """One query and one key block, partial (50 tokens) or a single token."""
    w = W.Workload(f"n{N}", 1, 2, N, 64, 64, 64, "normal", 20, "bf16", 0.5, 0.5)
    mask, _ = run_case(w, 0.5, 0.5)
    assert mask.Tq == 1 and mask.Tk == 1


@pytest.mark.parametrize("k_frac,p", [(1.0, 0.0), (0.0, 1.0), (0.3, 1.0)])
def test_dense_masks(k_frac, p):
    w = W.Workload("dense", 1, 1, 700, 64, 64, 64, "normal", 21, "bf16", k_frac, p)
    mask, _ = run_case(w, k_frac, p)
    assert mask.bitmap.all()


@pytest.mark.parametrize("k_frac,p", [(0.1, 0.0), (0.0, 0.4)])
def test_single_rule(k_frac, p):
    w = W.Workload("one_rule", 1, 2, 1024, 64, 64, 64, "normal", 22, "bf16", k_frac, p)
    run_case(w, k_frac, p)


ATOMIC_DQ = [w for w in SMALL if w.dtype == "bf16" and w.d == 128] + [
    W.Workload("atomic_split", 1, 2, 2000, 128, 128, 64, "normal", 33, "bf16", 1.0, 0.0)]


@pytest.mark.parametrize("w", ATOMIC_DQ, ids=[w.name for w in ATOMIC_DQ])
def test_atomic_dq_backward(w):
    """The fused backward (dQ by fp32 atomics inside the dK/dV pass): dQ, dK,
    dV against the oracle; dK and dV also against the deterministic backward
    (the same arithmetic apart from Delta's summation order)."""
    _say(f"[atomic dQ] {w.name} B{w.B} H{w.H} N{w.N} bq{w.bq} k{w.k_frac} p{w.p}")
    dev, ref = device_inputs(w) if w.B == 1 else _multi_batch(w)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    mask = sa2.build_mask(q, k, w.bq, w.bk, w.k_frac, w.p)
    o, lse = sa2.attn_fwd(q, k, v, mask)
    gq, gk, gv = sa2.attn_bwd_atomic_dq(q, k, v, o, lse, do, mask)
    dq, dk, dv = sa2.attn_bwd(q, k, v, o, lse, do, mask)
    torch.cuda.synchronize()
    bm = mask.bitmap.cpu().numpy()
    worst = dict(dq=0.0, dk=0.0, dv=0.0)
    for b in range(w.B):
        for h in range(w.H):
            Q, K, V, dO = (ref[t][b, h] for t in ("q", "k", "v", "do"))
            _, _, P = O.attention_dense(Q, K, V, bm[b, h], w.bq, w.bk)
            for name, mine, want in zip(("dq", "dk", "dv"), (gq, gk, gv),
                                        O.attention_dense_bwd(Q, K, V, dO, P)):
                worst[name] = max(worst[name], check_grad(f64(mine[b, h]), want,
                                                          f"atomic {w.name} b{b}h{h} {name}"))
    for a_, b_ in ((gk, dk), (gv, dv), (gq, dq)):
        assert float((a_.float() - b_.float()).norm() / b_.float().norm()) <= 1e-2
    log_parity("atomic_dq", w.name, **worst)


def test_both_rules_off_is_an_error():
    q = torch.zeros(1, 1, 128, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="SA2_EINVAL"):
        sa2.build_mask(q, q, 64, 64, 0.0, 0.0)


@pytest.mark.parametrize("N,bq", [(2000, 128), (1100, 64)])
def test_long_column_lists_are_split(N, bq):
    """Dense masks: every key block's column list is longer than the dK/dV
    plan's shortest segment, so each list is cut into segments whose fp32
    partial sums the reduce kernel adds; all of dK, dV against the oracle."""
    w = W.Workload(f"split{bq}", 1, 2, N, 128, bq, 64, "normal", 26, "bf16", 1.0, 0.0)
    mask, _ = run_case(w, 1.0, 0.0)
    assert int(mask.col_cnt.min().item()) > 8


@pytest.mark.parametrize("N,bq", [(2000, 128), (1100, 64)])
def test_long_row_lists_are_split(N, bq):
    """Dense masks on a small grid: every query block's row list is longer
    than the row plan's segment length, so every row of the forward and of
    dQ is cut into segments whose partials the last segment combines (and
    every column of dK/dV); the plans check out against the counts, and O,
    LSE, dQ, dK, dV match the oracle."""
    w = W.Workload(f"rowsplit{bq}", 1, 2, N, 128, bq, 64, "normal", 32, "bf16", 1.0, 0.0)
    dev, _ = device_inputs(w)
    mask = sa2.build_mask(dev["q"], dev["k"], w.bq, w.bk, 1.0, 0.0)
    torch.cuda.synchronize()
    rows_split, cols_split = check_plans(mask)
    assert rows_split == 2 * mask.Tq and cols_split == 2 * mask.Tk
    run_case(w, 1.0, 0.0)


@pytest.mark.parametrize("k_frac,p", [(0.1, 0.5), (1.0, 0.0)], ids=["hybrid", "dense_split"])
def test_reproducible_and_fully_written(k_frac, p):
    """Two runs agree bit for bit; outputs pre-filled with NaN are fully
    overwritten (with every block kept, every row list of the forward and dQ
    and every dK/dV column list is split and combined by its last segment)."""
    w = W.Workload("repro", 1, 2, 1500, 128, 128, 64, "normal", 23, "bf16", k_frac, p)
    dev, _ = device_inputs(w)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    outs = []
    for _ in range(2):
        mask = sa2.build_mask(q, k, w.bq, w.bk, w.k_frac, w.p)
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), device=q.device)
        sa2.attn_fwd(q, k, v, mask, o=o, lse=lse)
        grads = [torch.full_like(q, float("nan")) for _ in range(3)]
        sa2.attn_bwd(q, k, v, o, lse, do, mask, *grads)
        torch.cuda.synchronize()
        for t in (o, lse, *grads):
            assert torch.isfinite(t).all()
        outs.append([mask.bitmap.clone(), o, lse, *grads])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_caller_written_lists_get_plans():
    """A mask whose lists the caller wrote (here copied from a built mask)
    gets its plans from sa2_mask_plans; the attention results are the same."""
    w = W.Workload("ownlists", 1, 2, 1000, 128, 128, 64, "normal", 25, "bf16", 0.1, 0.5)
    dev, _ = device_inputs(w)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    built = sa2.build_mask(q, k, w.bq, w.bk, w.k_frac, w.p)
    own = sa2.BlockMask(1, 2, w.N, w.bq, w.bk, q.device)
    for name in ("bitmap", "row_cnt", "row_idx", "col_cnt", "col_idx"):
        getattr(own, name).copy_(getattr(built, name))
    own.remake_plans()
    outs = []
    for m in (built, own):
        o, lse = sa2.attn_fwd(q, k, v, m)
        grads = sa2.attn_bwd(q, k, v, o, lse, do, m)
        torch.cuda.synchronize()
        outs.append([o, lse, *grads])
    assert torch.equal(built.row_plan, own.row_plan) and torch.equal(built.col_plan, own.col_plan)
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_binding_refuses_malformed_outputs():
    """Caller-supplied outputs and workspaces of the wrong shape, dtype or
    layout are refused before any launch (the kernels would write past them)."""
    dev = torch.device("cuda:0")
    B, H, N, d = 1, 2, 256, 64
    g = torch.Generator().manual_seed(3)
    q, k, v, do = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
                   for _ in range(4))
    mask = sa2.build_mask(q, k, 64, 64, 0.25, 0.5)
    with pytest.raises(ValueError):
        sa2.attn_fwd(q, k, v, mask, o=torch.empty(B, H, N - 1, d, dtype=q.dtype, device=dev))
    with pytest.raises(ValueError):
        sa2.attn_fwd(q, k, v, mask, lse=torch.empty(B, H, N, dtype=torch.float16, device=dev))
    with pytest.raises(ValueError):
        sa2.attn_fwd(q, k, v, mask, o=torch.empty(B, H, d, N, dtype=q.dtype, device=dev).transpose(2, 3))
    o, lse = sa2.attn_fwd(q, k, v, mask)
    with pytest.raises(ValueError):
        sa2.attn_bwd(q, k, v, o, lse, do, mask, dk=torch.empty(B, H, N, d, dtype=torch.float32,
                                                               device=dev))
    with pytest.raises(ValueError):
        sa2.attn_bwd(q, k, v, o, lse, do, mask,
                     workspace=torch.empty(1 << 20, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        sa2.build_mask(q, k, 64, 64, 0.25, 0.5, workspace=torch.empty(4, dtype=torch.int64,
                                                                      device=dev))
    torch.cuda.synchronize()


def test_autograd_wrapper():
    w = W.Workload("autograd", 1, 1, 512, 64, 64, 64, "normal", 24, "bf16", 0.25, 0.5)
    dev, ref = device_inputs(w)
    q, k, v = (dev[t].clone().requires_grad_() for t in ("q", "k", "v"))
    mask = sa2.build_mask(q.detach(), k.detach(), 64, 64, 0.25, 0.5)
    out = sa2.sparse_attention(q, k, v, mask)
    out.backward(dev["do"])
    torch.cuda.synchronize()
    bm = mask.bitmap.cpu().numpy()[0, 0]
    Q, K, V, dO = (ref[t][0, 0] for t in ("q", "k", "v", "do"))
    _, _, P = O.attention_dense(Q, K, V, bm, 64, 64)
    for g, want, name in zip((q.grad, k.grad, v.grad), O.attention_dense_bwd(Q, K, V, dO, P),
                             ("dq", "dk", "dv")):
        check_grad(f64(g[0, 0]), want, name)


DISTILL_BF16 = W.Workload("distill_bf16_d128", 1, 2, 1000, 128, 128, 64, "normal", 27, "bf16",
                          0.1, 0.5)


@pytest.mark.parametrize("w,k_frac,p", [(W.WORKLOADS["c0"], 0.25, 0.0),
                                        (W.WORKLOADS["c0c"], 0.125, 0.3),
                                        (DISTILL_BF16, 0.1, 0.5)],
                         ids=["c0_f32_d64", "c0c_f32_d64", "bf16_d128"])
def test_distillation_step(w, k_frac, p):
    """Layer-level velocity distillation (gist.science 2B): the sparse student
    fitted to the dense teacher.  Loss within 2e-2 relative and the gradients
    within the backward bar of the oracle's step on the same masks; on the
    fp32/d = 64 kernels and on the bf16/d = 128 ones the layers use."""
    _say(f"[case] distill {w.name} k{k_frac} p{p}")
    dev, ref = device_inputs(w)
    q, k, v = dev["q"], dev["k"], dev["v"]
    mask = sa2.build_mask(q, k, w.bq, w.bk, k_frac, p)
    dense = sa2.build_mask(q, k, w.bq, w.bk, 1.0, 0.0)
    loss, dq, dk, dv, o_s, o_t = sa2.distill_step(q, k, v, mask, dense)
    torch.cuda.synchronize()
    assert dense.density() == 1.0
    rc, ri = mask.row_cnt.cpu().numpy(), mask.row_idx.cpu().numpy()
    total = 0.0
    grads = []
    for h in range(w.H):
        rows = [ri[0, h, i, :rc[0, h, i]] for i in range(rc.shape[2])]
        Q, K, V = (ref[t][0, h] for t in ("q", "k", "v"))
        lh, gq, gk, gv, _, _ = O.distill_step(Q, K, V, rows, w.bq, w.bk)
        total += lh
        grads.append((gq, gk, gv))
    want = total / w.H                     # the mean over every element of every head
    got = float(loss.item())
    assert abs(got - want) <= 2e-2 * want, (got, want)
    # the oracle's per-head gradients are of its per-head mean; the step's loss
    # is the mean over all H heads, so its gradients are 1/H of those
    for h in range(w.H):
        for name, mine, g in (("dq", dq, grads[h][0]), ("dk", dk, grads[h][1]),
                              ("dv", dv, grads[h][2])):
            check_grad(f64(mine[0, h]), g / w.H, f"distill {w.name} h{h} {name}")


# ---------------------------------------------------------------------------
# Rows of more than 256 key blocks take candidates first (each lane's best 4
# of its entries up to 512 key blocks, its best 8 beyond, the lanes holding
# every 64th key block); the candidates' prefix is used only when no lane's
# best left-out entry ranks inside it.
# Mask only (N x N attention would not fit the oracle's dense mode).
# ---------------------------------------------------------------------------

def _lane_cluster_inputs(N, d, seed):
    """Key blocks j with j % 64 == 0 score far above the rest: one lane of
    the selection holds every top block, so the candidates cannot be used."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    Q = np.tile(u, (N, 1)) + 0.1 * rng.standard_normal((N, d))
    K = 0.1 * rng.standard_normal((N, d))
    for j in range(0, -(-N // 64), 64):
        K[64 * j:64 * j + 64] += 3.0 * u
    return Q.astype(np.float32), K.astype(np.float32)


@pytest.mark.parametrize("case,N,k_frac,p", [
    ("candidates", 33000, 0.03, 0.3),
    ("topk_past_512", 33000, 0.995, 0.0),
    ("topp_past_512", 33000, 0.01, 0.999),
    ("lane_cluster", 40000, 0.03, 0.0),
    ("lane_cluster_topp", 40000, 0.0, 0.5),
    ("candidates_313", 20000, 0.03, 0.3),
    ("lane_cluster_313", 20000, 0.03, 0.0),
    ("lane_cluster_topp_313", 20000, 0.0, 0.5),
])
def test_long_row_selection(case, N, k_frac, p):
    d, bq, bk = 64, 128, 64
    if case.startswith("lane_cluster"):
        Qf, Kf = _lane_cluster_inputs(N, d, 28)
    else:
        rng = np.random.default_rng(29)
        Qf = rng.standard_normal((N, d)).astype(np.float32)
        Kf = rng.standard_normal((N, d)).astype(np.float32)
    q = torch.from_numpy(Qf).to(torch.bfloat16).reshape(1, 1, N, d).cuda()
    k = torch.from_numpy(Kf).to(torch.bfloat16).reshape(1, 1, N, d).cuda()
    _say(f"[long rows] {case} N{N} Tk{-(-N // bk)} k{k_frac} p{p}")
    mask = sa2.build_mask(q, k, bq, bk, k_frac, p)
    torch.cuda.synchronize()
    Q, K = (t.reshape(N, d).to(torch.float64).cpu().numpy() for t in (q, k))
    hm = O.build_mask_head(Q, K, bq, bk, k_frac, p)
    bm = mask.bitmap.cpu().numpy()[0, 0]
    compare_mask(hm, bm, p)
    check_lists(bm, mask.row_cnt.cpu().numpy()[0, 0], mask.row_idx.cpu().numpy()[0, 0],
                mask.col_cnt.cpu().numpy()[0, 0], mask.col_idx.cpu().numpy()[0, 0])


def test_graph_replay():
    """The whole step (mask, forward, backward) captured in one HIP graph:
    every replay, with eager work and synchronisations between replays,
    reproduces the eager results bit for bit (the library allocates nothing
    and writes no memset nodes)."""
    w = W.Workload("graph", 1, 2, 2000, 128, 128, 64, "normal", 30, "bf16", 0.1, 0.5)
    dev, _ = device_inputs(w)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    B, H, N, d = q.shape
    mask = sa2.BlockMask(B, H, N, w.bq, w.bk, q.device)
    mws = torch.empty(sa2.mask_workspace_bytes(B, H, N, d, w.bq, w.bk), dtype=torch.uint8,
                      device=q.device)
    bws = torch.empty(sa2.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    fws = torch.empty(sa2.fwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)

    def step():
        sa2.build_mask(q, k, w.bq, w.bk, w.k_frac, w.p, mask=mask, workspace=mws)
        sa2.attn_fwd(q, k, v, mask, o=o, lse=lse, workspace=fws)
        sa2.attn_bwd(q, k, v, o, lse, do, mask, dq=dq, dk=dk, dv=dv, workspace=bws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # eager, on the capture stream, before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    want = [t.clone() for t in (mask.bitmap, mask.row_cnt, o, lse, dq, dk, dv)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        mask.bitmap.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (mask.bitmap, mask.row_cnt, o, lse, dq, dk, dv)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep}"
        step()   # eager work between replays
        torch.cuda.synchronize()
