"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one call per step over all heads).

* Wan2.1-1.3B-shaped layer (H=12, N=32760 = 21x30x52, d=128, bf16, q-block
  128, k-block 64, k = 3%, p tuned for 5% density), forward and backward,
  and the same layer in a second block geometry (64 x 64 blocks): the whole
  mask of every head against the oracle; every element of O, LSE, dQ, dK and
  dV of every head against the oracle's gathered evaluation; closed-form
  invariants of the gradients on every head.
* 14B-720p-shaped layer (H=40, N=75600 = 21x45x80): the mask of all 40 heads
  against the oracle, and O, LSE, dQ, dK, dV of eight heads spread over the
  layer (0, 6, ..., 36, 39); on all 40 heads, the hybrid mask equals the
  union of the library's Top-k-only and Top-p-only masks, every row keeps at
  least kc blocks, and the gradient invariants hold (evaluated on the device
  in fp64).
* Mask-rule stress (H=8, N=16384): three score regimes x four densities; the
  hybrid mask contains the Top-k-only and Top-p-only masks on every head and
  equals their union; the three masks of every head against the oracle's;
  attention of head 0 against the oracle in full.
* The largest key-block count (4096) at one head.
* Many short rows over two batch entries (B=2, H=16, N=8192): the row plan
  goes head by head; one head per batch entry against the oracle.

Mask-comparison totals (rows compared, exact rows, score near-tie blocks,
mass near-tie rows) and the worst numeric errors are appended to the file
named by $SA2_PARITY_LOG when it is set.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_sa2_amd as sa2
import oracle as O
import workloads as W

from parity import (GRAD_REL_FRO, check_forward, check_grad, check_lists, check_plans,
                    compare_mask, device_inputs, f64, log_mask_exceptions, log_parity)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _head_np(ref, h, b=0):
    return tuple(ref[t][b, h] for t in ("q", "k", "v", "do") if t in ref)


def _row_lists(mask_np_bm):
    return [np.nonzero(r)[0] for r in mask_np_bm]


def _whole_head(w, ref, h, bm_h, o, lse, grads, b=0):
    """Every element of O, LSE (and dQ, dK, dV) of head h against the oracle's
    gathered evaluation (each query block over its kept key blocks only);
    returns the worst errors."""
    Q, K, V, dO = _head_np(ref, h, b)
    rows = _row_lists(bm_h)
    if grads is None:
        Oo, L = O.attention_gathered(Q, K, V, rows, w.bq, w.bk)
    else:
        Oo, L, rq, rk, rv = O.attention_gathered(Q, K, V, rows, w.bq, w.bk, dO=dO)
    om, oa = check_forward(f64(o[b, h]), f64(lse[b, h]), Oo, L, f"{w.name} h{h}")
    out = dict(o_max=om, o_mean=oa)
    if grads is not None:
        for name, g, want in zip(("dq", "dk", "dv"), grads, (rq, rk, rv)):
            out[name] = check_grad(f64(g[b, h]), want, f"{w.name} h{h} {name}")
    return out


def _worst(acc, e):
    for k_, v_ in e.items():
        acc[k_] = max(acc.get(k_, 0.0), v_)
    return acc


def _invariants(q, k, dq, dk, dv, do, h):
    """sum_u dK_u = 0, sum_u dV_u = sum_t dO_t, <Q, dQ> = <K, dK> (fixed mask),
    on the device in fp64."""
    Q, K, dQ, dK, dV, dO = (t[0, h].double() for t in (q, k, dq, dk, dv, do))
    scale = float(dK.abs().sum(dim=0).max())
    assert float(dK.sum(dim=0).abs().max()) <= GRAD_REL_FRO * scale, f"h{h}: sum dK"
    sv, so = dV.sum(dim=0), dO.sum(dim=0)
    assert float((sv - so).norm()) <= GRAD_REL_FRO * float(so.norm()), f"h{h}: sum dV"
    qd, kd = float((Q * dQ).sum()), float((K * dK).sum())
    floor = float((Q * dQ).abs().sum()) * 1e-3
    assert abs(qd - kd) <= GRAD_REL_FRO * max(abs(qd), abs(kd), floor), f"h{h}: <Q,dQ>"


def _mask_all_heads(test, w, mask, ref, k_frac, p, heads):
    """The mask of `heads` against the oracle (bitmap, lists), with the totals logged."""
    bm = mask.bitmap.cpu().numpy()
    rc, ri = mask.row_cnt.cpu().numpy(), mask.row_idx.cpu().numpy()
    cc, ci = mask.col_cnt.cpu().numpy(), mask.col_idx.cpu().numpy()
    exact = ties = mass = 0
    for h in heads:
        hm = O.build_mask_head(ref["q"][0, h], ref["k"][0, h], w.bq, w.bk, k_frac, p)
        e_, t_, m_ = compare_mask(hm, bm[0, h], p)
        exact += e_; ties += t_; mass += m_
        check_lists(bm[0, h], rc[0, h], ri[0, h], cc[0, h], ci[0, h])
    rows = len(heads) * mask.Tq
    _say(f"[{w.name}] mask: {rows} rows, {exact} exact, {ties} score near-tie blocks, "
         f"{mass} mass near-tie rows")
    log_mask_exceptions(test, w.name, len(heads), rows, exact, ties, mass)
    return bm


# ---------------------------------------------------------------------------
# Wan2.1-1.3B-shaped layer, forward + backward
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module", params=["c2", "c2_b64"], ids=["bq128_bk64", "bq64_bk64"])
def wan13(request):
    w = W.WORKLOADS[request.param]
    k_frac, p = W.tuned_params(request.param)
    _say(f"[wan1.3B] generating inputs H{w.H} N{w.N} d{w.d} bq{w.bq} bk{w.bk}")
    dev, ref = device_inputs(w)
    q, k, v, do = (dev[t] for t in ("q", "k", "v", "do"))
    mask = sa2.build_mask(q, k, w.bq, w.bk, k_frac, p)
    o, lse = sa2.attn_fwd(q, k, v, mask)
    grads = sa2.attn_bwd(q, k, v, o, lse, do, mask)
    torch.cuda.synchronize()
    return dict(w=w, k_frac=k_frac, p=p, dev=dev, ref=ref, mask=mask, o=o, lse=lse, grads=grads)


def test_wan13_mask_all_heads(wan13):
    w, mask, ref = wan13["w"], wan13["mask"], wan13["ref"]
    hm = {}
    check_plans(mask, hm)
    # rows are short against a slot's load: planned head by head; the
    # longest columns are as long as a slot's whole load: longest first
    assert hm == {"rows": [True, True], "cols": [False, False]}, hm
    _mask_all_heads("wan13_mask_all_heads", w, mask, ref, wan13["k_frac"], wan13["p"],
                    range(w.H))
    dens = mask.density()
    _say(f"[wan1.3B] density {dens:.5f}")
    assert abs(dens - 0.05) <= 0.02 * 0.05 + 1e-4


def test_wan13_attention_whole_layer(wan13):
    """O, LSE, dQ, dK, dV: every element of every head against the oracle."""
    w, ref = wan13["w"], wan13["ref"]
    bm = wan13["mask"].bitmap.cpu().numpy()
    worst = {}
    for h in range(w.H):
        _worst(worst, _whole_head(w, ref, h, bm[0, h], wan13["o"], wan13["lse"],
                                  wan13["grads"]))
    _say(f"[{w.name}] worst over {w.H} heads: " +
         ", ".join(f"{k_} {v_:.2e}" for k_, v_ in worst.items()))
    log_parity("wan13_attention_whole_layer", w.name, heads=w.H, **worst)


def test_wan13_atomic_dq_backward(wan13):
    """The fused backward (dQ by fp32 atomics in the dK/dV pass) on the
    full-size layer: dQ, dK, dV of heads 0 and H-1 against the oracle."""
    w, ref, dev = wan13["w"], wan13["ref"], wan13["dev"]
    q, k, v, do = (dev[t] for t in ("q", "k", "v", "do"))
    grads = sa2.attn_bwd_atomic_dq(q, k, v, wan13["o"], wan13["lse"], do, wan13["mask"])
    torch.cuda.synchronize()
    bm = wan13["mask"].bitmap.cpu().numpy()
    worst = {}
    for h in (0, w.H - 1):
        _worst(worst, _whole_head(w, ref, h, bm[0, h], wan13["o"], wan13["lse"], grads))
    log_parity("wan13_atomic_dq_backward", w.name, heads=2, **worst)


def test_wan13_gradient_invariants(wan13):
    w, dev = wan13["w"], wan13["dev"]
    dq, dk, dv = wan13["grads"]
    for h in range(w.H):
        _invariants(dev["q"], dev["k"], dq, dk, dv, dev["do"], h)


# ---------------------------------------------------------------------------
# 14B-720p-shaped layer
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def wan14():
    w = W.WORKLOADS["c3"]
    k_frac, p = W.tuned_params("c3")
    _say(f"[wan14B] generating inputs H{w.H} N{w.N} d{w.d}")
    dev, ref = device_inputs(w)
    q, k, v, do = (dev[t] for t in ("q", "k", "v", "do"))
    mask = sa2.build_mask(q, k, w.bq, w.bk, k_frac, p)
    o, lse = sa2.attn_fwd(q, k, v, mask)
    grads = sa2.attn_bwd(q, k, v, o, lse, do, mask)
    torch.cuda.synchronize()
    return dict(w=w, k_frac=k_frac, p=p, dev=dev, ref=ref, mask=mask, o=o, lse=lse, grads=grads)


def test_wan14_heads_against_the_oracle(wan14):
    """The mask of all 40 heads; O, LSE, dQ, dK, dV of eight heads spread over
    the layer."""
    w, mask, ref = wan14["w"], wan14["mask"], wan14["ref"]
    heads = tuple(range(0, w.H, 6)) + (w.H - 1,)
    bm = _mask_all_heads("wan14_heads_against_the_oracle", w, mask, ref, wan14["k_frac"],
                         wan14["p"], range(w.H))
    worst = {}
    for h in heads:
        _worst(worst, _whole_head(w, ref, h, bm[0, h], wan14["o"], wan14["lse"],
                                  wan14["grads"]))
    _say(f"[{w.name}] worst over heads {heads}: " +
         ", ".join(f"{k_} {v_:.2e}" for k_, v_ in worst.items()))
    log_parity("wan14_heads_against_the_oracle", w.name, heads=len(heads), **worst)
    dens = mask.density()
    _say(f"[wan14B] density {dens:.5f}")
    assert abs(dens - 0.05) <= 0.02 * 0.05 + 1e-4


def test_wan14_union_every_head(wan14):
    """On all 40 heads: the hybrid mask contains the library's Top-k-only and
    Top-p-only masks and equals their union (gist.science 2A), and every row
    keeps at least kc blocks.  Both work plans check out against the counts,
    and both are planned head by head."""
    w, mask, dev = wan14["w"], wan14["mask"], wan14["dev"]
    hm = {}
    check_plans(mask, hm)
    assert hm == {"rows": [True, True], "cols": [True, True]}, hm
    q, k = dev["q"], dev["k"]
    hy = mask.bitmap
    ko = sa2.build_mask(q, k, w.bq, w.bk, wan14["k_frac"], 0.0).bitmap
    po = sa2.build_mask(q, k, w.bq, w.bk, 0.0, wan14["p"]).bitmap
    torch.cuda.synchronize()
    assert torch.all(hy >= ko) and torch.all(hy >= po)
    assert torch.equal(hy, torch.maximum(ko, po))
    kc = O.topk_count(wan14["k_frac"], mask.Tk)
    assert int(ko.sum(dim=-1).min()) == kc and int(ko.sum(dim=-1).max()) == kc
    assert int(mask.row_cnt.min().item()) >= kc


def test_wan14_gradient_invariants_every_head(wan14):
    w, dev = wan14["w"], wan14["dev"]
    dq, dk, dv = wan14["grads"]
    for h in range(w.H):
        _invariants(dev["q"], dev["k"], dq, dk, dv, dev["do"], h)


# ---------------------------------------------------------------------------
# Many short rows over two batch entries: the row plan goes head by head
# ---------------------------------------------------------------------------

def test_head_major_rows_across_batches():
    """B=2, H=16, N=8192, Top-k 4 of 128 key blocks: 2048 rows of four blocks
    each, so both groups of the row plan are planned head by head, in (batch,
    head) order; both plans check out against the counts, and the mask, O,
    LSE, dQ, dK and dV of one head in each batch entry match the oracle."""
    from dataclasses import replace
    w = W.Workload("headmajor", 2, 16, 8192, 128, 128, 64, "normal", 41, "bf16", 4 / 128, 0.0)
    _say(f"[head-major] generating B{w.B} H{w.H} N{w.N}")
    dev1, ref1 = device_inputs(replace(w, B=1, H=w.B * w.H))
    dev = {k_: t.reshape(w.B, w.H, w.N, w.d).contiguous() for k_, t in dev1.items()}
    ref = {k_: a.reshape(w.B, w.H, w.N, w.d) for k_, a in ref1.items()}
    q, k, v, do = (dev[t] for t in ("q", "k", "v", "do"))
    mask = sa2.build_mask(q, k, w.bq, w.bk, w.k_frac, w.p)
    o, lse = sa2.attn_fwd(q, k, v, mask)
    grads = sa2.attn_bwd(q, k, v, o, lse, do, mask)
    torch.cuda.synchronize()
    hm = {}
    check_plans(mask, hm)
    assert hm["rows"] == [True, True], hm
    assert int(mask.row_cnt.min().item()) == 4 and int(mask.row_cnt.max().item()) == 4
    bm = mask.bitmap.cpu().numpy()
    rc, ri = mask.row_cnt.cpu().numpy(), mask.row_idx.cpu().numpy()
    cc, ci = mask.col_cnt.cpu().numpy(), mask.col_idx.cpu().numpy()
    worst = {}
    exact = ties = mass = 0
    for b, h in ((0, 3), (1, 12)):
        Q, K = ref["q"][b, h], ref["k"][b, h]
        e_, t_, m_ = compare_mask(O.build_mask_head(Q, K, w.bq, w.bk, w.k_frac, w.p), bm[b, h],
                                  w.p)
        exact += e_; ties += t_; mass += m_
        check_lists(bm[b, h], rc[b, h], ri[b, h], cc[b, h], ci[b, h])
        _worst(worst, _whole_head(w, ref, h, bm[b, h], o, lse, grads, b=b))
    log_mask_exceptions("head_major_rows_across_batches", w.name, 2, 2 * mask.Tq, exact, ties,
                        mass)
    log_parity("head_major_rows_across_batches", w.name, heads=2, **worst)


@pytest.mark.parametrize("H, N, quarters", [(288, 768, True), (288, 640, False)])
def test_head_major_rows_with_uneven_quarters(H, N, quarters):
    """Top-k 2 of the key blocks, so the row plan is head by head.  With six
    query blocks per head the quarters of a head hold 2, 1, 2 and 1 of them
    and fit the XCDs' item slots: XCD 4g + r holds quarter r.  With five per
    head, quarter 0 holds two of every five rows, more than an XCD's slots, so
    the group is dealt in turn.  The plans check out, and the mask, O, LSE,
    dQ, dK and dV of two heads match the oracle."""
    from dataclasses import replace
    Tk = -(-N // 64)
    w = W.Workload(f"uneven{H}", 1, H, N, 128, 128, 64, "normal", 43, "bf16", 2 / Tk, 0.0)
    _say(f"[head-major uneven] B1 H{H} N{N}")
    dev, ref = device_inputs(w)
    q, k, v, do = (dev[t] for t in ("q", "k", "v", "do"))
    mask = sa2.build_mask(q, k, w.bq, w.bk, w.k_frac, w.p)
    o, lse = sa2.attn_fwd(q, k, v, mask)
    grads = sa2.attn_bwd(q, k, v, o, lse, do, mask)
    torch.cuda.synchronize()
    hm = {}
    check_plans(mask, hm)
    assert hm["rows"] == [True, True], hm
    # XCD 0 holds only quarter-0 rows exactly when the plan uses quarters
    Tq = mask.Tq
    n = H * Tq
    J = (n + 7) // 8 + 2 * (((n + 7) // 8 + 15) // 16) + 64
    items = mask.row_plan.cpu().numpy()[:8 * J * 4].reshape(J, 8, 4)
    lists = items[:, 0, 0]
    lists = lists[lists >= 0]
    assert bool(np.all((lists % Tq) * 4 // Tq == 0)) == quarters
    bm = mask.bitmap.cpu().numpy()
    worst = {}
    exact = ties = mass = 0
    for h in (1, H - 2):
        e_, t_, m_ = compare_mask(O.build_mask_head(ref["q"][0, h], ref["k"][0, h], w.bq, w.bk,
                                                    w.k_frac, w.p), bm[0, h], w.p)
        exact += e_; ties += t_; mass += m_
        _worst(worst, _whole_head(w, ref, h, bm[0, h], o, lse, grads))
    log_mask_exceptions("head_major_rows_with_uneven_quarters", w.name, 2, 2 * Tq, exact, ties,
                        mass)
    log_parity("head_major_rows_with_uneven_quarters", w.name, heads=2, **worst)


# ---------------------------------------------------------------------------
# Mask-rule stress test
# ---------------------------------------------------------------------------

STRESS = [n for n in W.WORKLOADS if n.startswith("c4_")]


@pytest.fixture(scope="module")
def stress_inputs():
    cache = {}

    def get(regime):
        if regime not in cache:
            w = W.WORKLOADS[f"c4_{regime}_05"]
            _say(f"[stress] generating {regime} inputs")
            cache.clear()
            cache[regime] = device_inputs(w)
        return cache[regime]
    return get


@pytest.mark.parametrize("name", STRESS)
def test_stress_union_and_oracle(name, stress_inputs):
    w = W.WORKLOADS[name]
    k_frac, p = W.tuned_params(name)
    dev, ref = stress_inputs(w.gen)
    q, k, v, do = (dev[t] for t in ("q", "k", "v", "do"))
    _say(f"[stress] {name} k{k_frac:.5f} p{p:.5f}")
    hy = sa2.build_mask(q, k, w.bq, w.bk, k_frac, p)
    hy_bm = hy.bitmap.clone()
    ko = sa2.build_mask(q, k, w.bq, w.bk, k_frac, 0.0).bitmap.clone()
    po = sa2.build_mask(q, k, w.bq, w.bk, 0.0, p).bitmap.clone()
    torch.cuda.synchronize()
    assert torch.all(hy_bm >= ko) and torch.all(hy_bm >= po)
    assert torch.equal(hy_bm, torch.maximum(ko, po))
    o, lse = sa2.attn_fwd(q, k, v, hy)
    grads = sa2.attn_bwd(q, k, v, o, lse, do, hy)
    torch.cuda.synchronize()
    bm, ko_bm, po_bm = hy_bm.cpu().numpy(), ko.cpu().numpy(), po.cpu().numpy()
    # the hybrid mask and each rule on its own, as a mode of its own, against
    # the oracle on every head
    for tag, kf_, p_, got in (("", k_frac, p, bm), ("/top-k only", k_frac, 0.0, ko_bm),
                              ("/top-p only", 0.0, p, po_bm)):
        ex = ti = ma = 0
        for h in range(w.H):
            hm = O.build_mask_head(ref["q"][0, h], ref["k"][0, h], w.bq, w.bk, kf_, p_)
            e_, t_, m_ = compare_mask(hm, got[0, h], p_)
            ex += e_; ti += t_; ma += m_
        log_mask_exceptions("stress_union_and_oracle" + tag, name, w.H, w.H * w.Tq, ex, ti, ma)
    worst = _whole_head(w, ref, 0, bm[0, 0], o, lse, grads)
    log_parity("stress_union_and_oracle", name, heads=1, **worst)
    dens = hy.density()
    want = W.tuned_record(name)["density"]
    _say(f"[stress] {name} density {dens:.5f} (oracle {want:.5f}, target {w.target_density})")
    assert abs(dens - want) <= 1e-3 * want


# ---------------------------------------------------------------------------
# The largest key-block count the mask builder takes (4096: rows of 4096
# entries, 64 per lane, in the selection), at one head.  Top-k alone keeps 41
# blocks per row (the candidate path); with p = 0.3 rows keep about 1200
# (past the 512 candidates: the whole-row sort).
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def max_tk():
    w = W.Workload("max_tk", 1, 1, 4096 * 64, 64, 128, 64, "normal", 31, "bf16", 0.01, 0.0)
    _say(f"[max Tk] generating N{w.N} Tq{w.Tq} Tk{w.Tk}")
    dev, ref = device_inputs(w)
    return w, dev, ref


@pytest.mark.parametrize("p", [0.0, 0.3], ids=["candidates", "whole_rows"])
def test_max_key_blocks(max_tk, p):
    w, dev, ref = max_tk
    q, k, v, do = (dev[t] for t in ("q", "k", "v", "do"))
    mask = sa2.build_mask(q, k, w.bq, w.bk, w.k_frac, p)
    torch.cuda.synchronize()
    assert mask.Tk == 4096
    bm = _mask_all_heads(f"max_key_blocks p{p}", w, mask, ref, w.k_frac, p, [0])
    _say(f"[max Tk] p{p} kept per row {float(mask.row_cnt.float().mean()):.1f}")
    if p == 0.0:
        o, lse = sa2.attn_fwd(q, k, v, mask)
        grads = sa2.attn_bwd(q, k, v, o, lse, do, mask)
        torch.cuda.synchronize()
        worst = _whole_head(w, ref, 0, bm[0, 0], o, lse, grads)
        log_parity("max_key_blocks", w.name, heads=1, **worst)
