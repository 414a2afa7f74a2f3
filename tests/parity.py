"""Helpers for the GPU-vs-oracle parity tests (imported by the gpu tests).

Tolerances:
  mask   bit-exact, except blocks whose pooled score lies within 1e-6 of
         the row's selection threshold (the score of the row's last kept
         block), and rows whose cumulative mass at the Top-p cut lies within
         1e-12 of p ("mass near-ties": both sides sum in fp64, in different
         orders); such a row may keep one block more or fewer than the
         oracle's, and must still be a prefix of the oracle's ranking;
  O      max-abs <= 1e-2 and mean-abs <= 1e-3;
  dQ, dK, dV   relative Frobenius error <= 2e-2.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle as O
import workloads as W

SCORE_TOL = 1e-6
MASS_TOL = 1e-12
O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
GRAD_REL_FRO = 2e-2
LSE_MAX_ABS = 1e-2


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a (bf16 or fp32) tensor."""
    return t.detach().to("cpu", torch.float64).numpy()


def device_inputs(w: W.Workload, heads=None, tensors=W.TENSORS, device="cuda"):
    """Workload inputs as device tensors in the workload dtype, plus their fp64 values."""
    x = W.make_inputs(w, heads=heads, tensors=tensors)
    dev, ref = {}, {}
    for name, arr in x.items():
        t = W.to_device_dtype(arr, w.dtype)
        ref[name] = t.to(torch.float64).numpy()
        dev[name] = t.to(device)
    return dev, ref


def compare_mask(hm: O.HeadMask, bitmap_gpu: np.ndarray, p: float):
    """Compare one head's GPU bitmap with the oracle's.

    Returns (exact_rows, tie_blocks, mass_rows) and raises AssertionError for
    any difference the tolerance does not cover.
    """
    bm = hm.bitmap
    diff_rows = np.nonzero((bm != bitmap_gpu).any(axis=1))[0]
    if diff_rows.size == 0:
        return bm.shape[0], 0, 0
    tau = hm.threshold()
    allowed = hm.allowed_counts(p, MASS_TOL)
    ties = 0
    mass = 0
    for i in diff_rows:
        js = np.nonzero(bm[i] != bitmap_gpu[i])[0]
        if np.all(np.abs(hm.S[i, js] - tau[i]) <= SCORE_TOL):
            ties += len(js)
            continue
        n = int(bitmap_gpu[i].sum())
        if n != int(hm.count[i]) and n in allowed[i]:
            # the Top-p cut moved by one block: still a prefix of the ranking
            want = np.zeros_like(bm[i])
            want[hm.order[i, :n]] = 1
            assert np.array_equal(want, bitmap_gpu[i]), f"row {i}: not a ranking prefix"
            mass += 1
            continue
        raise AssertionError(
            f"row {i}: blocks {js.tolist()} differ; scores {hm.S[i, js].tolist()}, "
            f"threshold {tau[i]}, counts oracle {int(bm[i].sum())} gpu {n}")
    return bm.shape[0] - len(diff_rows), ties, mass


def log_mask_exceptions(test: str, workload: str, heads: int, rows: int, exact_rows: int,
                        tie_blocks: int, mass_rows: int) -> None:
    """Append one JSON line of mask-comparison totals to $SA2_PARITY_LOG (if set)."""
    path = os.environ.get("SA2_PARITY_LOG")
    if not path:
        return
    rec = dict(test=test, workload=workload, heads=heads, rows=rows, exact_rows=exact_rows,
               score_tie_blocks=tie_blocks, mass_near_tie_rows=mass_rows,
               score_tol=SCORE_TOL, mass_tol=MASS_TOL)
    with open(path, "a") as fh:
        fh.write(json.dumps(rec) + "\n")


def log_parity(test: str, workload: str, **errors) -> None:
    """Append one JSON line of worst-case numeric errors to $SA2_PARITY_LOG (if set)."""
    path = os.environ.get("SA2_PARITY_LOG")
    if not path:
        return
    with open(path, "a") as fh:
        fh.write(json.dumps(dict(test=test, workload=workload, **errors)) + "\n")


def check_lists(bitmap: np.ndarray, row_cnt, row_idx, col_cnt, col_idx):
    """Row and column lists must be exactly the ascending nonzeros of the bitmap."""
    Tq, Tk = bitmap.shape
    for i in range(Tq):
        want = np.nonzero(bitmap[i])[0]
        assert row_cnt[i] == len(want), f"row {i} count"
        assert np.array_equal(row_idx[i, :len(want)], want), f"row {i} list"
    for j in range(Tk):
        want = np.nonzero(bitmap[:, j])[0]
        assert col_cnt[j] == len(want), f"column {j} count"
        assert np.array_equal(col_idx[j, :len(want)], want), f"column {j} list"


ROW_PLAN = dict(slots=512, fair=1, extra=64, min_segment=16, imbalance=10, counters=2, quarters=True)
COL_PLAN = dict(slots=1024, fair=2, extra=128, min_segment=8, imbalance=0, counters=1,
                quarters=False)


def _items_per_xcd(n: int, kd: dict) -> int:
    return (n + 7) // 8 + 2 * (((n + 7) // 8 + 15) // 16) + kd["extra"]


def _equal_count_shares(n: int):
    q, r = divmod(n, 8)
    return [(x * q + min(x, r), q + (1 if x < r else 0)) for x in range(8)]


def _cut(c: int, L: int):
    """Segments of a list of c entries cut at L: nearly equal, in order."""
    ns = -(-c // L) if c > L else 1
    base, rem = divmod(c, ns)
    return [(s * base + min(s, rem), base + (1 if s < rem else 0)) for s in range(ns)]


def _check_items(cnt, lists, items, L, splits, ebase, ecap, slot_owner, what) -> int:
    """Items of `lists` (each list exactly once, as one item or as nearly equal
    segments of at most L entries) with split entries in [ebase, ebase + ecap)
    and partial slots in [2 ebase, 2 (ebase + ecap)).  Returns the split lists."""
    per_list: dict[int, list] = {}
    for it in items:
        per_list.setdefault(int(it[0]), []).append(tuple(int(v) for v in it))
    assert sorted(per_list) == [int(v) for v in lists], f"{what}: lists of the items"
    nsplit = 0
    for lst in lists:
        its_l = sorted(per_list[int(lst)], key=lambda t: t[1])
        c = int(cnt[lst])
        if c <= L:
            assert len(its_l) == 1 and its_l[0] == (lst, 0, c, -1), f"list {lst}: {its_l}"
            continue
        nsplit += 1
        want = _cut(c, L)
        ns = len(want)
        assert [(t[1], t[2]) for t in its_l] == want, f"list {lst}: segments {its_l}"
        entries = {t[3] >> 10 for t in its_l}
        assert len(entries) == 1, f"list {lst}: several split entries"
        e = entries.pop()
        assert ebase <= e < ebase + ecap, f"list {lst}: split entry outside its share"
        sp = splits[e]
        assert sp[0] == lst and sp[2] == ns, f"list {lst}: split entry {sp}"
        assert sorted(t[3] & 1023 for t in its_l) == list(range(ns))
        assert 2 * ebase <= sp[1] and sp[1] + ns <= 2 * (ebase + ecap), f"list {lst}: slots"
        for slot in range(sp[1], sp[1] + ns):
            assert slot not in slot_owner, f"slot {slot} shared"
            slot_owner[slot] = lst
    return nsplit


def check_plan(cnt, plan, kd: dict, cap: int, per_head: int, head_major_out=None) -> int:
    """A work plan (the int32 array the mask builder wrote) against the list
    counts it was made from (per_head consecutive lists per (batch, head)).

    Every list is covered by its items, as one item or as nearly equal
    segments; XCD x holds a contiguous share of the lists, and XCDs 4g..4g+3
    form group g, whose share is the union of theirs.  A group is head-major
    when 4 x its longest item (its lists cut at Lg = max(L0, ceil(group
    entries / (4 extra)))) x slots / 2 is at most the group's cost (entries +
    lists), L0 = max(min_segment, fair * ceil(total / slots)): then, for a
    plan kind with quarters, XCD 4g + r holds the items of the r-th
    contiguous quarter of every (batch, head)'s lists (list index within its
    head times 4 // lists per head = r), ordered by (batch, head) and longest
    first within each head (in the shared ranks of the plan: 4096 // (4
    heads) length ranks per quarter and head), unless a quarter holds more
    items than an XCD has slots; otherwise, or for a kind without, the group's items,
    in rank order k over (batch, head) and length (4096 // heads ranks per
    head), sit at slot 8 (k // 4) + 4g + k % 4.  Split entries and partial
    slots lie in the group's range.  Otherwise each XCD's
    items are its share longest first, cut at max(L0, ceil(share / extra)),
    with entries and slots in the XCD's range.  Every completion counter is
    zero.  Returns the number of split lists; appends each group's head-major
    decision to `head_major_out` when given."""
    cnt = np.clip(np.asarray(cnt).reshape(-1).astype(np.int64), 0, cap)
    n, ex = cnt.size, kd["extra"]
    J = _items_per_xcd(n, kd)
    buf = np.asarray(plan).reshape(-1).view(np.int32)
    items = buf[:8 * J * 4].reshape(J, 8, 4)
    splits = buf[8 * J * 4:8 * J * 4 + 8 * ex * 4].reshape(8 * ex, 4)
    done = buf[8 * J * 4 + 8 * ex * 4:8 * J * 4 + 8 * ex * 4 + kd["counters"] * 8 * ex]
    assert np.all(done == 0), "completion counters not zero"
    total = int(cnt.sum())
    L0 = max(kd["min_segment"], kd["fair"] * -(-total // kd["slots"]))
    costs = [int((cnt[a:a + ln] + 1).sum()) for a, ln in _equal_count_shares(n)]
    balanced = kd["imbalance"] == 0 or max(costs) * 800 > sum(costs) * (800 + 8 * kd["imbalance"])
    cols = []
    for x in range(8):
        its = items[:, x, :]
        k = int(np.count_nonzero(its[:, 0] >= 0))
        assert np.all(its[:k, 0] >= 0) and np.all(its[k:, 0] == -1), f"XCD {x}: gaps in items"
        cols.append(its[:k])
    lo, nsplit, slot_owner = 0, 0, {}
    for g in range(2):
        gcols = cols[4 * g:4 * g + 4]
        glists = np.unique(np.concatenate([c[:, 0] for c in gcols])) if any(len(c) for c in gcols) \
            else np.zeros(0, np.int64)
        if glists.size:
            assert glists[0] == lo and glists[-1] == lo + glists.size - 1, f"group {g}: not contiguous"
        if not balanced:
            want = sum(_equal_count_shares(n)[x][1] for x in range(4 * g, 4 * g + 4))
            assert glists.size == want, f"group {g}: share size"
        G0, G1 = lo, lo + glists.size
        lo = G1
        gshare = int(cnt[G0:G1].sum())
        Lg = max(L0, -(-gshare // (4 * ex)))
        glong = int(cnt[G0:G1].max()) if G1 > G0 else 0
        gseg = max((s for _, s in _cut(glong, Lg)), default=0)
        head_major = G1 > G0 and 4 * gseg * (kd["slots"] // 2) <= gshare + (G1 - G0)
        if head_major_out is not None:
            head_major_out.append(bool(head_major))
        if head_major:
            nitems = sum(len(c) for c in gcols)
            ph = max(per_head, 1)
            h0 = G0 // ph
            nh = (G1 - 1) // ph - h0 + 1
            qn = [0, 0, 0, 0]
            for lid in range(G0, G1):
                qn[(lid % ph) * 4 // ph] += len(_cut(int(cnt[lid]), Lg))
            if kd["quarters"] and max(qn) <= J:
                # XCD 4g + r: the r-th contiguous quarter of every head's lists
                nr = 4 * nh
                nb = 4096 // nr if nr <= 4096 else 1
                for r in range(4):
                    c = gcols[r]
                    assert len(c) == qn[r], f"group {g}: XCD {4 * g + r} does not hold quarter {r}"
                    assert np.all((c[:, 0] % ph) * 4 // ph == r), \
                        f"group {g}: item outside quarter {r}"
                    heads = c[:, 0] // ph
                    hh = r * nh + heads - h0
                    hb = hh if nr <= 4096 else hh * 4096 // nr
                    lr = nb - 1 - np.minimum(nb - 1, c[:, 2] * nb // (gseg + 1))
                    assert np.all(np.diff(hb * nb + lr) >= 0), \
                        f"group {g}: XCD {4 * g + r} not head by head, longest first"
                    assert np.all(np.diff(heads) >= 0), f"group {g}: heads out of order"
                    if nb > gseg:
                        same = heads[1:] == heads[:-1]
                        assert np.all(np.diff(c[:, 2])[same] <= 0), f"group {g}: not longest first"
                order = np.concatenate([c.reshape(-1, 4) for c in gcols])
            else:
                # a quarter larger than an XCD's slots: the items dealt in turn
                for r in range(4):
                    assert len(gcols[r]) == (-(-(nitems - r) // 4) if nitems > r else 0), \
                        f"group {g}: items not dealt in turn"
                order = np.array([gcols[k % 4][k // 4] for k in range(nitems)]).reshape(-1, 4)
                heads = order[:, 0] // ph
                nb = 4096 // nh if nh <= 4096 else 1
                hb = heads - h0 if nh <= 4096 else (heads - h0) * 4096 // nh
                lr = nb - 1 - np.minimum(nb - 1, order[:, 2] * nb // (gseg + 1))
                rank = hb * nb + lr
                assert np.all(np.diff(rank) >= 0), f"group {g}: not head by head, longest first"
                assert np.all(np.diff(heads) >= 0), f"group {g}: heads out of order"
                if nb > gseg:
                    same = heads[1:] == heads[:-1]
                    assert np.all(np.diff(order[:, 2])[same] <= 0), f"group {g}: not longest first"
            nsplit += _check_items(cnt, glists, order, Lg, splits, 4 * ex * g, 4 * ex,
                                   slot_owner, f"group {g}")
            continue
        xlo = G0
        for x in range(4 * g, 4 * g + 4):
            valid = cols[x]
            keys = np.minimum(valid[:, 2], 4095)
            assert np.all(np.diff(keys) <= 0), f"XCD {x}: not longest first"
            lists = np.unique(valid[:, 0])
            if lists.size:
                assert lists[0] == xlo and lists[-1] == xlo + lists.size - 1, \
                    f"XCD {x}: share not contiguous"
            if not balanced:
                assert lists.size == _equal_count_shares(n)[x][1], f"XCD {x}: share size"
            xlo += lists.size
            share = int(cnt[lists].sum()) if lists.size else 0
            L = max(L0, -(-share // ex))
            nsplit += _check_items(cnt, lists, valid, L, splits, ex * x, ex, slot_owner,
                                   f"XCD {x}")
        assert xlo == G1
    assert lo == n, "lists missing from the plan"
    return nsplit


def check_plans(mask, head_major: dict | None = None) -> tuple[int, int]:
    """Both plans of a BlockMask; returns (split rows, split columns) and,
    when `head_major` is a dict, sets its "rows" and "cols" entries to the
    two groups' head-major decisions."""
    hr, hc = [], []
    out = (check_plan(mask.row_cnt.cpu().numpy(), mask.row_plan.cpu().numpy(), ROW_PLAN,
                      mask.Tk, mask.Tq, hr),
           check_plan(mask.col_cnt.cpu().numpy(), mask.col_plan.cpu().numpy(), COL_PLAN,
                      mask.Tq, mask.Tk, hc))
    if head_major is not None:
        head_major.update(rows=hr, cols=hc)
    return out


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def check_forward(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray,
                  what: str = ""):
    """O within max-abs 1e-2 / mean-abs 1e-3 and LSE within 1e-2."""
    err = np.abs(o_gpu - o_ref)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    assert err.max() <= O_MAX_ABS, f"{what}: O max-abs {err.max():.3e}"
    assert err.mean() <= O_MEAN_ABS, f"{what}: O mean-abs {err.mean():.3e}"
    lerr = np.abs(lse_gpu - lse_ref).max()
    assert lerr <= LSE_MAX_ABS, f"{what}: LSE max-abs {lerr:.3e}"
    return float(err.max()), float(err.mean())


def check_grad(g_gpu: np.ndarray, g_ref: np.ndarray, what: str):
    assert np.isfinite(g_gpu).all(), f"{what}: non-finite"
    r = rel_fro(g_gpu, g_ref)
    assert r <= GRAD_REL_FRO, f"{what}: relative Frobenius error {r:.3e}"
    return r
