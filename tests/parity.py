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


ROW_PLAN = dict(slots=512, fair=1, extra=64, min_segment=16, imbalance=10, counters=2)
COL_PLAN = dict(slots=1024, fair=2, extra=128, min_segment=8, imbalance=0, counters=1)


def _items_per_xcd(n: int, kd: dict) -> int:
    return (n + 7) // 8 + 2 * (((n + 7) // 8 + 15) // 16) + kd["extra"]


def _equal_count_shares(n: int):
    q, r = divmod(n, 8)
    return [(x * q + min(x, r), q + (1 if x < r else 0)) for x in range(8)]


def check_plan(cnt, plan, kd: dict, cap: int) -> int:
    """A work plan (the int32 array the mask builder wrote) against the list
    counts it was made from: every list is covered by its items in order, as
    one item or as nearly equal segments; a list is cut exactly when it is
    longer than L = max(min_segment, fair * ceil(total / slots),
    ceil(share / extra)) of its XCD share, into ceil(n / L) segments; XCD x's
    items are the x-th contiguous share of the lists, longest first; each
    split owns partial slots inside its share's range; every completion
    counter is zero.  Returns the number of split lists."""
    cnt = np.clip(np.asarray(cnt).reshape(-1).astype(np.int64), 0, cap)
    n, ex = cnt.size, kd["extra"]
    J = _items_per_xcd(n, kd)
    buf = np.asarray(plan).reshape(-1).view(np.int32)
    items = buf[:8 * J * 4].reshape(J, 8, 4)
    splits = buf[8 * J * 4:8 * J * 4 + 8 * ex * 4].reshape(8 * ex, 4)
    done = buf[8 * J * 4 + 8 * ex * 4:8 * J * 4 + 8 * ex * 4 + kd["counters"] * 8 * ex]
    assert np.all(done == 0), "completion counters not zero"
    total = int(cnt.sum())
    costs = [int((cnt[a:a + ln] + 1).sum()) for a, ln in _equal_count_shares(n)]
    balanced = kd["imbalance"] == 0 or max(costs) * 800 > sum(costs) * (800 + 8 * kd["imbalance"])
    per_list: dict[int, list] = {}
    lo = 0
    nsplit = 0
    slot_owner = {}
    for x in range(8):
        its = items[:, x, :]
        k = int(np.count_nonzero(its[:, 0] >= 0))
        assert np.all(its[:k, 0] >= 0) and np.all(its[k:, 0] == -1), f"XCD {x}: gaps in items"
        valid = its[:k]
        keys = np.minimum(valid[:, 2], 4095)
        assert np.all(np.diff(keys) <= 0), f"XCD {x}: not longest first"
        lists = np.unique(valid[:, 0])
        if lists.size:
            assert lists[0] == lo and lists[-1] == lo + lists.size - 1, f"XCD {x}: share not contiguous"
        if not balanced:
            assert lists.size == _equal_count_shares(n)[x][1], f"XCD {x}: share size"
        lo += lists.size
        share = int(cnt[lists].sum()) if lists.size else 0
        L = max(kd["min_segment"], kd["fair"] * -(-total // kd["slots"]), -(-share // ex))
        for it in valid:
            per_list.setdefault(int(it[0]), []).append(tuple(int(v) for v in it))
        for lst in lists:
            its_l = sorted(per_list[int(lst)], key=lambda t: t[1])
            c = int(cnt[lst])
            if c <= L:
                assert len(its_l) == 1 and its_l[0] == (lst, 0, c, -1), f"list {lst}: {its_l}"
                continue
            nsplit += 1
            ns = -(-c // L)
            assert len(its_l) == ns, f"list {lst}: {len(its_l)} segments, expected {ns}"
            entries = {t[3] >> 10 for t in its_l}
            assert len(entries) == 1, f"list {lst}: several split entries"
            e = entries.pop()
            assert e // ex == x, f"list {lst}: split entry outside its share"
            sp = splits[e]
            assert sp[0] == lst and sp[2] == ns, f"list {lst}: split entry {sp}"
            assert sorted(t[3] & 1023 for t in its_l) == list(range(ns))
            assert its_l[0][1] == 0 and its_l[-1][1] + its_l[-1][2] == c
            for a, b in zip(its_l, its_l[1:]):
                assert a[1] + a[2] == b[1], f"list {lst}: segments not contiguous"
            sl = [t[2] for t in its_l]
            assert max(sl) - min(sl) <= 1, f"list {lst}: segments {sl}"
            assert 2 * ex * x <= sp[1] and sp[1] + ns <= 2 * ex * (x + 1), f"list {lst}: slots"
            for slot in range(sp[1], sp[1] + ns):
                assert slot not in slot_owner, f"slot {slot} shared"
                slot_owner[slot] = lst
    assert lo == n and sorted(per_list) == list(range(n)), "lists missing from the plan"
    return nsplit


def check_plans(mask) -> tuple[int, int]:
    """Both plans of a BlockMask; returns (split rows, split columns)."""
    return (check_plan(mask.row_cnt.cpu().numpy(), mask.row_plan.cpu().numpy(), ROW_PLAN,
                       mask.Tk),
            check_plan(mask.col_cnt.cpu().numpy(), mask.col_plan.cpu().numpy(), COL_PLAN,
                       mask.Tq))


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
