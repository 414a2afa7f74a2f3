"""The work-plan checker (tests/parity.py: check_plan) on plans made on the
host by a small planner written here from the plan rule, so that the checker
that the GPU tests rely on is itself pinned: it accepts every valid plan of
both orders (per-XCD longest first, and head by head over groups of four
XCDs, each XCD a quarter of every head or, where a quarter is too large, the
group dealt in turn), with and without cut lists, and rejects each
plausible defect (a missing or repeated item, items out of order, an item
outside its quarter, a group not dealt in turn, a split slot shared, a
counter left set)."""
from __future__ import annotations

import numpy as np
import pytest

import parity as P

NB = 4096


def _cut(ln, L):
    ns = -(-ln // L) if ln > L else 1
    base, rem = divmod(ln, ns)
    return [(s * base + min(s, rem), base + (1 if s < rem else 0)) for s in range(ns)]


def make_plan(cnt, kd, cap, per_head, rng):
    """A plan as the plan kernel lays it out (order inside a rank bucket
    drawn at random, as the kernel's atomics leave it); returns the int32
    array and the two groups' head-major decisions."""
    cnt = np.clip(np.asarray(cnt, np.int64), 0, cap)
    n, ex = cnt.size, kd["extra"]
    J = P._items_per_xcd(n, kd)
    items = np.zeros((J, 8, 4), np.int32)
    items[:, :, 0] = -1
    items[:, :, 3] = -1
    splits = np.zeros((8 * ex, 4), np.int32)
    splits[:, 0] = -1
    done = np.zeros(kd["counters"] * 8 * ex, np.int32)
    cost = cnt + 1
    total = int(cost.sum())
    q8, r8 = divmod(n, 8)

    def eq(k):
        return k * q8 + min(k, r8)
    pos = [int(cost[:eq(k)].sum()) for k in range(9)]
    worst = max(pos[k + 1] - pos[k] for k in range(8))
    balanced = kd["imbalance"] == 0 or worst * 800 > total * (800 + 8 * kd["imbalance"])
    pref = np.concatenate([[0], np.cumsum(cost)])
    slack = ((n + 7) // 8 + 15) // 16

    def bound(k):
        e = eq(k)
        if not balanced:
            return e
        target = (k * total + 7) // 8
        b = 0 if k == 0 else (int(np.nonzero(pref >= target)[0][0]) if target > 0 else n)
        return min(max(b, max(0, e - slack)), min(n, e + slack))
    b = [bound(k) for k in range(9)]
    L0 = max(kd["min_segment"], kd["fair"] * -(-int(cnt.sum()) // kd["slots"]))
    decisions = []
    for g in range(2):
        G0, G1 = b[4 * g], b[4 * g + 4]
        gshare = int(cnt[G0:G1].sum())
        glong = int(cnt[G0:G1].max()) if G1 > G0 else 0
        Lg = max(L0, -(-gshare // (4 * ex)))
        gseg = max(s for _, s in _cut(glong, Lg))
        hm = G1 > G0 and 4 * gseg * (kd["slots"] // 2) <= gshare + (G1 - G0)
        decisions.append(hm)
        units = [(None, G0, G1, Lg, 4 * ex * g)] if hm else \
            [(x, b[x], b[x + 1], max(L0, -(-int(cnt[b[x]:b[x + 1]].sum()) // ex)), ex * x)
             for x in range(4 * g, 4 * g + 4)]
        for x, c0, c1, L, ebase in units:
            h0 = c0 // per_head
            nh = (c1 - 1) // per_head - h0 + 1 if c1 > c0 else 1
            qn = [0, 0, 0, 0]
            for lid in range(c0, c1):
                qn[(lid % per_head) * 4 // per_head] += len(_cut(int(cnt[lid]), L))
            quarters = hm and kd["quarters"] and max(qn) <= J
            nr = 4 * nh if quarters else nh
            nb = NB // nr if nr <= NB else 1
            its, e_used, p_used = [], 0, 0
            for lid in range(c0, c1):
                segs = _cut(int(cnt[lid]), L)
                entry = -1
                if len(segs) > 1:
                    entry = ebase + e_used
                    e_used += 1
                    splits[entry] = (lid, 2 * ebase + p_used, len(segs), 0)
                    p_used += len(segs)
                for s2, (st, sl) in enumerate(segs):
                    if hm:
                        hh = ((lid % per_head) * 4 // per_head) * nh if quarters else 0
                        hh += lid // per_head - h0
                        hb = hh if nr <= NB else hh * NB // nr
                        key = NB - 1 - (hb * nb + nb - 1 - min(nb - 1, sl * nb // (gseg + 1)))
                    else:
                        key = min(sl, NB - 1)
                    its.append((key, rng.random(),
                                (lid, st, sl, entry * 1024 + s2 if len(segs) > 1 else -1)))
            its.sort(key=lambda t: (-t[0], t[1]))
            qpos = [0, 0, 0, 0]
            for k, (_, _, it) in enumerate(its):
                if quarters:   # XCD 4g + r: quarter r of every head
                    r = (it[0] % per_head) * 4 // per_head
                    items[qpos[r], 4 * g + r] = it
                    qpos[r] += 1
                elif hm:       # a quarter too large: dealt in turn
                    items[k // 4, 4 * g + k % 4] = it
                else:
                    items[k, x] = it
    return np.concatenate([items.reshape(-1), splits.reshape(-1), done]), decisions


def _cases():
    """(kind, counts, cap, per_head): both orders, cut lists, skewed heads."""
    rng = np.random.default_rng(7)
    out = []
    # many short lists: head by head
    out.append(("rows", rng.integers(0, 4, 300 * 32), 64, 32))
    out.append(("cols", rng.integers(0, 3, 200 * 64), 64, 64))
    # long lists, some cut: longest first per XCD
    c = rng.integers(1, 6, 24 * 40)
    c[rng.integers(0, c.size, 5)] = 300
    out.append(("rows", c, 400, 40))
    out.append(("cols", np.minimum(rng.geometric(0.05, 16 * 90), 512), 512, 90))
    # one head far denser than the rest (cost-balanced shares)
    c = rng.integers(0, 3, 12 * 128)
    c[:128] = 60
    out.append(("cols", c, 256, 128))
    # fewer lists than XCDs
    out.append(("rows", np.array([3, 0, 5]), 8, 3))
    # five lists per head: quarter 0 holds two of them, more than an XCD's
    # slots, so the head-major groups are dealt in turn
    out.append(("rows", rng.integers(0, 3, 500 * 5), 8, 5))
    return out


@pytest.mark.parametrize("case", range(len(_cases())))
def test_checker_accepts_valid_plans(case):
    kind, cnt, cap, per_head = _cases()[case]
    kd = P.ROW_PLAN if kind == "rows" else P.COL_PLAN
    plan, decisions = make_plan(cnt, kd, cap, per_head, np.random.default_rng(case))
    got = []
    P.check_plan(cnt, plan, kd, cap, per_head, got)
    assert got == decisions


def test_both_orders_are_exercised():
    kinds = set()
    for kind, cnt, cap, per_head in _cases():
        kd = P.ROW_PLAN if kind == "rows" else P.COL_PLAN
        _, dec = make_plan(cnt, kd, cap, per_head, np.random.default_rng(0))
        kinds.update(dec)
    assert kinds == {True, False}


def _plan_views(plan, n, kd):
    J = P._items_per_xcd(n, kd)
    ex = kd["extra"]
    items = plan[:8 * J * 4].reshape(J, 8, 4)
    splits = plan[8 * J * 4:8 * J * 4 + 8 * ex * 4].reshape(8 * ex, 4)
    done = plan[8 * J * 4 + 8 * ex * 4:]
    return items, splits, done


def _valid(case_index):
    kind, cnt, cap, per_head = _cases()[case_index]
    kd = P.ROW_PLAN if kind == "rows" else P.COL_PLAN
    plan, dec = make_plan(cnt, kd, cap, per_head, np.random.default_rng(1))
    return kd, cnt, cap, per_head, plan, dec


def _rejects(kd, cnt, cap, per_head, plan):
    with pytest.raises(AssertionError):
        P.check_plan(cnt, plan, kd, cap, per_head)


def test_rejects_a_missing_item():
    kd, cnt, cap, ph, plan, _ = _valid(0)
    items, _, _ = _plan_views(plan, cnt.size, kd)
    nz = np.argwhere(items[:, :, 0] >= 0)
    j, x = nz[len(nz) // 2]
    last = int(np.count_nonzero(items[:, x, 0] >= 0)) - 1
    items[j:last, x] = items[j + 1:last + 1, x].copy()   # close the gap
    items[last, x] = (-1, 0, 0, -1)
    _rejects(kd, cnt, cap, ph, plan)


def test_rejects_a_repeated_item():
    kd, cnt, cap, ph, plan, _ = _valid(2)
    items, _, _ = _plan_views(plan, cnt.size, kd)
    x = 0
    k = int(np.count_nonzero(items[:, x, 0] >= 0))
    items[k, x] = items[k - 1, x]
    _rejects(kd, cnt, cap, ph, plan)


def test_rejects_head_major_items_out_of_head_order():
    kd, cnt, cap, ph, plan, dec = _valid(0)
    assert dec == [True, True]
    items, _, _ = _plan_views(plan, cnt.size, kd)
    # swap the first item of the group with one of a later head
    a = items[0, 0].copy()
    j = np.nonzero(items[:, 1, 0] // ph > a[0] // ph)[0][0]
    items[0, 0], items[j, 1] = items[j, 1].copy(), a
    _rejects(kd, cnt, cap, ph, plan)


def test_rejects_an_item_outside_its_quarter():
    kd, cnt, cap, ph, plan, dec = _valid(0)   # rows: quarters
    assert dec == [True, True] and kd["quarters"]
    items, _, _ = _plan_views(plan, cnt.size, kd)
    # move XCD 3's last item to the end of XCD 0's column
    k3 = int(np.count_nonzero(items[:, 3, 0] >= 0))
    k0 = int(np.count_nonzero(items[:, 0, 0] >= 0))
    items[k0, 0] = items[k3 - 1, 3]
    items[k3 - 1, 3] = (-1, 0, 0, -1)
    _rejects(kd, cnt, cap, ph, plan)


def test_quarter_and_dealt_layouts_are_exercised():
    seen = set()
    for kind, cnt, cap, per_head in _cases():
        kd = P.ROW_PLAN if kind == "rows" else P.COL_PLAN
        plan, dec = make_plan(cnt, kd, cap, per_head, np.random.default_rng(0))
        items, _, _ = _plan_views(plan, cnt.size, kd)
        for g in range(2):
            if not dec[g]:
                continue
            lists = items[:, 4 * g, 0]
            lists = lists[lists >= 0]
            seen.add(bool(np.all((lists % per_head) * 4 // per_head == 0)))
    assert seen == {True, False}


def test_rejects_a_group_not_dealt_in_turn():
    kd, cnt, cap, ph, plan, dec = _valid(len(_cases()) - 1)
    assert dec == [True, True]
    items, _, _ = _plan_views(plan, cnt.size, kd)
    # move XCD 3's last item to the end of XCD 0's column
    k3 = int(np.count_nonzero(items[:, 3, 0] >= 0))
    k0 = int(np.count_nonzero(items[:, 0, 0] >= 0))
    items[k0, 0] = items[k3 - 1, 3]
    items[k3 - 1, 3] = (-1, 0, 0, -1)
    _rejects(kd, cnt, cap, ph, plan)


def test_rejects_longest_first_broken():
    kd, cnt, cap, ph, plan, dec = _valid(2)
    assert dec == [False, False]
    items, _, _ = _plan_views(plan, cnt.size, kd)
    x = 1
    k = int(np.count_nonzero(items[:, x, 0] >= 0))
    lens = items[:k, x, 2]
    i = int(np.argmax(lens > lens[-1]))     # an item longer than the last one
    items[[i, k - 1], x] = items[[k - 1, i], x]
    _rejects(kd, cnt, cap, ph, plan)


def test_rejects_a_shared_split_slot():
    kd, cnt, cap, ph, plan, _ = _valid(2)
    _, splits, _ = _plan_views(plan, cnt.size, kd)
    used = np.nonzero(splits[:, 0] >= 0)[0]
    assert len(used) >= 2
    splits[used[1], 1] = splits[used[0], 1]
    _rejects(kd, cnt, cap, ph, plan)


def test_rejects_a_counter_left_set():
    kd, cnt, cap, ph, plan, _ = _valid(3)
    _, _, done = _plan_views(plan, cnt.size, kd)
    done[5] = 1
    _rejects(kd, cnt, cap, ph, plan)
