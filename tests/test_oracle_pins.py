"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each test ties one part of the oracle to something the pages or the
mathematics fix: a hand-worked example, a closed form, a library routine,
brute force on tiny inputs, finite differences, or an invariant.  They are
chosen so that a plausible slip (a dropped 1/sqrt(d), a transposed operand, a
wrong sign, an off-by-one in the Top-p cut, the wrong tie-break) fails at
least one of them.  Pages: SpargeAttention2 on gist.science (section 1 for the
failure modes and the Top-p definition, 2A for the hybrid mask, 2C for the
tile-dropping kernel); the abstract (item ii: the sparse attention is
trainable).
"""
import itertools
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = Path(__file__).parent / "golden"


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def _hand_qk(m):
    """Q, K realising pooled scores m_j exactly (see the golden fixture)."""
    Tk = len(m)
    Q = np.zeros((8, 4))
    Q[:, 0] = 2.0
    K = np.zeros((2 * Tk, 4))
    for j, mj in enumerate(m):
        K[2 * j, 0] = mj - 0.5
        K[2 * j + 1, 0] = mj + 0.5
    return Q, K


# ---------------------------------------------------------------------------
# Mask builder
# ---------------------------------------------------------------------------

def test_hand_worked_masks():
    fx = json.loads((GOLDEN / "hybrid_mask_hand.json").read_text())
    n = 0
    for case in fx["cases"]:
        Q, K = _hand_qk(case["m"])
        for c in case["checks"]:
            # Q has 8 tokens and K 2*Tk: pool them with their own block sizes
            hm = O.build_mask_head(Q, K, 8, 2, c["k_frac"], c["p"])
            assert hm.kc == c["kc"], (case["name"], c)
            assert int(hm.pc[0]) == c["pc"], (case["name"], c)
            assert hm.bitmap[0].tolist() == c["bitmap"], (case["name"], c)
            n += 1
    assert n == 14


def _closed_form_runs():
    """r1..r3 of the row m = [0, 2, -1, 1] from their closed forms (see the fixture)."""
    e = math.e
    Z = e * e + e + 1.0 + 1.0 / e
    return {"r1": e * e / Z, "r2": (e * e + e) / Z, "r3": (e * e + e + 1.0) / Z}


def test_checker_threshold_hand_worked():
    """HeadMask.threshold(): the pooled score of each row's last kept block."""
    fx = json.loads((GOLDEN / "mask_checker_hand.json").read_text())
    for c in fx["threshold_cases"]:
        Q, K = _hand_qk(c["m"])
        hm = O.build_mask_head(Q, K, 8, 2, c["k_frac"], c["p"])
        assert int(hm.count[0]) == c["count"], c
        assert hm.threshold()[0] == c["threshold"], c


def test_checker_mass_near_p_hand_worked():
    """HeadMask.mass_near_p() and allowed_counts() at the Top-p cut: rows whose
    running mass lies 5e-7 and 2e-6 from p, on either side of the cut, and a
    Top-k count that hides a moved cut."""
    fx = json.loads((GOLDEN / "mask_checker_hand.json").read_text())
    runs = _closed_form_runs()
    Q, K = _hand_qk([0.0, 2.0, -1.0, 1.0])
    for c in fx["mass_cases"]:
        p = runs[c["base"]] + c["offset"]
        hm = O.build_mask_head(Q, K, 8, 2, c["k_frac"], p)
        assert int(hm.pc[0]) == c["pc"], c
        assert bool(hm.mass_near_p(p, c["tol"])[0]) == c["near"], c
        assert hm.allowed_counts(p, c["tol"])[0] == set(c["allowed"]), c
    # the rules are off: nothing is near, only the own count is allowed
    hm = O.build_mask_head(Q, K, 8, 2, 0.5, 0.0)
    assert not hm.mass_near_p(0.0, 1.0)[0] and hm.allowed_counts(0.0, 1.0)[0] == {2}


def test_pooling_brute_force_and_ragged():
    X = _rand((13, 3), 1)
    P = O.pool_blocks(X, 4)      # blocks of 4, 4, 4, 1
    assert P.shape == (4, 3)
    for i in range(4):
        toks = [X[t] for t in range(13) if t // 4 == i]
        want = [sum(v[c] for v in toks) / len(toks) for c in range(3)]
        assert np.allclose(P[i], want, rtol=0, atol=1e-15)
    assert np.array_equal(P[3], X[12])         # a one-token block is itself


def test_block_scores_scale_and_orientation():
    qb = _rand((3, 16), 2)
    kb = _rand((5, 16), 3)
    S = O.block_scores(qb, kb)
    for i in range(3):
        for j in range(5):
            assert abs(S[i, j] - sum(qb[i] * kb[j]) / 4.0) < 1e-13


def test_topk_count_rounding():
    assert O.topk_count(2 / 16, 16) == 2          # a stated count passes through
    assert O.topk_count(0.03, 512) == 16          # ceil(15.36)
    assert O.topk_count(0.03, 1182) == 36         # ceil(35.46)
    assert O.topk_count(1e-9, 100) == 1           # never below one block
    assert O.topk_count(0.0, 100) == 0
    assert O.topk_count(1.0, 100) == 100


def _mask_from_scores(S, k_frac, p):
    """Mask of a score matrix S [Tq, Tk], realised through the pooled path."""
    Tq, Tk = S.shape
    # d = Tq, q-bar_i = sqrt(d) e_i, k-bar_j = S[:, j]: scores are exactly S
    d = Tq
    Q = math.sqrt(d) * np.eye(Tq)
    K = S.T.copy()
    return O.build_mask_head(Q, K, 1, 1, k_frac, p)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_union_contains_both_rules(seed):
    S = _rand((24, 40), 10 + seed, 2.0)
    for k_frac, p in [(0.05, 0.5), (0.1, 0.9), (0.2, 0.3), (0.025, 0.97)]:
        h = _mask_from_scores(S, k_frac, p).bitmap
        k_only = _mask_from_scores(S, k_frac, 0.0).bitmap
        p_only = _mask_from_scores(S, 0.0, p).bitmap
        assert np.all(h >= k_only) and np.all(h >= p_only)
        assert np.array_equal(h, np.maximum(k_only, p_only))


def test_kept_set_is_a_score_prefix():
    S = _rand((30, 50), 20, 1.5)
    S[:, 7] = S[:, 8]                      # exact ties to exercise the tie-break
    hm = _mask_from_scores(S, 0.1, 0.6)
    bm = hm.bitmap
    for i in range(30):
        kept = np.nonzero(bm[i])[0]
        drop = np.nonzero(bm[i] == 0)[0]
        # every kept block beats every dropped one: higher score, or equal
        # score and a lower index
        for a in kept:
            for b in drop:
                assert S[i, a] > S[i, b] or (S[i, a] == S[i, b] and a < b)
        assert bm[i].sum() == max(hm.kc, hm.pc[i])


def _brute_topp(P_row, p):
    """Smallest subset with mass >= p; among those of that size the largest
    mass, then the lexicographically smallest index set."""
    Tk = len(P_row)
    for size in range(1, Tk + 1):
        best = None
        for sub in itertools.combinations(range(Tk), size):
            mass = sum(P_row[j] for j in sub)
            if mass >= p:
                key = (-mass, sub)
                if best is None or key < best[0]:
                    best = (key, sub)
        if best is not None:
            return set(best[1])
    return set(range(Tk))


@pytest.mark.parametrize("seed", range(6))
def test_topp_matches_brute_force(seed):
    Tk = 10
    S = _rand((4, Tk), 30 + seed, 1.0 + seed)
    for p in (0.3, 0.5, 0.8, 0.95):
        hm = _mask_from_scores(S, 0.0, p)
        for i in range(S.shape[0]):
            e = np.exp(S[i] - S[i].max())
            want = _brute_topp(e / e.sum(), p)
            assert set(np.nonzero(hm.bitmap[i])[0]) == want


def test_topk_matches_argpartition():
    S = _rand((16, 64), 40)
    for k_frac in (0.02, 0.1, 0.5):
        hm = _mask_from_scores(S, k_frac, 0.0)
        kc = hm.kc
        for i in range(16):
            want = set(np.argsort(-S[i], kind="stable")[:kc])
            assert set(np.nonzero(hm.bitmap[i])[0]) == want


def test_dense_special_cases():
    S = _rand((8, 12), 50)
    assert np.all(_mask_from_scores(S, 1.0, 0.0).bitmap == 1)
    assert np.all(_mask_from_scores(S, 0.05, 1.0).bitmap == 1)
    with pytest.raises(ValueError):
        _mask_from_scores(S, 0.0, 0.0)


def test_near_uniform_rows_closed_form():
    """Top-p on (almost) uniform rows keeps about p*Tk blocks (section 1)."""
    Tk = 256
    S = _rand((20, Tk), 60, 1e-7)
    for p in (0.3, 0.55, 0.9):
        hm = _mask_from_scores(S, 0.0, p)
        for i in range(20):
            assert abs(int(hm.pc[i]) - math.ceil(p * Tk)) <= 1


def test_sink_rows_closed_form():
    """A block holding mass >= p collapses Top-p to that block (section 1)."""
    S = _rand((10, 64), 70)
    S[:, 3] += 20.0
    hm = _mask_from_scores(S, 0.0, 0.9)
    assert np.all(hm.bitmap.sum(axis=1) == 1) and np.all(hm.bitmap[:, 3] == 1)
    hy = _mask_from_scores(S, 4 / 64, 0.9)
    assert np.all(hy.bitmap.sum(axis=1) == 4) and np.all(hy.bitmap[:, 3] == 1)


def test_density_monotone():
    S = _rand((16, 48), 80, 1.5)
    last = 0
    for p in np.linspace(0.05, 0.99, 12):
        dens = _mask_from_scores(S, 0.02, p).bitmap.sum()
        assert dens >= last
        last = dens
    last = 0
    for k in np.linspace(0.0, 1.0, 11):
        dens = _mask_from_scores(S, k, 0.4).bitmap.sum()
        assert dens >= last
        last = dens


def test_row_and_column_lists():
    S = _rand((9, 17), 90)
    hm = _mask_from_scores(S, 0.2, 0.5)
    bm = hm.bitmap
    rows = hm.row_lists()
    cols = hm.col_lists()
    for i in range(9):
        assert list(rows[i]) == [j for j in range(17) if bm[i, j]]
    for j in range(17):
        assert list(cols[j]) == [i for i in range(9) if bm[i, j]]


# ---------------------------------------------------------------------------
# Attention forward
# ---------------------------------------------------------------------------

def test_forward_all_ones_equals_sdpa_and_textbook():
    N, d = 96, 16
    Q, K, V = (_rand((N, d), s) for s in (1, 2, 3))
    ones = np.ones((3, 3), dtype=np.uint8)
    Oo, lse, P = O.attention_dense(Q, K, V, ones, 32, 32)
    t = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V))[0, 0].numpy()
    assert np.abs(Oo - ref).max() < 1e-12
    S = Q @ K.T / math.sqrt(d)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    assert np.abs(Oo - (E / E.sum(axis=1, keepdims=True)) @ V).max() < 1e-12
    from scipy.special import logsumexp
    assert np.abs(lse - logsumexp(S, axis=1)).max() < 1e-12


def test_forward_block_diagonal_is_per_block_attention():
    N, d, b = 96, 8, 32
    Q, K, V = (_rand((N, d), s) for s in (4, 5, 6))
    Oo, _, _ = O.attention_dense(Q, K, V, np.eye(3, dtype=np.uint8), b, b)
    for i in range(3):
        sl = slice(i * b, (i + 1) * b)
        want, _, _ = O.attention_dense(Q[sl], K[sl], V[sl], np.ones((1, 1), np.uint8), b, b)
        assert np.abs(Oo[sl] - want).max() < 1e-13


def test_forward_masked_matches_sdpa_with_bool_mask_and_ragged_blocks():
    N, d, bq, bk = 100, 8, 32, 16      # ragged: 4 q-blocks (last 4 rows), 7 k-blocks
    Q, K, V = (_rand((N, d), s) for s in (7, 8, 9))
    bm = (np.random.default_rng(3).random((4, 7)) < 0.4).astype(np.uint8)
    bm[np.arange(4), np.arange(4)] = 1
    Oo, lse, P = O.attention_dense(Q, K, V, bm, bq, bk)
    M = np.zeros((N, N), dtype=bool)
    for t in range(N):
        for u in range(N):
            M[t, u] = bool(bm[t // bq, u // bk])
    t_ = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t_(Q), t_(K), t_(V), attn_mask=torch.from_numpy(M)[None, None])[0, 0].numpy()
    assert np.abs(Oo - ref).max() < 1e-12
    assert np.abs(P.sum(axis=1) - 1).max() < 1e-13
    assert np.all(P[~M] == 0)


def test_forward_constant_v_rows():
    N, d = 64, 8
    Q, K = _rand((N, d), 10), _rand((N, d), 11)
    v = _rand((d,), 12)
    V = np.tile(v, (N, 1))
    bm = (np.random.default_rng(5).random((4, 4)) < 0.5).astype(np.uint8)
    bm[:, 0] = 1
    Oo, _, _ = O.attention_dense(Q, K, V, bm, 16, 16)
    assert np.abs(Oo - v).max() < 1e-14


def test_gathered_equals_dense():
    N, d, bq, bk = 200, 16, 64, 32
    Q, K, V, dO = (_rand((N, d), s) for s in (13, 14, 15, 16))
    hm = O.build_mask_head(Q, K, bq, bk, 0.2, 0.5)
    O1, l1, P = O.attention_dense(Q, K, V, hm.bitmap, bq, bk)
    g1 = O.attention_dense_bwd(Q, K, V, dO, P)
    O2, l2, *g2 = O.attention_gathered(Q, K, V, hm.row_lists(), bq, bk, dO=dO)
    assert np.abs(O1 - O2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13
    for a, b in zip(g1, g2):
        assert np.abs(a - b).max() < 1e-12


# ---------------------------------------------------------------------------
# Attention backward (the trainable path)
# ---------------------------------------------------------------------------

def _loss(Q, K, V, dO, bm, bq, bk):
    Oo, _, _ = O.attention_dense(Q, K, V, bm, bq, bk)
    return float((Oo * dO).sum())


def test_backward_finite_differences():
    N, d, b = 128, 16, 32
    Q, K, V, dO = (_rand((N, d), s) for s in (20, 21, 22, 23))
    bm = (np.random.default_rng(9).random((4, 4)) < 0.5).astype(np.uint8)
    bm[np.arange(4), (np.arange(4) + 1) % 4] = 1
    _, _, P = O.attention_dense(Q, K, V, bm, b, b)
    grads = O.attention_dense_bwd(Q, K, V, dO, P)
    rng = np.random.default_rng(0)
    h = 1e-6
    for which, g in zip(range(3), grads):
        for _ in range(6):
            t, c = int(rng.integers(N)), int(rng.integers(d))
            args = [Q.copy(), K.copy(), V.copy()]
            args[which][t, c] += h
            up = _loss(*args, dO, bm, b, b)
            args[which][t, c] -= 2 * h
            dn = _loss(*args, dO, bm, b, b)
            fd = (up - dn) / (2 * h)
            assert abs(fd - g[t, c]) <= 1e-6 * max(1.0, abs(g[t, c])), (which, t, c)


def test_backward_matches_torch_autograd():
    N, d, bq, bk = 96, 8, 32, 16
    Q, K, V, dO = (_rand((N, d), s) for s in (30, 31, 32, 33))
    bm = (np.random.default_rng(4).random((3, 6)) < 0.5).astype(np.uint8)
    bm[:, 0] = 1
    _, _, P = O.attention_dense(Q, K, V, bm, bq, bk)
    dQ, dK, dV = O.attention_dense_bwd(Q, K, V, dO, P)
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_() for a in (Q, K, V))
    M = torch.from_numpy(O.token_mask(bm, bq, bk, N))
    S = (tq @ tk.T) / math.sqrt(d)
    S = S.masked_fill(~M, float("-inf"))
    out = torch.softmax(S, dim=1) @ tv
    out.backward(torch.from_numpy(dO))
    for mine, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-12


def test_backward_invariants():
    N, d, bq, bk = 192, 16, 64, 32
    Q, K, V, dO = (_rand((N, d), s) for s in (40, 41, 42, 43))
    hm = O.build_mask_head(Q, K, bq, bk, 0.2, 0.4)
    _, _, P = O.attention_dense(Q, K, V, hm.bitmap, bq, bk)
    dQ, dK, dV = O.attention_dense_bwd(Q, K, V, dO, P)
    assert np.abs(dK.sum(axis=0)).max() < 1e-12          # softmax shift invariance
    assert np.abs(dV.sum(axis=0) - dO.sum(axis=0)).max() < 1e-12   # rows of P sum to 1
    assert abs((Q * dQ).sum() - (K * dK).sum()) < 1e-10


def test_per_block_functions_match_the_whole_head():
    N, d, bq, bk = 300, 16, 64, 32     # ragged on both axes
    Q, K, V, dO = (_rand((N, d), s) for s in (50, 51, 52, 53))
    hm = O.build_mask_head(Q, K, bq, bk, 0.15, 0.5)
    rows = hm.row_lists()
    Oo, lse, P = O.attention_dense(Q, K, V, hm.bitmap, bq, bk)
    dQ, dK, dV = O.attention_dense_bwd(Q, K, V, dO, P)
    for i in range(hm.S.shape[0]):
        lo, hi = O.block_range(i, bq, N)
        o_i, l_i = O.forward_query_block(Q, K, V, rows, bq, bk, i)
        assert np.abs(o_i - Oo[lo:hi]).max() < 1e-13 and np.abs(l_i - lse[lo:hi]).max() < 1e-13
        assert np.abs(O.dq_query_block(Q, K, V, dO, rows, bq, bk, i) - dQ[lo:hi]).max() < 1e-12
    for j in range(hm.S.shape[1]):
        lo, hi = O.block_range(j, bk, N)
        k_j, v_j = O.dkdv_key_block(Q, K, V, dO, rows, bq, bk, j)
        assert np.abs(k_j - dK[lo:hi]).max() < 1e-12 and np.abs(v_j - dV[lo:hi]).max() < 1e-12


# ---------------------------------------------------------------------------
# Layer-level velocity distillation (gist.science, section 2B)
# ---------------------------------------------------------------------------
def _rows_from_bitmap(bm):
    return [np.flatnonzero(r) for r in bm]


def test_distill_gradient_is_derivative_of_loss():
    """dO = 2 (O_s - O_t) / numel is d loss / d O_s (central differences)."""
    Os, Ot = _rand((40, 8), 50), _rand((40, 8), 51)
    loss, dO = O.distill_loss_grad(Os, Ot)
    assert loss == pytest.approx(float(((Os - Ot) ** 2).mean()), rel=1e-15)
    h = 1e-6
    for t, c in ((0, 0), (7, 3), (39, 7)):
        up, dn = Os.copy(), Os.copy()
        up[t, c] += h
        dn[t, c] -= h
        fd = (O.distill_loss_grad(up, Ot)[0] - O.distill_loss_grad(dn, Ot)[0]) / (2 * h)
        assert abs(fd - dO[t, c]) <= 1e-9


def test_distill_step_finite_differences():
    """Gradients of the whole distillation step (student through the sparse
    attention, teacher held fixed) against central differences of its loss."""
    N, d, b = 128, 16, 32
    Q, K, V = (_rand((N, d), s) for s in (60, 61, 62))
    bm = np.zeros((4, 4), np.uint8)
    bm[np.arange(4), np.arange(4)] = 1
    bm[np.arange(4), (np.arange(4) + 2) % 4] = 1
    rows = _rows_from_bitmap(bm)
    loss, dQ, dK, dV, Os, Ot = O.distill_step(Q, K, V, rows, b, b)
    assert loss > 1e-3                                   # the sparse student differs
    def loss_of(q, k, v):
        return O.distill_step(q, k, v, rows, b, b, O_teacher=Ot)[0]
    rng = np.random.default_rng(3)
    h = 1e-6
    for which, g in zip(range(3), (dQ, dK, dV)):
        for _ in range(5):
            t, c = int(rng.integers(N)), int(rng.integers(d))
            args = [Q.copy(), K.copy(), V.copy()]
            args[which][t, c] += h
            up = loss_of(*args)
            args[which][t, c] -= 2 * h
            dn = loss_of(*args)
            fd = (up - dn) / (2 * h)
            assert abs(fd - g[t, c]) <= 1e-7 * max(1.0, abs(g[t, c])) + 1e-10, (which, t, c)


def test_distill_with_every_block_kept_is_zero():
    """Student = teacher when the mask keeps every block: loss and gradients 0."""
    N, d, b = 96, 8, 32
    Q, K, V = (_rand((N, d), s) for s in (70, 71, 72))
    rows = [np.arange(3)] * 3
    loss, dQ, dK, dV, Os, Ot = O.distill_step(Q, K, V, rows, b, b)
    assert loss <= 1e-28
    for g in (dQ, dK, dV):
        assert np.abs(g).max() <= 1e-14
