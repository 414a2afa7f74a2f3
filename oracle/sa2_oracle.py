"""Plain fp64 CPU oracle for the SpargeAttention2 hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it; the two meet only through the seeded inputs of the
``workloads`` package.

What it computes, and where the pages say so (SpargeAttention2, arXiv
2602.13515; the method is stated on the gist.science page, section 2):

* Hybrid mask (section 2A and its formula): for every row i of the
  block-pooled attention matrix P-bar, block (i, j) is kept iff j is in
  Top-k(P-bar_i, k%) or in Top-p(P-bar_i, p%).  Top-p is the smallest set whose
  cumulative probability reaches p (section 1, first bullet).
* Block-sparse attention (section 2C): tiles are kept or dropped whole;
  dropped tiles contribute nothing.  The result is therefore ordinary softmax
  attention under the token-level mask that the block mask expands to, which
  is what ``attention_dense`` writes out.
* Trainable (abstract, item ii): gradients of that attention with respect to
  Q, K and V, with the mask held constant (selection is piecewise constant).

Readings taken where the pages are silent (each is listed in the design
notes): pooling is the mean over the tokens present in a block; block scores
use the same 1/sqrt(d) scale as attention; P-bar is the row softmax of the
pooled scores; k% is a fraction of the row's key blocks rounded up (with a
1e-6 guard) and clamped to [1, Tk]; ties in the sort are broken toward the
lower key-block index; "reaches p" means >= p; p >= 1 or k >= 1 select every
block; the attention is bidirectional; LSE is a natural log.

Parity with the authors' own implementation is unpinned (the pages print no
worked example, per-layer value or code); this oracle is pinned instead by
closed forms, library routines, brute force and finite differences in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# Block geometry
# ----------------------------------------------------------------------------

def n_blocks(N: int, b: int) -> int:
    """Number of blocks of size b covering N tokens; the last may be partial."""
    return -(-N // b)


def block_range(i: int, b: int, N: int) -> tuple[int, int]:
    """Token range [lo, hi) of block i (partial last block included)."""
    return i * b, min(N, (i + 1) * b)


# ----------------------------------------------------------------------------
# Mask builder (gist.science page, section 2A)
# ----------------------------------------------------------------------------

def pool_blocks(X: np.ndarray, b: int) -> np.ndarray:
    """Block pooling: mean of the tokens present in each block.

    X: float64 [N, d].  Returns float64 [ceil(N/b), d].
    """
    N = X.shape[0]
    T = n_blocks(N, b)
    out = np.empty((T, X.shape[1]), dtype=np.float64)
    for i in range(T):
        lo, hi = block_range(i, b, N)
        out[i] = X[lo:hi].sum(axis=0) / (hi - lo)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """S-bar = q-bar k-bar^T / sqrt(d): [Tq, Tk] float64."""
    d = qbar.shape[1]
    return (qbar @ kbar.T) / math.sqrt(d)


def row_softmax(S: np.ndarray) -> np.ndarray:
    """P-bar: softmax of each row of S-bar."""
    e = np.exp(S - S.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def topk_count(k_frac: float, Tk: int) -> int:
    """How many key blocks Top-k keeps per row: k% of Tk, rounded up."""
    if k_frac <= 0:
        return 0
    if k_frac >= 1:
        return Tk
    return min(Tk, max(1, math.ceil(k_frac * Tk - 1e-6)))


def row_order(S_row: np.ndarray) -> np.ndarray:
    """Key blocks by descending score; the lower index first on exact ties."""
    idx = np.arange(S_row.shape[0])
    return np.lexsort((idx, -S_row))


def topp_count(P_sorted: np.ndarray, p: float) -> int:
    """Smallest m >= 1 whose first m sorted probabilities sum to at least p.

    P_sorted is one row of P-bar in descending order.  The running sum is the
    plain left-to-right fp64 sum; if it never reaches p (rounding), every block
    is kept.
    """
    Tk = P_sorted.shape[0]
    if p <= 0:
        return 0
    if p >= 1:
        return Tk
    running = np.cumsum(P_sorted)
    hit = np.nonzero(running >= p)[0]
    return int(hit[0]) + 1 if hit.size else Tk


class HeadMask:
    """The hybrid block mask of one (batch, head), with the quantities behind it."""

    def __init__(self, S, P, order, kc, pc, keep):
        self.S = S              # [Tq, Tk] pooled scores
        self.P = P              # [Tq, Tk] P-bar
        self.order = order      # [Tq, Tk] descending-score order per row
        self.kc = kc            # Top-k count (same for every row)
        self.pc = pc            # [Tq] Top-p count per row
        self.count = keep       # [Tq] kept blocks per row = max(kc, pc)

    @property
    def bitmap(self) -> np.ndarray:
        Tq, Tk = self.S.shape
        bm = np.zeros((Tq, Tk), dtype=np.uint8)
        for i in range(Tq):
            bm[i, self.order[i, : self.count[i]]] = 1
        return bm

    def row_lists(self) -> list[np.ndarray]:
        """Kept key blocks of each query-block row, ascending."""
        bm = self.bitmap
        return [np.nonzero(bm[i])[0].astype(np.int32) for i in range(bm.shape[0])]

    def col_lists(self) -> list[np.ndarray]:
        """Query-block rows that kept each key block, ascending."""
        bm = self.bitmap
        return [np.nonzero(bm[:, j])[0].astype(np.int32) for j in range(bm.shape[1])]

    def threshold(self) -> np.ndarray:
        """Per row, the pooled score of the last kept block."""
        Tq = self.S.shape[0]
        return np.array([self.S[i, self.order[i, self.count[i] - 1]] for i in range(Tq)])

    def mass_near_p(self, p: float, tol: float) -> np.ndarray:
        """Rows whose cumulative sorted mass lies within tol of p at the Top-p cut."""
        Tq, Tk = self.S.shape
        out = np.zeros(Tq, dtype=bool)
        if p <= 0 or p >= 1:
            return out
        for i in range(Tq):
            run = np.cumsum(self.P[i, self.order[i]])
            m = self.pc[i]
            for r in (m - 2, m - 1):
                if 0 <= r < Tk and abs(run[r] - p) <= tol:
                    out[i] = True
        return out

    def allowed_counts(self, p: float, tol: float) -> list[set[int]]:
        """Per row, the kept counts that an exact evaluation in another
        summation order may give when the running mass at the Top-p cut lies
        within tol of p.

        The cut is pc = the first m whose running sum run[m-1] reaches p, so
        run[pc-2] < p <= run[pc-1].  If run[pc-2] is within tol of p, another
        order may already reach p there (Top-p keeps pc - 1); if run[pc-1] is
        within tol of p, another order may still fall short (Top-p keeps
        pc + 1).  The row keeps max(kc, that count), so a shifted cut below
        kc changes nothing.  Every set holds the row's own count.
        """
        Tq, Tk = self.S.shape
        out = [{int(c)} for c in self.count]
        if p <= 0 or p >= 1:
            return out
        for i in range(Tq):
            run = np.cumsum(self.P[i, self.order[i]])
            m = int(self.pc[i])
            if m >= 2 and abs(run[m - 2] - p) <= tol:
                out[i].add(max(int(self.kc), m - 1))
            if m <= Tk - 1 and abs(run[m - 1] - p) <= tol:
                out[i].add(max(int(self.kc), m + 1))
        return out


def build_mask_head(Q: np.ndarray, K: np.ndarray, bq: int, bk: int,
                    k_frac: float, p: float) -> HeadMask:
    """Hybrid Top-k + Top-p block mask of one head.

    Q, K: float64 [N, d].  Each row keeps the union of its Top-k and Top-p
    sets.  Both sets are prefixes of the same descending order, so their union
    is the longer prefix.
    """
    kc = topk_count(k_frac, n_blocks(K.shape[0], bk))
    if kc == 0 and p <= 0:
        raise ValueError("both selection rules are disabled: every row would be empty")
    S = block_scores(pool_blocks(Q, bq), pool_blocks(K, bk))
    P = row_softmax(S)
    Tq, Tk = S.shape
    order = np.empty((Tq, Tk), dtype=np.int64)
    pc = np.empty(Tq, dtype=np.int64)
    for i in range(Tq):
        order[i] = row_order(S[i])
        pc[i] = topp_count(P[i, order[i]], p)
    keep = np.maximum(kc, pc)
    return HeadMask(S, P, order, kc, pc, keep)


def build_mask(Q: np.ndarray, K: np.ndarray, bq: int, bk: int,
               k_frac: float, p: float) -> list[list[HeadMask]]:
    """Per (batch, head) masks for Q, K of shape [B, H, N, d]."""
    B, H = Q.shape[:2]
    return [[build_mask_head(Q[b, h], K[b, h], bq, bk, k_frac, p) for h in range(H)]
            for b in range(B)]


def density(masks) -> float:
    """Kept block pairs over all block pairs (sparsity = 1 - density)."""
    kept = 0
    total = 0
    for row in masks:
        for m in row:
            kept += int(m.count.sum())
            total += m.S.size
    return kept / total


# ----------------------------------------------------------------------------
# Block-sparse attention (gist.science page, section 2C; abstract item ii)
# ----------------------------------------------------------------------------

def token_mask(bitmap: np.ndarray, bq: int, bk: int, N: int) -> np.ndarray:
    """M[t, u] = bitmap[t // bq, u // bk] for t, u < N."""
    rows = np.arange(N) // bq
    cols = np.arange(N) // bk
    return bitmap[rows][:, cols].astype(bool)


def attention_dense(Q, K, V, bitmap, bq, bk):
    """Softmax attention of one head under the expanded block mask.

    Returns O [N, d], LSE [N] (natural log), P [N, N].
    """
    N, d = Q.shape
    M = token_mask(bitmap, bq, bk, N)
    S = (Q @ K.T) / math.sqrt(d)
    S = np.where(M, S, -np.inf)
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    l = E.sum(axis=1)
    P = E / l[:, None]
    O = P @ V
    lse = m + np.log(l)
    return O, lse, P


def attention_dense_bwd(Q, K, V, dO, P):
    """Gradients of O = softmax(QK^T/sqrt(d) masked) V for one head.

    dV = P^T dO;  dP = dO V^T;  Delta_t = sum_u P_tu dP_tu;
    dS = P * (dP - Delta);  dQ = dS K / sqrt(d);  dK = dS^T Q / sqrt(d).
    The mask is a constant (masked entries have P = 0, hence dS = 0).
    """
    d = Q.shape[1]
    dV = P.T @ dO
    dP = dO @ V.T
    delta = (P * dP).sum(axis=1)
    dS = P * (dP - delta[:, None])
    dQ = dS @ K / math.sqrt(d)
    dK = dS.T @ Q / math.sqrt(d)
    return dQ, dK, dV


def _kept_tokens(cols: np.ndarray, bk: int, N: int) -> np.ndarray:
    return np.concatenate([np.arange(*block_range(int(j), bk, N)) for j in cols])


def attention_gathered(Q, K, V, row_lists, bq, bk, dO=None, rows=None):
    """The same attention, evaluated per query block on its kept columns only.

    Identical to ``attention_dense`` in exact arithmetic (exp(-inf) = 0), but
    its cost grows with the kept blocks rather than N^2.  ``rows`` restricts
    the forward outputs to a subset of query blocks (their O/LSE entries; the
    rest are NaN); the backward needs every row.

    Returns O, LSE and, when dO is given, dQ, dK, dV.
    """
    N, d = Q.shape
    Tq = n_blocks(N, bq)
    scale = 1.0 / math.sqrt(d)
    O = np.full((N, d), np.nan)
    lse = np.full(N, np.nan)
    want = range(Tq) if rows is None else rows
    grads = dO is not None
    if grads:
        if rows is not None:
            raise ValueError("the backward needs every query block")
        dQ = np.zeros((N, d))
        dK = np.zeros((N, d))
        dV = np.zeros((N, d))
    for i in want:
        lo, hi = block_range(i, bq, N)
        cols = _kept_tokens(row_lists[i], bk, N)
        Qi, Kc, Vc = Q[lo:hi], K[cols], V[cols]
        S = (Qi @ Kc.T) * scale
        m = S.max(axis=1)
        E = np.exp(S - m[:, None])
        l = E.sum(axis=1)
        P = E / l[:, None]
        O[lo:hi] = P @ Vc
        lse[lo:hi] = m + np.log(l)
        if grads:
            dOi = dO[lo:hi]
            dV[cols] += P.T @ dOi
            dP = dOi @ Vc.T
            delta = (P * dP).sum(axis=1)
            dS = P * (dP - delta[:, None])
            dQ[lo:hi] = dS @ Kc * scale
            dK[cols] += dS.T @ Qi * scale
    if grads:
        return O, lse, dQ, dK, dV
    return O, lse


# ----------------------------------------------------------------------------
# One output block at a time (for spot checks at full size)
# ----------------------------------------------------------------------------

def _row_softmax_block(Q, K, row_lists, bq, bk, i):
    """P of query block i over its kept key tokens, with those token ids."""
    N, d = Q.shape
    lo, hi = block_range(i, bq, N)
    cols = _kept_tokens(row_lists[i], bk, N)
    S = (Q[lo:hi] @ K[cols].T) / math.sqrt(d)
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    l = E.sum(axis=1)
    return E / l[:, None], cols, (lo, hi), m + np.log(l)


def forward_query_block(Q, K, V, row_lists, bq, bk, i):
    """O and LSE of the rows of query block i."""
    P, cols, _, lse = _row_softmax_block(Q, K, row_lists, bq, bk, i)
    return P @ V[cols], lse


def dq_query_block(Q, K, V, dO, row_lists, bq, bk, i):
    """dQ of the rows of query block i: dS K / sqrt(d) over its kept keys."""
    d = Q.shape[1]
    P, cols, (lo, hi), _ = _row_softmax_block(Q, K, row_lists, bq, bk, i)
    dP = dO[lo:hi] @ V[cols].T
    delta = (P * dP).sum(axis=1)
    dS = P * (dP - delta[:, None])
    return dS @ K[cols] / math.sqrt(d)


def dkdv_key_block(Q, K, V, dO, row_lists, bq, bk, j):
    """dK and dV of the tokens of key block j.

    Sums, over every query block i whose row keeps block j, P_i^T dO_i and
    dS_i^T Q_i / sqrt(d) restricted to block j's columns; P_i and Delta_i come
    from query block i's whole kept row.
    """
    N, d = Q.shape
    jlo, jhi = block_range(j, bk, N)
    dK = np.zeros((jhi - jlo, d))
    dV = np.zeros((jhi - jlo, d))
    for i, lst in enumerate(row_lists):
        if j not in set(int(x) for x in lst):
            continue
        P, cols, (lo, hi), _ = _row_softmax_block(Q, K, row_lists, bq, bk, i)
        dP = dO[lo:hi] @ V[cols].T
        delta = (P * dP).sum(axis=1)
        dS = P * (dP - delta[:, None])
        sel = (cols >= jlo) & (cols < jhi)
        dV += P[:, sel].T @ dO[lo:hi]
        dK += dS[:, sel].T @ Q[lo:hi] / math.sqrt(d)
    return dK, dV


# ---------------------------------------------------------------------------
# Layer-level velocity distillation (gist.science, section 2B): the sparse
# student is fitted to the frozen full-attention teacher by the squared
# difference of their outputs.  At one attention layer the student output is
# the block-sparse attention and the teacher output the dense attention of the
# same Q, K, V; the expectation of the squared norm is taken as the mean over
# all output elements (a reading: the pages state the objective over a whole
# model's velocity prediction).
# ---------------------------------------------------------------------------
def distill_loss_grad(O_student: np.ndarray, O_teacher: np.ndarray):
    """loss = mean((O_s - O_t)^2); dO = d loss / d O_s = 2 (O_s - O_t) / numel."""
    diff = np.asarray(O_student, dtype=np.float64) - np.asarray(O_teacher, dtype=np.float64)
    n = diff.size
    return float((diff * diff).sum() / n), 2.0 * diff / n


def distill_step(Q, K, V, row_lists, bq, bk, O_teacher=None):
    """One layer-level distillation step on one head: the teacher output (dense
    attention unless given), the student forward over ``row_lists``, the loss,
    its gradient dO and the student's dQ, dK, dV for that dO (teacher fixed).

    Returns loss, dQ, dK, dV, O_student, O_teacher.
    """
    N, d = Q.shape
    if O_teacher is None:
        Tq, Tk = n_blocks(N, bq), n_blocks(N, bk)
        O_teacher, _ = attention_gathered(Q, K, V, [np.arange(Tk)] * Tq, bq, bk)
    O_s, _ = attention_gathered(Q, K, V, row_lists, bq, bk)
    loss, dO = distill_loss_grad(O_s, O_teacher)
    _, _, dQ, dK, dV = attention_gathered(Q, K, V, row_lists, bq, bk, dO=dO)
    return loss, dQ, dK, dV, O_s, O_teacher
