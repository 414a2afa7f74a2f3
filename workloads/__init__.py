"""Seeded synthetic inputs for the SpargeAttention2 hot path.

This module is the one piece of code that both sides of every parity check
use: it draws Q, K, V and dO for each workload, and it names the workload
shapes.  It holds none of the method's arithmetic (no pooling, no scores, no
masks, no attention): only random numbers, the smooth-grid signal that stands
in for video-diffusion activations, and the shape table.

Every draw is seeded with a numpy ``SeedSequence`` keyed on
``(seed, tensor, head)``, so each head of each tensor is an independent
stream.  That lets a caller regenerate only the heads it needs (the CPU oracle
checks a subset of heads at the large shapes) and lets the generator fan out
over threads, with identical values either way.

Workloads (shapes from the benchmark's statement of the problem; the pages
themselves fix no shapes, see SpargeAttention2 on gist.science, section 4,
for the Wan2.1 1.3B/480p and 14B/720p models they stand in for):

* ``c0``   B=1 H=2 N=1024 d=64, fp32 N(0,1) inputs, 64x64 blocks, k = 2 blocks
  per row, p = 0.9.
* ``c0b``  the smooth-grid signal on a 4x16x16 grid, d=64, Q and K sharing one
  signal at amplitude 2 (a row regime where Top-k keeps more than Top-p).
* ``c0c``  c0 with p = 0.3, so both rules are active.
* ``c1``   Wan2.1-1.3B-shaped layer: H=12, N=32760 (21x30x52 latent grid,
  frame-major), d=128, bf16, q-block 128, k-block 64, k = 3% plus Top-p with
  p tuned for 5% density.  Forward only.
* ``c2``   ``c1`` plus the backward pass (dO ~ N(0,1)).
* ``c3``   14B-720p-shaped layer: H=40, N=75600 (21x45x80), same generator.
* ``c4``   mask-rule stress: H=8, N=16384 (16x32x32), three score regimes
  (sink / near-uniform / smooth) and four target densities.
"""
from __future__ import annotations

import concurrent.futures as _cf
import json
import math
import os
from dataclasses import dataclass, field, replace
from pathlib import Path

import numpy as np

TENSORS = ("q", "k", "v", "do")
_TENSOR_ID = {name: i for i, name in enumerate(TENSORS)}

TUNED_PARAMS_PATH = Path(__file__).resolve().parent.parent / "tests" / "golden" / "tuned_params.json"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    bq: int
    bk: int
    gen: str                      # "normal" | "smooth" | "sink" | "uniform"
    seed: int
    dtype: str                    # "f32" | "bf16"
    k_frac: float
    p: float | None               # None: tuned for target_density
    target_density: float | None = None
    grid: tuple[int, int, int] | None = None
    shared_signal: bool = False   # Q and K share one smooth signal (c0b)
    amplitude: float = 0.5        # per-sinusoid amplitude of the smooth signal
    backward: bool = True
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def Tq(self) -> int:
        return -(-self.N // self.bq)

    @property
    def Tk(self) -> int:
        return -(-self.N // self.bk)


WORKLOADS: dict[str, Workload] = {
    "c0": Workload("c0", 1, 2, 1024, 64, 64, 64, "normal", 0, "f32", 2 / 16, 0.9),
    "c0b": Workload("c0b", 1, 2, 1024, 64, 64, 64, "smooth", 5, "f32", 2 / 16, 0.9,
                    grid=(4, 16, 16), shared_signal=True, amplitude=2.0),
    "c0c": Workload("c0c", 1, 2, 1024, 64, 64, 64, "normal", 0, "f32", 2 / 16, 0.3),
    "c1": Workload("c1", 1, 12, 32760, 128, 128, 64, "smooth", 1, "bf16", 0.03, None,
                   target_density=0.05, grid=(21, 30, 52), backward=False),
    "c2": Workload("c2", 1, 12, 32760, 128, 128, 64, "smooth", 1, "bf16", 0.03, None,
                   target_density=0.05, grid=(21, 30, 52), backward=True),
    # the 1.3B layer with square 64 x 64 blocks (a second block geometry)
    "c2_b64": Workload("c2_b64", 1, 12, 32760, 128, 64, 64, "smooth", 1, "bf16", 0.03, None,
                       target_density=0.05, grid=(21, 30, 52), backward=True),
    "c3": Workload("c3", 1, 40, 75600, 128, 128, 64, "smooth", 3, "bf16", 0.03, None,
                   target_density=0.05, grid=(21, 45, 80), backward=True),
}

C4_DENSITIES = (0.20, 0.10, 0.05, 0.03)
C4_REGIMES = {"sink": 40, "uniform": 41, "smooth": 42}
for _reg, _seed in C4_REGIMES.items():
    for _D in C4_DENSITIES:
        _name = f"c4_{_reg}_{int(round(_D * 100)):02d}"
        WORKLOADS[_name] = Workload(_name, 1, 8, 16384, 128, 128, 64, _reg, _seed, "bf16",
                                    round(0.6 * _D, 6), None, target_density=_D,
                                    grid=(16, 32, 32), backward=True)


def _rng(seed: int, tensor: str, head: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, _TENSOR_ID[tensor], head]))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def smooth_signal(grid, d: int, rng: np.random.Generator, amplitude: float = 0.5,
                  n_waves: int = 8) -> np.ndarray:
    """Low-frequency field on a T x Y x X token grid, flattened frame-major.

    Per channel: the sum of ``n_waves`` sinusoids
    ``amplitude * sin(2*pi*(f_t t/T + f_y y/Y + f_x x/X) + phi)`` with each
    frequency uniform in [0, 2) cycles per axis extent and phi uniform in
    [0, 2*pi).  At amplitude 0.5 and 8 waves the field has unit variance in
    expectation.  Returns float64 channel-major [d, T*Y*X].
    """
    T, Y, X = grid
    f = rng.uniform(0.0, 2.0, size=(n_waves, 3, d))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=(n_waves, d))
    t = (np.arange(T) / T)[:, None]
    yx_y = np.repeat(np.arange(Y) / Y, X)[:, None]
    yx_x = np.tile(np.arange(X) / X, Y)[:, None]
    # sin(a + b) = sin a cos b + cos a sin b, with a the frame term (plus
    # phase) and b the in-frame term: the field is then a per-channel product
    # of a [T, 2W] and a [2W, Y*X] factor, which avoids a sine per token.
    a = 2.0 * np.pi * f[:, 0, None, :] * t[None] + phi[:, None, :]          # [W, T, d]
    b = 2.0 * np.pi * (f[:, 1, None, :] * yx_y[None] + f[:, 2, None, :] * yx_x[None])  # [W, YX, d]
    left = amplitude * np.concatenate([np.sin(a), np.cos(a)], axis=0)      # [2W, T, d]
    right = np.concatenate([np.cos(b), np.sin(b)], axis=0)                  # [2W, YX, d]
    import torch
    s = torch.bmm(torch.from_numpy(np.ascontiguousarray(left.transpose(2, 1, 0))),
                  torch.from_numpy(np.ascontiguousarray(right.transpose(2, 0, 1)))).numpy()
    return s.reshape(d, T * Y * X)                                          # [d, T*YX]


def _head(w: Workload, tensor: str, head: int, out: np.ndarray | None = None) -> np.ndarray:
    """One head of one tensor, float32 [N, d], before any cross-head edit.

    Written into ``out`` (a float32 [N, d] array) when given.
    """
    rng = _rng(w.seed, tensor, head)
    N, d = w.N, w.d
    if out is None:
        out = np.empty((N, d), dtype=np.float32)
    if w.gen == "normal" or tensor == "do" or (w.gen == "uniform" and tensor == "v"):
        out[...] = rng.standard_normal((N, d))
        return out
    if w.gen == "uniform":
        out[...] = 0.05 * rng.standard_normal((N, d))
        return out
    # smooth / sink: smooth signal plus 0.5 N(0,1) noise, built channel-major
    if w.shared_signal and tensor in ("q", "k"):
        sig = smooth_signal(w.grid, d, _rng(w.seed, "q", head), w.amplitude)
    else:
        sig = smooth_signal(w.grid, d, rng, w.amplitude)
    sig += 0.5 * rng.standard_normal((d, N))
    if w.gen == "sink" and tensor == "q":
        # a per-head offset so that mean(Q) is far from zero and the sink
        # block really dominates its rows (drawn from its own stream)
        u = 0.5 * _rng(w.seed + 1000, "q", head).standard_normal(d)
        sig += u[:, None]
    step = 4096
    for lo in range(0, N, step):                 # blocked [d, N] -> [N, d]
        out[lo:lo + step] = sig[:, lo:lo + step].T
    return out


def head_inputs(w: Workload, head: int, tensors=TENSORS, out=None) -> dict[str, np.ndarray]:
    """All requested tensors of one head, float32 [N, d] (B = 1).

    ``out`` optionally maps tensor names to float32 [N, d] destinations.
    """
    res = {t: _head(w, t, head, None if out is None else out[t]) for t in tensors}
    if w.gen == "sink" and "k" in res:
        q = res["q"] if "q" in res else _head(w, "q", head)
        # attention sink: key tokens 0..63 (key block 0) += 6 * mean over tokens of Q
        res["k"][:64] += (6.0 * q.astype(np.float64).mean(axis=0)).astype(np.float32)
    return res


def make_inputs(w: Workload, heads=None, tensors=TENSORS) -> dict[str, np.ndarray]:
    """float32 arrays [B, len(heads), N, d] for the requested heads (default all).

    Heads are generated in parallel threads; the result does not depend on the
    thread count.
    """
    if w.B != 1:
        raise ValueError("workloads here have B = 1")
    heads = list(range(w.H)) if heads is None else list(heads)
    tensors = tuple(t for t in TENSORS if t in tensors and (t != "do" or w.backward))
    out = {t: np.empty((1, len(heads), w.N, w.d), dtype=np.float32) for t in tensors}
    import torch
    from threadpoolctl import threadpool_limits
    nthreads = torch.get_num_threads()
    torch.set_num_threads(1)          # parallel over heads instead
    try:
        with threadpool_limits(1), _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda ih: head_inputs(w, ih[1], tensors,
                                               {t: out[t][0, ih[0]] for t in tensors}),
                        enumerate(heads)))
    finally:
        torch.set_num_threads(nthreads)
    return out


def to_device_dtype(arr: np.ndarray, dtype: str):
    """float32 numpy -> torch CPU tensor in the workload's dtype (bf16 by RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def tuned_params(name: str) -> tuple[float, float]:
    """(k_frac, p) for a workload: fixed ones, or the stored tuned values."""
    w = WORKLOADS[name]
    if w.p is not None:
        return w.k_frac, w.p
    table = json.loads(TUNED_PARAMS_PATH.read_text())
    rec = table["workloads"][name]
    return float(rec["k_frac"]), float(rec["p"])


def tuned_record(name: str) -> dict:
    """The stored tuning record of a density-tuned workload (k_frac, p, density, ...)."""
    return json.loads(TUNED_PARAMS_PATH.read_text())["workloads"][name]


def with_heads(w: Workload, H: int) -> Workload:
    return replace(w, H=H)
