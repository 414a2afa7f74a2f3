"""SpargeAttention2 hot path on AMD Instinct MI355X (gfx950).

Python binding of libsa2 (include/sa2.h).  Every step of the path runs in the
library's HIP kernels; this module only checks tensors, allocates outputs with
PyTorch and passes pointers and the current stream through ctypes.

    mask = build_mask(q, k, bq=128, bk=64, k_frac=0.03, p=0.9)
    o, lse = attn_fwd(q, k, v, mask)
    dq, dk, dv = attn_bwd(q, k, v, o, lse, do, mask)
    out = sparse_attention(q, k, v, mask)          # autograd-aware

Tensors are CUDA (HIP) tensors of shape [B, H, N, d], contiguous, all
torch.bfloat16 or all torch.float32.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import Sa2Mask, check

__all__ = ["BlockMask", "build_mask", "build_mask_noalloc", "attn_fwd", "attn_bwd", "attn_bwd_dq",
           "attn_bwd_dkdv", "attn_bwd_atomic_dq", "sparse_attention", "SparseAttention",
           "distill_loss_grad", "distill_step", "version", "mask_workspace_bytes",
           "fwd_workspace_bytes", "bwd_workspace_bytes", "bwd_atomic_workspace_bytes",
           "distill_workspace_bytes"]

_DTYPES = {torch.bfloat16: _lib.SA2_BF16, torch.float32: _lib.SA2_F32}


def version() -> str:
    return _lib.lib().sa2_version().decode()


def _dtype_code(*ts: torch.Tensor) -> int:
    dt = ts[0].dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}: use bfloat16 or float32")
    for t in ts:
        if t.dtype != dt:
            raise TypeError("all tensors must share one dtype")
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
        if t.device != ts[0].device:
            raise ValueError("tensors must be on one device")
    return _DTYPES[dt]


def _shape(t: torch.Tensor):
    if t.dim() != 4:
        raise ValueError("expected a [B, H, N, d] tensor")
    return tuple(int(x) for x in t.shape)


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _out(t, shape, dtype, device, name: str):
    """A caller-supplied output: the kernels write exactly `shape` elements of
    `dtype` there, so anything else is refused before a launch."""
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")
    return t


def _workspace(ws, need: int, device):
    """A workspace tensor (new if None): contiguous bytes on `device`."""
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if (not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous()
            or ws.dtype != torch.uint8):
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    return ws


def _same_device(mask, device):
    if mask.device != device:
        raise ValueError(f"mask is on {mask.device}, tensors on {device}")


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


class BlockMask:
    """The hybrid block mask of every (batch, head): bitmap, row and column
    lists, and the attention kernels' work plans made from the list counts.

    Arrays (device, caller-owned through this object):
      bitmap  uint8 [B, H, Tq, Tk]
      row_cnt int32 [B, H, Tq];  row_idx int32 [B, H, Tq, Tk] (first row_cnt valid)
      col_cnt int32 [B, H, Tk];  col_idx int32 [B, H, Tk, Tq] (first col_cnt valid)
      row_plan, col_plan  int32 (sa2_mask_plan_bytes / 4 entries each)
    """

    def __init__(self, B: int, H: int, N: int, bq: int, bk: int, device):
        self.B, self.H, self.N, self.bq, self.bk = B, H, N, bq, bk
        self.Tq = -(-N // bq)
        self.Tk = -(-N // bk)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.bitmap = torch.empty((B, H, self.Tq, self.Tk), dtype=torch.uint8, device=dev)
        self.row_cnt = torch.empty((B, H, self.Tq), **i32)
        self.row_idx = torch.empty((B, H, self.Tq, self.Tk), **i32)
        self.col_cnt = torch.empty((B, H, self.Tk), **i32)
        self.col_idx = torch.empty((B, H, self.Tk, self.Tq), **i32)
        L = _lib.lib()
        self.row_plan = torch.empty((L.sa2_mask_plan_bytes(B, H, N, bq, bk, 0) // 4,), **i32)
        self.col_plan = torch.empty((L.sa2_mask_plan_bytes(B, H, N, bq, bk, 1) // 4,), **i32)
        self._c = Sa2Mask(B, H, N, bq, bk, self.Tq, self.Tk,
                          self.bitmap.data_ptr(), self.row_cnt.data_ptr(),
                          self.row_idx.data_ptr(), self.col_cnt.data_ptr(),
                          self.col_idx.data_ptr(), self.row_plan.data_ptr(),
                          self.col_plan.data_ptr())

    @property
    def device(self):
        return self.bitmap.device

    def c_struct(self) -> Sa2Mask:
        return self._c

    def remake_plans(self) -> None:
        """Remake the work plans from the list counts (sa2_mask_plans), after
        the caller wrote the lists itself."""
        check("sa2_mask_plans", _lib.lib().sa2_mask_plans(ctypes.byref(self._c),
                                                          _stream(self.device)))

    def density(self) -> float:
        """Kept block pairs over all block pairs (sparsity = 1 - density)."""
        return float(self.row_cnt.sum().item()) / float(self.B * self.H * self.Tq * self.Tk)

    def row_list(self, b: int, h: int, i: int) -> torch.Tensor:
        n = int(self.row_cnt[b, h, i].item())
        return self.row_idx[b, h, i, :n]

    def col_list(self, b: int, h: int, j: int) -> torch.Tensor:
        n = int(self.col_cnt[b, h, j].item())
        return self.col_idx[b, h, j, :n]


def mask_workspace_bytes(B, H, N, d, bq, bk) -> int:
    return int(_lib.lib().sa2_mask_workspace_bytes(B, H, N, d, bq, bk))


def build_mask(q: torch.Tensor, k: torch.Tensor, bq: int, bk: int, k_frac: float, p: float,
               mask: BlockMask | None = None, workspace: torch.Tensor | None = None) -> BlockMask:
    """Hybrid Top-k + Top-p block mask of q, k (sa2_build_mask)."""
    dt = _dtype_code(q, k)
    B, H, N, d = _shape(q)
    if _shape(k) != (B, H, N, d):
        raise ValueError("q and k must have the same shape")
    if mask is None:
        mask = BlockMask(B, H, N, bq, bk, q.device)
    _same_device(mask, q.device)
    workspace = _workspace(workspace, mask_workspace_bytes(B, H, N, d, bq, bk), q.device)
    L = _lib.lib()
    st = L.sa2_build_mask(_ptr(q), _ptr(k), dt, B, H, N, d, bq, bk, float(k_frac), float(p),
                          ctypes.byref(mask.c_struct()), _ptr(workspace), workspace.numel(),
                          _stream(q.device))
    check("sa2_build_mask", st)
    return mask


def build_mask_noalloc(q: torch.Tensor, k: torch.Tensor, bq: int, bk: int, k_frac: float,
                       p: float, mask: BlockMask) -> BlockMask:
    """The same mask as build_mask, written into the caller's `mask` with no
    workspace and no allocation by the library (sa2_build_mask_noalloc); for
    geometries whose workspace fits SA2_MASK_NOALLOC_MAX_BYTES."""
    dt = _dtype_code(q, k)
    B, H, N, d = _shape(q)
    if _shape(k) != (B, H, N, d):
        raise ValueError("q and k must have the same shape")
    _same_device(mask, q.device)
    st = _lib.lib().sa2_build_mask_noalloc(_ptr(q), _ptr(k), dt, B, H, N, d, bq, bk,
                                           float(k_frac), float(p),
                                           ctypes.byref(mask.c_struct()), _stream(q.device))
    check("sa2_build_mask_noalloc", st)
    return mask


def fwd_workspace_bytes(B, H, N, d) -> int:
    return int(_lib.lib().sa2_fwd_workspace_bytes(B, H, N, d))


def attn_fwd(q, k, v, mask: BlockMask, o=None, lse=None, workspace=None):
    """Block-sparse attention forward (sa2_attn_fwd) -> (o, lse)."""
    dt = _dtype_code(q, k, v)
    B, H, N, d = _shape(q)
    if _shape(k) != (B, H, N, d) or _shape(v) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    _same_device(mask, q.device)
    o = torch.empty_like(q) if o is None else _out(o, q.shape, q.dtype, q.device, "o")
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else
           _out(lse, (B, H, N), torch.float32, q.device, "lse"))
    workspace = _workspace(workspace, fwd_workspace_bytes(B, H, N, d), q.device)
    st = _lib.lib().sa2_attn_fwd(_ptr(q), _ptr(k), _ptr(v), dt, B, H, N, d,
                                 ctypes.byref(mask.c_struct()), _ptr(o), _ptr(lse),
                                 _ptr(workspace), workspace.numel(), _stream(q.device))
    check("sa2_attn_fwd", st)
    return o, lse


def bwd_workspace_bytes(B, H, N, d) -> int:
    return int(_lib.lib().sa2_bwd_workspace_bytes(B, H, N, d))


def attn_bwd(q, k, v, o, lse, dout, mask: BlockMask, dq=None, dk=None, dv=None,
             workspace=None):
    """Gradients of the block-sparse attention (sa2_attn_bwd) -> (dq, dk, dv)."""
    dt = _dtype_code(q, k, v, o, dout)
    B, H, N, d = _shape(q)
    for t in (k, v, o, dout):
        if _shape(t) != (B, H, N, d):
            raise ValueError("q, k, v, o, dout must have the same shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    _same_device(mask, q.device)
    if lse.device != q.device:
        raise ValueError("lse must be on the tensors' device")
    dq = torch.empty_like(q) if dq is None else _out(dq, q.shape, q.dtype, q.device, "dq")
    dk = torch.empty_like(k) if dk is None else _out(dk, k.shape, k.dtype, k.device, "dk")
    dv = torch.empty_like(v) if dv is None else _out(dv, v.shape, v.dtype, v.device, "dv")
    workspace = _workspace(workspace, bwd_workspace_bytes(B, H, N, d), q.device)
    st = _lib.lib().sa2_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), dt,
                                 B, H, N, d, ctypes.byref(mask.c_struct()), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _ptr(workspace), workspace.numel(),
                                 _stream(q.device))
    check("sa2_attn_bwd", st)
    return dq, dk, dv


def bwd_atomic_workspace_bytes(B, H, N, d) -> int:
    return int(_lib.lib().sa2_bwd_atomic_workspace_bytes(B, H, N, d))


def attn_bwd_atomic_dq(q, k, v, o, lse, dout, mask: BlockMask, dq=None, dk=None, dv=None,
                       workspace=None):
    """The backward with dQ accumulated by fp32 atomics inside the dK/dV pass
    (sa2_attn_bwd_atomic_dq; bf16, d = 128) -> (dq, dk, dv)."""
    dt, B, H, N, d = _bwd_prep(q, k, v, dout, lse, (o,))
    _same_device(mask, q.device)
    dq = torch.empty_like(q) if dq is None else _out(dq, q.shape, q.dtype, q.device, "dq")
    dk = torch.empty_like(k) if dk is None else _out(dk, k.shape, k.dtype, k.device, "dk")
    dv = torch.empty_like(v) if dv is None else _out(dv, v.shape, v.dtype, v.device, "dv")
    workspace = _workspace(workspace, bwd_atomic_workspace_bytes(B, H, N, d), q.device)
    st = _lib.lib().sa2_attn_bwd_atomic_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                           _ptr(dout), dt, B, H, N, d,
                                           ctypes.byref(mask.c_struct()), _ptr(dq), _ptr(dk),
                                           _ptr(dv), _ptr(workspace), workspace.numel(),
                                           _stream(q.device))
    check("sa2_attn_bwd_atomic_dq", st)
    return dq, dk, dv


def _bwd_prep(q, k, v, dout, lse, extra):
    dt = _dtype_code(q, k, v, dout, *extra)
    B, H, N, d = _shape(q)
    for t in (k, v, dout, *extra):
        if _shape(t) != (B, H, N, d):
            raise ValueError("q, k, v, o, dout must have the same shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if lse.device != q.device:
        raise ValueError("lse must be on the tensors' device")
    return dt, B, H, N, d


def attn_bwd_dq(q, k, v, o, lse, dout, mask: BlockMask, workspace: torch.Tensor, dq=None):
    """dQ, and Delta into `workspace` for attn_bwd_dkdv (sa2_attn_bwd_dq)."""
    dt, B, H, N, d = _bwd_prep(q, k, v, dout, lse, (o,))
    _same_device(mask, q.device)
    workspace = _workspace(workspace, bwd_workspace_bytes(B, H, N, d), q.device)
    dq = torch.empty_like(q) if dq is None else _out(dq, q.shape, q.dtype, q.device, "dq")
    st = _lib.lib().sa2_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                    dt, B, H, N, d, ctypes.byref(mask.c_struct()), _ptr(dq),
                                    _ptr(workspace), workspace.numel(), _stream(q.device))
    check("sa2_attn_bwd_dq", st)
    return dq


def attn_bwd_dkdv(q, k, v, lse, dout, mask: BlockMask, workspace: torch.Tensor, dk=None,
                  dv=None):
    """dK, dV using the Delta a prior attn_bwd_dq left in `workspace` (sa2_attn_bwd_dkdv)."""
    dt, B, H, N, d = _bwd_prep(q, k, v, dout, lse, ())
    _same_device(mask, q.device)
    workspace = _workspace(workspace, bwd_workspace_bytes(B, H, N, d), q.device)
    dk = torch.empty_like(k) if dk is None else _out(dk, k.shape, k.dtype, k.device, "dk")
    dv = torch.empty_like(v) if dv is None else _out(dv, v.shape, v.dtype, v.device, "dv")
    st = _lib.lib().sa2_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), dt, B, H,
                                      N, d, ctypes.byref(mask.c_struct()), _ptr(dk), _ptr(dv),
                                      _ptr(workspace), workspace.numel(), _stream(q.device))
    check("sa2_attn_bwd_dkdv", st)
    return dk, dv


class SparseAttention(torch.autograd.Function):
    """Trainable block-sparse attention: the mask is a constant of the graph."""

    @staticmethod
    def forward(ctx, q, k, v, mask):
        o, lse = attn_fwd(q, k, v, mask)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.mask = mask
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_bwd(q, k, v, o, lse, do.contiguous(), ctx.mask)
        return dq, dk, dv, None


def sparse_attention(q, k, v, mask: BlockMask):
    return SparseAttention.apply(q, k, v, mask)


def distill_workspace_bytes(B, H, N, d) -> int:
    return int(_lib.lib().sa2_distill_workspace_bytes(B, H, N, d))


def distill_loss_grad(o_student, o_teacher, dout=None, loss=None, workspace=None):
    """Layer-level velocity-distillation loss mean((o_s - o_t)^2) and its
    gradient 2 (o_s - o_t) / numel (sa2_distill_loss_grad) -> (loss, dout);
    loss is a one-element float64 device tensor."""
    dt = _dtype_code(o_student, o_teacher)
    B, H, N, d = _shape(o_student)
    if _shape(o_teacher) != (B, H, N, d):
        raise ValueError("o_student and o_teacher must have the same shape")
    dev = o_student.device
    dout = (torch.empty_like(o_student) if dout is None else
            _out(dout, o_student.shape, o_student.dtype, dev, "dout"))
    loss = (torch.empty((1,), dtype=torch.float64, device=dev) if loss is None else
            _out(loss, (1,), torch.float64, dev, "loss"))
    workspace = _workspace(workspace, distill_workspace_bytes(B, H, N, d), dev)
    st = _lib.lib().sa2_distill_loss_grad(_ptr(o_student), _ptr(o_teacher), dt, B, H, N, d,
                                          _ptr(dout), _ptr(loss), _ptr(workspace),
                                          workspace.numel(), _stream(o_student.device))
    check("sa2_distill_loss_grad", st)
    return loss, dout


def distill_step(q, k, v, mask: BlockMask, dense_mask: BlockMask):
    """One layer-level velocity-distillation step: the teacher is the same
    attention with every block kept (dense_mask), the student the sparse one
    (mask).  Returns (loss, dq, dk, dv, o_student, o_teacher); the gradients
    are those of the loss through the student, the teacher held fixed."""
    o_t, _ = attn_fwd(q, k, v, dense_mask)
    o_s, lse = attn_fwd(q, k, v, mask)
    loss, dout = distill_loss_grad(o_s, o_t)
    dq, dk, dv = attn_bwd(q, k, v, o_s, lse, dout, mask)
    return loss, dq, dk, dv, o_s, o_t
