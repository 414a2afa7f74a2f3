"""The allocation-free mask builder (sa2_build_mask_noalloc) against the
workspace one (sa2_build_mask): called through the C ABI, the mask must be
identical, on two calls in a row, the second with a smaller input.  (Its
refusal of an oversized geometry is checked on the host in test_abi.py.)"""
from __future__ import annotations

import ctypes

import pytest
import torch

import block_sparse_attention_sa2_amd as sa2
from block_sparse_attention_sa2_amd import _lib

from parity import check_plans

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, N, d, bq, bk, k_frac, p: the 1.3B-shaped layer, then a smaller call
    (1, 12, 32760, 128, 128, 64, 0.03, 0.08),
    (2, 3, 3000, 64, 64, 64, 0.1, 0.5),
]


def _noalloc():
    return _lib.lib().sa2_build_mask_noalloc


def _filled_mask(B, H, N, bq, bk, dev):
    m = sa2.BlockMask(B, H, N, bq, bk, dev)
    for t in (m.bitmap, m.row_cnt, m.row_idx, m.col_cnt, m.col_idx, m.row_plan, m.col_plan):
        t.fill_(7)   # list tails are left untouched: both masks start alike
    return m


def _same(a: sa2.BlockMask, b: sa2.BlockMask):
    for name in ("bitmap", "row_cnt", "row_idx", "col_cnt", "col_idx"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    # plans: list order among equal lengths within an XCD share may differ
    for m in (a, b):
        check_plans(m)


def test_noalloc_matches_workspace_build():
    dev = torch.device("cuda:0")
    fn = _noalloc()
    g = torch.Generator(device="cpu").manual_seed(5)
    for B, H, N, d, bq, bk, kf, p in CASES:
        print(f"[noalloc] B{B} H{H} N{N} d{d} bq{bq} bk{bk} k{kf} p{p}", flush=True)
        q = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
        k = torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(dev)
        want = _filled_mask(B, H, N, bq, bk, dev)
        sa2.build_mask(q, k, bq, bk, kf, p, mask=want)
        got = _filled_mask(B, H, N, bq, bk, dev)
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        st = fn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), _lib.SA2_BF16, B, H,
                N, d, bq, bk, kf, p, ctypes.byref(got.c_struct()), stream)
        assert st == _lib.SA2_OK, _lib.lib().sa2_last_error().decode()
        torch.cuda.synchronize()
        _same(want, got)
        assert 0 < want.density() < 1
