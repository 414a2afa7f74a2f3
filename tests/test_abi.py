"""The C ABI of libsa2 on a host without a GPU: it loads, exports what
include/sa2.h declares, and rejects malformed calls before touching a device.
"""
import ctypes
import re
from pathlib import Path

import pytest

from block_sparse_attention_sa2_amd import _lib

HEADER = Path(__file__).resolve().parents[1] / "include" / "sa2.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa2_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(_lib.SIGNATURES), names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.sa2_version().decode().startswith("sa2 ")


def test_workspace_sizes():
    L = _lib.lib()
    B, H, N, d, bq, bk = 1, 12, 32760, 128, 128, 64
    Tq, Tk = 256, 512
    up = lambda x: (x + 255) // 256 * 256
    want = up(B * H * Tq * d * 8) + up(B * H * Tk * d * 8) + up(B * H * Tq * Tk * 8)
    assert L.sa2_mask_workspace_bytes(B, H, N, d, bq, bk) == want
    assert L.sa2_mask_workspace_bytes(0, H, N, d, bq, bk) == 0
    stats = up(B * H * 4 * (-(-N // 128)) * 32 * 2 * 4)
    # d = 128 adds the partial-sum slots of split lists: 2 x 64 per XCD share
    # for dQ rows (128 x 128 fp32 each), 2 x 128 for dK/dV columns (64 keys
    # of dV and dK); the forward's slots also hold each row's max and sum
    dq_slots = up(8 * 2 * 64 * 128 * 128 * 4)
    dkdv_slots = up(8 * 2 * 128 * 2 * 64 * 128 * 4)
    assert L.sa2_bwd_workspace_bytes(B, H, N, d) == stats + dq_slots + dkdv_slots
    assert L.sa2_bwd_workspace_bytes(B, H, N, 64) == stats
    assert L.sa2_fwd_workspace_bytes(B, H, N, d) == up(8 * 2 * 64 * (128 * 128 + 256) * 4)
    assert L.sa2_fwd_workspace_bytes(B, H, N, 64) == 0
    # the mask's plans: items (one per list, plus slack for cost-balanced
    # column shares and the extra segments), split entries, counters
    nrows, ncols = B * H * Tq, B * H * Tk
    row_slack = ((nrows + 7) // 8 + 15) // 16
    row_plan = 8 * ((nrows + 7) // 8 + 2 * row_slack + 64) * 16 + 8 * 64 * 16 + 2 * 8 * 64 * 4
    slack = ((ncols + 7) // 8 + 15) // 16
    col_plan = 8 * ((ncols + 7) // 8 + 2 * slack + 128) * 16 + 8 * 128 * 16 + 8 * 128 * 4
    assert L.sa2_mask_plan_bytes(B, H, N, bq, bk, 0) == row_plan
    assert L.sa2_mask_plan_bytes(B, H, N, bq, bk, 1) == col_plan
    assert L.sa2_mask_plan_bytes(B, H, N, bq, bk, 2) == 0


def _mask(B=1, H=1, N=256, bq=64, bk=64):
    Tq, Tk = -(-N // bq), -(-N // bk)
    fake = 1 << 20   # never dereferenced: validation fails first
    return _lib.Sa2Mask(B, H, N, bq, bk, Tq, Tk, fake, fake, fake, fake, fake, fake, fake)


FAKE = ctypes.c_void_p(1 << 20)


def _status_and_msg(st):
    return st, _lib.lib().sa2_last_error().decode()


def test_build_mask_validation():
    L = _lib.lib()
    m = _mask()
    ws = ctypes.c_void_p(1 << 20)
    args = lambda **kw: dict(dict(q=FAKE, k=FAKE, dt=0, B=1, H=1, N=256, d=64, bq=64, bk=64,
                                  kf=0.1, p=0.5, m=ctypes.byref(m), ws=ws, wsb=1 << 30), **kw)
    call = lambda a: L.sa2_build_mask(a["q"], a["k"], a["dt"], a["B"], a["H"], a["N"], a["d"],
                                      a["bq"], a["bk"], a["kf"], a["p"], a["m"], a["ws"],
                                      a["wsb"], None)
    cases = [
        (dict(q=None), _lib.SA2_EINVAL),
        (dict(N=0), _lib.SA2_EINVAL),
        (dict(dt=7), _lib.SA2_EINVAL),
        (dict(d=60), _lib.SA2_EUNSUPPORTED),
        (dict(kf=0.0, p=0.0), _lib.SA2_EINVAL),
        (dict(kf=float("nan")), _lib.SA2_EINVAL),
        (dict(q=ctypes.c_void_p((1 << 20) + 4)), _lib.SA2_EINVAL),
        (dict(ws=ctypes.c_void_p((1 << 20) + 64)), _lib.SA2_EINVAL),
        (dict(N=300), _lib.SA2_EINVAL),          # mask geometry no longer matches
        (dict(wsb=16), _lib.SA2_EINVAL),
    ]
    # more (batch, head) pairs than a grid dimension holds
    big = _lib.Sa2Mask(1, 70000, 256, 64, 64, 4, 4, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                       1 << 20, 1 << 20)
    st = L.sa2_build_mask(FAKE, FAKE, 0, 1, 70000, 256, 64, 64, 64, 0.1, 0.5, ctypes.byref(big),
                          ws, 1 << 40, None)
    assert st == _lib.SA2_EUNSUPPORTED, st
    for kw, want in cases:
        st, msg = _status_and_msg(call(args(**kw)))
        assert st == want, (kw, st, msg)
        assert msg.startswith("sa2_build_mask"), msg


def test_attention_validation():
    L = _lib.lib()
    m = _mask()
    st, msg = _status_and_msg(L.sa2_attn_fwd(FAKE, FAKE, FAKE, 0, 1, 1, 256, 96,
                                             ctypes.byref(m), FAKE, FAKE, None, 0, None))
    assert st == _lib.SA2_EUNSUPPORTED and "d must be" in msg
    m2 = _mask(bk=32)
    st, msg = _status_and_msg(L.sa2_attn_fwd(FAKE, FAKE, FAKE, 0, 1, 1, 256, 64,
                                             ctypes.byref(m2), FAKE, FAKE, None, 0, None))
    assert st == _lib.SA2_EUNSUPPORTED and "key blocks" in msg
    st, msg = _status_and_msg(L.sa2_attn_fwd(FAKE, FAKE, None, 0, 1, 1, 256, 64,
                                             ctypes.byref(m), FAKE, FAKE, None, 0, None))
    assert st == _lib.SA2_EINVAL
    # d = 128 needs the forward workspace (row plan and partial slots)
    m3 = _mask(bq=128)
    need = L.sa2_fwd_workspace_bytes(1, 1, 256, 128)
    assert need > 0 and L.sa2_fwd_workspace_bytes(1, 1, 256, 64) == 0
    st, msg = _status_and_msg(L.sa2_attn_fwd(FAKE, FAKE, FAKE, 0, 1, 1, 256, 128,
                                             ctypes.byref(m3), FAKE, FAKE, None, 0, None))
    assert st == _lib.SA2_EINVAL and "workspace" in msg, msg
    st, msg = _status_and_msg(L.sa2_attn_fwd(FAKE, FAKE, FAKE, 0, 1, 1, 256, 128,
                                             ctypes.byref(m3), FAKE, FAKE, FAKE, need - 1, None))
    assert st == _lib.SA2_EINVAL and "workspace" in msg, msg
    st, msg = _status_and_msg(L.sa2_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 256,
                                             64, ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, 16,
                                             None))
    assert st == _lib.SA2_EINVAL and "workspace" in msg


def test_attention_refuses_a_mask_without_plans():
    """bf16, d = 128: the kernels walk the mask's plans, so a mask without
    them (or with a misaligned one) is refused before any launch (fake
    pointers, never read); the mask builder refuses one too."""
    L = _lib.lib()
    B, H, N, bq, bk = 1, 1, 256, 128, 64
    f = 1 << 20
    no_rows = _lib.Sa2Mask(B, H, N, bq, bk, 2, 4, f, f, f, f, f, None, f)
    no_cols = _lib.Sa2Mask(B, H, N, bq, bk, 2, 4, f, f, f, f, f, f, None)
    odd = _lib.Sa2Mask(B, H, N, bq, bk, 2, 4, f, f, f, f, f, f + 4, f)
    ws = ctypes.c_void_p(f)
    wsb = L.sa2_bwd_workspace_bytes(B, H, N, 128)
    fwb = L.sa2_fwd_workspace_bytes(B, H, N, 128)
    for m in (no_rows, odd):
        st, msg = _status_and_msg(L.sa2_attn_fwd(FAKE, FAKE, FAKE, 0, B, H, N, 128,
                                                 ctypes.byref(m), FAKE, FAKE, ws, fwb, None))
        assert st == _lib.SA2_EINVAL and "row plan" in msg, msg
        st, msg = _status_and_msg(L.sa2_attn_bwd_dq(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, B, H,
                                                    N, 128, ctypes.byref(m), FAKE, ws, wsb, None))
        assert st == _lib.SA2_EINVAL and "row plan" in msg, msg
    st, msg = _status_and_msg(L.sa2_attn_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, FAKE, 0, B, H, N, 128,
                                                  ctypes.byref(no_cols), FAKE, FAKE, ws, wsb,
                                                  None))
    assert st == _lib.SA2_EINVAL and "column plan" in msg, msg
    st, msg = _status_and_msg(L.sa2_build_mask(FAKE, FAKE, 0, B, H, N, 128, bq, bk, 0.1, 0.5,
                                               ctypes.byref(no_cols), ws, 1 << 30, None))
    assert st == _lib.SA2_EINVAL and "null" in msg, msg
    st, msg = _status_and_msg(L.sa2_mask_plans(ctypes.byref(no_rows), None))
    assert st == _lib.SA2_EINVAL, msg


def test_noalloc_mask_refuses_a_geometry_beyond_the_scratch():
    """The 14B-shaped layer needs 296 MB of mask workspace, more than the
    static scratch array: refused before anything touches a device."""
    L = _lib.lib()
    B, H, N, d, bq, bk = 1, 40, 75600, 128, 128, 64
    assert L.sa2_mask_workspace_bytes(B, H, N, d, bq, bk) > _lib.SA2_MASK_NOALLOC_MAX_BYTES
    m = _lib.Sa2Mask(B, H, N, bq, bk, -(-N // bq), -(-N // bk), 1 << 20, 1 << 20, 1 << 20,
                     1 << 20, 1 << 20, 1 << 20, 1 << 20)
    st, msg = _status_and_msg(L.sa2_build_mask_noalloc(FAKE, FAKE, 0, B, H, N, d, bq, bk, 0.03,
                                                       0.1, ctypes.byref(m), None))
    assert st == _lib.SA2_EUNSUPPORTED and "static scratch" in msg, msg
    # the 1.3B-shaped layer fits, in both block geometries; argument checks come first
    assert L.sa2_mask_workspace_bytes(1, 12, 32760, 128, 64, 64) <= _lib.SA2_MASK_NOALLOC_MAX_BYTES
    st, msg = _status_and_msg(L.sa2_build_mask_noalloc(FAKE, FAKE, 0, B, H, N, d, bq, bk, 0.0,
                                                       0.0, ctypes.byref(m), None))
    assert st == _lib.SA2_EINVAL and msg.startswith("sa2_build_mask_noalloc"), msg


def test_python_binding_refuses_cpu_tensors():
    import torch
    import block_sparse_attention_sa2_amd as sa2
    q = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        sa2.build_mask(q, q, 64, 64, 0.5, 0.5)


def test_distill_validation():
    L = _lib.lib()
    assert L.sa2_distill_workspace_bytes(1, 2, 64, 64) >= 8
    assert L.sa2_distill_workspace_bytes(0, 2, 64, 64) == 0
    ws = ctypes.c_void_p(1 << 20)
    loss = ctypes.c_void_p(1 << 20)
    call = lambda **kw: L.sa2_distill_loss_grad(
        kw.get("s", FAKE), kw.get("t", FAKE), kw.get("dt", 0), 1, 2, kw.get("N", 64),
        kw.get("d", 64), kw.get("o", FAKE), loss, kw.get("ws", ws), kw.get("wsb", 1 << 20), None)
    cases = [
        (dict(s=None), _lib.SA2_EINVAL),
        (dict(dt=5), _lib.SA2_EINVAL),
        (dict(d=12), _lib.SA2_EUNSUPPORTED),
        (dict(N=0), _lib.SA2_EINVAL),
        (dict(o=ctypes.c_void_p((1 << 20) + 8)), _lib.SA2_EINVAL),
        (dict(ws=ctypes.c_void_p((1 << 20) + 16)), _lib.SA2_EINVAL),
        (dict(wsb=8), _lib.SA2_EINVAL),
    ]
    for kw, want in cases:
        st, msg = _status_and_msg(call(**kw))
        assert st == want, (kw, st, msg)
        assert msg.startswith("sa2_distill_loss_grad"), msg


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    """No CPU fallback: with libsa2.so absent, every call through the binding
    raises ImportError before anything runs."""
    import torch
    import block_sparse_attention_sa2_amd as sa2
    monkeypatch.setattr(_lib, "LIB_PATH", tmp_path / "libsa2.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError, match="no fallback"):
        sa2.version()
    with pytest.raises(ImportError):
        sa2.mask_workspace_bytes(1, 1, 64, 64, 64, 64)
    q = torch.zeros(1, 1, 64, 64)
    with pytest.raises((ImportError, ValueError)):
        sa2.build_mask(q, q, 64, 64, 0.5, 0.5)
