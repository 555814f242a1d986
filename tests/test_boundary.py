"""The C-ABI library loads, exports every symbol include/mita.h declares, and
rejects invalid arguments before touching the GPU.

These run on the CPU: every mita_forward call below is invalid in some way,
and validation happens before any HIP call, so no kernel is launched and no
pointer is dereferenced (the device pointers are placeholders).
"""
import ctypes
import math
import os
import re

import pytest

from efficient_long_sequence_amd import mita

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

A = 0x10000  # 16-byte aligned placeholder address, never dereferenced


def _declared():
    src = open(os.path.join(ROOT, "include", "mita.h")).read()
    return sorted(set(re.findall(r"\b(mita_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = mita.lib()
    names = _declared()
    assert set(names) == set(mita.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert L.mita_version().startswith(b"mita-gfx950")


def _fwd(**kw):
    a = dict(Q=A, K=A, V=A, O=A, dt=mita.BF16, B=1, H=2, N=4096, d=64, pool=(1, 4096, 1, 64), m=64,
             k=64, s=1, ws=A, wsb=1 << 40)
    a.update(kw)
    P = mita.Pool(*a["pool"])
    return mita.lib().mita_forward(a["Q"], a["K"], a["V"], a["O"], a["dt"], a["B"], a["H"], a["N"], a["d"], P,
                                   a["m"], a["k"], a["s"], None, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=0), 1), (dict(O=0), 1), (dict(ws=0), 1),
    (dict(B=0), 2), (dict(N=4095), 2), (dict(m=63), 2), (dict(pool=(1, 4096, 2, 32)), 2),
    (dict(pool=(2, 2048, 1, 64), N=4096), 0),  # valid shape: checked separately below
    (dict(d=0), 2),
    (dict(k=0), 3), (dict(k=4097), 3), (dict(s=0), 3), (dict(s=65), 3), (dict(K=A + 8), 3),
    (dict(ws=A + 4), 3),
    (dict(d=48), 4), (dict(dt=7), 4), (dict(s=9, m=64), 4),
    (dict(N=1 << 20, pool=(1, 1 << 20, 1, 64), k=4096), 4),
    (dict(m=4097 * 1, pool=(1, 8192, 1, 4097), N=8192), 4),
    # more than 2^31 - 1 tokens in all: 64 * 512 * 2^16 = 2^31
    (dict(B=64, H=512, N=1 << 16, pool=(1, 1 << 16, 1, 64)), 4),
    (dict(wsb=100), 5),
])
def test_invalid_arguments_are_rejected(kw, code):
    if code == 0:
        # a valid pooling grid with an undersized workspace is reported as such
        kw = dict(kw, wsb=16)
        code = 5
    assert _fwd(**kw) == code


def test_workspace_bytes():
    L = mita.lib()
    P = mita.Pool(1, 1 << 20, 1, 512)
    big = L.mita_workspace_bytes(mita.BF16, 1, 2, 1 << 20, 64, P, 512, 512, 1)
    assert 50 << 20 < big < 1 << 30
    assert L.mita_workspace_bytes(mita.BF16, 1, 2, 1 << 20, 64, P, 511, 512, 1) == 0
    assert L.mita_workspace_bytes(mita.F32, 1, 1, 256, 32, mita.Pool(16, 16, 4, 4), 16, 16, 1) > 0
    s2 = L.mita_workspace_bytes(mita.BF16, 4, 2, 65536, 64, mita.Pool(1, 65536, 1, 128), 128, 128, 2)
    s1 = L.mita_workspace_bytes(mita.BF16, 4, 2, 65536, 64, mita.Pool(1, 65536, 1, 128), 128, 128, 1)
    assert s2 > s1


def test_status_strings_and_stages():
    L = mita.lib()
    for c in range(7):
        assert L.mita_status_str(c)
    n = L.mita_num_stages()
    names = [L.mita_stage_name(i).decode() for i in range(n)]
    assert names[0] == "pool" and "attend" in names and "score" in names
    assert L.mita_stage_name(99) == b"?"


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mita, "_lib", None)
    monkeypatch.setattr(mita, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        mita.lib()


def test_forward_variant_rejects_unknown_variant_before_any_launch():
    L = mita.lib()
    P = mita.Pool(1, 4096, 1, 64)
    args = (A, A, A, A, mita.BF16, 1, 2, 4096, 64, P, 64, 64, 1)
    assert L.mita_forward_variant(*args, 3, None, A, 1 << 40, None, None) == 3
    assert L.mita_forward_variant(*args, -1, None, A, 1 << 40, None, None) == 3
    # the shape checks run first, with the same codes as mita_forward
    bad = (A, A, A, A, mita.BF16, 1, 2, 4095, 64, P, 64, 64, 1)
    assert L.mita_forward_variant(*bad, 1, None, A, 1 << 40, None, None) == 2
    # and an undersized workspace is reported for a valid variant
    assert L.mita_forward_variant(*args, 1, None, A, 16, None, None) == 5


@pytest.mark.parametrize("kw,code", [
    (dict(Q=0), 1), (dict(O=0), 1), (dict(B=0), 2), (dict(N=0), 2), (dict(d=-1), 2),
    (dict(V=A + 4), 3), (dict(d=48), 4), (dict(dt=3), 4), (dict(N=(1 << 26) + 1), 4),
    (dict(B=300, H=300), 4),
])
def test_dense_attention_rejects_invalid_arguments(kw, code):
    a = dict(Q=A, K=A, V=A, O=A, dt=mita.BF16, B=1, H=2, N=4096, d=64)
    a.update(kw)
    got = mita.lib().mita_dense_attention(a["Q"], a["K"], a["V"], a["O"], a["dt"], a["B"], a["H"], a["N"],
                                          a["d"], None)
    assert got == code


def _saved(**kw):
    a = dict(qtilde=A, vtilde=A, topk=A, route=A, lse=A, lse_landmark=A, out_f32=A)
    a.update(kw)
    return mita.Saved(a["qtilde"], a["vtilde"], a["topk"], a["route"], a["lse"], a["lse_landmark"], a["out_f32"])


@pytest.mark.parametrize("variant,kw,code", [
    (0, dict(qtilde=0), 1), (0, dict(lse=0), 1), (0, dict(lse_landmark=0), 1), (1, dict(vtilde=0), 1),
    (0, dict(qtilde=A + 2), 3), (0, dict(vtilde=A + 8), 3), (5, {}, 3), (0, dict(out_f32=0), 1),
    (2, dict(out_f32=A + 4), 3),
    # the routing-only variant neither writes nor reads v~ and its normaliser
    (2, dict(vtilde=0, lse_landmark=0), 5),
    (0, {}, 5),  # valid saved set, undersized workspace
])
def test_forward_train_rejects_invalid_saved_tensors(variant, kw, code):
    L = mita.lib()
    P = mita.Pool(1, 4096, 1, 64)
    sv = _saved(**kw)
    got = L.mita_forward_train(A, A, A, A, mita.BF16, 1, 2, 4096, 64, P, 64, 64, 1, variant, ctypes.byref(sv),
                               A, 16, None)
    assert got == code
    assert L.mita_forward_train(A, A, A, A, mita.BF16, 1, 2, 4096, 64, P, 64, 64, 1, 0, None, A, 1 << 40,
                                None) == 1


def _bwd(variant=0, sv=None, **kw):
    a = dict(Q=A, K=A, V=A, O=A, dO=A, dQ=A, dK=A, dV=A, dt=mita.BF16, B=1, H=2, N=4096, d=64,
             pool=(1, 4096, 1, 64), m=64, k=64, s=1, ws=A, wsb=16)
    a.update(kw)
    sv = _saved() if sv is None else sv
    return mita.lib().mita_backward(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["dQ"], a["dK"], a["dV"], a["dt"],
                                    a["B"], a["H"], a["N"], a["d"], mita.Pool(*a["pool"]), a["m"], a["k"], a["s"],
                                    variant, ctypes.byref(sv), a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Q=0), 1), (dict(dO=0), 1), (dict(dQ=0), 1), (dict(dV=0), 1), (dict(ws=0), 1),
    (dict(N=4095), 2), (dict(k=0), 3), (dict(dK=A + 4), 3), (dict(dO=A + 2), 3), (dict(ws=A + 4), 3),
    (dict(variant=9), 3), (dict(sv=_saved(topk=0)), 1), (dict(sv=_saved(route=0)), 1),
    (dict(d=48), 4), (dict(s=9, m=64), 4), (dict(B=64, H=512, N=1 << 16, pool=(1, 1 << 16, 1, 64)), 4),
    ({}, 5), (dict(variant=2, sv=_saved(vtilde=0, lse_landmark=0)), 5),
    # a valid forward whose backward inverse lists would need 64-bit positions
    (dict(B=128, H=1, N=8192, pool=(1, 8192, 1, 4096), m=4096, k=8192), 4),
])
def test_backward_rejects_invalid_arguments(kw, code):
    assert _bwd(**kw) == code


def test_backward_workspace_bytes():
    L = mita.lib()
    P = mita.Pool(1, 1 << 20, 1, 512)
    big = L.mita_backward_workspace_bytes(mita.BF16, 1, 2, 1 << 20, 64, P, 512, 512, 1)
    # the routed key parts alone take s * B*H*m*k * 2d * 4 bytes
    assert 2 * 512 * 512 * 128 * 4 < big < 4 << 30
    assert L.mita_backward_workspace_bytes(mita.BF16, 1, 2, 1 << 20, 64, P, 511, 512, 1) == 0
    assert L.mita_backward_workspace_bytes(mita.BF16, 128, 1, 8192, 64, mita.Pool(1, 8192, 1, 4096), 4096, 8192,
                                           1) == 0
    s2 = L.mita_backward_workspace_bytes(mita.BF16, 1, 2, 4096, 64, mita.Pool(1, 4096, 1, 64), 64, 64, 2)
    s1 = L.mita_backward_workspace_bytes(mita.BF16, 1, 2, 4096, 64, mita.Pool(1, 4096, 1, 64), 64, 64, 1)
    assert s2 > s1


def test_probes_reject_invalid_arguments():
    L = mita.lib()
    assert L.mita_probe_mfma(None, 1, 1, None) == 1
    assert L.mita_probe_mfma(A, 0, 1, None) == 3
    assert L.mita_probe_mfma(A, 1, 0, None) == 3
    assert L.mita_probe_mfma(A + 4, 1, 1, None) == 3
    assert L.mita_probe_copy(None, A, 16, None) == 1
    assert L.mita_probe_copy(A, A, 17, None) == 3
    assert L.mita_probe_copy(A + 8, A, 16, None) == 3
    assert L.mita_probe_step(None, 0, 1, 1, None) == 1
    assert L.mita_probe_step(A, 4, 1, 1, None) == 3
    assert L.mita_probe_step(A, -1, 1, 1, None) == 3
    assert L.mita_probe_step(A, 0, 0, 1, None) == 3
    assert L.mita_probe_step(A, 1, 1, 0, None) == 3
    assert L.mita_probe_step(A + 4, 2, 1, 1, None) == 3


def test_events_elapsed_reports_nan_for_untimed_stages():
    """A stage whose two handles are NULL was not timed: NaN, no HIP call."""
    L = mita.lib()
    n = L.mita_num_stages()
    arr = (ctypes.c_void_p * (2 * n))()
    ms = (ctypes.c_float * n)()
    assert L.mita_events_elapsed(arr, n, ms) == 0
    assert all(math.isnan(x) for x in ms)
    assert L.mita_events_destroy(arr, 2 * n) == 0  # NULL handles are skipped


def test_saved_tensors_are_checked_before_the_call():
    """mita.backward checks every saved tensor against the call's sizes (the
    C ABI cannot see them); a mismatch raises before any launch."""
    import torch
    B, H, N, d, m, k, s = 1, 2, 64, 32, 4, 8, 1
    Q = torch.zeros(B, H, N, d, dtype=torch.bfloat16)
    good = dict(qtilde=torch.zeros(B, H, m, d, dtype=torch.bfloat16),
                vtilde=torch.zeros(B, H, m, d), topk=torch.zeros(B, H, m, k, dtype=torch.int32),
                route=torch.zeros(B, H, N, s, dtype=torch.int32), lse=torch.zeros(B, H, N),
                lse_landmark=torch.zeros(B, H, m), out_f32=torch.zeros(B, H, N, d))
    mita._check_saved(mita.SavedOut(**good), Q, m, k, s)
    for name, bad in (("topk", torch.zeros(B, H, m, k + 1, dtype=torch.int32)),
                      ("route", torch.zeros(B, H, N, s, dtype=torch.int64)),
                      ("out_f32", torch.zeros(B, H, N, d, dtype=torch.bfloat16)),
                      ("lse", torch.zeros(B, H, N + 1))):
        with pytest.raises(mita.MitaError):
            mita._check_saved(mita.SavedOut(**{**good, name: bad}), Q, m, k, s)



def _noalloc(**kw):
    a = dict(Q=A, K=A, V=A, O=A, dt=mita.BF16, B=1, H=2, N=65536, d=64, pool=(1, 65536, 1, 128), m=128,
             k=128, s=1)
    a.update(kw)
    P = mita.Pool(*a["pool"])
    return mita.lib().mita_forward_noalloc(a["Q"], a["K"], a["V"], a["O"], a["dt"], a["B"], a["H"], a["N"],
                                           a["d"], P, a["m"], a["k"], a["s"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(), 5),  # valid, but needs more than the static scratch: rejected before any launch
    (dict(Q=0), 1), (dict(N=65535), 2), (dict(k=0), 3), (dict(d=48), 4),
])
def test_noalloc_rejects_before_any_hip_call(kw, code):
    """The entry point without allocation validates like mita_forward and
    refuses a call whose workspace would exceed its static scratch, all on
    the host (no HIP call: these run on the CPU)."""
    assert _noalloc(**kw) == code
    import torch
    assert mita.workspace_bytes(torch.bfloat16, 1, 2, 65536, 64, (1, 65536, 1, 128), 128, 1) > \
        mita.NOALLOC_SCRATCH_BYTES
