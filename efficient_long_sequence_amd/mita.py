"""Python binding of libmita (ctypes): argument marshalling only.

Every step of the forward pass runs in the library's HIP kernels; this module
turns torch tensors into device pointers and the current HIP stream, sizes
the workspace, and raises on a non-OK status.  There is no CPU fallback: if
``libmita.so`` is missing, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmita.so")

F32, BF16 = 0, 1

STATUS = {
    0: "MITA_OK", 1: "MITA_ERR_NULL", 2: "MITA_ERR_SHAPE", 3: "MITA_ERR_PARAM",
    4: "MITA_ERR_UNSUPPORTED", 5: "MITA_ERR_WORKSPACE", 6: "MITA_ERR_HIP",
}

EXPORTS = [
    "mita_workspace_bytes", "mita_forward", "mita_forward_timed", "mita_forward_variant", "mita_dense_attention", "mita_num_stages",
    "mita_stage_name", "mita_events_create", "mita_events_destroy", "mita_events_elapsed",
    "mita_status_str", "mita_version", "mita_forward_train", "mita_backward_workspace_bytes", "mita_backward",
    "mita_probe_mfma", "mita_probe_copy", "mita_probe_step", "mita_forward_noalloc",
]


class Pool(ctypes.Structure):
    _fields_ = [("grid_h", ctypes.c_int), ("grid_w", ctypes.c_int),
                ("land_h", ctypes.c_int), ("land_w", ctypes.c_int)]


class Debug(ctypes.Structure):
    _fields_ = [("topk", ctypes.c_void_p), ("route", ctypes.c_void_p),
                ("vtilde", ctypes.c_void_p), ("qtilde", ctypes.c_void_p)]


class Saved(ctypes.Structure):
    _fields_ = [("qtilde", ctypes.c_void_p), ("vtilde", ctypes.c_void_p), ("topk", ctypes.c_void_p),
                ("route", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("lse_landmark", ctypes.c_void_p),
                ("out_f32", ctypes.c_void_p)]


class MitaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmita.so from the package directory (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m efficient_long_sequence_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    L.mita_workspace_bytes.restype = c_size
    L.mita_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, Pool, c_int, c_int, c_int]
    fwd = [vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, Pool, c_int, c_int, c_int,
           ctypes.POINTER(Debug), vp, c_size, vp]
    L.mita_forward.restype = c_int
    L.mita_forward.argtypes = fwd
    L.mita_forward_timed.restype = c_int
    L.mita_forward_timed.argtypes = fwd + [ctypes.POINTER(vp)]
    L.mita_forward_variant.restype = c_int
    L.mita_forward_variant.argtypes = fwd[:13] + [c_int] + fwd[13:] + [ctypes.POINTER(vp)]
    L.mita_forward_noalloc.restype = c_int
    L.mita_forward_noalloc.argtypes = fwd[:13] + [vp]
    L.mita_dense_attention.restype = c_int
    L.mita_dense_attention.argtypes = [vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, vp]
    L.mita_num_stages.restype = c_int
    L.mita_stage_name.restype = ctypes.c_char_p
    L.mita_stage_name.argtypes = [c_int]
    L.mita_events_create.restype = c_int
    L.mita_events_create.argtypes = [ctypes.POINTER(vp), c_int]
    L.mita_events_destroy.restype = c_int
    L.mita_events_destroy.argtypes = [ctypes.POINTER(vp), c_int]
    L.mita_events_elapsed.restype = c_int
    L.mita_events_elapsed.argtypes = [ctypes.POINTER(vp), c_int, ctypes.POINTER(ctypes.c_float)]
    L.mita_forward_train.restype = c_int
    L.mita_forward_train.argtypes = fwd[:13] + [c_int, ctypes.POINTER(Saved), vp, c_size, vp]
    L.mita_backward_workspace_bytes.restype = c_size
    L.mita_backward_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, Pool, c_int, c_int, c_int]
    L.mita_backward.restype = c_int
    L.mita_backward.argtypes = [vp] * 8 + [c_int, c_int, c_int, c_int, c_int, Pool, c_int, c_int, c_int, c_int,
                                           ctypes.POINTER(Saved), vp, c_size, vp]
    L.mita_probe_mfma.restype = c_int
    L.mita_probe_mfma.argtypes = [vp, c_int, c_int, vp]
    L.mita_probe_copy.restype = c_int
    L.mita_probe_copy.argtypes = [vp, vp, c_size, vp]
    L.mita_probe_step.restype = c_int
    L.mita_probe_step.argtypes = [vp, c_int, c_int, c_int, vp]
    L.mita_status_str.restype = ctypes.c_char_p
    L.mita_status_str.argtypes = [c_int]
    L.mita_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(code: int):
    if code != 0:
        raise MitaError(code, lib().mita_status_str(code).decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise MitaError(4, f"unsupported dtype {t}")


def workspace_bytes(dtype: torch.dtype, B: int, H: int, N: int, d: int, pool, k: int, s: int) -> int:
    gh, gw, lh, lw = pool
    return int(lib().mita_workspace_bytes(_dtype_code(dtype), B, H, N, d, Pool(gh, gw, lh, lw),
                                          lh * lw, k, s))


@dataclass
class DebugOut:
    topk: torch.Tensor    # int32 [B, H, m, k]
    route: torch.Tensor   # int32 [B, H, N, s]
    vtilde: torch.Tensor  # float32 [B, H, m, d]
    qtilde: torch.Tensor  # dtype [B, H, m, d]


class Events:
    """Per-stage HIP event pairs for mita_forward_timed: every stage, or only
    the stages named in `stages` (the others enqueue no record)."""

    def __init__(self, stages=None):
        L = lib()
        self.n = L.mita_num_stages()
        self.names = [L.mita_stage_name(i).decode() for i in range(self.n)]
        self.arr = (ctypes.c_void_p * (2 * self.n))()
        self.timed = [i for i, nm in enumerate(self.names) if stages is None or nm in stages]
        for i in self.timed:
            pair = (ctypes.c_void_p * 2)()
            _check(L.mita_events_create(pair, 2))
            self.arr[2 * i], self.arr[2 * i + 1] = pair[0], pair[1]

    def elapsed_ms(self) -> dict:
        ms = (ctypes.c_float * self.n)()
        _check(lib().mita_events_elapsed(self.arr, self.n, ms))
        return {self.names[i]: float(ms[i]) for i in self.timed}

    def close(self):
        if self.arr is not None:
            lib().mita_events_destroy(self.arr, 2 * self.n)
            self.arr = None


def dense_attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, out: torch.Tensor | None = None):
    """Full softmax attention softmax(Q K^T / sqrt(d)) V on the GPU (the
    baseline of the pages' long-sequence throughput test); [B, H, N, d]."""
    L = lib()
    B, H, N, d = Q.shape
    for t in (Q, K, V):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != Q.dtype or t.shape != Q.shape:
            raise MitaError(2, "Q, K, V must be contiguous device tensors of one shape and dtype")
    O = torch.empty_like(Q) if out is None else out
    stream = torch.cuda.current_stream(Q.device).cuda_stream
    _check(L.mita_dense_attention(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), _dtype_code(Q.dtype),
                                  B, H, N, d, stream))
    return O


# Entries and scales of the joint softmax: "paper" = shared logits 1/sqrt(d)
# like every other logit; "official" = shared logits 1/d, the authors' code
# path (MiTA tutorial, chapter 8, third check); "routed" = the routing-only
# ablation with no shared entries (the pages match entries per query by
# passing k + m / s as k).
VARIANTS = {"paper": 0, "official": 1, "routed": 2}


def official_params(grid_h: int, grid_w: int, pool_size: int, kv_topk: int):
    """Pool and k from the authors' side-length parameters: their module
    squares ``pool_size`` and ``kv_topk`` into m = pool_size**2 landmarks (a
    pool_size x pool_size landmark grid) and k = kv_topk**2 keys per expert
    (MiTA tutorial, chapter 8, third check)."""
    return (grid_h, grid_w, pool_size, pool_size), kv_topk * kv_topk


def forward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, pool, k: int, s: int,
            debug: bool = False, workspace: torch.Tensor | None = None,
            out: torch.Tensor | None = None, events: Events | None = None, m: int | None = None,
            variant: str = "paper"):
    """MiTA forward pass on the GPU.

    Q, K, V: contiguous device tensors [B, H, N, d] (bf16 or fp32).
    pool: (grid_h, grid_w, land_h, land_w); m = land_h * land_w unless given
    (a mismatching m is passed through so the library can reject it).
    variant: "paper", "official" or "routed" (see VARIANTS); with "routed" the
    debug v~ is not written (left as allocated).
    Returns O, or (O, DebugOut) when ``debug``.
    """
    L = lib()
    B, H, N, d = Q.shape
    gh, gw, lh, lw = pool
    m = lh * lw if m is None else m
    dt = _dtype_code(Q.dtype)
    P = Pool(gh, gw, lh, lw)
    need = int(L.mita_workspace_bytes(dt, B, H, N, d, P, m, k, s))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Q.device)
    O = torch.empty_like(Q) if out is None else out
    _check_qkv(Q, K, V, O)
    _check_workspace(workspace, Q)
    dbg_struct, dbg = None, None
    if debug:
        dev = Q.device
        dbg = DebugOut(
            topk=torch.empty((B, H, m, k), dtype=torch.int32, device=dev),
            route=torch.empty((B, H, N, s), dtype=torch.int32, device=dev),
            vtilde=torch.zeros((B, H, m, d), dtype=torch.float32, device=dev),
            qtilde=torch.empty((B, H, m, d), dtype=Q.dtype, device=dev),
        )
        dbg_struct = Debug(dbg.topk.data_ptr(), dbg.route.data_ptr(), dbg.vtilde.data_ptr(),
                           dbg.qtilde.data_ptr())
    stream = torch.cuda.current_stream(Q.device).cuda_stream
    args = (Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), dt, B, H, N, d, P, m, k, s,
            ctypes.byref(dbg_struct) if dbg_struct is not None else None,
            workspace.data_ptr(), workspace.numel(), stream)
    if variant not in VARIANTS:
        raise MitaError(3, f"unknown variant {variant!r}")
    if variant != "paper":
        code = L.mita_forward_variant(*args[:13], VARIANTS[variant], *args[13:],
                                      events.arr if events is not None else None)
    elif events is None:
        code = L.mita_forward(*args)
    else:
        code = L.mita_forward_timed(*args, events.arr)
    _check(code)
    return (O, dbg) if debug else O


# the library's own static scratch (bytes per GPU), for mita_forward_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, pool, k: int, s: int,
                    out: torch.Tensor | None = None, m: int | None = None):
    """MiTA forward pass through mita_forward_noalloc: no workspace, the
    library's static scratch instead (calls that overlap on one GPU race).
    Raises MitaError(MITA_ERR_WORKSPACE) when the call needs more than
    NOALLOC_SCRATCH_BYTES of it.  Pass ``out`` to allocate nothing here either."""
    L = lib()
    B, H, N, d = Q.shape
    gh, gw, lh, lw = pool
    m = lh * lw if m is None else m
    O = torch.empty_like(Q) if out is None else out
    _check_qkv(Q, K, V, O)
    stream = torch.cuda.current_stream(Q.device).cuda_stream
    _check(L.mita_forward_noalloc(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), _dtype_code(Q.dtype),
                                  B, H, N, d, Pool(gh, gw, lh, lw), m, k, s, stream))
    return O


# ---------------------------------------------------------------------------
# training: forward that keeps what the backward needs, and the backward
@dataclass
class SavedOut:
    """What mita_forward_train keeps for mita_backward (device tensors)."""
    qtilde: torch.Tensor        # dtype [B, H, m, d]
    vtilde: torch.Tensor        # float32 [B, H, m, d] (unused by the routing-only variant)
    topk: torch.Tensor          # int32 [B, H, m, k]
    route: torch.Tensor         # int32 [B, H, N, s]
    lse: torch.Tensor           # float32 [B, H, N]: log2 of each query's joint normaliser
    lse_landmark: torch.Tensor  # float32 [B, H, m]: log2 of each landmark row's normaliser
    out_f32: torch.Tensor       # float32 [B, H, N, d]: the output before rounding

    def struct(self) -> Saved:
        return Saved(self.qtilde.data_ptr(), self.vtilde.data_ptr(), self.topk.data_ptr(),
                     self.route.data_ptr(), self.lse.data_ptr(), self.lse_landmark.data_ptr(),
                     self.out_f32.data_ptr())


def _check_qkv(*ts):
    Q = ts[0]
    for t in ts:
        if (not t.is_cuda or not t.is_contiguous() or t.dtype != Q.dtype or t.shape != Q.shape
                or t.device != Q.device):
            raise MitaError(2, "tensors must be contiguous tensors of one shape and dtype on one device")


def _check_saved(saved: "SavedOut", Q: torch.Tensor, m: int, k: int, s: int):
    """The C ABI cannot see tensor sizes: every saved tensor must have the
    shape, dtype and device mita_forward_train wrote it with for this call's
    sizes (else the kernels would read outside it)."""
    B, H, N, d = Q.shape
    want = {"qtilde": ((B, H, m, d), Q.dtype), "vtilde": ((B, H, m, d), torch.float32),
            "topk": ((B, H, m, k), torch.int32), "route": ((B, H, N, s), torch.int32),
            "lse": ((B, H, N), torch.float32), "lse_landmark": ((B, H, m), torch.float32),
            "out_f32": ((B, H, N, d), torch.float32)}
    for name, (shape, dtype) in want.items():
        t = getattr(saved, name)
        if (not isinstance(t, torch.Tensor) or tuple(t.shape) != shape or t.dtype != dtype
                or t.device != Q.device or not t.is_contiguous()):
            raise MitaError(2, f"saved.{name} must be a contiguous {dtype} tensor of shape {shape} on {Q.device}")


def _check_workspace(ws: torch.Tensor, Q: torch.Tensor):
    if ws.device != Q.device or not ws.is_contiguous():
        raise MitaError(2, "workspace must be a contiguous tensor on the inputs' device")


def forward_train(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, pool, k: int, s: int,
                  variant: str = "paper", workspace: torch.Tensor | None = None):
    """Forward pass that also keeps the tensors the backward pass needs.
    Returns (O, SavedOut)."""
    L = lib()
    _check_qkv(Q, K, V)
    if variant not in VARIANTS:
        raise MitaError(3, f"unknown variant {variant!r}")
    B, H, N, d = Q.shape
    gh, gw, lh, lw = pool
    m = lh * lw
    dt = _dtype_code(Q.dtype)
    P = Pool(gh, gw, lh, lw)
    if workspace is None:
        workspace = torch.empty(max(int(L.mita_workspace_bytes(dt, B, H, N, d, P, m, k, s)), 16),
                                dtype=torch.uint8, device=Q.device)
    _check_workspace(workspace, Q)
    dev = Q.device
    sv = SavedOut(
        qtilde=torch.empty((B, H, m, d), dtype=Q.dtype, device=dev),
        vtilde=torch.empty((B, H, m, d), dtype=torch.float32, device=dev),
        topk=torch.empty((B, H, m, k), dtype=torch.int32, device=dev),
        route=torch.empty((B, H, N, s), dtype=torch.int32, device=dev),
        lse=torch.empty((B, H, N), dtype=torch.float32, device=dev),
        lse_landmark=torch.empty((B, H, m), dtype=torch.float32, device=dev),
        out_f32=torch.empty((B, H, N, d), dtype=torch.float32, device=dev),
    )
    O = torch.empty_like(Q)
    st = sv.struct()
    stream = torch.cuda.current_stream(dev).cuda_stream
    _check(L.mita_forward_train(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), dt, B, H, N, d, P, m, k, s,
                                VARIANTS[variant], ctypes.byref(st), workspace.data_ptr(), workspace.numel(),
                                stream))
    return O, sv


def backward_workspace_bytes(dtype: torch.dtype, B: int, H: int, N: int, d: int, pool, k: int, s: int) -> int:
    gh, gw, lh, lw = pool
    return int(lib().mita_backward_workspace_bytes(_dtype_code(dtype), B, H, N, d, Pool(gh, gw, lh, lw),
                                                   lh * lw, k, s))


def backward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor, dO: torch.Tensor, pool,
             k: int, s: int, saved: SavedOut, variant: str = "paper", workspace: torch.Tensor | None = None):
    """Gradients (dQ, dK, dV) of sum(O * dO), experts and routes held fixed."""
    L = lib()
    _check_qkv(Q, K, V, O, dO)
    if variant not in VARIANTS:
        raise MitaError(3, f"unknown variant {variant!r}")
    B, H, N, d = Q.shape
    gh, gw, lh, lw = pool
    m = lh * lw
    _check_saved(saved, Q, m, k, s)
    dt = _dtype_code(Q.dtype)
    P = Pool(gh, gw, lh, lw)
    if workspace is None:
        workspace = torch.empty(max(int(L.mita_backward_workspace_bytes(dt, B, H, N, d, P, m, k, s)), 16),
                                dtype=torch.uint8, device=Q.device)
    _check_workspace(workspace, Q)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(Q), torch.empty_like(Q)
    st = saved.struct()
    stream = torch.cuda.current_stream(Q.device).cuda_stream
    _check(L.mita_backward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), dO.data_ptr(), dQ.data_ptr(),
                           dK.data_ptr(), dV.data_ptr(), dt, B, H, N, d, P, m, k, s, VARIANTS[variant],
                           ctypes.byref(st), workspace.data_ptr(), workspace.numel(), stream))
    return dQ, dK, dV


class MitaFunction(torch.autograd.Function):
    """MiTA attention as an autograd function: forward_train / backward.

    ``MitaFunction.apply(Q, K, V, pool, k, s, variant)``; gradients flow to
    Q, K and V (experts and routes held fixed)."""

    @staticmethod
    def forward(ctx, Q, K, V, pool, k, s, variant="paper"):
        Q, K, V = Q.contiguous(), K.contiguous(), V.contiguous()
        O, sv = forward_train(Q, K, V, pool, k, s, variant=variant)
        ctx.save_for_backward(Q, K, V, O)
        ctx.sv, ctx.cfg = sv, (pool, k, s, variant)
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, O = ctx.saved_tensors
        pool, k, s, variant = ctx.cfg
        dQ, dK, dV = backward(Q, K, V, O, dO.contiguous(), pool, k, s, ctx.sv, variant=variant)
        return dQ, dK, dV, None, None, None, None


STEP_SHAPES = {0: (8, 4, 256), 1: (16, 1, 256), 2: (8, 2, 512), 3: (16, 2, 256)}  # shape: (waves, blocks per wave, workgroups)


def probe_peaks(mfma_blocks: int = 2048, mfma_iters: int = 16384, copy_mib: int = 1024, reps: int = 3,
                step_iters: int = 2000) -> dict:
    """Measured peaks of this GPU: bf16 matrix-core TFLOP/s (mita_probe_mfma),
    device-copy HBM GB/s (bytes read + written, mita_probe_copy) and the
    useful TFLOP/s of the bare online-softmax step at each launch shape
    (mita_probe_step: 8 useful 16x16x32 products per block-step); the best of
    `reps` timed launches after one warm-up."""
    L = lib()
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream(dev).cuda_stream
    out = torch.empty(mfma_blocks * 256, dtype=torch.float32, device=dev)
    src = torch.ones(copy_mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)

    def best(fn):
        fn()
        ms = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        return min(ms)

    t_mfma = best(lambda: _check(L.mita_probe_mfma(out.data_ptr(), mfma_blocks, mfma_iters, stream)))
    t_copy = best(lambda: _check(L.mita_probe_copy(src.data_ptr(), dst.data_ptr(), src.numel(), stream)))
    flops = mfma_blocks * 4 * mfma_iters * 8 * 16384.0
    step = {}
    sout = torch.empty(max(w * 64 * g for w, _, g in STEP_SHAPES.values()), dtype=torch.float32, device=dev)
    for shape, (nw, ib, grid) in STEP_SHAPES.items():
        t = best(lambda: _check(L.mita_probe_step(sout.data_ptr(), shape, grid, step_iters, stream)))
        step[f"{nw}x{ib}"] = grid * nw * ib * step_iters * 131072.0 / (t * 1e-3) * 1e-12
    return dict(mfma_bf16_tflops=flops / (t_mfma * 1e-3) * 1e-12, hbm_copy_gbs=2.0 * src.numel() / (t_copy * 1e-3) * 1e-9,
                step_bf16_tflops=step,
                probe="mita_probe_mfma (eight independent 16x16x32 bf16 MFMA chains on varied operands), "
                      "mita_probe_copy (16-byte copy, four loads in flight per thread), "
                      "mita_probe_step (the online-softmax step alone, operands in registers; "
                      "key: waves x 16-row blocks per wave)")
