"""Thin ctypes binding of the C ABI in include/kda.h (argument marshalling only).

Every step of the forward pass runs in the HIP kernels of libkda.so; this
module checks tensor dtypes, shapes, devices and contiguity, passes raw device
pointers and the current HIP stream, and turns negative status codes into
KdaError.  There is no fallback: if libkda.so is missing or was built for
another target, calls fail loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

KDA_BF16 = 0
KDA_FP32 = 1
D = 128

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")
_lib = None
_lock = threading.Lock()

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where} failed with status {status}: {detail}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so from the package directory (raises if it was never built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise FileNotFoundError(
                f"{_LIB_PATH} is missing: build it with `python -m linear_attention_kda_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.kda_fwd.restype = ctypes.c_int
        lib.kda_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, ctypes.c_int, _vp,
                                ctypes.c_int, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp]
        lib.kda_fwd_check.restype = ctypes.c_int
        lib.kda_fwd_check.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, ctypes.c_int,
                                      _vp, ctypes.c_int, _vp, _i32, _i32, _i64, _i32, _i32, _i32,
                                      _vp]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_decode.restype = ctypes.c_int
        lib.kda_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, ctypes.c_int, _vp,
                                   _i32, _i32, _i32, _i32, _vp, _vp]
        lib.kda_decode_check.restype = ctypes.c_int
        lib.kda_decode_check.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                         ctypes.c_int, _vp, _i32, _i32, _i32, _i32, _vp]
        for name in ("kda_gdn_fwd", "kda_gdn_fwd_check", "kda_gdn_decode", "kda_gdn_decode_check",
                     "kda_fwd_noalloc"):
            base = getattr(lib, name.replace("gdn_", "").replace("_noalloc", ""))
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = base.argtypes
        lib.kda_bwd.restype = ctypes.c_int
        lib.kda_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, ctypes.c_int, _vp,
                                _vp, ctypes.c_int, _vp, _i32, _i32, _i64, _i32, _i32, _i32,
                                _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        lib.kda_bwd_check.restype = ctypes.c_int
        lib.kda_bwd_check.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, ctypes.c_int,
                                      _vp, _vp, ctypes.c_int, _vp, _i32, _i32, _i64, _i32, _i32,
                                      _i32, _vp, _vp, _vp, _vp, _vp, _vp]
        lib.kda_bwd_workspace_bytes.restype = _i64
        lib.kda_bwd_workspace_bytes.argtypes = [_i32, _i64, _i32]
        lib.kda_dim_workspace_bytes.restype = _i64
        lib.kda_dim_workspace_bytes.argtypes = [_i32, _i64, _i32, _i32]
        lib.kda_release_workspaces.restype = ctypes.c_int
        lib.kda_release_workspaces.argtypes = []
        lib.kda_plan.restype = ctypes.c_int
        lib.kda_plan.argtypes = [_i32, _i64, _i32, _i32, _i32, ctypes.POINTER(_i32),
                                 ctypes.POINTER(_i32), ctypes.POINTER(_i64)]
        _lib = lib
        return lib


def _detail(lib, status: int) -> str:
    msg = lib.kda_last_error().decode()
    return msg or lib.kda_status_string(status).decode()


def _state_dtype(t) -> int:
    import torch
    if t is None:
        return KDA_FP32
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_FP32
    raise TypeError(f"states must be bfloat16 or float32, got {t.dtype}")


def release_workspaces(device=None):
    """Free the workspaces the library keeps between calls on `device` (default:
    torch's current device), after the calls that used them have finished."""
    import torch
    lib = load_library()
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        st = lib.kda_release_workspaces()
    if st != 0:
        raise KdaError(st, "kda_release_workspaces", _detail(lib, st))


def plan(n_sequences: int, T: int, heads: int, varlen: bool = False,
         cu_count: int = 0) -> tuple[int, int, int]:
    """(workgroups, value_splits, workspace_bytes) of kda_fwd for these sizes.

    T is tokens per batch row, or the packed total when varlen."""
    lib = load_library()
    wg, ns, ws = _i32(0), _i32(0), _i64(0)
    st = lib.kda_plan(n_sequences, T, heads, int(bool(varlen)), cu_count, ctypes.byref(wg),
                      ctypes.byref(ns), ctypes.byref(ws))
    if st != 0:
        raise KdaError(st, "kda_plan", _detail(lib, st))
    return wg.value, ns.value, ws.value


def fwd_check(*, B, T, H, K=D, V=D, q=0, k=0, v=0, g=0, beta=0, out=0, initial_state=0,
              initial_dtype=KDA_FP32, final_state=0, final_dtype=KDA_FP32, cu_seqlens=0,
              num_seqs=0, scale=1.0) -> int:
    """Host-only validation with raw (never dereferenced) addresses; returns the status."""
    lib = load_library()
    return lib.kda_fwd_check(q, k, v, g, beta, scale, initial_state, initial_dtype, final_state,
                             final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, out)


def gdn_fwd_check(*, B, T, H, K=D, V=D, q=0, k=0, v=0, g=0, beta=0, out=0, initial_state=0,
                  initial_dtype=KDA_FP32, final_state=0, final_dtype=KDA_FP32, cu_seqlens=0,
                  num_seqs=0, scale=1.0) -> int:
    """Host-only validation of the scalar-gate forward (g is [B, T, H])."""
    lib = load_library()
    return lib.kda_gdn_fwd_check(q, k, v, g, beta, scale, initial_state, initial_dtype,
                                 final_state, final_dtype, cu_seqlens, num_seqs, B, T, H, K, V, out)


def fwd(q, k, v, g, beta, scale: float | None = None, initial_state=None, final_state=None,
        cu_seqlens=None, out=None, output_final_state: bool = False):
    """KDA chunkwise forward pass on the current HIP stream.

    q, k, v: bf16 [B, T, H, d]; g: fp32 [B, T, H, d] (log-decay, alpha = exp(g));
    d = 128, 64 or 256; beta: fp32 [B, T, H]; scale defaults to 1/sqrt(d);
    initial_state / final_state: [N, H, d, d] bf16 or fp32 (same dtype when both given;
    final_state may be the same tensor as initial_state); cu_seqlens: int32
    [N+1] on the device (requires B = 1).  With output_final_state=True and no
    final_state tensor, one is allocated (dtype of initial_state, else fp32).
    Returns out, or (out, final_state) when a final state is produced.
    """
    return _fwd(q, k, v, g, beta, scale, initial_state, final_state, cu_seqlens, out,
                output_final_state, scalar_gate=False)


def fwd_noalloc(q, k, v, g, beta, scale: float | None = None, initial_state=None,
                final_state=None, cu_seqlens=None, out=None, output_final_state: bool = False):
    """fwd() through kda_fwd_noalloc: the library allocates no device memory and uses
    its static per-GPU scratch (KDA_NOALLOC_SCRATCH_BYTES) as the workspace.  out and
    final_state are allocated here (by torch) only when not given."""
    return _fwd(q, k, v, g, beta, scale, initial_state, final_state, cu_seqlens, out,
                output_final_state, scalar_gate=False, noalloc=True)


def gdn_fwd(q, k, v, g, beta, scale: float | None = None, initial_state=None, final_state=None,
            cu_seqlens=None, out=None, output_final_state: bool = False):
    """Scalar-gate (Gated DeltaNet) forward: as fwd() with g fp32 [B, T, H], one
    log-decay per token and head."""
    return _fwd(q, k, v, g, beta, scale, initial_state, final_state, cu_seqlens, out,
                output_final_state, scalar_gate=True)


def _fwd(q, k, v, g, beta, scale, initial_state, final_state, cu_seqlens, out,
         output_final_state, scalar_gate, noalloc=False):
    import torch
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("g", g, torch.float32),
                        ("beta", beta, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    g_shape = q.shape[:3] if scalar_gate else q.shape
    if k.shape != q.shape or g.shape != g_shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3]:
        raise ValueError("inconsistent shapes: q, k [B,T,H,K]; g [B,T,H,K] ([B,T,H] for the "
                         "scalar gate); v [B,T,H,V]; beta [B,T,H]")
    num_seqs = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev \
                or not cu_seqlens.is_contiguous():
            raise TypeError("cu_seqlens must be a contiguous int32 tensor on the same device")
        num_seqs = cu_seqlens.numel() - 1
    N = num_seqs if cu_seqlens is not None else B
    if out is None:
        out = torch.empty(B, T, H, V, dtype=torch.bfloat16, device=dev)
    elif out.shape != (B, T, H, V) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [B, T, H, V] tensor")
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and (t.shape != (N, H, K, V) or not t.is_contiguous() or t.device != dev):
            raise ValueError(f"{name} must be a contiguous [{N}, {H}, {K}, {V}] tensor on {dev}")
    if final_state is None and output_final_state:
        dt = initial_state.dtype if initial_state is not None else torch.float32
        final_state = torch.empty(N, H, K, V, dtype=dt, device=dev)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    stream = torch.cuda.current_stream(dev).cuda_stream
    entry = lib.kda_gdn_fwd if scalar_gate else lib.kda_fwd_noalloc if noalloc else lib.kda_fwd
    with torch.cuda.device(dev):
        st = entry(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), float(scale),
                   ptr(initial_state), _state_dtype(initial_state), ptr(final_state),
                   _state_dtype(final_state), ptr(cu_seqlens), num_seqs, B, T, H, K, V,
                   ptr(out), stream)
    if st != 0:
        raise KdaError(st, "kda_gdn_fwd" if scalar_gate else "kda_fwd_noalloc" if noalloc
                       else "kda_fwd", _detail(lib, st))
    return (out, final_state) if final_state is not None else out


def decode_check(*, N, H, K=D, V=D, q=0, k=0, v=0, g=0, beta=0, out=0, state=0,
                 state_dtype=KDA_FP32, state_indices=0, scale=1.0) -> int:
    """Host-only validation of a decode step with raw (never dereferenced) addresses."""
    lib = load_library()
    return lib.kda_decode_check(q, k, v, g, beta, scale, state, state_dtype, state_indices, N, H,
                                K, V, out)


def gdn_decode_check(*, N, H, K=D, V=D, q=0, k=0, v=0, g=0, beta=0, out=0, state=0,
                     state_dtype=KDA_FP32, state_indices=0, scale=1.0) -> int:
    """Host-only validation of a scalar-gate decode step (g is [N, H])."""
    lib = load_library()
    return lib.kda_gdn_decode_check(q, k, v, g, beta, scale, state, state_dtype, state_indices,
                                    N, H, K, V, out)


def decode(q, k, v, g, beta, state, scale: float | None = None, state_indices=None, out=None):
    """One recurrent KDA step per sequence on the current HIP stream; `state` is updated in place.

    q, k, v: bf16 [N, H, d] (one token per sequence, d = 128, 64 or 256); g: fp32
    [N, H, d]; beta: fp32 [N, H]; state: [slots, H, d, d] bf16 or fp32; state_indices:
    optional int32 [N] slot per sequence (negative: skip); scale defaults to
    1/sqrt(d).  Returns out (bf16 [N, H, d]).
    """
    return _decode(q, k, v, g, beta, state, scale, state_indices, out, scalar_gate=False)


def gdn_decode(q, k, v, g, beta, state, scale: float | None = None, state_indices=None, out=None):
    """Scalar-gate decode step: as decode() with g fp32 [N, H]."""
    return _decode(q, k, v, g, beta, state, scale, state_indices, out, scalar_gate=True)


def _decode(q, k, v, g, beta, state, scale, state_indices, out, scalar_gate):
    import torch
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d]")
    N, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("g", g, torch.float32),
                        ("beta", beta, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    g_shape = q.shape[:2] if scalar_gate else q.shape
    if k.shape != q.shape or g.shape != g_shape or v.shape[:2] != q.shape[:2] \
            or beta.shape != q.shape[:2]:
        raise ValueError("inconsistent shapes: q, k [N,H,K]; g [N,H,K] ([N,H] for the scalar "
                         "gate); v [N,H,V]; beta [N,H]")
    if state.dim() != 4 or state.shape[1:] != (H, K, V) or not state.is_contiguous() \
            or state.device != dev:
        raise ValueError(f"state must be a contiguous [slots, {H}, {K}, {V}] tensor on {dev}")
    if state_indices is not None:
        if state_indices.dtype != torch.int32 or state_indices.device != dev \
                or not state_indices.is_contiguous() or state_indices.shape != (N,):
            raise TypeError("state_indices must be a contiguous int32 [N] tensor on the same device")
    elif state.shape[0] < N:
        raise ValueError("without state_indices the state needs at least N slots")
    if out is None:
        out = torch.empty(N, H, V, dtype=torch.bfloat16, device=dev)
    elif out.shape != (N, H, V) or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [N, H, V] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    stream = torch.cuda.current_stream(dev).cuda_stream
    entry = lib.kda_gdn_decode if scalar_gate else lib.kda_decode
    with torch.cuda.device(dev):
        st = entry(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), float(scale), ptr(state),
                   _state_dtype(state), ptr(state_indices), N, H, K, V, ptr(out), stream)
    if st != 0:
        raise KdaError(st, "kda_gdn_decode" if scalar_gate else "kda_decode", _detail(lib, st))
    return out


def bwd_check(*, B, T, H, K=D, V=D, q=0, k=0, v=0, g=0, beta=0, d_out=0, initial_state=0,
              initial_dtype=KDA_FP32, d_final_state=0, d_final_dtype=KDA_FP32, cu_seqlens=0,
              num_seqs=0, dq=0, dk=0, dv=0, dg=0, dbeta=0, d_initial_state=0, scale=1.0) -> int:
    """Host-only validation of a backward call with raw (never dereferenced) addresses."""
    lib = load_library()
    return lib.kda_bwd_check(q, k, v, g, beta, scale, initial_state, initial_dtype, d_out,
                             d_final_state, d_final_dtype, cu_seqlens, num_seqs, B, T, H, K, V,
                             dq, dk, dv, dg, dbeta, d_initial_state)


def dim_workspace_bytes(n_sequences: int, rows: int, heads: int, head_dim: int) -> int:
    """Workspace bytes of fwd() at head dimension 64 or 256 (-1 for other sizes)."""
    return int(load_library().kda_dim_workspace_bytes(n_sequences, rows, heads, head_dim))


def bwd_workspace_bytes(n_sequences: int, rows: int, heads: int) -> int:
    return int(load_library().kda_bwd_workspace_bytes(n_sequences, rows, heads))


def bwd(q, k, v, g, beta, d_out, scale: float | None = None, initial_state=None,
        d_final_state=None, cu_seqlens=None, want_d_initial_state: bool = True):
    """Gradients of the KDA forward pass on the current HIP stream.

    Inputs as fwd(); d_out: bf16 [B, T, H, 128] (dL/do); d_final_state: dL/dS_final,
    [N, H, 128, 128] bf16 or fp32, or None.  Returns a dict with fp32 dq, dk, dv, dg
    ([B, T, H, 128]), dbeta ([B, T, H]) and dS0 ([N, H, 128, 128], the gradient of
    the initial state; None when want_d_initial_state is False).
    """
    import torch
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("g", g, torch.float32),
                        ("beta", beta, torch.float32), ("d_out", d_out, torch.bfloat16)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {dev}")
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3] or d_out.shape != v.shape:
        raise ValueError("inconsistent shapes")
    num_seqs = 0
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev \
                or not cu_seqlens.is_contiguous():
            raise TypeError("cu_seqlens must be a contiguous int32 tensor on the same device")
        num_seqs = cu_seqlens.numel() - 1
    N = num_seqs if cu_seqlens is not None else B
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None and (t.shape != (N, H, K, V) or not t.is_contiguous() or t.device != dev):
            raise ValueError(f"{name} must be a contiguous [{N}, {H}, {K}, {V}] tensor on {dev}")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty(B, T, H, K, **f32), "dk": torch.empty(B, T, H, K, **f32),
           "dv": torch.empty(B, T, H, V, **f32), "dg": torch.empty(B, T, H, K, **f32),
           "dbeta": torch.empty(B, T, H, **f32),
           "dS0": torch.empty(N, H, K, V, **f32) if want_d_initial_state else None}
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = lib.kda_bwd(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), float(scale),
                         ptr(initial_state), _state_dtype(initial_state), ptr(d_out),
                         ptr(d_final_state), _state_dtype(d_final_state), ptr(cu_seqlens),
                         num_seqs, B, T, H, K, V, ptr(out["dq"]), ptr(out["dk"]), ptr(out["dv"]),
                         ptr(out["dg"]), ptr(out["dbeta"]), ptr(out["dS0"]), stream)
    if st != 0:
        raise KdaError(st, "kda_bwd", _detail(lib, st))
    return out
