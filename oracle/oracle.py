"""ctypes binding of the fp64 KDA oracle (oracle/kda_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's cpu_baseline leg, never by the product path.  It shares no code
with the HIP implementation; both are fed by the seeded generator in
linear_attention_kda_amd/workloads.py, which holds none of the method's
arithmetic.

What the oracle computes is documented in kda_oracle.c: the Kimi Delta
Attention recurrence token by token in fp64
  S_t = (Diag(a_t) - b_t k_t (k_t * a_t)^T) S_{t-1} + b_t k_t v_t^T,  a_t = exp(g_t),
  o_t = scale * S_t^T q_t
[core.today "Kimi Linear 특집", ch.4 혁신 2 (state-update equation) and ch.2
(linear-attention readout)].  Inputs of any float dtype are upcast exactly to
float64 (bf16 -> fp64 is exact), so a comparison against the GPU measures only
the kernel's own rounding.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C99, OpenMP over independent tasks)."""
    stale = (not os.path.exists(_LIB_PATH)) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp, _dp,
                                       _ip, _ip, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, _ip, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int]
        lib.kda_oracle_fwd_literal.restype = ctypes.c_int
        lib.kda_oracle_fwd_literal.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp,
                                               _dp, _ip, _ip, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64]
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp, _dp,
                                       _ip, _ip, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int]
        lib.kda_oracle_bwd.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp, _dp,
                                       _dp, _dp, _dp, _dp, _dp, _dp, _ip, _ip, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int]
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _f64(x) -> np.ndarray:
    """Exact upcast to a contiguous float64 numpy array (accepts torch tensors)."""
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype, go via fp32 (exact)
        import torch
        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.to(torch.float32)
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(_dp)


def _sequences(B: int, T: int, cu_seqlens):
    if cu_seqlens is None:
        start = np.arange(B, dtype=np.int64) * T
        length = np.full(B, T, dtype=np.int64)
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                        dtype=np.int64)
        if cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] > T:
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end <= T")
        start = np.ascontiguousarray(cu[:-1])
        length = np.ascontiguousarray(np.diff(cu))
    return start, length


def fwd(q, k, v, g, beta, scale: float, initial_state=None, cu_seqlens=None, heads=None,
        nthreads: int = 0, literal: bool = False, col_block: int = 0):
    """Run the oracle.

    q, k, g: [B, T, H, DK]; v: [B, T, H, DV]; beta: [B, T, H]; initial_state:
    [N, H, DK, DV] or None (zero).  With cu_seqlens (B must be 1) sequence n is
    rows cu[n]:cu[n+1]; otherwise each batch row is one sequence (N = B).
    heads: optional list of head indices to evaluate (others stay zero).
    col_block: split every (sequence, head) into tasks of that many value
    columns (the columns of the state are independent; results are identical).
    Returns (o [B, T, H, DV] float64, final_state [N, H, DK, DV] float64).
    """
    lib = _load()
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3]:
        raise ValueError("inconsistent input shapes")
    start, length = _sequences(B, T, cu_seqlens)
    N = start.shape[0]
    S0 = None if initial_state is None else _f64(initial_state)
    if S0 is not None and S0.shape != (N, H, DK, DV):
        raise ValueError(f"initial_state must be {(N, H, DK, DV)}, got {S0.shape}")
    o = np.zeros((B, T, H, DV), dtype=np.float64)
    S_out = np.zeros((N, H, DK, DV), dtype=np.float64)
    if literal:
        if heads is not None:
            raise ValueError("the literal form evaluates all heads")
        rc = lib.kda_oracle_fwd_literal(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        float(scale), _ptr(S0), _ptr(S_out), _ptr(o),
                                        start.ctypes.data_as(_ip), length.ctypes.data_as(_ip),
                                        N, H, DK, DV)
    else:
        hs = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
        rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                _ptr(S0), _ptr(S_out), _ptr(o), start.ctypes.data_as(_ip),
                                length.ctypes.data_as(_ip), N, H, DK, DV,
                                None if hs is None else hs.ctypes.data_as(_ip),
                                0 if hs is None else hs.shape[0], int(col_block), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda oracle failed with code {rc}")
    return o, S_out


def gdn_fwd(q, k, v, g, beta, scale: float, initial_state=None, cu_seqlens=None, nthreads: int = 0):
    """Scalar-gate (Gated DeltaNet) oracle: one decay exp(g) per token and head.

    q, k: [B, T, H, DK]; v: [B, T, H, DV]; g, beta: [B, T, H]; initial_state:
    [N, H, DK, DV] or None.  Sequences as in fwd().  Returns (o, final_state)
    in float64.  The recurrence is documented at gdn_oracle_fwd in kda_oracle.c.
    """
    lib = _load()
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or g.shape != q.shape[:3] \
            or beta.shape != q.shape[:3]:
        raise ValueError("inconsistent input shapes")
    start, length = _sequences(B, T, cu_seqlens)
    N = start.shape[0]
    S0 = None if initial_state is None else _f64(initial_state)
    if S0 is not None and S0.shape != (N, H, DK, DV):
        raise ValueError(f"initial_state must be {(N, H, DK, DV)}, got {S0.shape}")
    o = np.zeros((B, T, H, DV), dtype=np.float64)
    S_out = np.zeros((N, H, DK, DV), dtype=np.float64)
    rc = lib.gdn_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                            _ptr(S0), _ptr(S_out), _ptr(o), start.ctypes.data_as(_ip),
                            length.ctypes.data_as(_ip), N, H, DK, DV, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"gdn oracle failed with code {rc}")
    return o, S_out


def bwd(q, k, v, g, beta, scale: float, do, initial_state=None, d_final_state=None,
        cu_seqlens=None, nthreads: int = 0):
    """Reverse-mode gradients of the KDA forward (oracle.fwd's recurrence) in fp64.

    do: dL/do, [B, T, H, DV]; d_final_state: dL/dS_final [N, H, DK, DV] or None.
    Returns a dict with dq, dk, dg ([B, T, H, DK]), dv ([B, T, H, DV]),
    dbeta ([B, T, H]) and dS0 ([N, H, DK, DV], the gradient of the initial state).
    Keeps every forward state of a running task: memory grows with the longest
    sequence (T * DK * DV * 8 bytes per thread).
    """
    lib = _load()
    q, k, v, g, beta, do = (_f64(x) for x in (q, k, v, g, beta, do))
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3] or do.shape != v.shape:
        raise ValueError("inconsistent input shapes")
    start, length = _sequences(B, T, cu_seqlens)
    N = start.shape[0]
    S0 = None if initial_state is None else _f64(initial_state)
    dST = None if d_final_state is None else _f64(d_final_state)
    for name, a in (("initial_state", S0), ("d_final_state", dST)):
        if a is not None and a.shape != (N, H, DK, DV):
            raise ValueError(f"{name} must be {(N, H, DK, DV)}, got {a.shape}")
    out = {n: np.zeros(x.shape, dtype=np.float64) for n, x in
           (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    out["dS0"] = np.zeros((N, H, DK, DV), dtype=np.float64)
    if nthreads <= 0:  # every running task holds its sequence's states
        per = (int(length.max()) + 1 if length.size else 1) * DK * DV * 8
        nthreads = max(1, min(max_threads(), int(8e9 // max(per, 1))))
    rc = lib.kda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(S0),
                            _ptr(do), _ptr(dST), _ptr(out["dq"]), _ptr(out["dk"]),
                            _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                            _ptr(out["dS0"]), start.ctypes.data_as(_ip),
                            length.ctypes.data_as(_ip), N, H, DK, DV, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"kda oracle backward failed with code {rc}")
    return out
