"""ctypes wrapper for the plain-C oracle (oracle/ref_cpu.c).

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Loads oracle/libssmoracle.so (built by
oracle/build.py); raises if it has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssmoracle.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"oracle library missing: {_LIB_PATH} (run oracle/build.py)")
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.ssm_oracle_fwd_rows.argtypes = [P, P, P, P, P, I64, P, P, P, P, P, ctypes.c_int,
                                          I64, I64, I64, I64, P, P, ctypes.c_int]
        L.ssm_oracle_fwd_rows.restype = ctypes.c_int
        L.ssm_oracle_fwd_rows_h0.argtypes = [P, P, P, P, P, I64, P, P, P, P, P, ctypes.c_int,
                                             I64, I64, I64, I64, P, I64, P, P, P, ctypes.c_int]
        L.ssm_oracle_fwd_rows_h0.restype = ctypes.c_int
        L.ssm_oracle_bwd.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P, I64, I64, I64, I64,
                                     P, P, P, P, P, P, P, P, P, ctypes.c_int]
        L.ssm_oracle_bwd.restype = ctypes.c_int
        L.affine_scan_serial_f32.argtypes = [P, P, P, P, I64, I64]
        L.affine_scan_serial_f32.restype = None
        L.affine_scan_replay_f32.argtypes = [P, P, P, P, I64, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.affine_scan_replay_f32.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _f32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float32).numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def fwd_rows(u_rows, delta_rows, z_rows, row_b, row_d, A, B, C, D, delta_bias,
             delta_softplus, batch, dim, dstate, L, want_y=True, nthreads=0, h0_rows=None, chunk=0):
    """float64 selective-scan forward for selected (batch, channel) rows.

    u_rows, delta_rows, z_rows: [nrows, L] (float32-representable values);
    row_b, row_d: [nrows] indices; A [dim, dstate]; B, C [batch, dstate, L];
    D, delta_bias [dim] or None; h0_rows: [nrows, dstate] start states or
    None (zero).  Returns (y [nrows, L] or None, last_state [nrows, dstate]),
    and with chunk > 0 also the chunk-boundary states
    [nrows, ceil(L/chunk), dstate] (state after step min((k+1)*chunk, L)-1).
    """
    u_rows = _f32(u_rows); delta_rows = _f32(delta_rows); z_rows = _f32(z_rows)
    A = _f32(A); B = _f32(B); C = _f32(C); D = _f32(D); delta_bias = _f32(delta_bias)
    row_b = np.ascontiguousarray(row_b, dtype=np.int64)
    row_d = np.ascontiguousarray(row_d, dtype=np.int64)
    nrows = row_b.shape[0]
    y = np.empty((nrows, L), dtype=np.float64) if want_y else None
    last = np.empty((nrows, dstate), dtype=np.float64)
    h0 = None if h0_rows is None else np.ascontiguousarray(
        h0_rows.detach().cpu().double().numpy() if hasattr(h0_rows, "detach") else h0_rows, dtype=np.float64)
    K = (L + chunk - 1) // chunk if chunk else 0
    bounds = np.empty((nrows, K, dstate), dtype=np.float64) if chunk else None
    rc = lib().ssm_oracle_fwd_rows_h0(_ptr(u_rows), _ptr(delta_rows), _ptr(z_rows), _ptr(row_b), _ptr(row_d),
                                      nrows, _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(delta_bias),
                                      int(bool(delta_softplus)), batch, dim, dstate, L, _ptr(h0), int(chunk),
                                      _ptr(bounds), _ptr(y), _ptr(last), int(nthreads))
    if rc != 0:
        raise ValueError("ssm_oracle_fwd_rows_h0 rejected its arguments")
    if chunk:
        return y, last, bounds
    return y, last


def fwd_full(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, nthreads=0):
    """All rows of a [b, d, L] problem; returns (y [b,d,L], last [b,d,n]) in float64."""
    u = _f32(u); delta = _f32(delta); z = _f32(z)
    bsz, dim, L = u.shape
    dstate = np.asarray(_f32(A)).shape[1]
    rb, rd = np.meshgrid(np.arange(bsz), np.arange(dim), indexing="ij")
    y, last = fwd_rows(u.reshape(bsz * dim, L), delta.reshape(bsz * dim, L),
                       None if z is None else z.reshape(bsz * dim, L), rb.ravel(), rd.ravel(),
                       A, B, C, D, delta_bias, delta_softplus, bsz, dim, dstate, L, nthreads=nthreads)
    return y.reshape(bsz, dim, L), last.reshape(bsz, dim, dstate)


def bwd_full(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
             h0=None, dy=None, dlast=None, nthreads=0):
    """float64 gradients of the whole [b, d, L] problem (ref_cpu.c
    ssm_oracle_bwd).  Inputs are taken at their float32 values (bfloat16
    tensors upcast exactly).  Returns a dict like oracle.ref.selective_scan_bwd:
    du, ddelta, dz (None without z) [b,d,L]; dA [d,n]; dB, dC [b,n,L];
    dD, ddelta_bias [d]; dh0 [b,d,n]."""
    u = _f32(u); delta = _f32(delta); z = _f32(z); A = _f32(A); B = _f32(B); C = _f32(C)
    D = _f32(D); delta_bias = _f32(delta_bias); h0 = _f32(h0); dy = _f32(dy); dlast = _f32(dlast)
    bsz, dim, L = u.shape
    n = A.shape[1]
    out = {k: np.empty(sh, dtype=np.float64) for k, sh in
           (("du", (bsz, dim, L)), ("ddelta", (bsz, dim, L)), ("dA", (dim, n)), ("dB", (bsz, n, L)),
            ("dC", (bsz, n, L)), ("dD", (dim,)), ("ddelta_bias", (dim,)), ("dh0", (bsz, dim, n)))}
    out["dz"] = np.empty((bsz, dim, L), dtype=np.float64) if z is not None else None
    rc = lib().ssm_oracle_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                              int(bool(delta_softplus)), _ptr(h0), _ptr(dy), _ptr(dlast), bsz, dim, n, L,
                              _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dz"]), _ptr(out["dA"]), _ptr(out["dB"]),
                              _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["ddelta_bias"]), _ptr(out["dh0"]),
                              int(nthreads))
    if rc != 0:
        raise ValueError("ssm_oracle_bwd rejected its arguments")
    return out


def affine_serial_f32(a, b):
    """Plain serial float32 fold with fmaf, [rows, L] -> (out_a, out_b)."""
    a = _f32(a); b = _f32(b)
    rows, L = a.shape
    oa = np.empty_like(a); ob = np.empty_like(b)
    lib().affine_scan_serial_f32(_ptr(a), _ptr(b), _ptr(oa), _ptr(ob), rows, L)
    return oa, ob


def affine_replay_f32(a, b, T, lanes, W):
    """float32 replay of the blocked scan order (see ref_cpu.c)."""
    a = _f32(a); b = _f32(b)
    rows, L = a.shape
    oa = np.empty_like(a); ob = np.empty_like(b)
    rc = lib().affine_scan_replay_f32(_ptr(a), _ptr(b), _ptr(oa), _ptr(ob), rows, L, int(T), int(lanes), int(W))
    if rc != 0:
        raise ValueError("bad replay parameters")
    return oa, ob
