"""MI355X (gfx950) selective-scan forward: thin Python binding of libssmscan.so.

Every function here only checks and marshals arguments (torch tensors ->
device pointers, the current HIP stream) and calls the C ABI declared in
``include/ssm_scan.h``; all arithmetic runs in the HIP kernels.  There is no
CPU fallback: if the library is missing or no GPU is present the calls raise.

    y, last_state = ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus=True)
    out_a, out_b  = affine_scan(a, b)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["SSMError", "ssm_scan_fwd", "ssm_scan_fwd_states", "ssm_scan_fwd_conv", "ssm_scan_bwd",
           "ssm_scan_bwd_conv", "ssm_step", "ssm_step_conv", "ssm_out_proj", "ssm_out_proj_bwd", "affine_scan",
           "affine_scan_order", "plan_for", "library_path", "load_library", "PLANS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssmscan.so")
_lib = None

SSM_OK, SSM_EINVAL, SSM_EUNSUPPORTED, SSM_EHIP, SSM_ENOMEM = 0, 1, 2, 3, 4
SSM_F32, SSM_BF16 = 0, 1
PLANS = {"auto": 0, "carry": 1, "twopass": 2, "mixed": 3, "lpar": 4}
_PLAN_NAMES = {v: k for k, v in PLANS.items()}
_STATUS = {SSM_EINVAL: "invalid argument", SSM_EUNSUPPORTED: "unsupported", SSM_EHIP: "HIP error",
           SSM_ENOMEM: "out of memory"}


class SSMError(RuntimeError):
    """A non-zero status from the C ABI; ``code`` is the SSM_* value."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, 'error')} ({code}): {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libssmscan.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(the selective scan has no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ssm_scan_fwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I64, I64, I64, I64, I, P]
    lib.ssm_scan_fwd.restype = I
    lib.ssm_scan_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I64, I64, I64, I64, I, P]
    lib.ssm_scan_fwd_noalloc.restype = I
    lib.ssm_scan_fwd_plan.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I64, I64, I64, I64, I, I, I, I64, P]
    lib.ssm_scan_fwd_plan.restype = I
    lib.ssm_scan_fwd_states.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, P, I64, I64, I64, I64, I64, I, I, P]
    lib.ssm_scan_fwd_states.restype = I
    lib.ssm_step.argtypes = [P, P, P, P, P, P, P, P, I, P, P, P, I64, I64, I64, I, P]
    lib.ssm_scan_fwd_conv.argtypes = [P, P, P, I, P, P, P, P, P, P, P, I, P, P, P, P, P, I64, I64, I64, I64, I64,
                                      I, I, P]
    lib.ssm_scan_fwd_conv.restype = I
    lib.ssm_step_conv.argtypes = [P, P, P, I, P, P, P, P, P, P, P, P, P, I, P, P, P, P, I64, I64, I64, I, P]
    lib.ssm_step_conv.restype = I
    lib.ssm_scan_bwd.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I64, P, P, P, P, P, P, P, P, P, P, P,
                                 I64, I64, I64, I64, I, I, P]
    lib.ssm_scan_bwd.restype = I
    lib.ssm_scan_bwd_conv.argtypes = [P, P, P, I, P, P, P, P, P, P, P, I, P, P, I64, P, P, P, P, P, P, P, P, P, P,
                                      P, P, P, I64, I64, I64, I64, I, I, P]
    lib.ssm_scan_bwd_conv.restype = I
    lib.ssm_step.restype = I
    lib.ssm_scan_plan_for.argtypes = [I64, I64, I64, I64, I, ctypes.POINTER(I), ctypes.POINTER(I),
                                      ctypes.POINTER(I64)]
    lib.ssm_scan_plan_for.restype = I
    lib.ssm_out_proj.argtypes = [P, P, P, I64, I64, I64, I64, I, P]
    lib.ssm_out_proj.restype = I
    lib.ssm_out_proj_bwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I, P]
    lib.ssm_out_proj_bwd.restype = I
    lib.affine_scan.argtypes = [P, P, P, P, I64, I64, P]
    lib.affine_scan.restype = I
    lib.affine_scan_order.argtypes = [ctypes.POINTER(I)] * 4
    lib.affine_scan_order.restype = I
    lib.ssm_last_error.argtypes = []
    lib.ssm_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int):
    if rc != SSM_OK:
        msg = load_library().ssm_last_error().decode(errors="replace")
        raise SSMError(rc, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, device, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def ssm_scan_fwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                 D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                 delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                 return_last_state: bool = True, plan: str = "auto", states_per_lane: int = 0,
                 chunk: int = 0, y: Optional[torch.Tensor] = None,
                 last_state: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Selective-scan forward on the GPU (see ``ssm_scan_fwd`` in include/ssm_scan.h).

    u, delta, z: [b, d, L]; B, C: [b, n, L] -- all float32 or all bfloat16.
    A: [d, n] float32; D, delta_bias: [d] float32 or None.
    Returns (y [b, d, L] in the input dtype, last_state [b, d, n] float32 or None).
    """
    device = u.device
    if device.type != "cuda":
        raise ValueError("ssm_scan_fwd needs CUDA/HIP tensors")
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [b, d, L] and A [d, n]")
    bsz, dim, L = u.shape
    n = A.shape[1]
    dt = u.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    _need(u, "u", dt, device, (bsz, dim, L))
    _need(delta, "delta", dt, device, (bsz, dim, L))
    _need(A, "A", torch.float32, device, (dim, n))
    _need(B, "B", dt, device, (bsz, n, L))
    _need(C, "C", dt, device, (bsz, n, L))
    if z is not None:
        _need(z, "z", dt, device, (bsz, dim, L))
    if D is not None:
        _need(D, "D", torch.float32, device, (dim,))
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", torch.float32, device, (dim,))
    if plan not in PLANS:
        raise ValueError(f"plan must be one of {list(PLANS)}")
    if y is None:
        y = torch.empty_like(u)
    else:
        _need(y, "y", dt, device, (bsz, dim, L))
    if return_last_state and last_state is None:
        last_state = torch.empty((bsz, dim, n), device=device, dtype=torch.float32)
    elif last_state is not None:
        _need(last_state, "last_state", torch.float32, device, (bsz, dim, n))
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_scan_fwd_plan(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                   _ptr(delta_bias), int(bool(delta_softplus)), _ptr(y), _ptr(last_state),
                                   bsz, dim, n, L, SSM_F32 if dt == torch.float32 else SSM_BF16,
                                   PLANS[plan], int(states_per_lane), int(chunk), _stream(device))
    _check(rc)
    return y, last_state


def ssm_scan_fwd_noalloc(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                         D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                         delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                         y: Optional[torch.Tensor] = None,
                         last_state: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``ssm_scan_fwd`` through the entry point that allocates no device
    memory (see ``ssm_scan_fwd_noalloc`` in include/ssm_scan.h): the library
    call itself allocates nothing; pass ``y`` (and ``last_state``) to keep
    this wrapper from allocating them with torch.  Calls that overlap on one
    GPU race on its fixed scratch."""
    device = u.device
    if device.type != "cuda":
        raise ValueError("ssm_scan_fwd_noalloc needs CUDA/HIP tensors")
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [b, d, L] and A [d, n]")
    bsz, dim, L = u.shape
    n = A.shape[1]
    dt = u.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    _need(u, "u", dt, device, (bsz, dim, L))
    _need(delta, "delta", dt, device, (bsz, dim, L))
    _need(A, "A", torch.float32, device, (dim, n))
    _need(B, "B", dt, device, (bsz, n, L))
    _need(C, "C", dt, device, (bsz, n, L))
    if z is not None:
        _need(z, "z", dt, device, (bsz, dim, L))
    if D is not None:
        _need(D, "D", torch.float32, device, (dim,))
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", torch.float32, device, (dim,))
    if y is None:
        y = torch.empty_like(u)
    else:
        _need(y, "y", dt, device, (bsz, dim, L))
    if last_state is not None:
        _need(last_state, "last_state", torch.float32, device, (bsz, dim, n))
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                      _ptr(delta_bias), int(bool(delta_softplus)), _ptr(y), _ptr(last_state),
                                      bsz, dim, n, L, SSM_F32 if dt == torch.float32 else SSM_BF16, _stream(device))
    _check(rc)
    return y, last_state


def ssm_scan_fwd_states(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                        C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                        delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                        h0: Optional[torch.Tensor] = None, state_chunk: int = 0, plan: str = "auto",
                        y: Optional[torch.Tensor] = None, last_state: Optional[torch.Tensor] = None,
                        chunk_states: Optional[torch.Tensor] = None):
    """Selective-scan forward from a start state h0 [b, d, n] (float32, or
    None for zero), also returning the states at every ``state_chunk`` steps
    (see ``ssm_scan_fwd_states`` in include/ssm_scan.h).

    Returns (y, last_state, chunk_states [b, ceil(L/state_chunk), d, n] or
    None when state_chunk is 0).
    """
    device = u.device
    if device.type != "cuda":
        raise ValueError("ssm_scan_fwd_states needs CUDA/HIP tensors")
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [b, d, L] and A [d, n]")
    bsz, dim, L = u.shape
    n = A.shape[1]
    dt = u.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    for t, name, shape in ((u, "u", (bsz, dim, L)), (delta, "delta", (bsz, dim, L)), (B, "B", (bsz, n, L)),
                           (C, "C", (bsz, n, L))):
        _need(t, name, dt, device, shape)
    _need(A, "A", torch.float32, device, (dim, n))
    if z is not None:
        _need(z, "z", dt, device, (bsz, dim, L))
    if D is not None:
        _need(D, "D", torch.float32, device, (dim,))
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", torch.float32, device, (dim,))
    if h0 is not None:
        _need(h0, "h0", torch.float32, device, (bsz, dim, n))
    if plan not in PLANS:
        raise ValueError(f"plan must be one of {list(PLANS)}")
    if state_chunk < 0:
        raise ValueError("state_chunk must be >= 0")
    if y is None:
        y = torch.empty_like(u)
    else:
        _need(y, "y", dt, device, (bsz, dim, L))
    if last_state is None:
        last_state = torch.empty((bsz, dim, n), device=device, dtype=torch.float32)
    else:
        _need(last_state, "last_state", torch.float32, device, (bsz, dim, n))
    if state_chunk > 0:
        K = -(-L // state_chunk)
        if chunk_states is None:
            chunk_states = torch.empty((bsz, K, dim, n), device=device, dtype=torch.float32)
        else:
            _need(chunk_states, "chunk_states", torch.float32, device, (bsz, K, dim, n))
    else:
        chunk_states = None
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_scan_fwd_states(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                     _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0), _ptr(y),
                                     _ptr(last_state), _ptr(chunk_states), int(state_chunk), bsz, dim, n, L,
                                     SSM_F32 if dt == torch.float32 else SSM_BF16, PLANS[plan], _stream(device))
    _check(rc)
    return y, last_state, chunk_states


def ssm_scan_fwd_conv(x: torch.Tensor, conv_w: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                      B: torch.Tensor, C: torch.Tensor, conv_b: Optional[torch.Tensor] = None,
                      D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                      delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                      h0: Optional[torch.Tensor] = None, state_chunk: int = 0, plan: str = "auto",
                      return_u: bool = False):
    """Selective scan with the causal depthwise conv1d + SiLU in front (see
    ``ssm_scan_fwd_conv`` in include/ssm_scan.h): u = silu(conv1d(x)) is
    computed in the kernel.  conv_w: [d, K] float32 (K = 1..4), conv_b: [d].

    Returns (y, last_state, chunk_states or None, u or None).
    """
    device = x.device
    if device.type != "cuda":
        raise ValueError("ssm_scan_fwd_conv needs CUDA/HIP tensors")
    if x.dim() != 3 or A.dim() != 2 or conv_w.dim() != 2:
        raise ValueError("x must be [b, d, L], A [d, n] and conv_w [d, K]")
    bsz, dim, L = x.shape
    n = A.shape[1]
    K = conv_w.shape[1]
    dt = x.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    for t, name, shape in ((x, "x", (bsz, dim, L)), (delta, "delta", (bsz, dim, L)), (B, "B", (bsz, n, L)),
                           (C, "C", (bsz, n, L))):
        _need(t, name, dt, device, shape)
    _need(A, "A", torch.float32, device, (dim, n))
    _need(conv_w, "conv_w", torch.float32, device, (dim, K))
    for t, name in ((conv_b, "conv_b"), (D, "D"), (delta_bias, "delta_bias")):
        if t is not None:
            _need(t, name, torch.float32, device, (dim,))
    if z is not None:
        _need(z, "z", dt, device, (bsz, dim, L))
    if h0 is not None:
        _need(h0, "h0", torch.float32, device, (bsz, dim, n))
    if plan not in PLANS:
        raise ValueError(f"plan must be one of {list(PLANS)}")
    y = torch.empty_like(x)
    last = torch.empty((bsz, dim, n), device=device, dtype=torch.float32)
    cs = (torch.empty((bsz, -(-L // state_chunk), dim, n), device=device, dtype=torch.float32)
          if state_chunk > 0 else None)
    u = torch.empty_like(x) if return_u else None
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_scan_fwd_conv(_ptr(x), _ptr(conv_w), _ptr(conv_b), int(K), _ptr(delta), _ptr(A), _ptr(B),
                                   _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0),
                                   _ptr(y), _ptr(last), _ptr(u), _ptr(cs), int(state_chunk), bsz, dim, n, L,
                                   SSM_F32 if dt == torch.float32 else SSM_BF16, PLANS[plan], _stream(device))
    _check(rc)
    return y, last, cs, u


def ssm_scan_bwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                 chunk_states: torch.Tensor, state_chunk: int, dy: torch.Tensor,
                 D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                 delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                 h0: Optional[torch.Tensor] = None, dlast: Optional[torch.Tensor] = None,
                 states_per_lane: int = 0, want_dD: bool = True, want_ddelta_bias: bool = True,
                 want_dh0: bool = True) -> dict:
    """Gradients of the selective scan (see ``ssm_scan_bwd`` in
    include/ssm_scan.h) from the chunk states that ``ssm_scan_fwd_states``
    wrote with the same inputs and ``state_chunk``.

    dy: gradient of y (dtype of u); dlast: gradient of last_state (float32,
    or None).  Returns a dict with du, ddelta, dz (dtype of u; dz None without
    z), dA [d, n], dB, dC [b, n, L] (float32), dD, ddelta_bias [d] and dh0
    [b, d, n] (float32; None where not asked for).
    """
    device = u.device
    if device.type != "cuda":
        raise ValueError("ssm_scan_bwd needs CUDA/HIP tensors")
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [b, d, L] and A [d, n]")
    bsz, dim, L = u.shape
    n = A.shape[1]
    dt = u.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    for t, name, shape in ((u, "u", (bsz, dim, L)), (delta, "delta", (bsz, dim, L)), (B, "B", (bsz, n, L)),
                           (C, "C", (bsz, n, L)), (dy, "dy", (bsz, dim, L))):
        _need(t, name, dt, device, shape)
    _need(A, "A", torch.float32, device, (dim, n))
    if state_chunk <= 0:
        raise ValueError("state_chunk must be positive")
    _need(chunk_states, "chunk_states", torch.float32, device, (bsz, -(-L // state_chunk), dim, n))
    if z is not None:
        _need(z, "z", dt, device, (bsz, dim, L))
    if D is not None:
        _need(D, "D", torch.float32, device, (dim,))
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", torch.float32, device, (dim,))
    if h0 is not None:
        _need(h0, "h0", torch.float32, device, (bsz, dim, n))
    if dlast is not None:
        _need(dlast, "dlast", torch.float32, device, (bsz, dim, n))
    f32 = dict(device=device, dtype=torch.float32)
    out = {
        "du": torch.empty_like(u), "ddelta": torch.empty_like(u),
        "dz": torch.empty_like(u) if z is not None else None,
        "dA": torch.empty((dim, n), **f32), "dB": torch.empty((bsz, n, L), **f32),
        "dC": torch.empty((bsz, n, L), **f32),
        "dD": torch.empty((dim,), **f32) if want_dD else None,
        "ddelta_bias": torch.empty((dim,), **f32) if want_ddelta_bias else None,
        "dh0": torch.empty((bsz, dim, n), **f32) if want_dh0 else None,
    }
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                              int(bool(delta_softplus)), _ptr(h0), _ptr(chunk_states), int(state_chunk), _ptr(dy),
                              _ptr(dlast), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
                              _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["ddelta_bias"]),
                              _ptr(out["dh0"]), bsz, dim, n, L, SSM_F32 if dt == torch.float32 else SSM_BF16,
                              int(states_per_lane), _stream(device))
    _check(rc)
    return out


def ssm_scan_bwd_conv(x: torch.Tensor, conv_w: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                      B: torch.Tensor, C: torch.Tensor, chunk_states: torch.Tensor, state_chunk: int,
                      dy: torch.Tensor, conv_b: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                      z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                      delta_softplus: bool = False, h0: Optional[torch.Tensor] = None,
                      dlast: Optional[torch.Tensor] = None, states_per_lane: int = 0) -> dict:
    """Gradients of ssm_scan_fwd_conv (see ``ssm_scan_bwd_conv`` in
    include/ssm_scan.h).  Returns a dict like ssm_scan_bwd with dx in place
    of du, plus dconv_w [d, K] and dconv_b [d] (float32; dconv_b None when
    conv_b is None)."""
    device = x.device
    if device.type != "cuda":
        raise ValueError("ssm_scan_bwd_conv needs CUDA/HIP tensors")
    bsz, dim, L = x.shape
    n = A.shape[1]
    K = conv_w.shape[1]
    dt = x.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    for t, name, shape in ((x, "x", (bsz, dim, L)), (delta, "delta", (bsz, dim, L)), (B, "B", (bsz, n, L)),
                           (C, "C", (bsz, n, L)), (dy, "dy", (bsz, dim, L))):
        _need(t, name, dt, device, shape)
    _need(A, "A", torch.float32, device, (dim, n))
    _need(conv_w, "conv_w", torch.float32, device, (dim, K))
    if state_chunk <= 0:
        raise ValueError("state_chunk must be positive")
    _need(chunk_states, "chunk_states", torch.float32, device, (bsz, -(-L // state_chunk), dim, n))
    for t, name in ((conv_b, "conv_b"), (D, "D"), (delta_bias, "delta_bias")):
        if t is not None:
            _need(t, name, torch.float32, device, (dim,))
    if z is not None:
        _need(z, "z", dt, device, (bsz, dim, L))
    for t, name in ((h0, "h0"), (dlast, "dlast")):
        if t is not None:
            _need(t, name, torch.float32, device, (bsz, dim, n))
    f32 = dict(device=device, dtype=torch.float32)
    out = {
        "dx": torch.empty_like(x), "ddelta": torch.empty_like(x),
        "dz": torch.empty_like(x) if z is not None else None,
        "dconv_w": torch.empty((dim, K), **f32),
        "dconv_b": torch.empty((dim,), **f32) if conv_b is not None else None,
        "dA": torch.empty((dim, n), **f32), "dB": torch.empty((bsz, n, L), **f32),
        "dC": torch.empty((bsz, n, L), **f32), "dD": torch.empty((dim,), **f32),
        "ddelta_bias": torch.empty((dim,), **f32), "dh0": torch.empty((bsz, dim, n), **f32),
    }
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_scan_bwd_conv(_ptr(x), _ptr(conv_w), _ptr(conv_b), int(K), _ptr(delta), _ptr(A), _ptr(B),
                                   _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(h0),
                                   _ptr(chunk_states), int(state_chunk), _ptr(dy), _ptr(dlast), _ptr(out["dx"]),
                                   _ptr(out["dconv_w"]), _ptr(out["dconv_b"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
                                   _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
                                   _ptr(out["ddelta_bias"]), _ptr(out["dh0"]), bsz, dim, n, L,
                                   SSM_F32 if dt == torch.float32 else SSM_BF16, int(states_per_lane),
                                   _stream(device))
    _check(rc)
    return out


def ssm_step(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
             state: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
             delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
             state_out: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None):
    """One recurrent step (see ``ssm_step`` in include/ssm_scan.h).

    u, delta, z: [b, d]; B, C: [b, n]; A: [d, n] float32; state: [b, d, n]
    float32.  The new state goes to ``state_out`` (default: ``state`` itself,
    updated in place).  Returns (y [b, d], state_out).
    """
    device = u.device
    if device.type != "cuda":
        raise ValueError("ssm_step needs CUDA/HIP tensors")
    if u.dim() != 2 or A.dim() != 2:
        raise ValueError("u must be [b, d] and A [d, n]")
    bsz, dim = u.shape
    n = A.shape[1]
    dt = u.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    _need(u, "u", dt, device, (bsz, dim))
    _need(delta, "delta", dt, device, (bsz, dim))
    _need(A, "A", torch.float32, device, (dim, n))
    _need(B, "B", dt, device, (bsz, n))
    _need(C, "C", dt, device, (bsz, n))
    _need(state, "state", torch.float32, device, (bsz, dim, n))
    if z is not None:
        _need(z, "z", dt, device, (bsz, dim))
    if D is not None:
        _need(D, "D", torch.float32, device, (dim,))
    if delta_bias is not None:
        _need(delta_bias, "delta_bias", torch.float32, device, (dim,))
    if state_out is None:
        state_out = state
    else:
        _need(state_out, "state_out", torch.float32, device, (bsz, dim, n))
    if y is None:
        y = torch.empty_like(u)
    else:
        _need(y, "y", dt, device, (bsz, dim))
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_step(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                          int(bool(delta_softplus)), _ptr(state), _ptr(state_out), _ptr(y), bsz, dim, n,
                          SSM_F32 if dt == torch.float32 else SSM_BF16, _stream(device))
    _check(rc)
    return y, state_out


def ssm_step_conv(x: torch.Tensor, conv_w: torch.Tensor, conv_state: Optional[torch.Tensor], delta: torch.Tensor,
                  A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, state: torch.Tensor,
                  conv_b: Optional[torch.Tensor] = None, D: Optional[torch.Tensor] = None,
                  z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                  delta_softplus: bool = False, conv_state_out: Optional[torch.Tensor] = None,
                  state_out: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                  return_u: bool = False):
    """One decode step with the causal conv1d + SiLU in front (see
    ``ssm_step_conv`` in include/ssm_scan.h).  conv_state: [b, d, K-1]
    float32 (None when K = 1), updated in place unless conv_state_out is
    given; state likewise.  Returns (y, conv_state_out, state_out, u or None).
    """
    device = x.device
    if device.type != "cuda":
        raise ValueError("ssm_step_conv needs CUDA/HIP tensors")
    bsz, dim = x.shape
    n = A.shape[1]
    K = conv_w.shape[1]
    dt = x.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    for t, name, shape in ((x, "x", (bsz, dim)), (delta, "delta", (bsz, dim)), (B, "B", (bsz, n)),
                           (C, "C", (bsz, n))):
        _need(t, name, dt, device, shape)
    _need(A, "A", torch.float32, device, (dim, n))
    _need(conv_w, "conv_w", torch.float32, device, (dim, K))
    _need(state, "state", torch.float32, device, (bsz, dim, n))
    if K > 1:
        _need(conv_state, "conv_state", torch.float32, device, (bsz, dim, K - 1))
    for t, name in ((conv_b, "conv_b"), (D, "D"), (delta_bias, "delta_bias")):
        if t is not None:
            _need(t, name, torch.float32, device, (dim,))
    if z is not None:
        _need(z, "z", dt, device, (bsz, dim))
    if conv_state_out is None:
        conv_state_out = conv_state
    if state_out is None:
        state_out = state
    if y is None:
        y = torch.empty_like(x)
    u = torch.empty_like(x) if return_u else None
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_step_conv(_ptr(x), _ptr(conv_w), _ptr(conv_b), int(K), _ptr(conv_state if K > 1 else None),
                               _ptr(conv_state_out if K > 1 else None), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                               _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(delta_softplus)), _ptr(state),
                               _ptr(state_out), _ptr(y), _ptr(u), bsz, dim, n,
                               SSM_F32 if dt == torch.float32 else SSM_BF16, _stream(device))
    _check(rc)
    return y, conv_state_out, state_out, u


def ssm_out_proj(y: torch.Tensor, W: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Linear projection after the gated scan (see ``ssm_out_proj`` in
    include/ssm_scan.h): out[b, t, m] = sum_k W[m, k] * y[b, k, t].

    y: [b, d_inner, L] (the scan's output), W: [d_model, d_inner], both
    float32 or both bfloat16.  Returns out [b, L, d_model] in their dtype."""
    device = y.device
    if device.type != "cuda":
        raise ValueError("ssm_out_proj needs CUDA/HIP tensors")
    if y.dim() != 3 or W.dim() != 2:
        raise ValueError("y must be [b, d_inner, L] and W [d_model, d_inner]")
    bsz, dk, L = y.shape
    dm = W.shape[0]
    dt = y.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("y must be float32 or bfloat16")
    _need(y, "y", dt, device, (bsz, dk, L))
    _need(W, "W", dt, device, (dm, dk))
    if out is None:
        out = torch.empty((bsz, L, dm), device=device, dtype=dt)
    else:
        _need(out, "out", dt, device, (bsz, L, dm))
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_out_proj(_ptr(y), _ptr(W), _ptr(out), bsz, dk, dm, L,
                              SSM_F32 if dt == torch.float32 else SSM_BF16, _stream(device))
    _check(rc)
    return out


def ssm_out_proj_bwd(y: torch.Tensor, W: torch.Tensor, dout: torch.Tensor, want_dy: bool = True,
                     want_dW: bool = True) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Gradients of ssm_out_proj (see ``ssm_out_proj_bwd`` in
    include/ssm_scan.h) for dout [b, L, d_model]: returns (dy [b, d_inner, L]
    or None, dW [d_model, d_inner] or None), in the dtype of y."""
    device = y.device
    if device.type != "cuda":
        raise ValueError("ssm_out_proj_bwd needs CUDA/HIP tensors")
    if y.dim() != 3 or W.dim() != 2 or dout.dim() != 3:
        raise ValueError("y must be [b, d_inner, L], W [d_model, d_inner] and dout [b, L, d_model]")
    if not (want_dy or want_dW):
        raise ValueError("ask for dy, dW or both")
    bsz, dk, L = y.shape
    dm = W.shape[0]
    dt = y.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("y must be float32 or bfloat16")
    _need(y, "y", dt, device, (bsz, dk, L))
    _need(W, "W", dt, device, (dm, dk))
    _need(dout, "dout", dt, device, (bsz, L, dm))
    dy = torch.empty_like(y) if want_dy else None
    dW = torch.empty_like(W) if want_dW else None
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.ssm_out_proj_bwd(_ptr(y), _ptr(W), _ptr(dout), _ptr(dy), _ptr(dW), bsz, dk, dm, L,
                                  SSM_F32 if dt == torch.float32 else SSM_BF16, _stream(device))
    _check(rc)
    return dy, dW


def affine_scan(a: torch.Tensor, b: torch.Tensor, return_a: bool = True,
                out_a: Optional[torch.Tensor] = None,
                out_b: Optional[torch.Tensor] = None) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """Inclusive scan of affine pairs along the last axis of [rows, L] float32
    tensors (see ``affine_scan`` in include/ssm_scan.h).  Returns (out_a or
    None, out_b).  out_a / out_b may be given, including a / b themselves."""
    device = a.device
    if device.type != "cuda":
        raise ValueError("affine_scan needs CUDA/HIP tensors")
    if a.dim() != 2:
        raise ValueError("a must be [rows, L]")
    rows, L = a.shape
    _need(a, "a", torch.float32, device, (rows, L))
    _need(b, "b", torch.float32, device, (rows, L))
    if out_b is None:
        out_b = torch.empty_like(b)
    else:
        _need(out_b, "out_b", torch.float32, device, (rows, L))
    if return_a and out_a is None:
        out_a = torch.empty_like(a)
    elif out_a is not None:
        _need(out_a, "out_a", torch.float32, device, (rows, L))
    lib = load_library()
    with torch.cuda.device(device):
        rc = lib.affine_scan(_ptr(a), _ptr(b), _ptr(out_a), _ptr(out_b), rows, L, _stream(device))
    _check(rc)
    return out_a, out_b


def affine_scan_order() -> dict:
    """Constants of affine_scan's association order (host only)."""
    lib = load_library()
    vals = [ctypes.c_int() for _ in range(4)]
    _check(lib.affine_scan_order(*[ctypes.byref(v) for v in vals]))
    return dict(zip(("items_per_lane", "lanes", "waves", "chunk"), (v.value for v in vals)))


def plan_for(batch: int, d_inner: int, d_state: int, L: int, dtype=torch.float32) -> dict:
    """The plan the library's automatic choice takes for a size (host only)."""
    lib = load_library()
    pl, s = ctypes.c_int(), ctypes.c_int()
    ch = ctypes.c_int64()
    code = SSM_F32 if dtype in (torch.float32, "f32") else SSM_BF16
    _check(lib.ssm_scan_plan_for(batch, d_inner, d_state, L, code, ctypes.byref(pl), ctypes.byref(s),
                                 ctypes.byref(ch)))
    return {"plan": _PLAN_NAMES[pl.value], "states_per_lane": s.value, "chunk": ch.value}
