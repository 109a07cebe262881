"""CPU oracle for the selective-scan forward pass and the affine-pair scan.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code, constants or helpers with the
HIP library; the only thing both sides see is the seeded input tensors.

Everything here is plain, slow and written to be checked by eye against the
pages it cites.  Floating point is float64 unless a function says otherwise;
inputs in narrower types are upcast exactly before any arithmetic.

Pages cited (by title, then section / equation / table):

* [Scan page]   "Hardware-aware parallel associative scan for Mamba"
                (http://www.pwwt.cn/news/6375169/)
* [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
                optimisation" (https://scwacadex.pages.dev/posts/blog8_mamba_parallel_scan/)
* [Truth page]  "The hardware truth of Mamba's parallel scan"
                (http://www.sheratonhq.com/news/137962)

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):

* A is a real diagonal per (channel, state): a_t = exp(delta_t * A[d, n])
  ([Scan page] §1.2, last paragraph).  The Truth page's dense d x d A is not
  used.
* b_t = delta_t * B_t * x_t, the Euler-style input term the Scan page states
  in §1.2 (not the exact zero-order-hold integral).
* B and C are per time step and shared by every channel of a batch row.
* The optional D skip adds D[d] * u_t to C_t . h_t; the optional gate
  multiplies that sum by silu(z_t).
* delta_bias is added to delta before the optional softplus.
* The initial state h_0 is zero unless an explicit h0 is given.

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
except where its docstring says "parity unpinned".
"""
from __future__ import annotations

from fractions import Fraction
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "IDENTITY",
    "compose",
    "scan_serial",
    "scan_hillis_steele",
    "scan_blelloch",
    "scan_chunked_two_pass",
    "softplus",
    "silu",
    "selective_scan_fwd",
    "selective_scan_bruteforce",
    "selective_scan_bwd",
    "causal_conv1d",
    "causal_conv1d_silu_bwd",
    "out_proj",
    "out_proj_tokens",
    "out_proj_bwd",
    "affine_scan",
    "lti_closed_form",
]

# The identity element of the affine-pair monoid ([Scan page] §1.2): the map
# h -> 1*h + 0 leaves every state unchanged.
IDENTITY = (1, 0)


# --------------------------------------------------------------------------
# The monoid of affine pairs
# --------------------------------------------------------------------------

def compose(p2, p1):
    """Composition of two affine steps, later step on the left.

    A pair (a, b) stands for the map h -> a*h + b ([Scan page] §1.2;
    [Mamba-2 page] §2.1).  Applying p1 first and p2 second gives
    a2*(a1*h + b1) + b2 = (a2*a1)*h + (a2*b1 + b2), so
    (a2, b2) o (a1, b1) = (a2*a1, a2*b1 + b2)   ([Mamba-2 page] §2.2).

    Works elementwise on scalars, Fractions or numpy arrays.
    """
    a2, b2 = p2
    a1, b1 = p1
    return (a2 * a1, a2 * b1 + b2)


def _as_pairs(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        raise ValueError("a and b must have the same shape")
    return a, b


def scan_serial(a, b):
    """Inclusive prefix compositions along the last axis, left to right.

    Output (A_t, B_t) = (a_t, b_t) o ... o (a_1, b_1), so that
    h_t = A_t * h_0 + B_t for any start state h_0 ([Scan page] §2.1).
    Object arrays of Fractions are supported for exact checks.
    """
    a, b = _as_pairs(a, b)
    outA = np.empty_like(a)
    outB = np.empty_like(b)
    accA = None
    accB = None
    for t in range(a.shape[-1]):
        if t == 0:
            accA, accB = a[..., 0], b[..., 0]
        else:
            accA, accB = compose((a[..., t], b[..., t]), (accA, accB))
        outA[..., t] = accA
        outB[..., t] = accB
    return outA, outB


def _identity_like(x):
    if x.dtype == object:
        return (np.full(x.shape, Fraction(1), dtype=object),
                np.full(x.shape, Fraction(0), dtype=object))
    return np.ones_like(x), np.zeros_like(x)


def scan_hillis_steele(a, b):
    """Hillis-Steele inclusive scan ([Scan page] §2.1).

    Round d = 1, 2, 4, ...: every position i >= d becomes
    (a[i], b[i]) o (a[i-d], b[i-d]) using the values of the previous round
    (double buffering), ceil(log2 L) rounds in total.
    """
    a, b = _as_pairs(a, b)
    cur_a = a.copy()
    cur_b = b.copy()
    L = a.shape[-1]
    d = 1
    while d < L:
        nxt_a = cur_a.copy()
        nxt_b = cur_b.copy()
        for i in range(d, L):
            nxt_a[..., i], nxt_b[..., i] = compose(
                (cur_a[..., i], cur_b[..., i]), (cur_a[..., i - d], cur_b[..., i - d]))
        cur_a, cur_b = nxt_a, nxt_b
        d *= 2
    return cur_a, cur_b


def scan_blelloch(a, b):
    """Work-efficient (Blelloch) scan: up-sweep, then down-sweep.

    [Scan page] §2.1 describes the two sweeps and suggests padding the front
    of the sequence with identities (1, 0) up to a power of two so the tree is
    regular.  The down-sweep yields exclusive prefixes; the inclusive result
    is the exclusive prefix composed with the element itself.
    """
    a, b = _as_pairs(a, b)
    L = a.shape[-1]
    if L == 0:
        return a.copy(), b.copy()
    n = 1
    while n < L:
        n *= 2
    pad = n - L
    one, zero = _identity_like(a[..., :1])
    ta = np.concatenate([np.repeat(one, pad, axis=-1), a], axis=-1) if pad else a.copy()
    tb = np.concatenate([np.repeat(zero, pad, axis=-1), b], axis=-1) if pad else b.copy()
    ta = ta.copy()
    tb = tb.copy()
    # Up-sweep: node at the right end of each block of width 2*s accumulates
    # its left sibling (earlier elements are on the right of the operator).
    s = 1
    while s < n:
        for r in range(2 * s - 1, n, 2 * s):
            l = r - s
            ta[..., r], tb[..., r] = compose((ta[..., r], tb[..., r]), (ta[..., l], tb[..., l]))
        s *= 2
    # Down-sweep for exclusive prefixes: root gets the identity.
    ta[..., n - 1] = one[..., 0]
    tb[..., n - 1] = zero[..., 0]
    s = n // 2
    while s >= 1:
        for r in range(2 * s - 1, n, 2 * s):
            l = r - s
            left_a, left_b = ta[..., l].copy(), tb[..., l].copy()
            # left child receives the parent's prefix; right child receives
            # (left subtree total) applied after the parent's prefix.
            ta[..., l], tb[..., l] = ta[..., r], tb[..., r]
            ta[..., r], tb[..., r] = compose((left_a, left_b), (ta[..., r], tb[..., r]))
        s //= 2
    excl_a = ta[..., pad:]
    excl_b = tb[..., pad:]
    inc_a, inc_b = compose((a, b), (excl_a, excl_b))
    return inc_a, inc_b


def scan_chunked_two_pass(a, b, chunk: int, h0=None):
    """Chunked two-pass scan with the fix-up of [Scan page] §2.2 and §3.3.

    Pass 1 scans each chunk of ``chunk`` steps from the identity, giving
    local prefixes and the chunk total (A_tot^(k), B_tot^(k)).  Pass 2 runs
    the recurrence over chunk totals:
        h_init^(0) = h0,
        h_init^(k) = A_tot^(k-1) * h_init^(k-1) + B_tot^(k-1).
    Pass 3 fixes up every position: h_t = A_loc_t * h_init^(k) + B_loc_t.

    Returns (h, boundary) where h[..., t] is the state after step t and
    boundary[..., k] = h_init^(k) for k = 0..K (boundary[..., K] is the final
    state), i.e. the chunk-boundary states the Mamba-2 page §4.3 keeps for
    recomputation.
    """
    a, b = _as_pairs(a, b)
    L = a.shape[-1]
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    K = (L + chunk - 1) // chunk
    if h0 is None:
        h0 = np.zeros(a.shape[:-1], dtype=b.dtype)
        if b.dtype == object:
            h0 = np.full(a.shape[:-1], Fraction(0), dtype=object)
    locA = np.empty_like(a)
    locB = np.empty_like(b)
    totals = []
    for k in range(K):
        s, e = k * chunk, min(L, (k + 1) * chunk)
        la, lb = scan_serial(a[..., s:e], b[..., s:e])
        locA[..., s:e] = la
        locB[..., s:e] = lb
        totals.append((np.asarray(la[..., -1]), np.asarray(lb[..., -1])))
    boundary = [np.asarray(h0)]
    for k in range(K):
        tot_a, tot_b = totals[k]
        boundary.append(np.asarray(tot_a * boundary[k] + tot_b))
    h = np.empty_like(b)
    for k in range(K):
        s, e = k * chunk, min(L, (k + 1) * chunk)
        h[..., s:e] = locA[..., s:e] * boundary[k][..., None] + locB[..., s:e]
    return h, np.stack(boundary, axis=-1)


# --------------------------------------------------------------------------
# Elementwise functions
# --------------------------------------------------------------------------

def softplus(x):
    """softplus(x) = log(1 + e^x), in the overflow-safe form
    max(x, 0) + log1p(exp(-|x|)).  [Scan page] §1.2 uses softplus to keep the
    step size delta positive.
    """
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z), the gate nonlinearity the
    Mamba-2 page §4.1 names.  Written as z * (1 / (1 + e^-z)) in float64;
    e^-z overflows to inf for z < -709 and the quotient then is -0.0, which
    is the correct limit."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# Selective scan forward
# --------------------------------------------------------------------------

def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: upcast exactly on the CPU
        x = x.detach().to("cpu")
        import torch  # local import: the oracle itself does not need torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def selective_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       delta_softplus=False, h0=None, chunk: Optional[int] = None):
    """Plain definition of the selective-scan forward pass, float64.

    Shapes: u, delta, z: [b, d, L]; A: [d, n]; B, C: [b, n, L]; D,
    delta_bias: [d]; h0: [b, d, n].  For every batch row b, channel d and
    step t, with h starting at h0 (zero by default):

        x      = delta[b,d,t] + delta_bias[d]
        Delta  = softplus(x) if delta_softplus else x
        a      = exp(Delta * A[d,n])                 ([Scan page] §1.2)
        bb     = Delta * B[b,n,t] * u[b,d,t]         ([Scan page] §1.2)
        h[n]   = a * h[n] + bb                       ([Scan page] §1, eq. of h_t)
        y      = sum_n C[b,n,t] * h[n] + D[d]*u       (output eq. of h_t, D skip)
        y     *= silu(z[b,d,t]) if z is given         ([Mamba-2 page] §4.1 gate)

    Returns (y [b,d,L], last_state [b,d,n]); with ``chunk`` also the states at
    every chunk boundary, [b, d, n, K+1] (h_0, h_chunk, h_2chunk, ..., h_L),
    the checkpoint set of the Mamba-2 page §4.3.

    The loop is over t only; channels and states are vectorised, which does
    not change any arithmetic (each element is an independent recurrence).
    """
    u = _f64(u)
    delta = _f64(delta)
    A = _f64(A)
    B = _f64(B)
    C = _f64(C)
    D = _f64(D)
    z = _f64(z)
    delta_bias = _f64(delta_bias)
    bsz, dim, L = u.shape
    n = A.shape[1]
    if delta.shape != u.shape or A.shape != (dim, n) or B.shape != (bsz, n, L) or C.shape != (bsz, n, L):
        raise ValueError("inconsistent shapes")
    x = delta + (delta_bias[None, :, None] if delta_bias is not None else 0.0)
    dt = softplus(x) if delta_softplus else x
    h = np.zeros((bsz, dim, n)) if h0 is None else _f64(h0).copy()
    y = np.empty((bsz, dim, L))
    bounds = [h.copy()] if chunk else None
    for t in range(L):
        a = np.exp(dt[:, :, t, None] * A[None, :, :])                 # [b,d,n]
        bb = dt[:, :, t, None] * B[:, None, :, t] * u[:, :, t, None]  # [b,d,n]
        h = a * h + bb
        yt = np.einsum("bdn,bn->bd", h, C[:, :, t])
        if D is not None:
            yt = yt + D[None, :] * u[:, :, t]
        if z is not None:
            yt = yt * silu(z[:, :, t])
        y[:, :, t] = yt
        if chunk and ((t + 1) % chunk == 0 or t + 1 == L):
            bounds.append(h.copy())
    if chunk:
        return y, h, np.stack(bounds, axis=-1)
    return y, h


def selective_scan_bruteforce(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                              delta_softplus=False):
    """Independent closed expansion of the same recurrence, for tiny L.

    Unrolling h_t = a_t h_{t-1} + b_t from h_0 = 0 gives
        h_t[n] = sum_{j<=t} exp(A[d,n] * sum_{j<s<=t} Delta_s) * Delta_j B_j[n] u_j,
    i.e. each input is carried forward by the product of the later decays,
    written here as one exponential of a sum (a different rounding path from
    the step-by-step loop).  Pure Python loops: use only for L <= ~16.
    """
    u = _f64(u); delta = _f64(delta); A = _f64(A); B = _f64(B); C = _f64(C)
    D = _f64(D); z = _f64(z); delta_bias = _f64(delta_bias)
    bsz, dim, L = u.shape
    n = A.shape[1]
    y = np.zeros((bsz, dim, L))
    last = np.zeros((bsz, dim, n))
    for bi in range(bsz):
        for di in range(dim):
            x = delta[bi, di] + (delta_bias[di] if delta_bias is not None else 0.0)
            dt = softplus(x) if delta_softplus else x
            for t in range(L):
                acc = 0.0
                for k in range(n):
                    hk = 0.0
                    for j in range(t + 1):
                        decay = float(np.exp(A[di, k] * float(np.sum(dt[j + 1:t + 1]))))
                        hk += decay * dt[j] * B[bi, k, j] * u[bi, di, j]
                    acc += C[bi, k, t] * hk
                    if t == L - 1:
                        last[bi, di, k] = hk
                if D is not None:
                    acc += D[di] * u[bi, di, t]
                if z is not None:
                    acc *= float(silu(z[bi, di, t]))
                y[bi, di, t] = acc
    return y, last


def selective_scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                       delta_softplus=False, h0=None, dy=None, dlast=None):
    """Gradients of the selective scan, float64, by reverse-mode chain rule.

    The forward pass is the one of ``selective_scan_fwd``; the loss is
    sum(dy * y) + sum(dlast * last_state), i.e. dy and dlast are the incoming
    gradients of y [b,d,L] and of the final state [b,d,n] (either may be
    None: zero).  The states h_t are kept for every step (this is the plain
    definition; the chunked recomputation of [Scan page] §4.2 and the
    Mamba-2 page §4.3 reaches the same values with only chunk-boundary
    states stored).

    With s_t the sum before the gate (s_t = C_t . h_t + D u_t, y_t = s_t *
    silu(z_t)) and g_t = dL/dh_t:

        gs_t   = dy_t * silu(z_t)                (dy_t without a gate)
        dz_t   = dy_t * s_t * silu'(z_t),  silu'(z) = sig(z) (1 + z (1 - sig(z)))
        g_t    = C_t gs_t + a_{t+1} g_{t+1},  starting from g_L = dlast
        dC_t  += gs_t h_t                        (summed over channels d)
        dB_t  += g_t Delta_t u_t                 (summed over channels d)
        du_t   = D gs_t + Delta_t sum_n g_t B_t
        dDelta = sum_n g_t (A a_t h_{t-1} + B_t u_t)
        dA    += g_t a_t h_{t-1} Delta_t         (summed over b and t)
        dD    += gs_t u_t                        (summed over b and t)
        dx_t   = dDelta_t * sig(x_t) with softplus (softplus' = sigmoid),
                 else dDelta_t;  ddelta_t = dx_t,  ddelta_bias += dx_t
        dh0    = a_0 g_0

    where h_{-1} is h0 (zero by default).  Returns a dict with keys du,
    ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0 (dz None without a gate;
    dD and ddelta_bias are computed whether or not D and delta_bias are
    given, as the gradients at zero).
    """
    u = _f64(u); delta = _f64(delta); A = _f64(A); B = _f64(B); C = _f64(C)
    D = _f64(D); z = _f64(z); delta_bias = _f64(delta_bias)
    bsz, dim, L = u.shape
    n = A.shape[1]
    dy = np.zeros((bsz, dim, L)) if dy is None else _f64(dy)
    dlast = np.zeros((bsz, dim, n)) if dlast is None else _f64(dlast)
    x = delta + (delta_bias[None, :, None] if delta_bias is not None else 0.0)
    dt = softplus(x) if delta_softplus else x
    Dv = np.zeros(dim) if D is None else D
    # forward, keeping every state: hs[t+1] = h_t, hs[0] = h0
    hs = np.empty((L + 1, bsz, dim, n))
    hs[0] = 0.0 if h0 is None else _f64(h0)
    aa = np.empty((L, bsz, dim, n))
    s = np.empty((bsz, dim, L))
    for t in range(L):
        aa[t] = np.exp(dt[:, :, t, None] * A[None, :, :])
        bb = dt[:, :, t, None] * B[:, None, :, t] * u[:, :, t, None]
        hs[t + 1] = aa[t] * hs[t] + bb
        s[:, :, t] = np.einsum("bdn,bn->bd", hs[t + 1], C[:, :, t]) + Dv[None, :] * u[:, :, t]
    if z is not None:
        sig = 1.0 / (1.0 + np.exp(-z))
        gs = dy * z * sig
        dz = dy * s * sig * (1.0 + z * (1.0 - sig))
    else:
        gs = dy
        dz = None
    du = np.empty((bsz, dim, L))
    ddt = np.empty((bsz, dim, L))
    dA = np.zeros((dim, n))
    dB = np.zeros((bsz, n, L))
    dC = np.zeros((bsz, n, L))
    g = dlast.copy()
    a_next = np.ones((bsz, dim, n))
    for t in range(L - 1, -1, -1):
        g = C[:, None, :, t] * gs[:, :, t, None] + a_next * g
        h_prev = hs[t]
        dC[:, :, t] = np.einsum("bd,bdn->bn", gs[:, :, t], hs[t + 1])
        dB[:, :, t] = np.einsum("bdn,bd->bn", g, dt[:, :, t] * u[:, :, t])
        du[:, :, t] = Dv[None, :] * gs[:, :, t] + dt[:, :, t] * np.einsum("bdn,bn->bd", g, B[:, :, t])
        ga = g * aa[t] * h_prev
        ddt[:, :, t] = np.einsum("bdn,dn->bd", ga, A) + u[:, :, t] * np.einsum("bdn,bn->bd", g, B[:, :, t])
        dA += np.einsum("bdn,bd->dn", ga, dt[:, :, t])
        a_next = aa[t]
    dh0 = aa[0] * g if L > 0 else g
    dD = np.einsum("bdl,bdl->d", gs, u)
    dx = ddt * (1.0 / (1.0 + np.exp(-x))) if delta_softplus else ddt
    return {"du": du, "ddelta": dx, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "dz": dz,
            "ddelta_bias": dx.sum(axis=(0, 2)), "dh0": dh0}


def causal_conv1d(x, w, b=None, activation: Optional[str] = "silu"):
    """Depthwise causal 1-D convolution of every channel, float64, then the
    activation (SiLU by default, None for none): the Conv1D in front of the
    SSM in the Mamba block ([Mamba-2 page] §4.1 names Conv1D and SiLU among
    the fused operators).  The pages give no formula; the reading taken is
    the usual causal one with K-1 steps of zero left padding:

        out[b,d,t] = b[d] + sum_{k=0}^{K-1} w[d,k] * x[b,d,t-(K-1)+k],

    x at steps below 0 being zero, so w[d, K-1] multiplies the current step.
    x: [b, d, L]; w: [d, K]; b: [d] or None.
    """
    x = _f64(x)
    w = _f64(w)
    bsz, dim, L = x.shape
    K = w.shape[1]
    out = np.zeros((bsz, dim, L)) if b is None else np.broadcast_to(_f64(b)[None, :, None], (bsz, dim, L)).copy()
    for k in range(K):
        shift = K - 1 - k              # w[:, k] multiplies x[t - shift]
        if shift >= L:
            continue
        out[:, :, shift:] += w[None, :, k, None] * x[:, :, :L - shift]
    if activation == "silu":
        out = silu(out)
    elif activation is not None:
        raise ValueError("activation must be 'silu' or None")
    return out


def causal_conv1d_silu_bwd(x, w, b, du):
    """Gradients through u = silu(causal_conv1d(x, w, b)) (the reading of
    ``causal_conv1d``), float64, for an incoming gradient du of u:

        pre_t   = b + sum_k w[k] x_{t-(K-1)+k}
        dpre_t  = du_t * silu'(pre_t),  silu'(p) = sig(p) (1 + p (1 - sig(p)))
        dx_t    = sum_k w[k] dpre_{t+(K-1)-k}      (terms past the end are zero)
        dw[d,k] = sum_{b,t} dpre_t x_{t-(K-1)+k},  db[d] = sum_{b,t} dpre_t

    Returns (dx [b,d,L], dw [d,K], db [d])."""
    x = _f64(x)
    w = _f64(w)
    du = _f64(du)
    bsz, dim, L = x.shape
    K = w.shape[1]
    pre = causal_conv1d(x, w, b, activation=None)
    sig = 1.0 / (1.0 + np.exp(-pre))
    dpre = du * sig * (1.0 + pre * (1.0 - sig))
    dx = np.zeros_like(x)
    dw = np.zeros((dim, K))
    for k in range(K):
        shift = K - 1 - k                 # w[:, k] multiplies x[t - shift]
        if shift >= L:
            continue
        dx[:, :, :L - shift] += w[None, :, k, None] * dpre[:, :, shift:]
        dw[:, k] = np.einsum("bdl,bdl->d", dpre[:, :, shift:], x[:, :, :L - shift])
    return dx, dw, dpre.sum(axis=(0, 2))


def out_proj(y, W):
    """The Linear projection that closes the Mamba block after the gated
    scan ([Mamba-2 page] §4.1 lists it last in the fused chain: Conv1D, SSM,
    SiLU gate, Linear).  The pages give no shapes; the reading taken is the
    usual Linear on every token's d_inner vector, with the weight stored
    [d_model, d_inner], applied to y in the scan's [b, d_inner, L] layout and
    written token-major:

        out[b, t, m] = sum_k W[m, k] * y[b, k, t]

    float64, one library matrix product per batch row.  Returns
    [b, L, d_model]."""
    y = _f64(y)
    W = _f64(W)
    out = np.empty((y.shape[0], y.shape[2], W.shape[0]))
    for b in range(y.shape[0]):
        out[b] = (W @ y[b]).T
    return out


def out_proj_tokens(y, W, bt):
    """``out_proj`` for a list of (batch row, step) pairs only: row i of the
    result is out[bt[i][0], bt[i][1], :] (the same definition, for sampled
    outputs of large problems)."""
    y = _f64(y) if isinstance(y, np.ndarray) else y
    W = _f64(W)
    cols = np.stack([_f64(y[b, :, t]) for b, t in bt])     # [n, d_inner]
    return cols @ W.T


def out_proj_bwd(y, W, dout):
    """Gradients of ``out_proj`` for an incoming gradient dout [b, L, d_model]
    of its output, float64 (the chain rule of a linear map, one library
    matrix product per term):

        dy[b, k, t] = sum_m W[m, k] * dout[b, t, m]
        dW[m, k]    = sum_{b, t} dout[b, t, m] * y[b, k, t]

    Returns (dy [b, d_inner, L], dW [d_model, d_inner])."""
    y = _f64(y)
    W = _f64(W)
    dout = _f64(dout)
    dy = np.empty_like(y)
    dW = np.zeros_like(W)
    for b in range(y.shape[0]):
        dy[b] = W.T @ dout[b].T
        dW += dout[b].T @ y[b].T
    return dy, dW


def lti_closed_form(a: float, b):
    """Closed form for a constant decay a (constant Delta and A):
    h_t = sum_{j<=t} a^(t-j) b_j, the causal kernel with weights a^(i-j) that
    the Truth page §1 writes for the time-invariant case.  Evaluated as a
    dense lower-triangular matrix product, float64."""
    b = _f64(b)
    L = b.shape[-1]
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    expo = (i - j).astype(np.float64)
    K = np.where(i >= j, np.power(float(a), np.maximum(expo, 0.0)), 0.0)
    return b @ K.T


# --------------------------------------------------------------------------
# Bare affine scan
# --------------------------------------------------------------------------

def affine_scan(a, b):
    """Serial float64 left fold over each row of a, b ([rows, L]).

    out_a[t] = a_t * out_a[t-1], out_b[t] = a_t * out_b[t-1] + b_t starting
    from the identity (1, 0), i.e. the inclusive prefix compositions of
    [Scan page] §2.1 with h_0 = 0.
    """
    a = _f64(a)
    b = _f64(b)
    out_a = np.empty_like(a)
    out_b = np.empty_like(b)
    pa = np.ones(a.shape[:-1])
    pb = np.zeros(a.shape[:-1])
    for t in range(a.shape[-1]):
        pa = a[..., t] * pa
        pb = a[..., t] * pb + b[..., t]
        out_a[..., t] = pa
        out_b[..., t] = pb
    return out_a, out_b
