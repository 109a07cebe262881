"""Pins of the gradient oracle (oracle.ref.selective_scan_bwd and the C
oracle's ssm_oracle_bwd) against things other than itself:

* central finite differences of the forward oracle (float64), element by
  element for every input that has a gradient;
* reverse-mode automatic differentiation (torch.autograd, float64, CPU) of a
  plain transcription of the forward recurrence of [Scan page] §1.2;
* the closed form at L = 1 with a zero start state, where h = Delta B u and
  every gradient is a short product;
* agreement of the C oracle with the NumPy one;
* for the causal conv1d + SiLU in front (oracle.ref.causal_conv1d_silu_bwd):
  central finite differences of the conv, and autograd through torch's
  grouped conv1d composed with the forward transcription.

The loss is sum(dy * y) + sum(dlast * last_state) throughout.
"""
import numpy as np
import pytest
import torch

from oracle import cpu, ref

KEYS_D = ("u", "delta", "z", "h0")


def _problem(seed, b=2, d=3, n=4, L=6, gated=True, softplus=True, with_D=True, with_bias=True,
             with_h0=True, with_dlast=True):
    rng = np.random.default_rng(seed)
    p = {
        "u": rng.normal(size=(b, d, L)),
        "delta": rng.normal(size=(b, d, L)) * 0.5,
        "A": -rng.uniform(0.3, 2.0, size=(d, n)),
        "B": rng.normal(size=(b, n, L)),
        "C": rng.normal(size=(b, n, L)),
        "D": rng.normal(size=d) if with_D else None,
        "z": rng.normal(size=(b, d, L)) if gated else None,
        "delta_bias": rng.normal(size=d) * 0.3 if with_bias else None,
        "h0": rng.normal(size=(b, d, n)) if with_h0 else None,
    }
    dy = rng.normal(size=(b, d, L))
    dlast = rng.normal(size=(b, d, n)) if with_dlast else None
    return p, dy, dlast, softplus


def _loss(p, dy, dlast, softplus):
    y, last = ref.selective_scan_fwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                                     delta_bias=p["delta_bias"], delta_softplus=softplus, h0=p["h0"])
    val = float(np.sum(dy * y))
    if dlast is not None:
        val += float(np.sum(dlast * last))
    return val


def _grads(p, dy, dlast, softplus):
    return ref.selective_scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], D=p["D"], z=p["z"],
                                  delta_bias=p["delta_bias"], delta_softplus=softplus, h0=p["h0"],
                                  dy=dy, dlast=dlast)


GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
           "delta_bias": "ddelta_bias", "h0": "dh0"}

CASES = [
    dict(),
    dict(gated=False, softplus=False, with_D=False, with_bias=False, with_h0=False, with_dlast=False),
    dict(L=1, with_h0=False),
    dict(b=1, d=2, n=3, L=9, softplus=True, with_h0=True, with_dlast=False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bwd_oracle_matches_finite_differences(case):
    p, dy, dlast, sp = _problem(10 + case, **CASES[case])
    g = _grads(p, dy, dlast, sp)
    eps = 1e-5
    for name, gname in GRAD_OF.items():
        if p[name] is None:
            continue
        x = p[name]
        fd = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(p, dy, dlast, sp)
            x[idx] = old - eps
            lm = _loss(p, dy, dlast, sp)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        got = g[gname]
        scale = max(1.0, float(np.max(np.abs(fd))))
        err = float(np.max(np.abs(got - fd))) / scale
        assert err < 1e-7, (name, err)


def _torch_forward(t, softplus):
    """Plain transcription of the forward recurrence in torch float64, so that
    autograd differentiates it independently of the hand-derived backward."""
    u, delta, A, B, C = t["u"], t["delta"], t["A"], t["B"], t["C"]
    b, d, L = u.shape
    x = delta + (t["delta_bias"][None, :, None] if t["delta_bias"] is not None else 0.0)
    dt = torch.nn.functional.softplus(x) if softplus else x
    h = t["h0"] if t["h0"] is not None else torch.zeros(b, d, A.shape[1], dtype=torch.float64)
    ys = []
    for i in range(L):
        a = torch.exp(dt[:, :, i, None] * A[None])
        h = a * h + dt[:, :, i, None] * B[:, None, :, i] * u[:, :, i, None]
        y = (h * C[:, None, :, i]).sum(-1)
        if t["D"] is not None:
            y = y + t["D"][None] * u[:, :, i]
        if t["z"] is not None:
            y = y * torch.nn.functional.silu(t["z"][:, :, i])
        ys.append(y)
    return torch.stack(ys, dim=-1), h


@pytest.mark.parametrize("case", range(len(CASES)))
def test_bwd_oracle_matches_autograd(case):
    p, dy, dlast, sp = _problem(20 + case, **CASES[case])
    g = _grads(p, dy, dlast, sp)
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=True)) for k, v in p.items()}
    y, last = _torch_forward(t, sp)
    loss = (y * torch.tensor(dy)).sum()
    if dlast is not None:
        loss = loss + (last * torch.tensor(dlast)).sum()
    names = [k for k in GRAD_OF if t[k] is not None]
    grads = torch.autograd.grad(loss, [t[k] for k in names], allow_unused=True)
    for name, gt in zip(names, grads):
        want = np.zeros_like(p[name]) if gt is None else gt.numpy()
        np.testing.assert_allclose(g[GRAD_OF[name]], want, rtol=1e-10, atol=1e-12, err_msg=name)


def test_bwd_oracle_closed_form_single_step():
    """L = 1, h0 = 0, no gate: h = Delta B u, y = C.h + D u, so
    dC_n = sum_d dy Delta B_n u, dB_n = sum_d dy C_n Delta u,
    du = dy (Delta C.B + D), dDelta = dy u C.B (the decay term vanishes with a
    zero start state), dA = 0, dD = dy u, dh0 = a dy C."""
    rng = np.random.default_rng(3)
    b, d, n = 2, 5, 4
    u = rng.normal(size=(b, d, 1)); delta = rng.uniform(0.1, 1.0, size=(b, d, 1))
    A = -rng.uniform(0.5, 1.5, size=(d, n)); B = rng.normal(size=(b, n, 1)); C = rng.normal(size=(b, n, 1))
    D = rng.normal(size=d); dy = rng.normal(size=(b, d, 1))
    g = ref.selective_scan_bwd(u, delta, A, B, C, D=D, dy=dy)
    dt = delta[:, :, 0]
    CB = np.einsum("bn,bn->b", C[:, :, 0], B[:, :, 0])
    np.testing.assert_allclose(g["dC"][:, :, 0], np.einsum("bd,bd,bn->bn", dy[:, :, 0], dt * u[:, :, 0], B[:, :, 0]),
                               rtol=1e-13)
    np.testing.assert_allclose(g["dB"][:, :, 0], np.einsum("bd,bd,bn->bn", dy[:, :, 0], dt * u[:, :, 0], C[:, :, 0]),
                               rtol=1e-13)
    np.testing.assert_allclose(g["du"][:, :, 0], dy[:, :, 0] * (dt * CB[:, None] + D[None]), rtol=1e-13)
    np.testing.assert_allclose(g["ddelta"][:, :, 0], dy[:, :, 0] * u[:, :, 0] * CB[:, None], rtol=1e-13)
    assert np.all(g["dA"] == 0.0)
    np.testing.assert_allclose(g["dD"], np.sum(dy[:, :, 0] * u[:, :, 0], axis=0), rtol=1e-13)
    a = np.exp(dt[:, :, None] * A[None])
    np.testing.assert_allclose(g["dh0"], a * dy[:, :, 0, None] * C[:, None, :, 0], rtol=1e-13)


@pytest.mark.parametrize("gated,softplus,h0", [(True, True, True), (False, False, False)])
def test_bwd_c_oracle_matches_numpy(gated, softplus, h0):
    rng = np.random.default_rng(7)
    b, d, n, L = 2, 5, 16, 37
    f = lambda *s: rng.normal(size=s).astype(np.float32)
    u, delta, z, dy = f(b, d, L), f(b, d, L) * np.float32(0.5), f(b, d, L), f(b, d, L)
    A = (-rng.uniform(0.5, 4.0, size=(d, n))).astype(np.float32)
    B, C, D, bias = f(b, n, L), f(b, n, L), f(d), f(d) * np.float32(0.2)
    hh = f(b, d, n) if h0 else None
    dlast = f(b, d, n)
    kw = dict(D=D, z=z if gated else None, delta_bias=bias, delta_softplus=softplus, h0=hh, dy=dy, dlast=dlast)
    want = ref.selective_scan_bwd(u, delta, A, B, C, **kw)
    for nth in (1, 3):
        got = cpu.bwd_full(u, delta, A, B, C, nthreads=nth, **kw)
        for k, v in want.items():
            if v is None:
                assert got[k] is None
                continue
            scale = max(1e-30, float(np.max(np.abs(v))))
            assert float(np.max(np.abs(got[k] - v))) / scale < 1e-12, (k, nth)


# ------------------------------------------------------- conv1d + SiLU in front

def _conv_loss(x, w, b, g):
    return float(np.sum(g * ref.causal_conv1d(x, w, b)))


@pytest.mark.parametrize("K", [1, 2, 4])
def test_conv_bwd_matches_finite_differences(K):
    rng = np.random.default_rng(30 + K)
    x = rng.normal(size=(2, 3, 9))
    w = rng.normal(size=(3, K))
    b = rng.normal(size=3)
    g = rng.normal(size=(2, 3, 9))
    dx, dw, db = ref.causal_conv1d_silu_bwd(x, w, b, g)
    eps = 1e-6
    for arr, grad in ((x, dx), (w, dw), (b, db)):
        fd = np.empty_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = _conv_loss(x, w, b, g)
            arr[idx] = old - eps
            lm = _conv_loss(x, w, b, g)
            arr[idx] = old
            fd[idx] = (lp - lm) / (2 * eps)
        assert float(np.max(np.abs(grad - fd))) / max(1.0, float(np.max(np.abs(fd)))) < 1e-7


def test_conv_then_scan_bwd_matches_autograd():
    """The composed gradient (conv + SiLU, then the scan) against
    torch.autograd through torch's grouped conv1d and a plain float64
    transcription of the forward recurrence."""
    rng = np.random.default_rng(33)
    b, d, n, L, K = 2, 3, 4, 7, 4
    p, dy, dlast, sp = _problem(34, b=b, d=d, n=n, L=L)
    x = rng.normal(size=(b, d, L))
    w = rng.normal(size=(d, K)) * 0.5
    cb = rng.normal(size=d) * 0.1
    u = ref.causal_conv1d(x, w, cb)
    pp = dict(p)
    pp["u"] = u
    g = _grads(pp, dy, dlast, sp)
    dx, dw, dcb = ref.causal_conv1d_silu_bwd(x, w, cb, g["du"])
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(cb, requires_grad=True)
    ut = torch.nn.functional.silu(torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (K - 1, 0)), wt[:, None, :],
                                                             bt, groups=d))
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64)) for k, v in p.items()}
    t["u"] = ut
    y, last = _torch_forward(t, sp)
    loss = (y * torch.tensor(dy)).sum() + (last * torch.tensor(dlast)).sum()
    gx, gw, gb = torch.autograd.grad(loss, [xt, wt, bt])
    np.testing.assert_allclose(dx, gx.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw, gw.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dcb, gb.numpy(), rtol=1e-10, atol=1e-12)
