"""GPU parity of the torch.autograd wrappers (selective_scan,
selective_scan_conv): the gradients that loss.backward() leaves in .grad are
compared with the float64 gradient oracle.

The loss is sum(y * dy) + sum(last_state * dlast), so the gradients of y
and of the last state that reach the backward are exactly dy and dlast.
Bounds as for the direct backward tests (max |gpu - oracle| / max |oracle|):
1e-4 for float32 results, 2e-2 for those stored in bfloat16 (du, ddelta, dz,
and with bfloat16 I/O also dB and dC, which the wrapper returns in the dtype
of B and C).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref
from selective_state_space_ssm_amd.autograd import out_proj, selective_scan, selective_scan_conv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / (scale if scale > 0 else 1.0))


def _host(t):
    return t.detach().float().cpu().numpy()


def make(b, d, n, L, dtype, seed, with_h0=True):
    w = workloads.Workload("t", b, d, n, L, "f32" if dtype == torch.float32 else "bf16", True, "normal",
                           "dt_init", softplus=True)
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    inp["A"] = workloads.random_A(d, n, device=DEV, seed=seed + 1)
    gr = workloads.make_grads(w, device=DEV, seed=seed)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 2)
    inp["h0"] = torch.randn((b, d, n), generator=g, device=DEV) if with_h0 else None
    return inp, gr["dy"], gr["dlast"]


def leaves(inp, names):
    return {k: (inp[k].detach().clone().requires_grad_(True) if inp[k] is not None else None) for k in names}


def check(got, want, dtype, label):
    for k, g in got.items():
        if g is None or want.get(k) is None:
            continue
        bf16_stored = dtype == torch.bfloat16 and k in ("u", "x", "delta", "z", "B", "C")
        bound = 2e-2 if bf16_stored else 1e-4
        e = rel_err(_host(g), want[k])
        assert e <= bound, f"{label}: d{k} rel err {e:.3g}"


CASES = [
    # b, d, n, L, state_chunk
    (1, 16, 16, 64, 32),
    (2, 40, 16, 150, 64),
    (1, 33, 16, 517, 128),
]
NAMES = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}sc{c[4]}" for c in CASES])
def test_autograd_matches_oracle(case, dtype):
    b, d, n, L, sc = case
    inp, dy, dlast = make(b, d, n, L, dtype, seed=30 + L)
    p = leaves(inp, NAMES)
    y, last = selective_scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"], p["delta_bias"],
                             delta_softplus=True, h0=p["h0"], state_chunk=sc)
    loss = (y.float() * dy.float()).sum() + (last * dlast).sum()
    loss.backward()
    torch.cuda.synchronize(DEV)
    want = ref.selective_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                                  delta_bias=inp["delta_bias"], delta_softplus=True, h0=inp["h0"], dy=dy,
                                  dlast=dlast)
    want = {"u": want["du"], "delta": want["ddelta"], "A": want["dA"], "B": want["dB"], "C": want["dC"],
            "D": want["dD"], "z": want["dz"], "delta_bias": want["ddelta_bias"], "h0": want["dh0"]}
    check({k: p[k].grad for k in NAMES}, want, dtype, str(case))
    # forward values are the library's forward
    y_ref, last_ref = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"],
                                             z=inp["z"], delta_bias=inp["delta_bias"], delta_softplus=True,
                                             h0=inp["h0"])
    assert rel_err(_host(y), y_ref) <= (2e-2 if dtype == torch.bfloat16 else 1e-4)
    assert rel_err(_host(last), last_ref) <= 1e-4


def test_autograd_only_y_used():
    """last_state unused (its gradient is None) and no h0: the backward runs
    with dlast absent and the parameters without inputs get no gradient."""
    inp, dy, _ = make(2, 24, 16, 200, torch.float32, seed=7, with_h0=False)
    p = leaves(inp, ("u", "delta", "A", "B", "C"))
    y, _ = selective_scan(p["u"], p["delta"], p["A"], p["B"], p["C"], inp["D"], inp["z"], inp["delta_bias"],
                          delta_softplus=True, state_chunk=64)
    (y * dy).sum().backward()
    torch.cuda.synchronize(DEV)
    want = ref.selective_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                                  delta_bias=inp["delta_bias"], delta_softplus=True, dy=dy)
    want = {"u": want["du"], "delta": want["ddelta"], "A": want["dA"], "B": want["dB"], "C": want["dC"]}
    check({k: p[k].grad for k in want}, want, torch.float32, "only-y")


def test_autograd_chains_through_torch_ops():
    """The wrapper sits inside an ordinary autograd graph: delta comes from a
    torch product with a weight, y goes through a torch reduction.  The
    weight's gradient equals the oracle's ddelta contracted with the product's
    other operand."""
    b, d, n, L = 1, 32, 16, 96
    inp, dy, _ = make(b, d, n, L, torch.float32, seed=11, with_h0=False)
    g = torch.Generator(device=DEV)
    g.manual_seed(123)
    xin = torch.randn((b, 8, L), generator=g, device=DEV)
    W = (torch.randn((d, 8), generator=g, device=DEV) * 0.2).requires_grad_(True)
    delta = torch.matmul(W, xin)                                  # [b, d, L]
    y, _ = selective_scan(inp["u"], delta, inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"],
                          delta_softplus=True, state_chunk=32)
    (y * dy).sum().backward()
    torch.cuda.synchronize(DEV)
    want = ref.selective_scan_bwd(inp["u"], delta.detach(), inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                                  delta_bias=inp["delta_bias"], delta_softplus=True, dy=dy)
    dW = np.einsum("bdl,bkl->dk", want["ddelta"], _host(xin).astype(np.float64))
    assert rel_err(_host(W.grad), dW) <= 1e-4


CONV_CASES = [
    # b, d, n, L, state_chunk, K
    (1, 16, 16, 64, 32, 4),
    (2, 40, 16, 150, 64, 3),
]
CONV_NAMES = ("x", "conv_w", "conv_b", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CONV_CASES, ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}sc{c[4]}K{c[5]}"
                                                   for c in CONV_CASES])
def test_autograd_conv_matches_oracle(case, dtype):
    b, d, n, L, sc, K = case
    inp, dy, dlast = make(b, d, n, L, dtype, seed=60 + L + K)
    g = torch.Generator(device=DEV)
    g.manual_seed(5 + K)
    inp["x"] = inp["u"]
    inp["conv_w"] = torch.randn((d, K), generator=g, device=DEV) * (1.0 / K)
    inp["conv_b"] = torch.randn((d,), generator=g, device=DEV) * 0.1
    p = leaves(inp, CONV_NAMES)
    y, last = selective_scan_conv(p["x"], p["conv_w"], p["conv_b"], p["delta"], p["A"], p["B"], p["C"], p["D"],
                                  p["z"], p["delta_bias"], delta_softplus=True, h0=p["h0"], state_chunk=sc)
    loss = (y.float() * dy.float()).sum() + (last * dlast).sum()
    loss.backward()
    torch.cuda.synchronize(DEV)
    u = ref.causal_conv1d(inp["x"], inp["conv_w"], inp["conv_b"])
    w = ref.selective_scan_bwd(u, inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                               delta_bias=inp["delta_bias"], delta_softplus=True, h0=inp["h0"], dy=dy, dlast=dlast)
    dx, dcw, dcb = ref.causal_conv1d_silu_bwd(inp["x"], inp["conv_w"], inp["conv_b"], w["du"])
    want = {"x": dx, "conv_w": dcw, "conv_b": dcb, "delta": w["ddelta"], "A": w["dA"], "B": w["dB"],
            "C": w["dC"], "D": w["dD"], "z": w["dz"], "delta_bias": w["ddelta_bias"], "h0": w["dh0"]}
    check({k: p[k].grad for k in CONV_NAMES}, want, dtype, str(case))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_autograd_scan_then_out_proj(dtype):
    """The tail of the block in one graph: the gated scan, then the output
    projection, then a loss on the projected tokens.  The gradients of the
    scan inputs and of W against the oracle chain (projection gradients,
    then the scan's gradients for that dy)."""
    b, d, n, L, sc = 2, 48, 16, 130, 64
    inp, _, _ = make(b, d, n, L, dtype, seed=77, with_h0=False)
    Wt = workloads.make_proj_inputs(1, d, d // 2, 1, dtype=dtype, device=DEV, seed=5)["W"]
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    R = torch.randn((b, L, d // 2), generator=g, device=DEV).to(dtype)
    names = ("u", "delta", "B", "C", "z")
    p = leaves(inp, names)
    W = Wt.detach().clone().requires_grad_(True)
    y, _ = selective_scan(p["u"], p["delta"], inp["A"], p["B"], p["C"], inp["D"], p["z"], inp["delta_bias"],
                          delta_softplus=True, state_chunk=sc)
    out = out_proj(y, W)
    (out.float() * R.float()).sum().backward()
    torch.cuda.synchronize(DEV)
    # oracle chain, on the stored (rounded) y the projection saw
    dy_ref, dW_ref = ref.out_proj_bwd(y.detach(), Wt, R)
    want = ref.selective_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                                  delta_bias=inp["delta_bias"], delta_softplus=True, dy=dy_ref)
    want = {"u": want["du"], "delta": want["ddelta"], "B": want["dB"], "C": want["dC"], "z": want["dz"]}
    bound = 2e-2 if dtype == torch.bfloat16 else 1e-4
    assert rel_err(_host(W.grad), dW_ref) <= bound
    if dtype == torch.float32:
        check({k: p[k].grad for k in names}, want, dtype, "scan+proj")
    else:
        # the scan's backward sees dy rounded to bfloat16 (one 2^-9 relative
        # rounding per element); that enters every gradient, so the bfloat16
        # bound holds for all of them
        for k in names:
            assert rel_err(_host(p[k].grad), want[k]) <= 2e-2, k
