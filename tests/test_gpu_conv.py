"""GPU parity of ssm_scan_fwd_conv (causal depthwise conv1d + SiLU fused in
front of the scan) against the float64 oracle: u = oracle.ref.causal_conv1d
then oracle.ref.selective_scan_fwd, through the C ABI.

Bounds as for the forward: max |gpu - oracle| / max |oracle| <= 1e-4 with
float32 storage, 2e-2 with bfloat16 storage (y and u_out are rounded to
bfloat16 once; the kernel's u itself stays float32).
"""
import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads
from oracle import ref

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / (scale if scale > 0 else 1.0))


def _host(t):
    return t.detach().double().cpu().numpy()


def make(b, d, n, L, dtype, K, seed, with_bias=True, with_h0=False):
    w = workloads.Workload("t", b, d, n, L, "f32" if dtype == torch.float32 else "bf16", True, "normal", "dt_init")
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 3)
    inp["conv_w"] = torch.randn((d, K), generator=g, device=DEV) * (1.0 / K)
    inp["conv_b"] = torch.randn((d,), generator=g, device=DEV) * 0.1 if with_bias else None
    inp["h0"] = torch.randn((b, d, n), generator=g, device=DEV) if with_h0 else None
    return inp


def oracle(inp, state_chunk=0):
    u = ref.causal_conv1d(inp["u"], inp["conv_w"], inp["conv_b"])
    out = ref.selective_scan_fwd(u, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                 inp["delta_bias"], True, h0=inp["h0"], chunk=state_chunk or None)
    return u, out


CASES = [
    # b, d, n, L, K, plan
    (1, 16, 16, 64, 4, "carry"),
    (2, 40, 16, 150, 4, "carry"),
    (2, 40, 16, 150, 3, "mixed"),
    (1, 33, 16, 517, 2, "auto"),
    (2, 24, 8, 77, 1, "carry"),
    (1, 16, 16, 5000, 4, "twopass"),
    (1, 20, 16, 3, 4, "carry"),
    (2, 40, 16, 150, 4, "lpar"),
    (1, 37, 16, 700, 3, "lpar"),
    (2, 9, 5, 1029, 1, "lpar"),
    (1, 64, 16, 2048, 4, "lpar"),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}K{c[4]}{c[5]}" for c in CASES])
def test_conv_scan_matches_oracle(case, dtype):
    b, d, n, L, K, plan = case
    inp = make(b, d, n, L, dtype, K, seed=L + K)
    y, last, cs, u = ssm.ssm_scan_fwd_conv(inp["u"], inp["conv_w"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                           conv_b=inp["conv_b"], D=inp["D"], z=inp["z"],
                                           delta_bias=inp["delta_bias"], delta_softplus=True, plan=plan,
                                           return_u=True)
    torch.cuda.synchronize(DEV)
    u_ref, (y_ref, last_ref) = oracle(inp)
    tol = TOL[dtype]
    assert rel_err(_host(u), u_ref) <= tol, "u"
    assert rel_err(_host(y), y_ref) <= tol, "y"
    assert rel_err(_host(last), last_ref) <= 1e-4, "last_state"


@pytest.mark.parametrize("plan", ["auto", "lpar"])
def test_conv_scan_states_and_no_u_output(plan):
    """h0, chunk-boundary states, no conv bias, no u output."""
    inp = make(2, 48, 16, 320, torch.float32, 4, seed=2, with_bias=False, with_h0=True)
    y, last, cs, u = ssm.ssm_scan_fwd_conv(inp["u"], inp["conv_w"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                           D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], delta_softplus=True,
                                           h0=inp["h0"], state_chunk=64, plan=plan)
    torch.cuda.synchronize(DEV)
    assert u is None
    _, (y_ref, last_ref, bounds) = oracle(inp, state_chunk=64)
    assert rel_err(_host(y), y_ref) <= 1e-4
    assert rel_err(_host(last), last_ref) <= 1e-4
    assert rel_err(_host(cs).transpose(0, 2, 3, 1), bounds[..., 1:]) <= 1e-4


def test_conv_scan_full_size_130m():
    """The 130m shape (b=8, d=1536, L=2048, float32) with a 4-tap conv, in the
    launch configuration of the benchmark's --conv mode: every element of
    the conv output u, of y and of last_state against the oracle.  The
    oracle's conv output (float64) feeds its scan rounded to float32, a
    relative change of at most 2^-24 per element."""
    import fullcheck
    w = workloads.WORKLOADS["130m"]
    inp = workloads.make_inputs(w, device=DEV, seed=0)
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    inp["conv_w"] = torch.randn((w.dim, 4), generator=g, device=DEV) * 0.25
    inp["conv_b"] = torch.randn((w.dim,), generator=g, device=DEV) * 0.1
    y, last, _, u = ssm.ssm_scan_fwd_conv(inp["u"], inp["conv_w"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                          conv_b=inp["conv_b"], D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                          delta_softplus=True, return_u=True)
    torch.cuda.synchronize(DEV)
    u_ref = ref.causal_conv1d(inp["u"], inp["conv_w"], inp["conv_b"])
    eu = rel_err(_host(u), u_ref)
    err = fullcheck.compare_forward(inp, y, last, u_override=torch.from_numpy(u_ref))
    print(f"[conv full-size] u {eu:.3e} y {err['y']:.3e} last {err['last_state']:.3e}", flush=True)
    assert eu <= 1e-4 and err["y"] <= 1e-4 and err["last_state"] <= 1e-4
