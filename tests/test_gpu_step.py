"""GPU parity of ssm_step (one recurrent decode step) against the float64
oracle's recurrence, through the C ABI.  One step from state h equals the
oracle's selective scan over L = 1 with h0 = h; T steps in a row equal the
oracle (and the GPU forward pass) over T steps.

Metric: max |gpu - oracle| / max |oracle| <= 1e-4 (float32 storage) or
2e-2 (bfloat16 storage) for y, and 1e-4 for the float32 state.
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
    return None if t is None else t.detach().float().cpu().numpy()


def seq_inputs(b, d, n, L, dtype, seed, gated=True, with_D=True, with_bias=True):
    w = workloads.Workload("t", b, d, n, L, "f32" if dtype == torch.float32 else "bf16", gated,
                           "normal" if with_D else None, "dt_init")
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    inp["A"] = workloads.random_A(d, n, device=DEV, seed=seed + 1)
    if not with_bias:
        inp["delta_bias"] = None
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 2)
    inp["h0"] = torch.randn((b, d, n), generator=g, device=DEV, dtype=torch.float32)
    return inp


def step_at(inp, t, state, softplus=True, state_out=None):
    pick = lambda x: None if x is None else x[..., t].clone(memory_format=torch.contiguous_format)
    return ssm.ssm_step(pick(inp["u"]), pick(inp["delta"]), inp["A"], pick(inp["B"]), pick(inp["C"]), state,
                        D=inp["D"], z=pick(inp["z"]), delta_bias=inp["delta_bias"], delta_softplus=softplus,
                        state_out=state_out)


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 70, 16), (3, 130, 5), (1, 64, 3), (8, 1536, 16)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("opts", [dict(), dict(gated=False, with_D=False, with_bias=False)], ids=["full", "bare"])
def test_one_step(shape, dtype, opts):
    b, d, n = shape
    inp = seq_inputs(b, d, n, 1, dtype, seed=b + d + n, **opts)
    state = inp["h0"].clone()
    y, st = step_at(inp, 0, state)
    torch.cuda.synchronize(DEV)
    y_ref, h_ref = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                          inp["delta_bias"], True, h0=inp["h0"])
    assert st.data_ptr() == state.data_ptr()  # in place by default
    assert rel_err(_host(y), y_ref[..., 0]) <= TOL[dtype]
    assert rel_err(_host(st), h_ref) <= 1e-4


def test_softplus_off():
    inp = seq_inputs(2, 96, 16, 1, torch.float32, seed=5)
    # without softplus, delta + bias itself must be a valid (positive) step
    inp["delta"] = (inp["delta"].abs() * 0.05).contiguous()
    inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
    state = inp["h0"].clone()
    y, st = step_at(inp, 0, state, softplus=False)
    torch.cuda.synchronize(DEV)
    y_ref, h_ref = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                          inp["delta_bias"], False, h0=inp["h0"])
    assert rel_err(_host(y), y_ref[..., 0]) <= 1e-4 and rel_err(_host(st), h_ref) <= 1e-4


def test_out_of_place_equals_in_place():
    inp = seq_inputs(4, 200, 16, 1, torch.float32, seed=6)
    s1 = inp["h0"].clone()
    out = torch.empty_like(s1)
    y2, _ = step_at(inp, 0, inp["h0"], state_out=out)
    y1, _ = step_at(inp, 0, s1)
    torch.cuda.synchronize(DEV)
    assert torch.equal(y1, y2) and torch.equal(s1, out)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_decode_loop_equals_scan(dtype):
    """T decode steps from h0 give the oracle's scan over T steps and agree
    with the GPU forward pass started from the same state."""
    b, d, n, T = 2, 96, 16, 64
    inp = seq_inputs(b, d, n, T, dtype, seed=9)
    state = inp["h0"].clone()
    ys = []
    for t in range(T):
        y, _ = step_at(inp, t, state)
        ys.append(y)
    torch.cuda.synchronize(DEV)
    y_dec = torch.stack(ys, dim=-1)
    y_ref, h_ref = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                          inp["delta_bias"], True, h0=inp["h0"])
    assert rel_err(_host(y_dec), y_ref) <= TOL[dtype]
    assert rel_err(_host(state), h_ref) <= 1e-4
    y_fwd, h_fwd, _ = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                                              inp["z"], inp["delta_bias"], delta_softplus=True, h0=inp["h0"])
    torch.cuda.synchronize(DEV)
    assert rel_err(_host(state), _host(h_fwd)) <= 1e-4
    assert rel_err(_host(y_dec), _host(y_fwd)) <= TOL[dtype]


# ------------------------------------------------------------ decode with the conv

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("K,inplace", [(4, True), (4, False), (3, True), (2, False), (1, True)])
def test_step_conv_sequence_matches_conv_scan(K, inplace, dtype):
    """T decode steps with the conv, from zero conv and SSM states, equal the
    oracle's causal conv1d + SiLU followed by the scan over the same T steps;
    the conv state ends holding the last K-1 inputs."""
    b, d, n, T = 2, 40, 16, 12
    inp = seq_inputs(b, d, n, T, dtype, seed=40 + K)
    g = torch.Generator(device=DEV)
    g.manual_seed(5 + K)
    conv_w = torch.randn((d, K), generator=g, device=DEV) * (1.0 / K)
    conv_b = torch.randn((d,), generator=g, device=DEV) * 0.1
    cs = torch.zeros((b, d, K - 1), device=DEV) if K > 1 else None
    state = torch.zeros((b, d, n), device=DEV)
    ys, us = [], []
    for t in range(T):
        pick = lambda x: None if x is None else x[..., t].clone(memory_format=torch.contiguous_format)
        kw = dict(conv_b=conv_b, D=inp["D"], z=pick(inp["z"]), delta_bias=inp["delta_bias"], delta_softplus=True,
                  return_u=True)
        if not inplace:
            kw["conv_state_out"] = torch.empty_like(cs) if cs is not None else None
            kw["state_out"] = torch.empty_like(state)
        y, cs2, st2, u = ssm.ssm_step_conv(pick(inp["u"]), conv_w, cs, pick(inp["delta"]), inp["A"],
                                           pick(inp["B"]), pick(inp["C"]), state, **kw)
        cs, state = cs2, st2
        ys.append(y.clone())
        us.append(u.clone())
    torch.cuda.synchronize(DEV)
    u_ref = ref.causal_conv1d(inp["u"], conv_w, conv_b)
    y_ref, last_ref = ref.selective_scan_fwd(u_ref, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                             inp["delta_bias"], True)
    tol = TOL[dtype]
    assert rel_err(np.stack([_host(v) for v in us], -1), u_ref) <= tol
    assert rel_err(np.stack([_host(v) for v in ys], -1), y_ref) <= tol
    assert rel_err(_host(state), last_ref) <= 1e-4
    if K > 1:
        x_host = inp["u"].float().cpu().numpy()
        np.testing.assert_array_equal(_host(cs), x_host[:, :, T - (K - 1):])


def test_step_conv_matches_conv_forward_on_gpu():
    """Decode over T steps reproduces ssm_scan_fwd_conv's y and last state."""
    b, d, n, T = 1, 64, 16, 40
    inp = seq_inputs(b, d, n, T, torch.float32, seed=77)
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    conv_w = torch.randn((d, 4), generator=g, device=DEV) * 0.25
    y_fwd, last_fwd, _, _ = ssm.ssm_scan_fwd_conv(inp["u"], conv_w, inp["delta"], inp["A"], inp["B"], inp["C"],
                                                  D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                                  delta_softplus=True)
    cs = torch.zeros((b, d, 3), device=DEV)
    state = torch.zeros((b, d, n), device=DEV)
    for t in range(T):
        pick = lambda x: x[..., t].clone(memory_format=torch.contiguous_format)
        y, cs, state, _ = ssm.ssm_step_conv(pick(inp["u"]), conv_w, cs, pick(inp["delta"]), inp["A"], pick(inp["B"]),
                                            pick(inp["C"]), state, D=inp["D"], z=pick(inp["z"]),
                                            delta_bias=inp["delta_bias"], delta_softplus=True)
        assert rel_err(_host(y), _host(y_fwd[..., t])) <= 1e-5
    torch.cuda.synchronize(DEV)
    assert rel_err(_host(state), _host(last_fwd)) <= 1e-5
