"""GPU parity when every step size is tiny: delta + bias uniform on [-30, -9],
so Delta = softplus(delta + bias) lies between about 1e-13 and 1.2e-4.

This is the edge of the method where softplus(x) ~ e^x: a float32
log(1 + e^x) rounds 1 + e^x and loses Delta's digits (all of them below
x ~ -16.6).  With no D and no gate, y = C . h is built from Delta alone, so
an error in Delta is the error in y.  Every forward plan, the start-state /
chunk-state variant, the decode step and the backward are compared with the
float64 oracle, element by element, at the float32 bound 1e-4 (2e-2 for
bfloat16 storage).
"""
import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads
from oracle import cpu, ref

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.max(np.abs(want))
    assert scale > 0
    return float(np.max(np.abs(got - want)) / scale)


def _host(t):
    return None if t is None else t.detach().float().cpu().numpy()


def tiny_delta_inputs(b, d, n, L, dtype=torch.float32, seed=0, with_bias=True):
    """u, B, C ~ N(0, 1); A = -(n+1); delta + bias ~ U[-30, -9] (with the
    bias, delta ~ U[-26, -5] and bias ~ U[-4, -4]); no D, no gate."""
    w = workloads.Workload("t", b, d, n, L, "f32" if dtype == torch.float32 else "bf16", False, None, "dt_init")
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 100)
    x = torch.rand((b, d, L), generator=g, device=DEV) * 21.0 - 30.0
    if with_bias:
        bias = torch.full((d,), -4.0, device=DEV)
        inp["delta"] = (x - bias[None, :, None]).to(dtype).contiguous()
        inp["delta_bias"] = bias
    else:
        inp["delta"] = x.to(dtype).contiguous()
        inp["delta_bias"] = None
    inp["D"] = None
    inp["z"] = None
    inp["delta_softplus"] = True
    return inp


def oracle_full(inp, h0=None):
    u = inp["u"]
    bsz, dim, L = u.shape
    n = inp["A"].shape[1]
    rb, rd = np.meshgrid(np.arange(bsz), np.arange(dim), indexing="ij")
    h0_rows = None if h0 is None else h0.reshape(bsz * dim, n)
    y, last = cpu.fwd_rows(u.reshape(bsz * dim, L), inp["delta"].reshape(bsz * dim, L), None, rb.ravel(),
                           rd.ravel(), inp["A"], inp["B"], inp["C"], None, inp["delta_bias"], True, bsz, dim, n, L,
                           h0_rows=h0_rows)
    return y.reshape(bsz, dim, L), last.reshape(bsz, dim, n)


PLANS = [dict(plan="carry", states_per_lane=1), dict(plan="carry", states_per_lane=2),
         dict(plan="carry", states_per_lane=4), dict(plan="mixed"),
         dict(plan="twopass", states_per_lane=2, chunk=128), dict(plan="twopass", states_per_lane=4, chunk=256)]


@pytest.mark.parametrize("kw", PLANS, ids=lambda k: "-".join(str(v) for v in k.values()))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_forward_every_plan(kw, dtype):
    inp = tiny_delta_inputs(2, 80, 16, 1000, dtype=dtype, seed=31)
    y, last = ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], None, None, inp["delta_bias"],
                               delta_softplus=True, **kw)
    torch.cuda.synchronize(DEV)
    y_ref, last_ref = oracle_full(inp)
    ey, eh = rel_err(_host(y), y_ref), rel_err(_host(last), last_ref)
    assert ey <= TOL[dtype] and eh <= 1e-4, f"y {ey:.3e} last_state {eh:.3e}"


def test_forward_no_bias():
    """The same range reached by delta alone (no bias)."""
    inp = tiny_delta_inputs(1, 64, 16, 700, seed=32, with_bias=False)
    y, last = ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], None, None, None,
                               delta_softplus=True)
    torch.cuda.synchronize(DEV)
    y_ref, last_ref = oracle_full(inp)
    assert rel_err(_host(y), y_ref) <= 1e-4 and rel_err(_host(last), last_ref) <= 1e-4


def test_forward_states():
    """From a start state, keeping the state every 64 steps."""
    inp = tiny_delta_inputs(2, 48, 16, 512, seed=33)
    g = torch.Generator(device=DEV)
    g.manual_seed(34)
    h0 = torch.randn((2, 48, 16), generator=g, device=DEV) * 1e-6
    y, last, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], None, None,
                                          inp["delta_bias"], delta_softplus=True, h0=h0, state_chunk=64)
    torch.cuda.synchronize(DEV)
    y_ref, last_ref = oracle_full(inp, h0=h0.double().cpu().numpy())
    assert rel_err(_host(y), y_ref) <= 1e-4 and rel_err(_host(last), last_ref) <= 1e-4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_decode_steps(dtype):
    """Thirty-two decode steps in a row from a zero state against the
    oracle's recurrence over the same 32 steps."""
    inp = tiny_delta_inputs(3, 70, 16, 32, dtype=dtype, seed=35)
    state = torch.zeros((3, 70, 16), device=DEV)
    ys = []
    for t in range(32):
        pick = lambda x: x[..., t].clone(memory_format=torch.contiguous_format)
        y, state = ssm.ssm_step(pick(inp["u"]), pick(inp["delta"]), inp["A"], pick(inp["B"]), pick(inp["C"]), state,
                                delta_bias=inp["delta_bias"], delta_softplus=True)
        ys.append(y)
    torch.cuda.synchronize(DEV)
    y_ref, last_ref = oracle_full(inp)
    assert rel_err(_host(torch.stack(ys, -1)), y_ref) <= TOL[dtype]
    assert rel_err(_host(state), last_ref) <= 1e-4


@pytest.mark.parametrize("S", [1, 2, 4])
def test_backward(S):
    """Gradients of every input, from the forward's chunk states."""
    inp = tiny_delta_inputs(2, 48, 16, 384, seed=36)
    w = workloads.Workload("t", 2, 48, 16, 384, "f32", False, None, "dt_init")
    gr = workloads.make_grads(w, device=DEV, seed=37)
    _, _, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], None, None,
                                       inp["delta_bias"], delta_softplus=True, state_chunk=128)
    got = ssm.ssm_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], cs, 128, gr["dy"],
                           delta_bias=inp["delta_bias"], delta_softplus=True, dlast=gr["dlast"], states_per_lane=S)
    torch.cuda.synchronize(DEV)
    want = ref.selective_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], None, None,
                                  inp["delta_bias"], True, dy=gr["dy"], dlast=gr["dlast"])
    for k, v in want.items():
        if v is None or got.get(k) is None:
            continue
        e = rel_err(_host(got[k]), v)
        assert e <= 1e-4, f"{k}: {e:.3e}"
