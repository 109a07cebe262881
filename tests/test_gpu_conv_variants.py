"""Every compiled variant of the conv-in-front kernels against the float64
oracle, every output element: the forward plans (carry at two and at four
states per lane, mixed, two-pass, L-parallel) and the backward at one, two
and four states per lane, each with float32 and bfloat16 storage, with and
without the gate, and with L a multiple of 8 (vector loads and stores) or
not.  Each case spans several channel groups, the last one ragged, so the
first channel of every workgroup runs its first tile: the halo there reaches
before step 0, where the conv reads zero (causal padding), and whose load
offsets must not wrap.

Bounds as in the other conv tests: max |gpu - oracle| / max |oracle| <= 1e-4
for float32 results, 2e-2 for bfloat16-stored ones.
"""
import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads
from oracle import ref

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / (scale if scale > 0 else 1.0))


def _host(t):
    return t.detach().double().cpu().numpy()


def _make(b, d, n, L, dtype, gated, K, seed):
    w = workloads.Workload("t", b, d, n, L, dtype, gated, "normal", "dt_init")
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 3)
    inp["conv_w"] = torch.randn((d, K), generator=g, device=DEV) * (1.0 / K)
    inp["conv_b"] = torch.randn((d,), generator=g, device=DEV) * 0.1
    return w, inp


# plan, b, d (ragged last group), n, L (a multiple of 8), K; the plan that
# ssm_scan_fwd_conv picks for these sizes is checked in the test
FWD = [
    ("carry", 2, 40, 16, 96, 3),      # 6 groups: carry, two states per lane
    ("carry", 4, 6136, 16, 40, 4),    # 1536 groups: carry, four states per lane
    ("mixed", 4, 2552, 16, 40, 3),    # 640 groups: blocks at two and at one state per lane
    ("twopass", 1, 40, 16, 2304, 3),  # 3 groups, long: chunk aggregates, carry, fix-up
    ("lpar", 2, 40, 16, 600, 4),      # L-parallel
]


@pytest.mark.parametrize("vec", [True, False], ids=["vec", "novec"])
@pytest.mark.parametrize("gated", [True, False], ids=["gated", "ungated"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", FWD, ids=[f"{c[0]}-b{c[1]}d{c[2]}L{c[4]}K{c[5]}" for c in FWD])
def test_conv_forward_variant(case, dtype, gated, vec):
    plan, b, d, n, L, K = case
    if not vec:
        L += 3
    w, inp = _make(b, d, n, L, dtype, gated, K, seed=d + L + K)
    chosen = ssm.plan_for(b, d, n, L)["plan"]
    if plan in ("carry", "mixed"):
        assert chosen == plan, f"sizes meant for the {plan} plan chose {chosen}"
    print(f"[conv fwd variant] {plan} b{b} d{d} L{L} K{K} {dtype} gated={gated}", flush=True)
    y, last, _, u = ssm.ssm_scan_fwd_conv(inp["u"], inp["conv_w"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                          conv_b=inp["conv_b"], D=inp["D"], z=inp["z"],
                                          delta_bias=inp["delta_bias"], delta_softplus=True, plan=plan,
                                          return_u=True)
    torch.cuda.synchronize(DEV)
    u_ref = ref.causal_conv1d(inp["u"], inp["conv_w"], inp["conv_b"])
    y_ref, last_ref = ref.selective_scan_fwd(u_ref, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                                             inp["z"], inp["delta_bias"], True)
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert rel_err(_host(u), u_ref) <= tol, "u"
    assert rel_err(_host(y), y_ref) <= tol, "y"
    assert rel_err(_host(last), last_ref) <= 1e-4, "last_state"


@pytest.mark.parametrize("vec", [True, False], ids=["vec", "novec"])
@pytest.mark.parametrize("gated", [True, False], ids=["gated", "ungated"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S", [1, 2, 4])
def test_conv_backward_variant(S, dtype, gated, vec):
    b, d, n, L, sc, K = 2, 40, 15, 200, 64, 3
    if not vec:
        L += 3
    w, inp = _make(b, d, n, L, dtype, gated, K, seed=100 + 10 * S + L)
    gr = workloads.make_grads(w, device=DEV, seed=7 + S)
    x = inp["u"]
    print(f"[conv bwd variant] S{S} b{b} d{d} L{L} sc{sc} K{K} {dtype} gated={gated}", flush=True)
    _, _, cs, _ = ssm.ssm_scan_fwd_conv(x, inp["conv_w"], inp["delta"], inp["A"], inp["B"], inp["C"],
                                        conv_b=inp["conv_b"], D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                        delta_softplus=True, state_chunk=sc)
    got = ssm.ssm_scan_bwd_conv(x, inp["conv_w"], inp["delta"], inp["A"], inp["B"], inp["C"], cs, sc, gr["dy"],
                                conv_b=inp["conv_b"], D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                delta_softplus=True, dlast=gr["dlast"], states_per_lane=S)
    torch.cuda.synchronize(DEV)
    u = ref.causal_conv1d(x, inp["conv_w"], inp["conv_b"])
    want = ref.selective_scan_bwd(u, inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                                  delta_bias=inp["delta_bias"], delta_softplus=True, dy=gr["dy"],
                                  dlast=gr["dlast"])
    dx, dw, db = ref.causal_conv1d_silu_bwd(x, inp["conv_w"], inp["conv_b"], want["du"])
    want.update(dx=dx, dconv_w=dw, dconv_b=db)
    checked = 0
    for k in ("dx", "dconv_w", "dconv_b", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias"):
        if want.get(k) is None or got.get(k) is None:
            continue
        bound = 2e-2 if (dtype == "bf16" and k in ("dx", "ddelta", "dz")) else 1e-4
        e = rel_err(_host(got[k]), want[k])
        assert e <= bound, f"{k}: rel err {e:.3g}"
        checked += 1
    assert checked >= 9
