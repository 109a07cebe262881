"""The library's launches inside a captured HIP graph (torch.cuda.CUDAGraph):
the decode step (the launch-bound path a serving loop would capture), the
decode step with the conv in front, the single-launch forward plans and the
output projection's forward.

Each graph is replayed several times with the program's own eager work
(in-place updates of the inputs) and synchronizations between the replays,
and every replay is compared bit for bit with the same launch made eagerly
on the same inputs.  The library records only kernel launches on the
caller's stream for these calls (no memset, allocation or synchronization).
"""
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _step_inputs(b, d, n, dtype, seed):
    w = workloads.Workload("t", b, d, n, 1, "f32" if dtype == torch.float32 else "bf16", True, "normal",
                           "dt_init", softplus=True)
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    pick = lambda x: x[..., 0].contiguous()
    out = {k: pick(inp[k]) for k in ("u", "delta", "z", "B", "C")}
    out.update(A=workloads.random_A(d, n, device=DEV, seed=seed + 1), D=inp["D"], delta_bias=inp["delta_bias"])
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 2)
    out["state"] = torch.randn((b, d, n), generator=g, device=DEV)
    return out


def _capture(fn):
    """Warm up on a side stream (as torch requires), then capture fn."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize(DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_decode_step_replays_match_eager(dtype):
    inp = _step_inputs(8, 96, 16, dtype, seed=3)
    state0 = inp["state"].clone()
    st_g = state0.clone()
    y_g = torch.empty_like(inp["u"])

    def step_g():
        ssm.ssm_step(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], st_g, D=inp["D"], z=inp["z"],
                     delta_bias=inp["delta_bias"], delta_softplus=True, y=y_g)

    graph = _capture(step_g)
    st_g.copy_(state0)                       # the warm-up and capture stepped it
    st_e = state0.clone()
    y_e = torch.empty_like(y_g)
    for r in range(4):
        graph.replay()
        ssm.ssm_step(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], st_e, D=inp["D"], z=inp["z"],
                     delta_bias=inp["delta_bias"], delta_softplus=True, y=y_e)
        torch.cuda.synchronize(DEV)
        assert torch.equal(st_g, st_e) and torch.equal(y_g, y_e), f"replay {r}"
        # eager work between replays: the next token's inputs, in place
        inp["u"].mul_(0.5).add_(0.25)
        inp["delta"].mul_(0.9)
        torch.cuda.synchronize(DEV)


def test_decode_step_with_conv_replays_match_eager():
    inp = _step_inputs(4, 64, 16, torch.float32, seed=5)
    K = 4
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    conv_w = torch.randn((64, K), generator=g, device=DEV) * 0.25
    conv_b = torch.randn((64,), generator=g, device=DEV) * 0.1
    cs0 = torch.randn((4, 64, K - 1), generator=g, device=DEV)
    state0 = inp["state"].clone()
    cs_g, st_g = cs0.clone(), state0.clone()
    y_g = torch.empty_like(inp["u"])

    def step_g():
        ssm.ssm_step_conv(inp["u"], conv_w, cs_g, inp["delta"], inp["A"], inp["B"], inp["C"], st_g, conv_b=conv_b,
                          D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], delta_softplus=True, y=y_g)

    graph = _capture(step_g)
    cs_g.copy_(cs0)
    st_g.copy_(state0)
    cs_e, st_e = cs0.clone(), state0.clone()
    y_e = torch.empty_like(y_g)
    for r in range(4):
        graph.replay()
        ssm.ssm_step_conv(inp["u"], conv_w, cs_e, inp["delta"], inp["A"], inp["B"], inp["C"], st_e, conv_b=conv_b,
                          D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], delta_softplus=True, y=y_e)
        torch.cuda.synchronize(DEV)
        assert torch.equal(cs_g, cs_e) and torch.equal(st_g, st_e) and torch.equal(y_g, y_e), f"replay {r}"
        inp["u"].add_(0.1)
        torch.cuda.synchronize(DEV)


@pytest.mark.parametrize("plan", ["carry", "mixed"])
def test_forward_replays_match_eager(plan):
    w = workloads.Workload("t", 2, 64, 16, 300, "f32", True, "normal", "dt_init", softplus=True)
    inp = workloads.make_inputs(w, device=DEV, seed=9)
    y_g = torch.empty_like(inp["u"])
    last_g = torch.empty((2, 64, 16), device=DEV)

    def fwd(y, last):
        ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                         inp["delta_bias"], delta_softplus=True, plan=plan, y=y, last_state=last)

    graph = _capture(lambda: fwd(y_g, last_g))
    y_e = torch.empty_like(y_g)
    last_e = torch.empty_like(last_g)
    for r in range(3):
        graph.replay()
        fwd(y_e, last_e)
        torch.cuda.synchronize(DEV)
        assert torch.equal(y_g, y_e) and torch.equal(last_g, last_e), f"replay {r}"
        inp["u"].mul_(-1.0)
        torch.cuda.synchronize(DEV)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_out_proj_replays_match_eager(dtype):
    """The output projection allocates nothing for its forward (bfloat16 with
    every size a multiple of 8 takes the kernel that loads into LDS
    directly): captured once, replayed with in-place updates of y between
    replays, each replay equal to the eager launch bit for bit."""
    inp = workloads.make_proj_inputs(2, 520, 264, 264, dtype=dtype, device=DEV, seed=17)
    out_g = torch.empty((2, 264, 264), device=DEV, dtype=dtype)
    graph = _capture(lambda: ssm.ssm_out_proj(inp["y"], inp["W"], out=out_g))
    out_e = torch.empty_like(out_g)
    for r in range(3):
        graph.replay()
        ssm.ssm_out_proj(inp["y"], inp["W"], out=out_e)
        torch.cuda.synchronize(DEV)
        assert torch.equal(out_g, out_e), f"replay {r}"
        inp["y"].mul_(-0.5)
        torch.cuda.synchronize(DEV)
