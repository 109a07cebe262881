"""GPU parity of ssm_scan_fwd_states (start state h0 and chunk-boundary
states) against the float64 oracle, through the C ABI.

Metric and bounds as in test_gpu_ssm.py: max |gpu - oracle| / max |oracle|
<= 1e-4 (float32 storage) or 2e-2 (bfloat16 storage), per output tensor.
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


def inputs(b, d, n, L, dtype, seed):
    w = workloads.Workload("t", b, d, n, L, "f32" if dtype == torch.float32 else "bf16", True, "normal", "dt_init")
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    inp["A"] = workloads.random_A(d, n, device=DEV, seed=seed + 1)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 2)
    inp["h0"] = torch.randn((b, d, n), generator=g, device=DEV, dtype=torch.float32)
    return inp


def run_states(inp, state_chunk, plan="auto", h0=True):
    y, last, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                          inp["delta_bias"], delta_softplus=True,
                                          h0=inp["h0"] if h0 else None, state_chunk=state_chunk, plan=plan)
    torch.cuda.synchronize(DEV)
    return y, last, cs


def oracle(inp, state_chunk, h0=True):
    return ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                  inp["delta_bias"], True, h0=inp["h0"] if h0 else None,
                                  chunk=state_chunk or None)


CASES = [
    # b, d, n, L, state_chunk, plan
    (1, 64, 16, 256, 64, "auto"),
    (2, 70, 16, 300, 32, "auto"),
    (1, 48, 16, 256, 96, "mixed"),
    (2, 130, 5, 1000, 128, "mixed"),
    (2, 80, 16, 1000, 256, "twopass"),
    (1, 64, 16, 4096, 512, "twopass"),
    (16, 1536, 16, 64, 32, "auto"),       # 1536 groups: four states per lane
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:5])) + "-" + c[5])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_start_state_and_chunk_states(case, dtype):
    b, d, n, L, sc, plan = case
    inp = inputs(b, d, n, L, dtype, seed=L + d)
    y, last, cs = run_states(inp, sc, plan)
    y_ref, last_ref, bnd_ref = oracle(inp, sc)
    tol = TOL[dtype]
    assert rel_err(_host(y), y_ref) <= tol
    assert rel_err(_host(last), last_ref) <= 1e-4
    K = -(-L // sc)
    assert cs.shape == (b, K, d, n)
    # oracle boundaries: [b, d, n, K+1] with h0 first
    want = bnd_ref[..., 1:].transpose(0, 3, 1, 2)
    assert rel_err(_host(cs), want) <= 1e-4
    assert torch.equal(cs[:, -1], last)


def test_zero_start_state_matches_plain_call():
    """h0 = NULL and no chunk states is exactly ssm_scan_fwd."""
    inp = inputs(2, 96, 16, 300, torch.float32, seed=4)
    y1, l1, cs = run_states(inp, 0, h0=False)
    assert cs is None
    y2, l2 = ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                              inp["delta_bias"], delta_softplus=True)
    torch.cuda.synchronize(DEV)
    assert torch.equal(y1, y2) and torch.equal(l1, l2)


@pytest.mark.parametrize("plan", ["auto", "mixed", "twopass"])
def test_split_runs_compose(plan):
    """Steps [0, t1) and then [t1, L) from the state reached give the whole
    run (h_t = A_t h_0 + B_t for any h_0)."""
    inp = inputs(2, 96, 16, 2048, torch.float32, seed=8)
    t1 = 1024
    y, last, _ = run_states(inp, 0, plan)
    first = {k: (v[..., :t1].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    y1, l1, _ = run_states(first, 0, plan)
    second = {k: (v[..., t1:].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    second["h0"] = l1
    y2, l2, _ = run_states(second, 0, plan)
    assert rel_err(_host(torch.cat([y1, y2], dim=-1)), _host(y)) <= 1e-5
    assert rel_err(_host(l2), _host(last)) <= 1e-5


@pytest.mark.parametrize("name,sc", [("130m", 256), ("long", 4096)])
def test_full_size(name, sc):
    """Full-size workload with a random start state and chunk states, in the
    automatic launch configuration: every element of y, last_state and the
    chunk states against the C oracle."""
    import fullcheck
    w = workloads.WORKLOADS[name]
    print(f"[states full-size] {name}: b={w.batch} d={w.dim} L={w.L} state_chunk={sc}", flush=True)
    inp = workloads.make_inputs(w, device=DEV, seed=0)
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    inp["h0"] = torch.randn((w.batch, w.dim, w.dstate), generator=g, device=DEV, dtype=torch.float32)
    y, last, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                          inp["delta_bias"], delta_softplus=w.softplus, h0=inp["h0"],
                                          state_chunk=sc)
    torch.cuda.synchronize(DEV)
    err = fullcheck.compare_forward(inp, y, last, h0=inp["h0"], chunk_states=cs, state_chunk=sc)
    tol = TOL[w.torch_dtype]
    print(f"[states full-size] {name}: y {err['y']:.3e} last {err['last_state']:.3e} "
          f"chunk states {err['chunk_states']:.3e}", flush=True)
    assert err["y"] <= tol and err["last_state"] <= 1e-4 and err["chunk_states"] <= 1e-4
