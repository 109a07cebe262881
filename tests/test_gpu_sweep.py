"""Seeded random sweep over the forward, the start-state / chunk-state forward
and the backward: sizes, dtypes, optional inputs, plans and states per lane
drawn from fixed generators, every element of every output compared with
the C oracle (float64).  The cases are small (the oracle finishes each in
milliseconds) but span several 16-channel groups, 32-step tiles and chunks
with ragged ends, n < 16 and L = 1.

Bounds as in the per-entry-point tests: max |gpu - oracle| / max |oracle|
<= 1e-4 for float32 results and 2e-2 for bfloat16-stored ones.
"""
import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads
from oracle import cpu

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PLANS = ("auto", "carry", "mixed", "twopass")


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / (scale if scale > 0 else 1.0))


def _host(t):
    return None if t is None else t.detach().float().cpu().numpy()


def _draw(rng, with_plan):
    c = dict(b=int(rng.integers(1, 5)), d=int(rng.integers(1, 130)), n=int(rng.integers(1, 17)),
             L=int(rng.choice([1, int(rng.integers(2, 64)), int(rng.integers(64, 1200))])),
             dtype=("f32", "bf16")[int(rng.integers(2))],
             gated=bool(rng.integers(2)), with_D=bool(rng.integers(2)), with_bias=bool(rng.integers(2)),
             softplus=bool(rng.integers(2)), seed=int(rng.integers(1 << 20)))
    if with_plan:
        c["plan"] = PLANS[int(rng.integers(len(PLANS)))]
        c["S"] = int(rng.choice([0, 1, 2, 4])) if c["plan"] in ("carry", "twopass") else 0
        c["chunk"] = int(rng.choice([0, 64, 128, 320])) if c["plan"] == "twopass" else 0
    return c


def _cases(seed, count, with_plan):
    rng = np.random.default_rng(seed)
    return [_draw(rng, with_plan) for _ in range(count)]


def _id(c):
    s = f"b{c['b']}d{c['d']}n{c['n']}L{c['L']}-{c['dtype']}"
    if "plan" in c:
        s += f"-{c['plan']}{c['S'] or ''}" + (f"c{c['chunk']}" if c["chunk"] else "")
    return s + f"-{'g' if c['gated'] else ''}{'D' if c['with_D'] else ''}{'b' if c['with_bias'] else ''}" \
               f"{'s' if c['softplus'] else ''}"


def _inputs(c):
    w = workloads.Workload("t", c["b"], c["d"], c["n"], c["L"], c["dtype"], c["gated"],
                           "normal" if c["with_D"] else None, "dt_init", softplus=c["softplus"])
    inp = workloads.make_inputs(w, device=DEV, seed=c["seed"])
    inp["A"] = workloads.random_A(c["d"], c["n"], device=DEV, seed=c["seed"] + 1)
    if not c["with_bias"]:
        inp["delta_bias"] = None
    if not c["softplus"]:  # without softplus, delta + bias itself is the (positive) step
        inp["delta"] = (inp["delta"].float().abs() * 0.05).to(inp["u"].dtype)
        if inp["delta_bias"] is not None:
            inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
    inp["delta_softplus"] = c["softplus"]
    return inp, w


def _bound(dtype):
    return 2e-2 if dtype == "bf16" else 1e-4


FWD = _cases(7101, 36, with_plan=True)


@pytest.mark.parametrize("c", FWD, ids=[_id(c) for c in FWD])
def test_forward_sweep(c):
    inp, _ = _inputs(c)
    print(f"[sweep fwd] {_id(c)} seed {c['seed']}", flush=True)
    y, last = ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                               inp["delta_bias"], delta_softplus=c["softplus"], plan=c["plan"],
                               states_per_lane=c["S"], chunk=c["chunk"])
    torch.cuda.synchronize(DEV)
    y_ref, last_ref = cpu.fwd_full(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                                   delta_bias=inp["delta_bias"], delta_softplus=c["softplus"])
    ey, eh = rel_err(_host(y), y_ref), rel_err(_host(last), last_ref)
    assert ey <= _bound(c["dtype"]) and eh <= 1e-4, f"y {ey:.3e} last {eh:.3e}"


STATES = _cases(7202, 16, with_plan=True)


@pytest.mark.parametrize("c", STATES, ids=[_id(c) for c in STATES])
def test_start_state_sweep(c):
    inp, _ = _inputs(c)
    g = torch.Generator(device=DEV)
    g.manual_seed(c["seed"] + 5)
    h0 = torch.randn((c["b"], c["d"], c["n"]), generator=g, device=DEV)
    sc = 32 * int(np.random.default_rng(c["seed"]).integers(1, 9))
    print(f"[sweep states] {_id(c)} state_chunk {sc} seed {c['seed']}", flush=True)
    plan = c["plan"]
    y, last, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                          inp["delta_bias"], delta_softplus=c["softplus"], h0=h0, state_chunk=sc,
                                          plan=plan)
    torch.cuda.synchronize(DEV)
    bsz, dim, L = inp["u"].shape
    rb, rd = np.meshgrid(np.arange(bsz), np.arange(dim), indexing="ij")
    rb, rd = rb.ravel(), rd.ravel()
    flat = lambda x: None if x is None else x.reshape(bsz * dim, L)
    y_ref, last_ref, bounds = cpu.fwd_rows(flat(inp["u"]), flat(inp["delta"]), flat(inp["z"]), rb, rd,
                                           _host(inp["A"]), _host(inp["B"]), _host(inp["C"]), _host(inp["D"]),
                                           _host(inp["delta_bias"]), c["softplus"], bsz, dim, c["n"], L,
                                           h0_rows=h0.reshape(bsz * dim, c["n"]), chunk=sc)
    K = bounds.shape[1]
    want_cs = bounds.reshape(bsz, dim, K, c["n"]).transpose(0, 2, 1, 3)
    assert rel_err(_host(y).reshape(bsz * dim, L), y_ref) <= _bound(c["dtype"])
    assert rel_err(_host(last).reshape(bsz * dim, c["n"]), last_ref) <= 1e-4
    assert rel_err(_host(cs), want_cs) <= 1e-4


BWD = _cases(7303, 16, with_plan=False)
IO_KEYS = ("du", "ddelta", "dz")


@pytest.mark.parametrize("c", BWD, ids=[_id(c) for c in BWD])
def test_backward_sweep(c):
    inp, w = _inputs(c)
    rng = np.random.default_rng(c["seed"])
    sc = 32 * int(rng.integers(1, 17))
    S = int(rng.choice([0, 1, 2, 4]))
    gr = workloads.make_grads(w, device=DEV, seed=c["seed"])
    g = torch.Generator(device=DEV)
    g.manual_seed(c["seed"] + 6)
    h0 = torch.randn((c["b"], c["d"], c["n"]), generator=g, device=DEV) if rng.integers(2) else None
    dlast = gr["dlast"] if rng.integers(2) else None
    print(f"[sweep bwd] {_id(c)} state_chunk {sc} S {S} h0 {h0 is not None} dlast {dlast is not None} "
          f"seed {c['seed']}", flush=True)
    _, _, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                       inp["delta_bias"], delta_softplus=c["softplus"], h0=h0, state_chunk=sc)
    got = ssm.ssm_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], cs, sc, gr["dy"], D=inp["D"],
                           z=inp["z"], delta_bias=inp["delta_bias"], delta_softplus=c["softplus"], h0=h0,
                           dlast=dlast, states_per_lane=S)
    torch.cuda.synchronize(DEV)
    want = cpu.bwd_full(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                        delta_bias=inp["delta_bias"], delta_softplus=c["softplus"], h0=h0, dy=gr["dy"], dlast=dlast)
    for k, v in want.items():
        if v is None or got.get(k) is None:
            continue
        bound = 2e-2 if (c["dtype"] == "bf16" and k in IO_KEYS) else 1e-4
        e = rel_err(_host(got[k]), v)
        assert e <= bound, f"{k}: {e:.3e}"
