"""Seeded random sweep over every entry point (forward plans, start states and
chunk states, backward, the conv in front forward and backward, decode steps
with and without the conv, the output projection and its gradients, the
affine scan): sizes, dtypes, optional inputs, plans and states per lane
drawn from fixed generators, every element of every output compared with
the float64 oracle (the affine scan bit for bit with its float32 replay).  The cases are small (the oracle finishes each in
milliseconds) but span several 16-channel groups, 32-step tiles, chunks and
matrix tiles with ragged ends, n < 16 and L = 1.

Bounds as in the per-entry-point tests: max |gpu - oracle| / max |oracle|
<= 1e-4 for float32 results and 2e-2 for bfloat16-stored ones.
"""
import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads
from oracle import cpu, ref

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PLANS = ("auto", "carry", "mixed", "twopass", "lpar")


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


FWD = _cases(7101, 72, with_plan=True)


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


STATES = _cases(7202, 32, with_plan=True)


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


BWD = _cases(7303, 32, with_plan=False)
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


# ------------------------------------------------------- conv1d + SiLU in front

CONV = _cases(7404, 32, with_plan=True)


@pytest.mark.parametrize("c", CONV, ids=[_id(c) for c in CONV])
def test_conv_forward_sweep(c):
    inp, _ = _inputs(c)
    rng = np.random.default_rng(c["seed"] + 1)
    K = int(rng.integers(1, 5))
    g = torch.Generator(device=DEV)
    g.manual_seed(c["seed"] + 7)
    conv_w = torch.randn((c["d"], K), generator=g, device=DEV) * (1.0 / K)
    conv_b = torch.randn((c["d"],), generator=g, device=DEV) * 0.1 if rng.integers(2) else None
    h0 = torch.randn((c["b"], c["d"], c["n"]), generator=g, device=DEV) if rng.integers(2) else None
    print(f"[sweep conv] {_id(c)} K {K} bias {conv_b is not None} h0 {h0 is not None} seed {c['seed']}",
          flush=True)
    y, last, _, u = ssm.ssm_scan_fwd_conv(inp["u"], conv_w, inp["delta"], inp["A"], inp["B"], inp["C"],
                                          conv_b=conv_b, D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                          delta_softplus=c["softplus"], h0=h0, plan=c["plan"], return_u=True)
    torch.cuda.synchronize(DEV)
    u_ref = ref.causal_conv1d(inp["u"], conv_w, conv_b)
    y_ref, last_ref = ref.selective_scan_fwd(u_ref, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                             inp["delta_bias"], c["softplus"], h0=h0)
    assert rel_err(_host(u), u_ref) <= _bound(c["dtype"])
    assert rel_err(_host(y), y_ref) <= _bound(c["dtype"])
    assert rel_err(_host(last), last_ref) <= 1e-4


CONV_BWD = _cases(7505, 40, with_plan=False)


@pytest.mark.parametrize("c", CONV_BWD, ids=[_id(c) for c in CONV_BWD])
def test_conv_backward_sweep(c):
    inp, w = _inputs(c)
    rng = np.random.default_rng(c["seed"] + 2)
    K = int(rng.integers(1, 5))
    sc = 32 * int(rng.integers(1, 17))
    S = int(rng.choice([0, 1, 2, 4]))
    g = torch.Generator(device=DEV)
    g.manual_seed(c["seed"] + 8)
    conv_w = torch.randn((c["d"], K), generator=g, device=DEV) * (1.0 / K)
    conv_b = torch.randn((c["d"],), generator=g, device=DEV) * 0.1 if rng.integers(2) else None
    h0 = torch.randn((c["b"], c["d"], c["n"]), generator=g, device=DEV) if rng.integers(2) else None
    gr = workloads.make_grads(w, device=DEV, seed=c["seed"])
    dlast = gr["dlast"] if rng.integers(2) else None
    print(f"[sweep conv bwd] {_id(c)} K {K} state_chunk {sc} S {S} seed {c['seed']}", flush=True)
    x = inp["u"]
    _, _, cs, _ = ssm.ssm_scan_fwd_conv(x, conv_w, inp["delta"], inp["A"], inp["B"], inp["C"], conv_b=conv_b,
                                        D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                        delta_softplus=c["softplus"], h0=h0, state_chunk=sc)
    got = ssm.ssm_scan_bwd_conv(x, conv_w, inp["delta"], inp["A"], inp["B"], inp["C"], cs, sc, gr["dy"],
                                conv_b=conv_b, D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                delta_softplus=c["softplus"], h0=h0, dlast=dlast, states_per_lane=S)
    torch.cuda.synchronize(DEV)
    u = ref.causal_conv1d(x, conv_w, conv_b)
    want = ref.selective_scan_bwd(u, inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                                  delta_bias=inp["delta_bias"], delta_softplus=c["softplus"], h0=h0, dy=gr["dy"],
                                  dlast=dlast)
    dx, dw, db = ref.causal_conv1d_silu_bwd(x, conv_w, conv_b, want["du"])
    want.update(dx=dx, dconv_w=dw, dconv_b=db)
    for k in ("dx", "dconv_w", "dconv_b", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        if want.get(k) is None or got.get(k) is None:
            continue
        bound = 2e-2 if (c["dtype"] == "bf16" and k in ("dx", "ddelta", "dz")) else 1e-4
        e = rel_err(_host(got[k]), want[k])
        assert e <= bound, f"{k}: {e:.3e}"


# ------------------------------------------------------- decode steps

STEP = _cases(7606, 24, with_plan=False)


@pytest.mark.parametrize("c", STEP, ids=[_id(c) for c in STEP])
def test_decode_sweep(c):
    """T = min(L, 24) decode steps from a random state, with the conv in front
    for half of the cases, against the oracle's scan over the same steps."""
    inp, _ = _inputs(c)
    T = min(c["L"], 24)
    rng = np.random.default_rng(c["seed"] + 3)
    K = int(rng.integers(0, 5))   # 0: no conv
    g = torch.Generator(device=DEV)
    g.manual_seed(c["seed"] + 9)
    h0 = torch.randn((c["b"], c["d"], c["n"]), generator=g, device=DEV)
    conv_w = torch.randn((c["d"], K), generator=g, device=DEV) * (1.0 / K) if K else None
    conv_b = torch.randn((c["d"],), generator=g, device=DEV) * 0.1 if K else None
    print(f"[sweep decode] {_id(c)} T {T} K {K} seed {c['seed']}", flush=True)
    state = h0.clone()
    cstate = torch.zeros((c["b"], c["d"], K - 1), device=DEV) if K > 1 else None
    ys = []
    for t in range(T):
        pick = lambda v: None if v is None else v[..., t].clone(memory_format=torch.contiguous_format)
        if K:
            y, cstate, state, _ = ssm.ssm_step_conv(pick(inp["u"]), conv_w, cstate, pick(inp["delta"]), inp["A"],
                                                    pick(inp["B"]), pick(inp["C"]), state, conv_b=conv_b,
                                                    D=inp["D"], z=pick(inp["z"]), delta_bias=inp["delta_bias"],
                                                    delta_softplus=c["softplus"])
        else:
            y, state = ssm.ssm_step(pick(inp["u"]), pick(inp["delta"]), inp["A"], pick(inp["B"]), pick(inp["C"]),
                                    state, D=inp["D"], z=pick(inp["z"]), delta_bias=inp["delta_bias"],
                                    delta_softplus=c["softplus"])
        ys.append(y.clone())
    torch.cuda.synchronize(DEV)
    sl = lambda v: None if v is None else v[..., :T]
    u_ref = ref.causal_conv1d(sl(inp["u"]), conv_w, conv_b) if K else sl(inp["u"])
    y_ref, last_ref = ref.selective_scan_fwd(u_ref, sl(inp["delta"]), inp["A"], sl(inp["B"]), sl(inp["C"]), inp["D"],
                                             sl(inp["z"]), inp["delta_bias"], c["softplus"], h0=h0)
    assert rel_err(np.stack([_host(v) for v in ys], -1), y_ref) <= _bound(c["dtype"])
    assert rel_err(_host(state), last_ref) <= 1e-4


# ------------------------------------------------------- output projection

def _proj_cases(seed, count):
    """Half of the cases have every size a multiple of 8 (the block's own
    shapes, which bfloat16 runs on the kernel that loads into LDS directly),
    the rest any size."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        c = dict(b=int(rng.integers(1, 5)), k=int(rng.integers(1, 700)), m=int(rng.integers(1, 400)),
                 L=int(rng.integers(1, 600)), dtype=("f32", "bf16")[int(rng.integers(2))],
                 seed=int(rng.integers(1 << 20)))
        if i % 2 == 0:
            for key in ("k", "m", "L"):
                c[key] = 8 * ((c[key] + 7) // 8)
        out.append(c)
    return out


PROJ = _proj_cases(7707, 30)


@pytest.mark.parametrize("c", PROJ, ids=[f"b{c['b']}k{c['k']}m{c['m']}L{c['L']}-{c['dtype']}" for c in PROJ])
def test_out_proj_sweep(c):
    dtype = torch.float32 if c["dtype"] == "f32" else torch.bfloat16
    inp = workloads.make_proj_inputs(c["b"], c["k"], c["m"], c["L"], dtype=dtype, device=DEV, seed=c["seed"])
    g = torch.Generator(device=DEV)
    g.manual_seed(c["seed"] + 7)
    dout = torch.randn((c["b"], c["L"], c["m"]), generator=g, device=DEV).to(dtype).contiguous()
    print(f"[sweep proj] {c}", flush=True)
    out = ssm.ssm_out_proj(inp["y"], inp["W"])
    dy, dW = ssm.ssm_out_proj_bwd(inp["y"], inp["W"], dout)
    torch.cuda.synchronize(DEV)
    want_dy, want_dW = ref.out_proj_bwd(inp["y"], inp["W"], dout)
    assert rel_err(_host(out), ref.out_proj(inp["y"], inp["W"])) <= _bound(c["dtype"])
    assert rel_err(_host(dy), want_dy) <= _bound(c["dtype"])
    assert rel_err(_host(dW), want_dW) <= _bound(c["dtype"])


# ------------------------------------------------------- affine scan

def _affine_cases(seed, count):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 300)), int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 20000))])),
             int(rng.integers(1 << 20))) for _ in range(count)]


AFFINE = _affine_cases(7808, 24)


@pytest.mark.parametrize("rows,L,seed", AFFINE, ids=[f"r{r}L{l}" for r, l, _ in AFFINE])
def test_affine_scan_sweep(rows, L, seed):
    """Bit for bit against the float32 replay of the documented association
    order (any NaN matching any NaN), for inputs with decays, growth, exact
    zeros and subnormal-range values."""
    g = torch.Generator().manual_seed(seed)
    a = torch.exp(torch.randn((rows, L), generator=g) * 1.5)
    a[torch.rand((rows, L), generator=g) < 0.01] = 0.0
    a[torch.rand((rows, L), generator=g) < 0.01] = 1e-30
    b = torch.randn((rows, L), generator=g)
    a, b = a.float().contiguous(), b.float().contiguous()
    print(f"[sweep affine] rows {rows} L {L} seed {seed}", flush=True)
    oa, ob = ssm.affine_scan(a.to(DEV), b.to(DEV))
    torch.cuda.synchronize(DEV)
    o = ssm.affine_scan_order()
    ra, rb = cpu.affine_replay_f32(a.numpy(), b.numpy(), o["items_per_lane"], o["lanes"], o["waves"])
    for got, want in ((oa.cpu().numpy(), ra), (ob.cpu().numpy(), rb)):
        nx, ny = np.isnan(got), np.isnan(want)
        assert np.array_equal(nx, ny)
        assert np.array_equal(got[~nx].view(np.uint32), np.asarray(want, np.float32)[~ny].view(np.uint32))
