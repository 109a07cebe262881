"""GPU parity of ssm_scan_fwd against the float64 oracle (through the C ABI).

Metric (per output tensor): max |gpu - oracle| / max |oracle|, bound 1e-4 for
float32 storage and 2e-2 for bfloat16 storage (float32 state in both).
Every test compares every element; the full-size workloads run exactly as
the benchmark launches them and are compared block by block of channels.
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


def run_gpu(inp, **kw):
    y, last = ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                               inp["delta_bias"], delta_softplus=inp["delta_softplus"], **kw)
    torch.cuda.synchronize(DEV)
    return y, last


def oracle_rows(inp, rows_b, rows_d):
    from oracle import cpu
    u, dl, z = inp["u"], inp["delta"], inp["z"]
    rb = torch.as_tensor(rows_b, device=u.device)
    rd = torch.as_tensor(rows_d, device=u.device)
    sel = lambda x: None if x is None else x[rb, rd].float().cpu().numpy()
    bsz, dim, L = u.shape
    n = inp["A"].shape[1]
    return cpu.fwd_rows(sel(u), sel(dl), sel(z), np.asarray(rows_b), np.asarray(rows_d), _host(inp["A"]),
                        _host(inp["B"]), _host(inp["C"]), _host(inp["D"]), _host(inp["delta_bias"]),
                        inp["delta_softplus"], bsz, dim, n, L)


def oracle_all(inp):
    bsz, dim, L = inp["u"].shape
    rb, rd = np.meshgrid(np.arange(bsz), np.arange(dim), indexing="ij")
    y, last = oracle_rows(inp, rb.ravel(), rd.ravel())
    n = inp["A"].shape[1]
    return y.reshape(bsz, dim, L), last.reshape(bsz, dim, n)


def check_all(inp, tol=None, **kw):
    y, last = run_gpu(inp, **kw)
    y_ref, last_ref = oracle_all(inp)
    tol = tol or TOL[inp["u"].dtype]
    ey, eh = rel_err(_host(y), y_ref), rel_err(_host(last), last_ref)
    assert ey <= tol and eh <= tol, f"y err {ey:.3e}, last_state err {eh:.3e} (tol {tol:g}) {kw}"
    return ey, eh


def small_inputs(b, d, n, L, dtype=torch.float32, gated=True, with_D=True, with_bias=True, softplus=True,
                 random_A=True, seed=0):
    w = workloads.Workload("t", b, d, n, L, "f32" if dtype == torch.float32 else "bf16", gated,
                           "normal" if with_D else None, "dt_init")
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    if random_A:
        inp["A"] = workloads.random_A(d, n, device=DEV, seed=seed + 1)
    if not with_bias:
        inp["delta_bias"] = None
    inp["delta_softplus"] = softplus
    if not softplus:  # without softplus, delta + bias itself must be a valid (positive) step
        inp["delta"] = (inp["delta"].float().abs() * 0.05).to(dtype)
        if inp["delta_bias"] is not None:
            inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
    return inp


# ------------------------------------------------------------ small, complete

@pytest.mark.parametrize("plan,S,chunk", [("auto", 0, 0), ("carry", 1, 0), ("carry", 2, 0), ("carry", 4, 0),
                                          ("mixed", 0, 0), ("twopass", 1, 64), ("twopass", 2, 64),
                                          ("twopass", 4, 128)])
def test_tiny_workload(plan, S, chunk):
    """The tiny workload (b=1, d=64, n=16, L=256, float32, gated, S4D-real A)
    against the NumPy float64 oracle, element by element."""
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"], device=DEV)
    y, last = run_gpu(inp, plan=plan, states_per_lane=S, chunk=chunk)
    y_ref, last_ref = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                                             inp["z"], inp["delta_bias"], True)
    assert rel_err(_host(y), y_ref) <= 1e-4
    assert rel_err(_host(last), last_ref) <= 1e-4


SHAPES = [
    # b, d, n, L
    (1, 1, 1, 1),
    (1, 3, 2, 5),
    (2, 70, 4, 7),
    (1, 64, 16, 31),
    (1, 64, 16, 33),
    (2, 65, 16, 255),
    (1, 128, 16, 257),
    (3, 130, 5, 1000),
    (1, 200, 16, 4097),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_ragged_shapes(shape, dtype):
    inp = small_inputs(*shape, dtype=dtype, seed=sum(shape))
    check_all(inp)


@pytest.mark.parametrize("shape", [(1, 64, 16, 100), (2, 130, 16, 257), (3, 200, 5, 1000), (1, 48, 16, 64),
                                   (2, 16, 16, 100), (3, 20, 7, 45)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_mixed_plan(shape, dtype):
    """Blocks of two 16-channel groups at two states per lane next to blocks
    of one group at one state per lane (ragged channel and step tails
    included) give the oracle's result; with fewer than three groups every
    block has one group."""
    inp = small_inputs(*shape, dtype=dtype, seed=3 + sum(shape))
    check_all(inp, plan="mixed")


@pytest.mark.parametrize("gated,with_D,with_bias,softplus", [
    (False, False, False, True), (True, False, True, False), (False, True, False, False), (True, True, True, True)])
def test_optional_inputs(gated, with_D, with_bias, softplus):
    inp = small_inputs(2, 96, 16, 300, gated=gated, with_D=with_D, with_bias=with_bias, softplus=softplus, seed=7)
    check_all(inp)


@pytest.mark.parametrize("S", [1, 2, 4])
@pytest.mark.parametrize("n", [1, 3, 8, 16])
def test_states_per_lane_and_dstate(S, n):
    inp = small_inputs(2, 64, n, 160, seed=11 + n)
    check_all(inp, plan="carry", states_per_lane=S)


@pytest.mark.parametrize("L,chunk", [(256, 64), (1000, 128), (4097, 1024), (5000, 64 * 7)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_two_pass_matches_oracle_and_carry(L, chunk, dtype):
    """Chunk aggregates -> scan over chunks -> fix-up gives the same result as
    the carry plan and the oracle (ragged last chunk included)."""
    inp = small_inputs(2, 80, 16, L, dtype=dtype, seed=L)
    check_all(inp, plan="twopass", chunk=chunk)
    y1, l1 = run_gpu(inp, plan="carry")
    y2, l2 = run_gpu(inp, plan="twopass", chunk=chunk)
    assert rel_err(_host(y2), _host(y1)) <= TOL[dtype] and rel_err(_host(l2), _host(l1)) <= 1e-4


def test_repeat_runs_are_bit_identical():
    """A missing barrier shows up as run-to-run differences; every plan must
    give identical bits on every run."""
    inp = small_inputs(4, 256, 16, 1024, seed=3)
    for kw in (dict(plan="carry", states_per_lane=1), dict(plan="carry", states_per_lane=4), dict(plan="mixed"),
               dict(plan="twopass", chunk=256)):
        y0, l0 = run_gpu(inp, **kw)
        for _ in range(5):
            y1, l1 = run_gpu(inp, **kw)
            assert torch.equal(y0, y1) and torch.equal(l0, l1), kw


def test_identity_padding_varlen_small():
    """End padding with identity steps (softplus(-inf) = 0, so a = 1, b = 0)
    leaves each row's final state equal to the unpadded run's."""
    w = workloads.WORKLOADS["varlen"].with_sizes(batch=4, dim=64, L=1024)
    inp = workloads.make_inputs(w, device=DEV, seed=5)
    lengths = inp["lengths"].cpu().numpy()
    _, last = run_gpu(inp)
    for bi, ln in enumerate(lengths):
        trunc = {k: (v[bi:bi + 1, :, :ln].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
                 for k, v in inp.items()}
        _, last_t = run_gpu(trunc)
        assert rel_err(_host(last[bi]), _host(last_t[0])) <= 1e-4
        rb = np.full(8, 0)
        rd = np.arange(8)
        _, lref = oracle_rows(trunc, rb, rd)
        assert rel_err(_host(last[bi, :8]), lref) <= 1e-4


@pytest.mark.parametrize("plan", ["carry", "lpar"])
def test_softplus_off_zero_delta_pads(plan):
    """Softplus off with delta = 0 exactly at the padded steps (and no bias):
    under one plan, the final state equals the truncated run's bit for bit."""
    inp = small_inputs(3, 64, 16, 512, softplus=False, with_bias=False, seed=9)
    inp["delta"][:, :, 400:] = 0
    check_all(inp, plan=plan)
    _, last = run_gpu(inp, plan=plan)
    trunc = {k: (v[..., :400].contiguous() if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    _, last_t = run_gpu(trunc, plan=plan)
    assert torch.equal(last, last_t)


# ------------------------------------------------------------ full sizes

def _sample_rows(bsz, dim, count, seed):
    rng = np.random.default_rng(seed)
    rb = rng.integers(0, bsz, count)
    rd = rng.integers(0, dim, count)
    rb[:2] = [0, bsz - 1]
    rd[:2] = [0, dim - 1]
    return rb, rd


@pytest.mark.parametrize("name", ["130m", "1.4b", "long", "varlen"])
def test_full_size_workload(name):
    """Each full-size workload in the launch configuration the benchmark uses
    (automatic plan): every element of y and last_state against the C
    oracle, compared block by block of channels."""
    import fullcheck
    w = workloads.WORKLOADS[name]
    print(f"[full-size] {name}: b={w.batch} d={w.dim} n={w.dstate} L={w.L} {w.dtype} "
          f"plan {ssm.plan_for(w.batch, w.dim, w.dstate, w.L, w.dtype)}", flush=True)
    inp = workloads.make_inputs(w, device=DEV, seed=0)
    y, last = run_gpu(inp)
    err = fullcheck.compare_forward(inp, y, last)
    tol = TOL[w.torch_dtype]
    print(f"[full-size] {name}: y err {err['y']:.3e}, last_state err {err['last_state']:.3e} (tol {tol:g}) "
          f"over all {w.batch * w.dim} channels", flush=True)
    assert err["y"] <= tol and err["last_state"] <= 1e-4
    if w.varlen:
        # per-sequence final states equal those of the unpadded rows
        lengths = inp["lengths"].cpu().numpy()
        for bi in (0, w.batch - 1):
            ln = int(lengths[bi])
            trunc = {k: (v[bi:bi + 1, :, :ln].contiguous() if k in ("u", "delta", "z", "B", "C") else v)
                     for k, v in inp.items()}
            _, lt = oracle_rows(trunc, np.zeros(4, int), np.array([0, 1, w.dim - 2, w.dim - 1]))
            assert rel_err(_host(last[bi, [0, 1, w.dim - 2, w.dim - 1]]), lt) <= 1e-4
    del inp, y, last
    torch.cuda.empty_cache()


# ------------------------------------------------------------ extreme values

@pytest.mark.parametrize("S", [1, 2, 4])
def test_extreme_values(S):
    """delta spread over [-80, 80] (softplus's linear branch above 44 and a
    step near zero far below), A as negative as -400 (decays that underflow
    to zero within a step), and inputs of magnitude 1e3: the recurrence
    stays finite and matches the oracle."""
    inp = small_inputs(2, 32, 16, 300, seed=11)
    g = torch.Generator(device=DEV)
    g.manual_seed(12)
    inp["delta"] = (torch.rand(inp["delta"].shape, generator=g, device=DEV) * 160.0 - 80.0).contiguous()
    inp["A"] = -torch.exp(torch.randn(inp["A"].shape, generator=g, device=DEV) * 2.0).clamp(max=400.0)
    inp["u"] = (inp["u"] * 1e3).contiguous()
    y, last = run_gpu(inp, plan="carry", states_per_lane=S)
    assert torch.isfinite(y).all() and torch.isfinite(last).all()
    y_ref, last_ref = oracle_all(inp)
    assert rel_err(_host(y), y_ref) <= 1e-4
    assert rel_err(_host(last), last_ref) <= 1e-4


def test_nan_propagates_like_the_oracle():
    """A NaN in u at one step of one channel makes that channel's outputs NaN
    from that step on and nowhere else (each (b, d) row is an independent
    recurrence); every other value matches the oracle."""
    inp = small_inputs(1, 32, 16, 200, seed=13)
    u = inp["u"].clone()
    u[0, 5, 120] = float("nan")
    inp["u"] = u
    y, last = run_gpu(inp)
    y_ref, last_ref = oracle_all(inp)
    yg = _host(y)
    np.testing.assert_array_equal(np.isnan(yg), np.isnan(y_ref))
    assert np.isnan(yg[0, 5, 120:]).all() and not np.isnan(yg[0, 5, :120]).any()
    ok = ~np.isnan(y_ref)
    assert rel_err(yg[ok], y_ref[ok]) <= 1e-4
    np.testing.assert_array_equal(np.isnan(_host(last)), np.isnan(last_ref))


# ------------------------------------------------------------ large sizes

def test_very_long_sequence_few_channels():
    """b=1, d=16, L=2^22 (4.2M steps): the automatic plan splits L into
    thousands of chunks (two-pass) and the per-row byte offsets reach 268 MB;
    every channel's output against the C oracle."""
    L = 1 << 22
    inp = small_inputs(1, 16, 16, L, seed=21)
    print(f"[long] L={L} plan {ssm.plan_for(1, 16, 16, L, 'f32')}", flush=True)
    y, last = run_gpu(inp)
    y_ref, last_ref = oracle_all(inp)
    assert rel_err(_host(last), last_ref) <= 1e-4
    assert rel_err(_host(y), y_ref) <= 1e-4
    del inp, y, last
    torch.cuda.empty_cache()


@pytest.mark.parametrize("b,d,L", [(4096, 16, 64), (1, 16384, 128)], ids=["batch4096", "d16384"])
def test_large_batch_or_width(b, d, L):
    inp = small_inputs(b, d, 16, L, dtype=torch.bfloat16, seed=22)
    y, last = run_gpu(inp)
    rb, rd = _sample_rows(b, d, 64, seed=3)
    y_ref, last_ref = oracle_rows(inp, rb, rd)
    idx = (torch.as_tensor(rb, device=DEV), torch.as_tensor(rd, device=DEV))
    assert rel_err(_host(y[idx]), y_ref) <= 2e-2
    assert rel_err(_host(last[idx]), last_ref) <= 1e-4


def test_longest_accepted_sequence():
    """L at the library's limit, (2^32 - 4096) / 64 = 67108800 steps, with
    one 16-channel group and 16 states: the last channel's row of u, delta
    and y and the last state's row of B and C end 4096 bytes short of 2^32,
    the top of the 32-bit offsets the kernels address rows with.  Channels 0
    and 15 against the C oracle over every step (L + 1 is refused, see the
    host tests)."""
    L = ((1 << 32) - 4096) // 64
    inp = small_inputs(1, 16, 16, L, gated=False, seed=23)
    print(f"[max L] L={L} plan {ssm.plan_for(1, 16, 16, L, 'f32')}", flush=True)
    y, last = run_gpu(inp)
    rb, rd = np.array([0, 0]), np.array([0, 15])
    y_ref, last_ref = oracle_rows(inp, rb, rd)
    idx = (torch.as_tensor(rb, device=DEV), torch.as_tensor(rd, device=DEV))
    assert rel_err(_host(last[idx]), last_ref) <= 1e-4
    for i in range(2):
        assert rel_err(_host(y[idx][i]), y_ref[i]) <= 1e-4, f"channel {rd[i]}"
    del inp, y, last
    torch.cuda.empty_cache()
