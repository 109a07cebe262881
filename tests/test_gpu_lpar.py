"""GPU parity of the L-parallel forward plan (plan "lpar": a tile cut into
16 time segments per channel, folded thread-serially, joined by a wave64 DPP
scan of the segment pairs and refolded from registers) against the float64
oracle, through the C ABI.

Metric as in test_gpu_ssm.py: max |gpu - oracle| / max |oracle| per output
tensor, bound 1e-4 for float32 storage and 2e-2 for bfloat16 storage.  The
shapes put ragged tails on every tiling level: channels (4 per workgroup),
states (4 per lane, one wavefront per 4 states), segments (8 steps) and
tiles (128 steps).
"""
import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads
from oracle import ref
from test_gpu_ssm import DEV, TOL, _host, check_all, oracle_all, rel_err, run_gpu, small_inputs

pytestmark = pytest.mark.gpu


def test_tiny_workload_lpar():
    """The tiny workload (b=1, d=64, n=16, L=256: two tiles) against the
    NumPy float64 oracle."""
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"], device=DEV)
    y, last = run_gpu(inp, plan="lpar")
    y_ref, last_ref = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                                             inp["z"], inp["delta_bias"], True)
    assert rel_err(_host(y), y_ref) <= 1e-4
    assert rel_err(_host(last), last_ref) <= 1e-4


SHAPES = [
    # b, d, n, L
    (1, 1, 1, 1),
    (1, 3, 2, 5),
    (2, 70, 4, 7),
    (1, 4, 16, 8),
    (1, 5, 16, 9),
    (1, 64, 16, 127),
    (1, 64, 16, 128),
    (2, 65, 16, 129),
    (1, 8, 16, 255),
    (3, 130, 5, 1000),
    (1, 200, 16, 4097),
    (2, 6, 13, 3000),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_lpar_ragged_shapes(shape, dtype):
    inp = small_inputs(*shape, dtype=dtype, seed=40 + sum(shape))
    check_all(inp, plan="lpar")


@pytest.mark.parametrize("gated,with_D,with_bias,softplus", [
    (False, False, False, True), (True, False, True, True), (False, True, True, False), (True, True, False, False)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_lpar_optional_inputs(gated, with_D, with_bias, softplus, dtype):
    inp = small_inputs(2, 36, 16, 300, dtype=dtype, gated=gated, with_D=with_D, with_bias=with_bias,
                       softplus=softplus, seed=50)
    check_all(inp, plan="lpar")


@pytest.mark.parametrize("n", [1, 3, 4, 5, 8, 12, 16])
def test_lpar_dstate(n):
    """d_state below 16: whole wavefronts past d_state skip the scan, and the
    last active one runs with some states empty."""
    inp = small_inputs(1, 20, n, 700, seed=60 + n)
    check_all(inp, plan="lpar")


@pytest.mark.parametrize("L", [64, 1000, 2048])
def test_lpar_start_state(L):
    """A given start state h0 (ssm_scan_fwd_states with the L-parallel plan)
    enters the first segment's carry."""
    inp = small_inputs(2, 24, 16, L, seed=70)
    g = torch.Generator(device=DEV)
    g.manual_seed(71)
    h0 = torch.randn((2, 24, 16), generator=g, device=DEV, dtype=torch.float32)
    y, last, _ = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                         inp["delta_bias"], delta_softplus=True, h0=h0, plan="lpar")
    torch.cuda.synchronize(DEV)
    y_ref, last_ref = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                                             inp["z"], inp["delta_bias"], True, h0=h0)
    assert rel_err(_host(y), y_ref) <= 1e-4
    assert rel_err(_host(last), last_ref) <= 1e-4


@pytest.mark.parametrize("L,sc", [(64, 32), (256, 32), (1000, 32), (1000, 96), (1024, 128), (1500, 128),
                                  (2048, 224), (3000, 512), (700, 4096), (2048, 2048)],
                         ids=lambda v: str(v))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_lpar_chunk_states(L, sc, dtype):
    """The states at every state_chunk boundary (the checkpoints the backward
    recomputes from) through the L-parallel plan, from a start state: spacings
    below, at and above the 256-step tile, not dividing it (96, 224), L a
    multiple of the spacing or not, and a spacing longer than L (one entry,
    the final state).  Every entry against the oracle's states at the same
    steps."""
    b, d, n = 2, 21, 13
    inp = small_inputs(b, d, n, L, dtype=dtype, seed=80 + L + sc)
    g = torch.Generator(device=DEV)
    g.manual_seed(81)
    h0 = torch.randn((b, d, n), generator=g, device=DEV, dtype=torch.float32)
    y, last, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                          inp["delta_bias"], delta_softplus=True, h0=h0, state_chunk=sc, plan="lpar")
    torch.cuda.synchronize(DEV)
    y_ref, last_ref, bounds = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"],
                                                     inp["z"], inp["delta_bias"], True, h0=h0, chunk=sc)
    K = -(-L // sc)
    assert cs.shape == (b, K, d, n)
    cs_ref = bounds[..., 1:].transpose(0, 3, 1, 2)  # [b, K, d, n]
    assert rel_err(_host(cs), cs_ref) <= 1e-4
    assert rel_err(_host(y), y_ref) <= TOL[dtype]
    assert rel_err(_host(last), last_ref) <= 1e-4
    np.testing.assert_array_equal(_host(cs)[:, -1], _host(last))


def test_lpar_chunk_states_feed_the_backward():
    """The backward from the L-parallel plan's chunk states gives the same
    gradients as from the carry plan's (both are the state after the same
    steps, to float32 rounding)."""
    inp = small_inputs(1, 40, 16, 1024, seed=82)
    sc = 128
    g = torch.Generator(device=DEV)
    g.manual_seed(83)
    dy = torch.randn(inp["u"].shape, generator=g, device=DEV, dtype=inp["u"].dtype)
    grads = []
    for plan in ("lpar", "carry"):
        _, _, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                           inp["delta_bias"], delta_softplus=True, state_chunk=sc, plan=plan)
        gr = ssm.ssm_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], cs, sc, dy, D=inp["D"],
                              z=inp["z"], delta_bias=inp["delta_bias"], delta_softplus=True)
        grads.append(gr)
    torch.cuda.synchronize(DEV)
    for name in grads[0]:
        if grads[0][name] is None:
            continue
        a, c = _host(grads[0][name]), _host(grads[1][name])
        assert rel_err(a, c) <= 1e-4, name


def test_lpar_conv_chunk_states_feed_the_backward():
    """With the conv in front: the conv backward from the L-parallel plan's
    chunk states gives the gradients it gives from the carry plan's."""
    inp = small_inputs(2, 24, 16, 1000, seed=84)
    g = torch.Generator(device=DEV)
    g.manual_seed(85)
    conv_w = torch.randn((24, 4), generator=g, device=DEV) * 0.25
    conv_b = torch.randn((24,), generator=g, device=DEV) * 0.1
    dy = torch.randn(inp["u"].shape, generator=g, device=DEV, dtype=inp["u"].dtype)
    sc = 128
    grads, ys = [], []
    for plan in ("lpar", "carry"):
        y, _, cs, _ = ssm.ssm_scan_fwd_conv(inp["u"], conv_w, inp["delta"], inp["A"], inp["B"], inp["C"],
                                            conv_b=conv_b, D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                            delta_softplus=True, state_chunk=sc, plan=plan)
        gr = ssm.ssm_scan_bwd_conv(inp["u"], conv_w, inp["delta"], inp["A"], inp["B"], inp["C"], cs, sc, dy,
                                   conv_b=conv_b, D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                   delta_softplus=True)
        grads.append(gr)
        ys.append(y)
    torch.cuda.synchronize(DEV)
    assert rel_err(_host(ys[0]), _host(ys[1])) <= 1e-4
    for name in grads[0]:
        if grads[0][name] is None:
            continue
        assert rel_err(_host(grads[0][name]), _host(grads[1][name])) <= 1e-4, name


def test_lpar_extreme_values():
    """delta over [-80, 80], A down to -400 (decays that underflow within a
    step, so segment products of exactly zero) and inputs of magnitude 1e3."""
    inp = small_inputs(2, 32, 16, 300, seed=11)
    g = torch.Generator(device=DEV)
    g.manual_seed(12)
    inp["delta"] = (torch.rand(inp["delta"].shape, generator=g, device=DEV) * 160.0 - 80.0).contiguous()
    inp["A"] = -torch.exp(torch.randn(inp["A"].shape, generator=g, device=DEV) * 2.0).clamp(max=400.0)
    inp["u"] = (inp["u"] * 1e3).contiguous()
    y, last = run_gpu(inp, plan="lpar")
    assert torch.isfinite(y).all() and torch.isfinite(last).all()
    y_ref, last_ref = oracle_all(inp)
    assert rel_err(_host(y), y_ref) <= 1e-4
    assert rel_err(_host(last), last_ref) <= 1e-4


def test_lpar_small_delta():
    """delta + bias uniform over [-30, -9] (Delta from about 1e-13 up), no D,
    no gate: the scan of segment products close to one."""
    inp = small_inputs(1, 16, 16, 1000, gated=False, with_D=False, with_bias=False, seed=73)
    g = torch.Generator(device=DEV)
    g.manual_seed(74)
    inp["delta"] = (torch.rand(inp["delta"].shape, generator=g, device=DEV) * 21.0 - 30.0).contiguous()
    check_all(inp, plan="lpar")


def test_lpar_nan_stays_in_its_channel():
    """A NaN in u at one step of one channel makes that channel's outputs NaN
    from that step on (the scan joins segments of one channel only)."""
    inp = small_inputs(1, 8, 16, 400, seed=13)
    u = inp["u"].clone()
    u[0, 5, 120] = float("nan")
    inp["u"] = u
    y, last = run_gpu(inp, plan="lpar")
    y_ref, last_ref = oracle_all(inp)
    yg = _host(y)
    np.testing.assert_array_equal(np.isnan(yg), np.isnan(y_ref))
    ok = ~np.isnan(y_ref)
    assert rel_err(yg[ok], y_ref[ok]) <= 1e-4


def test_lpar_repeat_runs_are_bit_identical():
    """A missing barrier or an unordered LDS access shows up as run-to-run
    differences."""
    inp = small_inputs(2, 40, 16, 1500, seed=75)
    y0, l0 = run_gpu(inp, plan="lpar")
    for _ in range(3):
        y1, l1 = run_gpu(inp, plan="lpar")
        assert torch.equal(y0, y1) and torch.equal(l0, l1)


def test_twopass_long_workload_full():
    """The long workload (b=1, d=2048, n=16, L=65536, float32, no gate, no D),
    which the automatic choice runs with the L-parallel plan, through the
    two-pass plan: every element against the C oracle."""
    import fullcheck
    w = workloads.WORKLOADS["long"]
    print(f"[two-pass full-size] long: b={w.batch} d={w.dim} n={w.dstate} L={w.L}", flush=True)
    inp = workloads.make_inputs(w, device=DEV, seed=0)
    y, last = run_gpu(inp, plan="twopass")
    err = fullcheck.compare_forward(inp, y, last)
    print(f"[two-pass full-size] long: y err {err['y']:.3e}, last_state err {err['last_state']:.3e}", flush=True)
    assert err["y"] <= 1e-4 and err["last_state"] <= 1e-4
    del inp, y, last
    torch.cuda.empty_cache()


def _sweep_cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        out.append(dict(b=int(rng.integers(1, 4)), d=int(rng.integers(1, 70)), n=int(rng.integers(1, 17)),
                        L=int(rng.choice([1, int(rng.integers(2, 300)), int(rng.integers(300, 3000))])),
                        dtype=(torch.float32, torch.bfloat16)[int(rng.integers(2))],
                        gated=bool(rng.integers(2)), with_D=bool(rng.integers(2)),
                        with_bias=bool(rng.integers(2)), softplus=bool(rng.integers(2)),
                        h0=bool(rng.integers(2)), seed=int(rng.integers(1 << 20)),
                        sc=int(rng.choice([0, 32, 96, 128, 512]))))
    return out


SWEEP = _sweep_cases(7909, 24)


@pytest.mark.parametrize("c", SWEEP, ids=lambda c: f"b{c['b']}d{c['d']}n{c['n']}L{c['L']}"
                         f"{'-bf16' if c['dtype'] == torch.bfloat16 else ''}{'-h0' if c['h0'] else ''}"
                         f"{'-sc' + str(c['sc']) if c['sc'] else ''}")
def test_lpar_seeded_sweep(c):
    """Seeded random sizes (ragged channels, states, segments and tiles, L
    from 1), storage types, optional inputs, start states and chunk-state
    spacings through the L-parallel plan, every element against the float64
    oracle."""
    inp = small_inputs(c["b"], c["d"], c["n"], c["L"], dtype=c["dtype"], gated=c["gated"], with_D=c["with_D"],
                       with_bias=c["with_bias"], softplus=c["softplus"], seed=c["seed"])
    h0 = None
    if c["h0"]:
        g = torch.Generator(device=DEV)
        g.manual_seed(c["seed"] + 7)
        h0 = torch.randn((c["b"], c["d"], c["n"]), generator=g, device=DEV, dtype=torch.float32)
    sc = c["sc"]
    y, last, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                          inp["delta_bias"], delta_softplus=inp["delta_softplus"], h0=h0,
                                          state_chunk=sc, plan="lpar")
    torch.cuda.synchronize(DEV)
    res = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                 inp["delta_bias"], inp["delta_softplus"], h0=h0, chunk=sc or None)
    y_ref, last_ref = res[0], res[1]
    tol = TOL[c["dtype"]]
    assert rel_err(_host(y), y_ref) <= tol
    assert rel_err(_host(last), last_ref) <= 1e-4
    if sc:
        assert rel_err(_host(cs), res[2][..., 1:].transpose(0, 3, 1, 2)) <= 1e-4
