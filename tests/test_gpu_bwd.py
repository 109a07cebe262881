"""GPU parity of ssm_scan_bwd (gradients by chunked recomputation) against
the float64 gradient oracle, through the C ABI.

The chunk states come from the GPU forward (ssm_scan_fwd_states with the
same state_chunk), as in training.  Metric per output tensor:
max |gpu - oracle| / max |oracle|, bounded by 1e-4 for float32 results and
2e-2 for the bfloat16-stored ones (du, ddelta, dz with bfloat16 I/O: one
bfloat16 rounding is 2^-9 relative).  dB and dC are float32 for either
dtype, but with bfloat16 I/O their terms carry the bfloat16-rounded
recomputed inputs no more than the forward does, so they keep 1e-4.
"""
import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads
from oracle import cpu, ref

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GKEYS = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0")
IO_KEYS = ("du", "ddelta", "dz")


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    scale = np.max(np.abs(want))
    return float(np.max(np.abs(got - want)) / (scale if scale > 0 else 1.0))


def tol(key, dtype):
    return 2e-2 if (dtype == torch.bfloat16 and key in IO_KEYS) else 1e-4


def _host(t):
    return None if t is None else t.detach().float().cpu().numpy()


def make(b, d, n, L, dtype, seed, gated=True, softplus=True, with_D=True, with_bias=True, with_h0=True,
         with_dlast=True, A_random=True):
    w = workloads.Workload("t", b, d, n, L, "f32" if dtype == torch.float32 else "bf16", gated,
                           "normal" if with_D else None, "dt_init", softplus=softplus)
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    if A_random:
        inp["A"] = workloads.random_A(d, n, device=DEV, seed=seed + 1)
    if not with_bias:
        inp["delta_bias"] = None
    gr = workloads.make_grads(w, device=DEV, seed=seed)
    inp["dy"] = gr["dy"]
    inp["dlast"] = gr["dlast"] if with_dlast else None
    if with_h0:
        g = torch.Generator(device=DEV)
        g.manual_seed(seed + 2)
        inp["h0"] = torch.randn((b, d, n), generator=g, device=DEV, dtype=torch.float32)
    else:
        inp["h0"] = None
    return inp


def run_gpu(inp, state_chunk, S=0):
    _, _, cs = ssm.ssm_scan_fwd_states(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                       inp["delta_bias"], delta_softplus=inp["delta_softplus"], h0=inp["h0"],
                                       state_chunk=state_chunk)
    g = ssm.ssm_scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], cs, state_chunk, inp["dy"],
                         D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                         delta_softplus=inp["delta_softplus"], h0=inp["h0"], dlast=inp["dlast"], states_per_lane=S)
    torch.cuda.synchronize(DEV)
    return g


def run_oracle(inp, use_c=False):
    args = (inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"])
    kw = dict(D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], delta_softplus=inp["delta_softplus"],
              h0=inp["h0"], dy=inp["dy"], dlast=inp["dlast"])
    if use_c:
        return cpu.bwd_full(*args, **kw)
    return ref.selective_scan_bwd(*args, **kw)


def check(got, want, dtype, label):
    for k in GKEYS:
        if want[k] is None or got[k] is None:
            continue
        e = rel_err(_host(got[k]), want[k])
        assert e <= tol(k, dtype), f"{label}: {k} rel err {e:.3g}"


CASES = [
    # b, d, n, L, state_chunk, S
    (1, 16, 16, 64, 32, 1),
    (1, 16, 16, 64, 32, 2),
    (1, 16, 16, 64, 32, 4),
    (2, 40, 16, 150, 64, 1),
    (2, 40, 16, 150, 64, 2),
    (2, 40, 16, 150, 64, 4),
    (1, 32, 16, 517, 128, 0),
    (2, 24, 8, 300, 512, 2),
    (1, 16, 5, 97, 32, 4),
    (3, 17, 16, 1, 32, 2),
    (1, 20, 16, 16, 32, 4),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}sc{c[4]}S{c[5]}" for c in CASES])
def test_bwd_matches_oracle(case, dtype):
    b, d, n, L, sc, S = case
    inp = make(b, d, n, L, dtype, seed=17 + L)
    check(run_gpu(inp, sc, S), run_oracle(inp), dtype, str(case))


@pytest.mark.parametrize("flags", [
    dict(gated=False, softplus=False, with_D=False, with_bias=False, with_h0=False, with_dlast=False),
    dict(gated=False, softplus=True, with_D=True, with_bias=True, with_h0=False, with_dlast=True),
    dict(gated=True, softplus=False, with_D=False, with_bias=True, with_h0=True, with_dlast=False),
], ids=["bare", "nogate", "nosoftplus"])
@pytest.mark.parametrize("S", [1, 2, 4])
def test_bwd_optional_inputs(flags, S):
    inp = make(2, 33, 16, 200, torch.float32, seed=5, **flags)
    if not flags["softplus"]:
        # without softplus Delta = delta + bias must stay positive for a
        # bounded recurrence: take |delta| * 0.05 and a small positive bias
        inp["delta"] = inp["delta"].abs() * 0.05
        if inp["delta_bias"] is not None:
            inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
    check(run_gpu(inp, 64, S), run_oracle(inp), torch.float32, str(flags))


def test_bwd_state_chunks_agree():
    """The result does not depend on state_chunk beyond float32 rounding."""
    inp = make(1, 32, 16, 700, torch.float32, seed=9)
    want = run_oracle(inp)
    for sc in (32, 96, 256, 512):
        check(run_gpu(inp, sc), want, torch.float32, f"sc={sc}")


def test_bwd_repeat_is_stable():
    """Two runs agree to float32 rounding (the atomic sums may differ in the
    last bits); the per-element gradients are identical."""
    inp = make(2, 48, 16, 256, torch.float32, seed=4)
    g1 = run_gpu(inp, 128)
    g2 = run_gpu(inp, 128)
    for k in ("du", "ddelta", "dz", "dh0"):
        assert torch.equal(g1[k], g2[k]), k
    for k in ("dA", "dB", "dC", "dD", "ddelta_bias"):
        assert rel_err(_host(g1[k]), _host(g2[k])) < 1e-6, k


@pytest.mark.parametrize("name,sc", [("130m", 128), ("1.4b", 128)])
def test_bwd_full_size(name, sc):
    """Full benchmark shapes (b=8, d=1536 / 4096, n=16, L=2048), every
    gradient element against the C oracle."""
    w = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(w, device=DEV, seed=0)
    gr = workloads.make_grads(w, device=DEV, seed=0)
    inp.update(dy=gr["dy"], dlast=gr["dlast"], h0=None)
    print(f"[bwd full] {name} sc={sc}", flush=True)
    got = run_gpu(inp, sc)
    want = run_oracle(inp, use_c=True)
    check(got, want, w.torch_dtype, name)


# ------------------------------------------------------- conv1d + SiLU in front

CONV_CASES = [
    # b, d, n, L, state_chunk, S, K
    (1, 16, 16, 64, 32, 1, 4),
    (2, 40, 16, 150, 64, 2, 4),
    (2, 40, 16, 150, 64, 4, 3),
    (1, 33, 16, 517, 128, 0, 2),
    (2, 24, 8, 77, 32, 2, 1),
    (1, 20, 16, 3, 32, 1, 4),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CONV_CASES,
                         ids=[f"b{c[0]}d{c[1]}n{c[2]}L{c[3]}sc{c[4]}S{c[5]}K{c[6]}" for c in CONV_CASES])
def test_bwd_conv_matches_oracle(case, dtype):
    b, d, n, L, sc, S, K = case
    inp = make(b, d, n, L, dtype, seed=50 + L + K)
    g = torch.Generator(device=DEV)
    g.manual_seed(9 + K)
    conv_w = torch.randn((d, K), generator=g, device=DEV) * (1.0 / K)
    conv_b = torch.randn((d,), generator=g, device=DEV) * 0.1
    x = inp["u"]
    _, _, cs, _ = ssm.ssm_scan_fwd_conv(x, conv_w, inp["delta"], inp["A"], inp["B"], inp["C"], conv_b=conv_b,
                                        D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                        delta_softplus=inp["delta_softplus"], h0=inp["h0"], state_chunk=sc)
    got = ssm.ssm_scan_bwd_conv(x, conv_w, inp["delta"], inp["A"], inp["B"], inp["C"], cs, sc, inp["dy"],
                                conv_b=conv_b, D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"],
                                delta_softplus=inp["delta_softplus"], h0=inp["h0"], dlast=inp["dlast"],
                                states_per_lane=S)
    torch.cuda.synchronize(DEV)
    u = ref.causal_conv1d(x, conv_w, conv_b)
    want = ref.selective_scan_bwd(u, inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                                  delta_bias=inp["delta_bias"], delta_softplus=inp["delta_softplus"], h0=inp["h0"],
                                  dy=inp["dy"], dlast=inp["dlast"])
    dx, dw, db = ref.causal_conv1d_silu_bwd(x, conv_w, conv_b, want["du"])
    want.update(dx=dx, dconv_w=dw, dconv_b=db)
    for k in ("dx", "dconv_w", "dconv_b", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dh0"):
        if want.get(k) is None or got.get(k) is None:
            continue
        bound = 2e-2 if (dtype == torch.bfloat16 and k in ("dx", "ddelta", "dz")) else 1e-4
        e = rel_err(_host(got[k]), want[k])
        assert e <= bound, f"{case}: {k} rel err {e:.3g}"
