"""GPU parity of the row kernel's identity tiles against the float64 oracle.

A tile whose Delta2 and Delta*u are all zero and whose B is finite leaves the
states unchanged, and the one-wave (four states per lane) groups skip its
recurrence.  These cases pad one batch row with delta = -inf (softplus gives
Delta = 0 exactly), so that most of its tiles are such tiles, and plant the
non-finite values that must keep a tile on the full recurrence because the
plain definition turns them into NaN: B non-finite at a padded step (0 * B),
u infinite at a padded step (Delta * u), A infinite (exp(0 * A)).  Every
output element is compared: the NaN pattern exactly, the rest within the
forward's bound.
"""
import numpy as np
import pytest
import torch

from test_gpu_ssm import DEV, TOL, _host, oracle_all, rel_err, run_gpu, small_inputs

pytestmark = pytest.mark.gpu

B_, D_, N_, L_ = 2, 40, 16, 512
PAD = 200  # batch row 0 is padded from this step on


def padded(dtype, seed):
    inp = small_inputs(B_, D_, N_, L_, dtype=dtype, seed=seed)
    delta = inp["delta"].clone()
    delta[0, :, PAD:] = float("-inf")
    inp["delta"] = delta.contiguous()
    return inp


def check(inp):
    y, last = run_gpu(inp, plan="carry", states_per_lane=4)
    y_ref, last_ref = oracle_all(inp)
    yg, lg = _host(y), _host(last)
    np.testing.assert_array_equal(np.isnan(yg), np.isnan(y_ref))
    np.testing.assert_array_equal(np.isnan(lg), np.isnan(last_ref))
    ok, okl = ~np.isnan(y_ref), ~np.isnan(last_ref)
    assert rel_err(yg[ok], y_ref[ok]) <= TOL[inp["u"].dtype]
    assert rel_err(lg[okl], last_ref[okl]) <= 1e-4
    return y_ref, last_ref


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_padded_rows(dtype):
    y_ref, last_ref = check(padded(dtype, 90))
    assert np.isfinite(y_ref).all() and np.isfinite(last_ref).all()


@pytest.mark.parametrize("value", [float("nan"), float("inf")], ids=["nan", "inf"])
def test_non_finite_B_at_a_padded_step(value):
    inp = padded(torch.float32, 91)
    Bm = inp["B"].clone()
    Bm[0, 3, 300] = value
    inp["B"] = Bm.contiguous()
    y_ref, _ = check(inp)
    assert np.isnan(y_ref[0, :, 300:]).all() and not np.isnan(y_ref[1]).any()


def test_infinite_u_at_a_padded_step():
    inp = padded(torch.float32, 92)
    u = inp["u"].clone()
    u[0, 5, 400] = float("inf")
    inp["u"] = u.contiguous()
    y_ref, _ = check(inp)
    assert np.isnan(y_ref[0, 5, 400:]).all() and not np.isnan(y_ref[0, 4]).any()


def test_infinite_A_with_padding():
    inp = padded(torch.float32, 93)
    A = inp["A"].clone()
    A[7, 2] = float("-inf")
    inp["A"] = A.contiguous()
    y_ref, _ = check(inp)
    assert np.isnan(y_ref[0, 7, PAD:]).all() and not np.isnan(y_ref[1, 7]).any()


def _pad_cases(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        b = int(rng.integers(1, 5))
        L = int(rng.integers(32, 3000))
        out.append(dict(b=b, d=int(rng.integers(1, 70)), n=int(rng.integers(1, 17)), L=L,
                        dtype=(torch.float32, torch.bfloat16)[int(rng.integers(2))],
                        gated=bool(rng.integers(2)), with_D=bool(rng.integers(2)), with_bias=bool(rng.integers(2)),
                        lens=[int(x) for x in rng.integers(0, L + 1, size=b)], seed=int(rng.integers(1 << 20))))
    return out


PADS = _pad_cases(8801, 16)


@pytest.mark.parametrize("c", PADS, ids=lambda c: f"b{c['b']}d{c['d']}n{c['n']}L{c['L']}"
                         f"{'-bf16' if c['dtype'] == torch.bfloat16 else ''}")
def test_padded_rows_seeded_sweep(c):
    """Random sizes and a random length per batch row (delta = -inf past it,
    lengths from 0 to L), through the four-states-per-lane carry plan:
    every element against the float64 oracle."""
    inp = small_inputs(c["b"], c["d"], c["n"], c["L"], dtype=c["dtype"], gated=c["gated"], with_D=c["with_D"],
                       with_bias=c["with_bias"], seed=c["seed"])
    delta = inp["delta"].clone()
    for bi, ln in enumerate(c["lens"]):
        delta[bi, :, ln:] = float("-inf")
    inp["delta"] = delta.contiguous()
    check(inp)
