"""GPU test of ssm_scan_fwd_noalloc, the forward entry point that allocates
no device memory (its two-pass workspace lives in a fixed per-device scratch
array), called through the C ABI.

Its outputs must equal those of ssm_scan_fwd bit for bit (same plan, same
kernels) and match the float64 oracle within the float32 / bfloat16
bounds, on calls in a row whose second input is smaller than the first
(the scratch keeps the first call's contents), and on a shape whose plan
uses no scratch at all.
"""
import ctypes

import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads
from oracle import cpu

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))


def inputs(b, d, n, L, dtype, seed):
    w = workloads.Workload("t", b, d, n, L, "f32" if dtype == torch.float32 else "bf16", True, "normal", "dt_init")
    return workloads.make_inputs(w, device=DEV, seed=seed)


def call_noalloc(inp):
    """ssm_scan_fwd_noalloc through ctypes; outputs preallocated by the test."""
    lib = ssm.load_library()
    u = inp["u"]
    b, d, L = u.shape
    n = inp["A"].shape[1]
    y = torch.full_like(u, float("nan"))
    last = torch.full((b, d, n), float("nan"), device=DEV)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    dtype = ssm.SSM_F32 if u.dtype == torch.float32 else ssm.SSM_BF16
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    print(f"[noalloc] b={b} d={d} n={n} L={L} {u.dtype} plan {ssm.plan_for(b, d, n, L, u.dtype)}", flush=True)
    rc = lib.ssm_scan_fwd_noalloc(P(u), P(inp["delta"]), P(inp["A"]), P(inp["B"]), P(inp["C"]), P(inp["D"]),
                                  P(inp["z"]), P(inp["delta_bias"]), int(inp["delta_softplus"]), P(y), P(last),
                                  b, d, n, L, dtype, stream)
    assert rc == 0, lib.ssm_last_error().decode()
    torch.cuda.synchronize(DEV)
    return y, last


def check_against_fwd_and_oracle(inp):
    y, last = call_noalloc(inp)
    y_ref, last_ref = ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                       inp["delta_bias"], delta_softplus=inp["delta_softplus"])
    torch.cuda.synchronize(DEV)
    assert torch.equal(y, y_ref) and torch.equal(last, last_ref)
    yo, lo = cpu.fwd_full(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                          inp["delta_bias"], inp["delta_softplus"])
    assert rel_err(y.float().cpu().numpy(), yo) <= TOL[inp["u"].dtype]
    assert rel_err(last.cpu().numpy(), lo) <= 1e-4


def test_two_calls_second_smaller():
    """Two-pass plans (few channels, long L): the first call's workspace
    (16 chunks of 64 channels x 16 states) is larger than the second's
    (32 chunks of 16 channels x 8 states), which runs over the first call's
    leftovers."""
    big = inputs(1, 64, 16, 16384, torch.float32, seed=41)
    assert ssm.plan_for(1, 64, 16, 16384, torch.float32)["plan"] == "twopass"
    check_against_fwd_and_oracle(big)
    small = inputs(1, 16, 8, 32768, torch.bfloat16, seed=42)
    assert ssm.plan_for(1, 16, 8, 32768, torch.bfloat16)["plan"] == "twopass"
    check_against_fwd_and_oracle(small)


def test_thousand_chunks_then_single_pass():
    """The automatic plan at 1024 chunks (3 MiB of scratch), then a shape
    whose plan needs no scratch."""
    inp = inputs(1, 16, 16, 1 << 20, torch.float32, seed=43)
    check_against_fwd_and_oracle(inp)
    inp = inputs(2, 1536, 16, 512, torch.float32, seed=44)
    assert ssm.plan_for(2, 1536, 16, 512, torch.float32)["plan"] != "twopass"
    check_against_fwd_and_oracle(inp)


def test_binding_same_name():
    """The Python binding of the same name gives the same bits."""
    inp = inputs(1, 48, 16, 8192, torch.float32, seed=45)
    y, last = call_noalloc(inp)
    last2 = torch.empty_like(last)
    y2, _ = ssm.ssm_scan_fwd_noalloc(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                     inp["delta_bias"], delta_softplus=True, last_state=last2)
    torch.cuda.synchronize(DEV)
    assert torch.equal(y, y2) and torch.equal(last, last2)
