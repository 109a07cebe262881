"""GPU parity of ssm_out_proj (the Linear after the gated scan, on the
matrix cores) against the float64 oracle, through the C ABI.

Metric: max |gpu - oracle| / max |oracle| over the compared outputs.  Bound
1e-4 for float32 storage (float32 products summed in float32 over d_inner
terms); 2e-2 for bfloat16 storage (the products of bfloat16 values are exact
in float32; the one bfloat16 rounding of the result is 2^-9 relative).  The
oracle sees the stored (bfloat16-rounded) inputs, upcast exactly.
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


def tol(dtype):
    return 2e-2 if dtype == torch.bfloat16 else 1e-4


CASES = [
    # batch, d_inner, d_model, L
    (1, 64, 64, 64),          # one partial tile
    (2, 256, 256, 256),       # whole bfloat16 tiles
    (2, 200, 136, 300),       # ragged in every dimension, vector path (multiples of 8 / 4)
    (1, 1536, 768, 517),      # 130m widths, ragged length (element path)
    (3, 100, 72, 96),         # d_inner not a multiple of 8: element path for bfloat16
    (2, 37, 30, 19),          # nothing aligned: element path, partial stores
    (3, 40, 24, 1),           # one step
    (1, 1, 16, 40),           # d_inner = 1
    (1, 520, 260, 260),       # one past a tile in every dimension
    # every size a multiple of 8: the bfloat16 path that loads straight into
    # LDS, with a K tail shorter than its 32-value stage (forward K = d_inner,
    # dy K = d_model, dW K = L) and ragged M and N tiles
    (2, 200, 136, 304),
    (3, 520, 264, 264),
    (4, 320, 136, 200),
    (1, 8, 8, 8),
    (2, 1544, 776, 520),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}k{c[1]}m{c[2]}L{c[3]}" for c in CASES])
def test_out_proj_matches_oracle(case, dtype):
    b, dk, dm, L = case
    print(f"[proj] {case} {dtype}", flush=True)
    inp = workloads.make_proj_inputs(b, dk, dm, L, dtype=dtype, device=DEV, seed=sum(case))
    out = ssm.ssm_out_proj(inp["y"], inp["W"])
    torch.cuda.synchronize(DEV)
    assert out.shape == (b, L, dm) and out.dtype == dtype
    want = ref.out_proj(inp["y"], inp["W"])
    e = rel_err(out.float().cpu().numpy(), want)
    assert e <= tol(dtype), f"{case}: rel err {e:.3g}"


def test_out_proj_writes_nothing_outside_out():
    """A given out buffer inside a larger allocation: the guard bands around
    it keep their values (partial tiles store nothing past the edges)."""
    b, dk, dm, L = 2, 72, 36, 70
    inp = workloads.make_proj_inputs(b, dk, dm, L, dtype=torch.float32, device=DEV, seed=3)
    n = b * L * dm
    big = torch.full((n + 2048,), 7.0, device=DEV)
    out = big[1024:1024 + n].view(b, L, dm)
    ssm.ssm_out_proj(inp["y"], inp["W"], out=out)
    torch.cuda.synchronize(DEV)
    assert torch.all(big[:1024] == 7.0) and torch.all(big[1024 + n:] == 7.0)
    e = rel_err(out.cpu().numpy(), ref.out_proj(inp["y"], inp["W"]))
    assert e <= 1e-4


def test_out_proj_repeat_is_bitwise_stable():
    inp = workloads.make_proj_inputs(2, 512, 256, 384, dtype=torch.bfloat16, device=DEV, seed=8)
    o1 = ssm.ssm_out_proj(inp["y"], inp["W"])
    o2 = ssm.ssm_out_proj(inp["y"], inp["W"])
    torch.cuda.synchronize(DEV)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("name", ["130m", "1.4b"])
def test_out_proj_full_size_sampled(name):
    """The layer shapes (130m: d_inner 1536 -> d_model 768, float32; 1.4b:
    4096 -> 2048, bfloat16; b=8, L=2048), the launch the benchmark times:
    every d_model output of 96 sampled (batch row, step) tokens against the
    oracle, the first and last token of every row included."""
    w = workloads.WORKLOADS[name]
    dm = workloads.d_model_of(w)
    inp = workloads.make_proj_inputs(w.batch, w.dim, dm, w.L, dtype=w.torch_dtype, device=DEV, seed=0)
    print(f"[proj full] {name}", flush=True)
    out = ssm.ssm_out_proj(inp["y"], inp["W"])
    torch.cuda.synchronize(DEV)
    rng = np.random.default_rng(0)
    pairs = [(b, 0) for b in range(w.batch)] + [(b, w.L - 1) for b in range(w.batch)]
    pairs += [(int(rng.integers(w.batch)), int(rng.integers(w.L))) for _ in range(96 - len(pairs))]
    want = ref.out_proj_tokens(inp["y"], inp["W"], pairs)
    got = np.stack([out[b, t].float().cpu().numpy() for b, t in pairs])
    e = rel_err(got, want)
    assert e <= tol(w.torch_dtype), f"{name}: rel err {e:.3g}"


# ------------------------------------------------------------------ gradients

def _bwd_inputs(b, dk, dm, L, dtype, seed):
    inp = workloads.make_proj_inputs(b, dk, dm, L, dtype=dtype, device=DEV, seed=seed)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 7)
    inp["dout"] = torch.randn((b, L, dm), generator=g, device=DEV).to(dtype).contiguous()
    return inp


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"b{c[0]}k{c[1]}m{c[2]}L{c[3]}" for c in CASES])
def test_out_proj_bwd_matches_oracle(case, dtype):
    """dy and dW against the float64 gradient oracle (ragged sizes; with
    several batch rows the dW sum is split over workgroups and reduced)."""
    b, dk, dm, L = case
    print(f"[proj bwd] {case} {dtype}", flush=True)
    inp = _bwd_inputs(b, dk, dm, L, dtype, seed=3 * sum(case))
    dy, dW = ssm.ssm_out_proj_bwd(inp["y"], inp["W"], inp["dout"])
    torch.cuda.synchronize(DEV)
    want_dy, want_dW = ref.out_proj_bwd(inp["y"], inp["W"], inp["dout"])
    e1 = rel_err(dy.float().cpu().numpy(), want_dy)
    e2 = rel_err(dW.float().cpu().numpy(), want_dW)
    assert e1 <= tol(dtype) and e2 <= tol(dtype), f"{case}: dy {e1:.3g} dW {e2:.3g}"


def test_out_proj_bwd_one_output_and_repeatability():
    """dy alone and dW alone give what the joint call gives; dW (split over
    the batch rows and summed in a fixed order) is bitwise repeatable."""
    inp = _bwd_inputs(4, 320, 136, 200, torch.bfloat16, seed=21)
    dy, dW = ssm.ssm_out_proj_bwd(inp["y"], inp["W"], inp["dout"])
    dy1, none1 = ssm.ssm_out_proj_bwd(inp["y"], inp["W"], inp["dout"], want_dW=False)
    none2, dW1 = ssm.ssm_out_proj_bwd(inp["y"], inp["W"], inp["dout"], want_dy=False)
    _, dW2 = ssm.ssm_out_proj_bwd(inp["y"], inp["W"], inp["dout"], want_dy=False)
    torch.cuda.synchronize(DEV)
    assert none1 is None and none2 is None
    assert torch.equal(dy, dy1) and torch.equal(dW, dW1) and torch.equal(dW1, dW2)


@pytest.mark.parametrize("name", ["130m", "1.4b"])
def test_out_proj_bwd_full_size_sampled(name):
    """The layer shapes, the launches the benchmark times: 24 sampled (batch
    row, channel) rows of dy and 24 sampled rows of dW, every element of each,
    against the oracle's definition evaluated for those rows."""
    w = workloads.WORKLOADS[name]
    dm = workloads.d_model_of(w)
    print(f"[proj bwd full] {name}", flush=True)
    inp = _bwd_inputs(w.batch, w.dim, dm, w.L, w.torch_dtype, seed=0)
    dy, dW = ssm.ssm_out_proj_bwd(inp["y"], inp["W"], inp["dout"])
    torch.cuda.synchronize(DEV)
    rng = np.random.default_rng(1)
    W_h = inp["W"].double().cpu().numpy()
    rows = [(int(rng.integers(w.batch)), int(rng.integers(w.dim))) for _ in range(24)]
    got = np.stack([dy[b, k].double().cpu().numpy() for b, k in rows])
    want = np.stack([W_h[:, k] @ inp["dout"][b].double().cpu().numpy().T for b, k in rows])
    e1 = rel_err(got, want)
    ms = [int(v) for v in rng.integers(dm, size=24)]
    dout_h = [inp["dout"][b].double().cpu().numpy() for b in range(w.batch)]
    y_h = [inp["y"][b].double().cpu().numpy() for b in range(w.batch)]
    want_w = np.stack([sum(dout_h[b][:, m] @ y_h[b].T for b in range(w.batch)) for m in ms])
    got_w = np.stack([dW[m].double().cpu().numpy() for m in ms])
    e2 = rel_err(got_w, want_w)
    assert e1 <= tol(w.torch_dtype) and e2 <= tol(w.torch_dtype), f"{name}: dy {e1:.3g} dW {e2:.3g}"
