"""GPU affine_scan against (1) the float32 CPU replay of its documented
association order -- bit for bit -- and (2) the float64 serial oracle."""
import numpy as np
import pytest
import torch

import selective_state_space_ssm_amd as ssm
from oracle import ref

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(rows, L, seed, kind="decay"):
    g = torch.Generator().manual_seed(seed)
    if kind == "decay":
        a = torch.exp(-torch.rand((rows, L), generator=g) * 0.2)
    elif kind == "wide":  # decays, growth, exact zeros and tiny values (subnormal products)
        a = torch.exp(torch.randn((rows, L), generator=g) * 2.0)
        a[torch.rand((rows, L), generator=g) < 0.01] = 0.0
        a[torch.rand((rows, L), generator=g) < 0.01] = 1e-30
    else:
        raise ValueError(kind)
    b = torch.randn((rows, L), generator=g)
    return a.float().contiguous(), b.float().contiguous()


def bits_equal(x, y):
    """Same float32 bit patterns everywhere, except that any NaN matches any
    NaN (x86 and the GPU produce different default NaN encodings)."""
    x = np.asarray(x, np.float32)
    y = np.asarray(y, np.float32)
    nx, ny = np.isnan(x), np.isnan(y)
    return bool(np.array_equal(nx, ny) and np.array_equal(x[~nx].view(np.uint32), y[~ny].view(np.uint32)))


def _replay(a, b):
    from oracle import cpu
    o = ssm.affine_scan_order()
    return cpu.affine_replay_f32(a.numpy(), b.numpy(), o["items_per_lane"], o["lanes"], o["waves"])


SHAPES = [(1, 1), (3, 7), (2, 64), (5, 2048), (2, 2049), (4, 10000), (64, 4096), (300, 777), (1, 65536)]


@pytest.mark.parametrize("rows,L", SHAPES)
@pytest.mark.parametrize("kind", ["decay", "wide"])
def test_bit_exact_against_replay(rows, L, kind):
    a, b = _inputs(rows, L, seed=rows * 1000 + L, kind=kind)
    oa, ob = ssm.affine_scan(a.to(DEV), b.to(DEV))
    torch.cuda.synchronize(DEV)
    ra, rb = _replay(a, b)
    got_a, got_b = oa.cpu().numpy(), ob.cpu().numpy()
    # compare bit patterns (distinguishes -0 from +0)
    assert bits_equal(got_b, rb)
    assert bits_equal(got_a, ra)


@pytest.mark.parametrize("rows,L", [(4, 5000), (16, 2048)])
def test_close_to_float64(rows, L):
    a, b = _inputs(rows, L, seed=7)
    oa, ob = ssm.affine_scan(a.to(DEV), b.to(DEV))
    ea, eb = ref.affine_scan(a.numpy(), b.numpy())
    got_b = ob.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_b - eb)) <= 1e-5 * np.max(np.abs(eb))
    got_a = oa.cpu().numpy().astype(np.float64)
    normal = ea > 1e-30
    assert np.max(np.abs(got_a - ea)[normal] / ea[normal]) <= 1e-4


def test_in_place_and_no_products():
    a, b = _inputs(8, 3000, seed=9)
    ra, rb = _replay(a, b)
    ad, bd = a.to(DEV), b.to(DEV)
    oa, ob = ssm.affine_scan(ad, bd, out_a=ad, out_b=bd)  # in place
    torch.cuda.synchronize(DEV)
    assert oa.data_ptr() == ad.data_ptr() and ob.data_ptr() == bd.data_ptr()
    assert bits_equal(ob.cpu().numpy(), rb)
    assert bits_equal(oa.cpu().numpy(), ra)
    oa2, ob2 = ssm.affine_scan(a.to(DEV), b.to(DEV), return_a=False)
    assert oa2 is None
    assert bits_equal(ob2.cpu().numpy(), rb)


def test_forgetting_steps_exact():
    """a_t = 0 gives h_t = b_t exactly, whatever came before."""
    a, b = _inputs(4, 4096, seed=11)
    a[:, ::97] = 0.0
    _, ob = ssm.affine_scan(a.to(DEV), b.to(DEV), return_a=False)
    got = ob.cpu()
    assert torch.equal(got[:, ::97], b[:, ::97])


def test_repeatable():
    a, b = _inputs(32, 6000, seed=13, kind="wide")
    ad, bd = a.to(DEV), b.to(DEV)
    oa0, ob0 = ssm.affine_scan(ad, bd)
    for _ in range(5):
        oa1, ob1 = ssm.affine_scan(ad, bd)
        assert bits_equal(oa0.cpu().numpy(), oa1.cpu().numpy()) and bits_equal(ob0.cpu().numpy(), ob1.cpu().numpy())
