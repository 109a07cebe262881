"""The plain-C oracle: its float64 recurrence against the NumPy oracle and
the brute-force expansion, and its float32 replay of the blocked scan order
against exact and serial results."""
import numpy as np
import pytest
import torch

import workloads
from oracle import ref


def _rows(inp):
    u, dl, z = inp["u"], inp["delta"], inp["z"]
    b, d, L = u.shape
    return b, d, L


@pytest.mark.parametrize("gated,softplus,with_D", [(True, True, True), (False, True, False),
                                                   (True, False, True), (False, False, False)])
def test_c_oracle_matches_numpy_oracle(oracle_lib, gated, softplus, with_D):
    from oracle import cpu
    rng = np.random.default_rng(20)
    bsz, d, n, L = 3, 7, 5, 97
    u = rng.normal(size=(bsz, d, L)).astype(np.float32)
    dl = (rng.normal(size=(bsz, d, L)) if softplus else rng.uniform(0.001, 0.3, (bsz, d, L))).astype(np.float32)
    z = rng.normal(size=(bsz, d, L)).astype(np.float32) if gated else None
    A = (-np.exp(rng.normal(size=(d, n)))).astype(np.float32)
    B = rng.normal(size=(bsz, n, L)).astype(np.float32)
    C = rng.normal(size=(bsz, n, L)).astype(np.float32)
    D = rng.normal(size=d).astype(np.float32) if with_D else None
    bias = (rng.normal(size=d) * 0.3).astype(np.float32)
    y1, l1 = ref.selective_scan_fwd(u, dl, A, B, C, D, z, bias, softplus)
    y2, l2 = cpu.fwd_full(u, dl, A, B, C, D, z, bias, softplus)
    assert np.max(np.abs(y1 - y2)) <= 1e-12 * np.max(np.abs(y1))
    assert np.max(np.abs(l1 - l2)) <= 1e-12 * np.max(np.abs(l1))


def test_c_oracle_matches_bruteforce(oracle_lib):
    from oracle import cpu
    rng = np.random.default_rng(21)
    bsz, d, n, L = 1, 2, 3, 7
    u = rng.normal(size=(bsz, d, L)).astype(np.float32)
    dl = rng.normal(size=(bsz, d, L)).astype(np.float32)
    z = rng.normal(size=(bsz, d, L)).astype(np.float32)
    A = (-np.exp(rng.normal(size=(d, n)))).astype(np.float32)
    B = rng.normal(size=(bsz, n, L)).astype(np.float32)
    C = rng.normal(size=(bsz, n, L)).astype(np.float32)
    D = rng.normal(size=d).astype(np.float32)
    y1, l1 = ref.selective_scan_bruteforce(u, dl, A, B, C, D, z, None, True)
    y2, l2 = cpu.fwd_full(u, dl, A, B, C, D, z, None, True)
    assert np.max(np.abs(y1 - y2)) <= 1e-12 * np.max(np.abs(y1))
    assert np.max(np.abs(l1 - l2)) <= 1e-12 * np.max(np.abs(l1))


def test_c_oracle_row_selection_and_threads(oracle_lib):
    """Selected rows equal the same rows of the full problem; thread count
    does not change the (per-row serial) result."""
    from oracle import cpu
    w = workloads.WORKLOADS["tiny"].with_sizes(batch=2, dim=16, L=64)
    inp = workloads.make_inputs(w)
    yf, lf = cpu.fwd_full(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                          inp["delta_bias"], True, nthreads=1)
    rb = np.array([1, 0, 1]); rd = np.array([3, 15, 0])
    ys, ls = cpu.fwd_rows(inp["u"][rb, rd], inp["delta"][rb, rd], inp["z"][rb, rd], rb, rd, inp["A"], inp["B"],
                          inp["C"], inp["D"], inp["delta_bias"], True, 2, 16, 16, 64, nthreads=4)
    assert np.array_equal(ys, yf[rb, rd]) and np.array_equal(ls, lf[rb, rd])


def test_c_oracle_rejects_bad_rows(oracle_lib):
    from oracle import cpu
    x = np.zeros((1, 4), np.float32)
    with pytest.raises(ValueError):
        cpu.fwd_rows(x, x, None, [0], [5], np.zeros((2, 1)), np.zeros((1, 1, 4)), np.zeros((1, 1, 4)),
                     None, None, False, 1, 2, 1, 4)


def test_tiny_workload_numpy_vs_c(oracle_lib):
    from oracle import cpu
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"])
    y1, l1 = ref.selective_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                    inp["delta_bias"], True)
    y2, l2 = cpu.fwd_full(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                          inp["delta_bias"], True)
    assert np.max(np.abs(y1 - y2)) <= 1e-12 * np.max(np.abs(y1))
    assert np.max(np.abs(l1 - l2)) <= 1e-12 * np.max(np.abs(l1))


# ------------------------------------------------------------ float32 replay

def test_replay_single_lane_is_the_serial_fold(oracle_lib):
    """With one lane, one wave and T = L the blocked order degenerates to the
    plain serial fold; the replay must then be bit-identical to it."""
    from oracle import cpu
    rng = np.random.default_rng(30)
    for L in (1, 5, 64, 333):
        a = rng.uniform(0, 1.2, (4, L)).astype(np.float32)
        b = rng.normal(size=(4, L)).astype(np.float32)
        sa, sb = cpu.affine_serial_f32(a, b)
        ra, rb = cpu.affine_replay_f32(a, b, T=L, lanes=1, W=1)
        assert np.array_equal(sa, ra) and np.array_equal(sb, rb)


@pytest.mark.parametrize("T,lanes,W", [(8, 64, 4), (4, 64, 1), (1, 64, 2), (3, 16, 3), (8, 32, 2)])
def test_replay_exact_on_integer_resets(oracle_lib, T, lanes, W):
    """a in {0, 1} and small integer b keep every partial result an integer
    below 2^24, so any association order is exact: the replay must equal the
    float64 serial scan bit for bit (a wrong index, lane partner or carry
    would change some integer)."""
    from oracle import cpu
    rng = np.random.default_rng(31)
    for L in (1, 63, 64 * T * W, 64 * T * W + 1, 3 * 64 * T * W - 17, 5000):
        a = (rng.uniform(0, 1, (3, L)) < 0.97).astype(np.float32)
        b = rng.integers(-8, 9, (3, L)).astype(np.float32)
        ra, rb = cpu.affine_replay_f32(a, b, T, lanes, W)
        ea, eb = ref.affine_scan(a, b)
        assert np.array_equal(ra.astype(np.float64), ea) and np.array_equal(rb.astype(np.float64), eb)


def test_replay_exact_on_power_of_two_products(oracle_lib):
    """a in {1/2, 1, 2} with b = 0: every prefix product is an exact power of
    two (kept within float32 range), so out_a must be exact in any order."""
    from oracle import cpu
    rng = np.random.default_rng(32)
    L = 7000
    a = np.empty((2, L), np.float32)
    for r in range(2):
        e = 0
        for t in range(L):
            step = rng.integers(-1, 2)
            if abs(e + step) > 60:
                step = -step
            e += step
            a[r, t] = 2.0 ** step
    ra, rb = cpu.affine_replay_f32(a, np.zeros_like(a), 8, 64, 4)
    ea, _ = ref.affine_scan(a, np.zeros_like(a))
    assert np.array_equal(ra.astype(np.float64), ea) and np.all(rb == 0)


def test_replay_close_to_float64_and_order_specific(oracle_lib):
    """Random inputs: the replay agrees with the float64 scan to float32
    rounding, and differs in some bits from the serial float32 fold
    (it really follows its own order)."""
    from oracle import cpu
    rng = np.random.default_rng(33)
    L = 6000
    a = np.exp(-rng.uniform(0, 0.05, (4, L))).astype(np.float32)
    b = rng.normal(size=(4, L)).astype(np.float32)
    ra, rb = cpu.affine_replay_f32(a, b, 8, 64, 4)
    ea, eb = ref.affine_scan(a, b)
    assert np.max(np.abs(rb - eb)) <= 2e-5 * np.max(np.abs(eb))
    normal = ea > 1e-30  # below that float32 products flush through the subnormal range
    assert np.max(np.abs(ra - ea)[normal] / ea[normal]) <= 2e-4
    assert np.all(np.abs(ra - ea)[~normal] <= 1e-30)
    sa, sb = cpu.affine_serial_f32(a, b)
    assert not np.array_equal(sb, rb)


def test_c_oracle_start_state_and_chunk_states(oracle_lib):
    """The C recurrence from a given start state, with the chunk-boundary
    states, equals the NumPy oracle's."""
    rng = np.random.default_rng(31)
    bsz, d, n, L, ch = 2, 5, 6, 70, 16
    u = rng.normal(size=(bsz, d, L)).astype(np.float32)
    dl = rng.normal(size=(bsz, d, L)).astype(np.float32)
    z = rng.normal(size=(bsz, d, L)).astype(np.float32)
    A = (-np.exp(rng.normal(size=(d, n)))).astype(np.float32)
    B = rng.normal(size=(bsz, n, L)).astype(np.float32)
    C = rng.normal(size=(bsz, n, L)).astype(np.float32)
    D = rng.normal(size=d).astype(np.float32)
    h0 = rng.normal(size=(bsz, d, n))
    y_ref, last_ref, bnd_ref = ref.selective_scan_fwd(u, dl, A, B, C, D=D, z=z, delta_softplus=True, h0=h0,
                                                      chunk=ch)
    rb, rd = np.meshgrid(np.arange(bsz), np.arange(d), indexing="ij")
    from oracle import cpu
    y, last, bnd = cpu.fwd_rows(u.reshape(-1, L), dl.reshape(-1, L), z.reshape(-1, L), rb.ravel(), rd.ravel(),
                                A, B, C, D, None, True, bsz, d, n, L, h0_rows=h0.reshape(-1, n), chunk=ch)
    K = -(-L // ch)
    assert bnd.shape == (bsz * d, K, n)
    assert np.max(np.abs(y.reshape(bsz, d, L) - y_ref)) <= 1e-12 * np.max(np.abs(y_ref))
    assert np.max(np.abs(last.reshape(bsz, d, n) - last_ref)) <= 1e-12 * np.max(np.abs(last_ref))
    # the NumPy oracle also keeps h_0 in front: its entries 1..K are the C oracle's 0..K-1
    got = bnd.reshape(bsz, d, K, n).transpose(0, 1, 3, 2)
    assert np.max(np.abs(got - bnd_ref[..., 1:])) <= 1e-12 * np.max(np.abs(bnd_ref))
