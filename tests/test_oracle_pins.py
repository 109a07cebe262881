"""Pins for the CPU oracle: facts the pages and the mathematics fix, each
chosen so that a plausible mistake in the oracle (a dropped term, a wrong
sign or index, swapped operands) fails at least one of them.

Pages: [Scan page] "Hardware-aware parallel associative scan for Mamba";
[Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
optimisation"; [Truth page] "The hardware truth of Mamba's parallel scan".
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac_pairs(rng, shape, L):
    """Random exact rationals: a in {0, 1/8, ..., 2}, b in {-4, ..., 4}/4."""
    a = np.empty(shape + (L,), dtype=object)
    b = np.empty(shape + (L,), dtype=object)
    for idx in np.ndindex(a.shape):
        a[idx] = Fraction(rng.randint(0, 16), 8)
        b[idx] = Fraction(rng.randint(-16, 16), 4)
    return a, b


# ---------------------------------------------------------------- monoid

def test_compose_matches_sequential_application():
    """[Scan page] §1.2 checks (a2,b2)o(a1,b1) by applying step 1 then step 2
    to h; do that on exact rationals."""
    rng = random.Random(0)
    for _ in range(500):
        a1, b1, a2, b2, h = (Fraction(rng.randint(-50, 50), rng.randint(1, 9)) for _ in range(5))
        h1 = a1 * h + b1
        h2 = a2 * h1 + b2
        pa, pb = ref.compose((a2, b2), (a1, b1))
        assert pa * h + pb == h2
    # the order matters: o is not commutative
    assert ref.compose((2, 1), (3, 5)) != ref.compose((3, 5), (2, 1))


def test_associativity_exact_random_triples():
    """o is associative ([Scan page] §1.2; proof in [Mamba-2 page] §2.3):
    brute force on 10^4 random triples in exact rationals."""
    rng = random.Random(1)
    for _ in range(10000):
        p, q, r = ((Fraction(rng.randint(-30, 30), rng.randint(1, 7)),
                    Fraction(rng.randint(-30, 30), rng.randint(1, 7))) for _ in range(3))
        left = ref.compose(ref.compose(r, q), p)
        right = ref.compose(r, ref.compose(q, p))
        assert left == right


def test_associativity_fp64_is_close_not_exact():
    """In floating point the two bracketings agree only up to rounding
    ([Scan page] §1.2 warning): a few ulp, and not always bit-equal."""
    rng = np.random.default_rng(2)
    a = rng.uniform(0, 1, (3, 100000))
    b = rng.normal(size=(3, 100000))
    p, q, r = [(a[i], b[i]) for i in range(3)]
    la, lb = ref.compose(ref.compose(r, q), p)
    ra, rb = ref.compose(r, ref.compose(q, p))
    scale = np.abs(b).sum(axis=0) + 1
    assert np.max(np.abs(lb - rb) / scale) < 4 * np.finfo(np.float64).eps
    assert np.max(np.abs(la - ra) / np.maximum(np.abs(la), 1e-300)) < 4 * np.finfo(np.float64).eps
    assert np.any(lb != rb)


def test_identity_exact():
    """(1, 0) is a two-sided identity, exactly in float64 ([Scan page] §1.2)."""
    rng = np.random.default_rng(3)
    a = rng.uniform(-2, 2, 1000)
    b = rng.normal(size=1000)
    one, zero = np.ones(1000), np.zeros(1000)
    la, lb = ref.compose((one, zero), (a, b))
    ra, rb = ref.compose((a, b), (one, zero))
    assert np.array_equal(la, a) and np.array_equal(lb, b)
    assert np.array_equal(ra, a) and np.array_equal(rb, b)


# ---------------------------------------------------------------- scans

@pytest.mark.parametrize("L", list(range(1, 65)))
def test_scans_agree_exactly(L):
    """Serial, Hillis-Steele and Blelloch scans ([Scan page] §2.1) and the
    chunked two-pass scan ([Scan page] §2.2, §3.3) give identical prefixes
    in exact arithmetic, for every L <= 64 (non-powers of two included)."""
    rng = random.Random(100 + L)
    a, b = _frac_pairs(rng, (2,), L)
    sa, sb = ref.scan_serial(a, b)
    for fn in (ref.scan_hillis_steele, ref.scan_blelloch):
        xa, xb = fn(a, b)
        assert (xa == sa).all() and (xb == sb).all(), fn.__name__
    for chunk in (1, 2, 3, 4, 8, 16):
        h0 = np.array([Fraction(0)] * 2, dtype=object)
        h, bnd = ref.scan_chunked_two_pass(a, b, chunk, h0=h0)
        assert (h == sb).all()
        assert (bnd[..., -1] == sb[..., -1]).all()


def test_scans_fp64_long():
    rng = np.random.default_rng(4)
    for L in (257, 1000, 4097):
        a = rng.uniform(0.5, 1.0, (3, L))
        b = rng.normal(size=(3, L))
        sa, sb = ref.scan_serial(a, b)
        for fn in (ref.scan_hillis_steele, ref.scan_blelloch):
            xa, xb = fn(a, b)
            assert np.max(np.abs(xb - sb)) <= 1e-12 * np.max(np.abs(sb))
            assert np.max(np.abs(xa - sa) / np.maximum(sa, 1e-300)) <= 1e-12
        h, _ = ref.scan_chunked_two_pass(a, b, 64)
        assert np.max(np.abs(h - sb)) <= 1e-12 * np.max(np.abs(sb))


def test_two_pass_seq8_chunk4_and_planted_fixup_mistakes():
    """The two-chunk case seq_len = 8, chunk = 4 that [Scan page] §3.3 and
    §5.1 recommend checking by hand.  The correct fix-up is
    h_init^(1) = A_tot^(0) h_init^(0) + B_tot^(0).  Each mistake §5.1 warns
    about, planted in a copy of the fix-up here on the CPU, changes the
    second chunk and leaves the first one correct."""
    rng = random.Random(5)
    a, b = _frac_pairs(rng, (), 8)
    a = np.array([Fraction(x) + Fraction(1, 2) for x in a], dtype=object)  # no zero decays
    h0 = Fraction(3, 2)
    # hand recurrence
    hand = []
    h = h0
    for t in range(8):
        h = a[t] * h + b[t]
        hand.append(h)
    hch, bnd = ref.scan_chunked_two_pass(a, b, 4, h0=np.array(h0, dtype=object))
    assert list(hch) == hand
    assert bnd[0] == h0 and bnd[1] == hand[3] and bnd[2] == hand[7]

    la0, lb0 = ref.scan_serial(a[:4], b[:4])
    la1, lb1 = ref.scan_serial(a[4:], b[4:])
    A0, B0 = la0[-1], lb0[-1]
    A1, B1 = la1[-1], lb1[-1]
    good = A0 * h0 + B0
    wrong = {
        "local state of the previous chunk's last element": B0,
        "own chunk's total instead of the previous one": A1 * h0 + B1,
        "index shifted by one position": la0[-2] * h0 + lb0[-2],
    }
    assert good == hand[3]
    for name, init in wrong.items():
        second = [la1[j] * init + lb1[j] for j in range(4)]
        assert second != hand[4:], name


def test_boundary_states_L12_chunk4():
    """[Mamba-2 page] §4.3: L = 12, chunk 4 keeps h0, h4, h8, h12; those equal
    the serial states at t = 4, 8, 12 (selective scan with chunk output)."""
    rng = np.random.default_rng(6)
    bsz, d, n, L = 2, 3, 4, 12
    u = rng.normal(size=(bsz, d, L))
    dl = rng.normal(size=(bsz, d, L))
    A = -np.exp(rng.normal(size=(d, n)))
    B = rng.normal(size=(bsz, n, L))
    C = rng.normal(size=(bsz, n, L))
    y, last, bnd = ref.selective_scan_fwd(u, dl, A, B, C, delta_softplus=True, chunk=4)
    assert bnd.shape == (bsz, d, n, 4)
    assert np.all(bnd[..., 0] == 0)
    for k, t in ((1, 4), (2, 8), (3, 12)):
        _, hk = ref.selective_scan_fwd(u[..., :t], dl[..., :t], A, B[..., :t], C[..., :t], delta_softplus=True)
        assert np.array_equal(bnd[..., k], hk)
    assert np.array_equal(bnd[..., 3], last)


def test_two_pass_L16384_chunk256():
    """The [Scan page] §3.3 measurement shape: L = 16384, chunk 256, K = 64
    chunk totals; the two-pass result equals the serial scan in float64."""
    rng = np.random.default_rng(7)
    L = 16384
    a = np.exp(-0.01 * rng.uniform(0, 1, (2, L)))
    b = rng.normal(size=(2, L))
    sa, sb = ref.scan_serial(a, b)
    h, bnd = ref.scan_chunked_two_pass(a, b, 256)
    assert bnd.shape[-1] == 65
    assert np.max(np.abs(h - sb)) <= 1e-12 * np.max(np.abs(sb))


# ---------------------------------------------------------------- closed forms

def test_lti_closed_form_matches_recurrence():
    """Constant delta and A make the scan time invariant: h_t =
    sum_j a^(t-j) b_j with a = exp(delta*A), the causal kernel of
    [Truth page] §1.  Checked on h (last_state) and y = C.h."""
    rng = np.random.default_rng(8)
    L, n = 512, 3
    dval = 0.037
    A = np.array([[-0.5, -1.0, -3.0]])
    u = rng.normal(size=(1, 1, L))
    dl = np.full((1, 1, L), dval)
    B = rng.normal(size=(1, n, L))
    C = rng.normal(size=(1, n, L))
    y, last = ref.selective_scan_fwd(u, dl, A, B, C, delta_softplus=False)
    yc = np.zeros(L)
    for k in range(n):
        a = math.exp(dval * A[0, k])
        bseq = dval * B[0, k] * u[0, 0]
        hk = ref.lti_closed_form(a, bseq)
        assert abs(hk[-1] - last[0, 0, k]) <= 1e-12 * np.max(np.abs(hk))
        yc += C[0, k] * hk
    assert np.max(np.abs(yc - y[0, 0])) <= 1e-12 * np.max(np.abs(yc))


def test_forgetting_step_is_exact():
    """a_t = 0 gives h_t = b_t exactly: (0, b2) o (a1, b1) = (0, b2)."""
    rng = np.random.default_rng(9)
    a = rng.uniform(0.1, 1.0, (4, 50))
    b = rng.normal(size=(4, 50))
    zeros = [7, 20, 21, 49]
    a[:, zeros] = 0.0
    oa, ob = ref.affine_scan(a, b)
    for t in zeros:
        assert np.array_equal(ob[:, t], b[:, t])
        assert np.all(oa[:, t] == 0)
    # and through the selective scan: A = -inf makes a = exp(-inf) = 0
    u = rng.normal(size=(1, 2, 6)); dl = rng.uniform(0.1, 1, (1, 2, 6))
    B = rng.normal(size=(1, 1, 6)); C = np.ones((1, 1, 6))
    y, last = ref.selective_scan_fwd(u, dl, np.full((2, 1), -np.inf), B, C)
    assert np.array_equal(y[0], dl[0] * B[0, 0][None, :] * u[0])


@pytest.mark.parametrize("softplus", [False, True])
@pytest.mark.parametrize("gated", [False, True])
def test_bruteforce_expansion_tiny(softplus, gated):
    """Loop vs the unrolled sum h_t = sum_j exp(A sum_{j<s<=t} dt_s) dt_j B_j u_j,
    with every per-step input, D, bias and gate present; L <= 8."""
    rng = np.random.default_rng(10 + 2 * softplus + gated)
    bsz, d, n, L = 2, 3, 4, 8
    u = rng.normal(size=(bsz, d, L))
    dl = rng.normal(size=(bsz, d, L)) if softplus else rng.uniform(0.01, 1.0, (bsz, d, L))
    A = -np.exp(rng.normal(size=(d, n)))
    B = rng.normal(size=(bsz, n, L))
    C = rng.normal(size=(bsz, n, L))
    D = rng.normal(size=d)
    z = rng.normal(size=(bsz, d, L)) if gated else None
    bias = rng.normal(size=d) * 0.5
    y1, l1 = ref.selective_scan_fwd(u, dl, A, B, C, D, z, bias, softplus)
    y2, l2 = ref.selective_scan_bruteforce(u, dl, A, B, C, D, z, bias, softplus)
    assert np.max(np.abs(y1 - y2)) <= 1e-12 * np.max(np.abs(y2))
    assert np.max(np.abs(l1 - l2)) <= 1e-12 * np.max(np.abs(l2))


def test_underflow_products_printed_on_page():
    """[Scan page] §4.3: over a 256-step chunk the decay product is about
    e^-12.8 = 2.8e-6 when delta*A = -0.05, and about e^-76.8 = 4e-34 when
    delta*A = -0.3.  The oracle's cumulative product must match both the
    exact exponential and the page's printed digits."""
    with open(os.path.join(GOLDEN, "underflow_products.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        a = np.full((1, c["steps"]), math.exp(c["delta_times_A"]))
        oa, _ = ref.affine_scan(a, np.zeros_like(a))
        exact = math.exp(c["steps"] * c["delta_times_A"])
        assert abs(oa[0, -1] - exact) <= 1e-12 * exact
        sig = c["printed_sig_digits"]
        assert float(f"{oa[0, -1]:.{sig - 1}e}") == c["printed"]


def test_padding_with_identity_steps():
    """End padding with delta = 0 (a = 1, b = 0) leaves last_state unchanged
    and front padding leaves the later outputs unchanged, exactly
    ([Scan page] §2.1 pads with identities)."""
    rng = np.random.default_rng(11)
    bsz, d, n, L, P = 2, 3, 4, 40, 13
    u = rng.normal(size=(bsz, d, L)); dl = rng.uniform(0.01, 0.5, (bsz, d, L))
    z = rng.normal(size=(bsz, d, L)); D = rng.normal(size=d)
    A = -np.exp(rng.normal(size=(d, n)))
    B = rng.normal(size=(bsz, n, L)); C = rng.normal(size=(bsz, n, L))
    y, last = ref.selective_scan_fwd(u, dl, A, B, C, D, z)

    def padded(x, front, fill):
        padw = [(0, 0)] * (x.ndim - 1) + ([(P, 0)] if front else [(0, P)])
        return np.pad(x, padw, constant_values=fill)

    for front in (False, True):
        up = padded(u, front, 0.7); zp = padded(z, front, -0.3)
        dp = padded(dl, front, 0.0)
        Bp = padded(B, front, 1.5); Cp = padded(C, front, 2.5)
        yp, lp = ref.selective_scan_fwd(up, dp, A, Bp, Cp, D, zp)
        assert np.array_equal(lp, last)
        if front:
            assert np.array_equal(yp[..., P:], y)
        else:
            assert np.array_equal(yp[..., :L], y)
    # softplus on with raw delta = -inf gives delta = 0 exactly
    dinf = padded(dl, False, -np.inf)
    assert np.all(ref.softplus(dinf[..., L:]) == 0.0)


def test_softplus_silu_against_torch():
    """Textbook functions checked against an independent library (torch,
    float64, CPU)."""
    x = np.concatenate([np.linspace(-40, 19.9, 20001), np.array([-700.0, -1e-8, 0.0, 1e-8])])
    sp_t = torch.nn.functional.softplus(torch.from_numpy(x), threshold=1e9).numpy()
    assert np.max(np.abs(ref.softplus(x) - sp_t) / np.maximum(sp_t, 1e-300)) < 1e-14
    zz = np.concatenate([np.linspace(-60, 60, 20001), np.array([-800.0, 800.0])])
    si_t = torch.nn.functional.silu(torch.from_numpy(zz)).numpy()
    assert np.max(np.abs(ref.silu(zz) - si_t) / np.maximum(np.abs(si_t), 1e-300)) < 1e-14
    assert ref.softplus(np.array([-np.inf]))[0] == 0.0


def test_affine_scan_matches_tree_scans():
    rng = np.random.default_rng(12)
    a = rng.uniform(0, 1, (5, 300)); b = rng.normal(size=(5, 300))
    oa, ob = ref.affine_scan(a, b)
    xa, xb = ref.scan_blelloch(a, b)
    assert np.max(np.abs(ob - xb)) <= 1e-13 * np.max(np.abs(ob))
    assert np.max(np.abs(oa - xa) / np.maximum(oa, 1e-300)) <= 1e-12


def test_chunk_state_sizes_printed_on_page():
    """[Scan page] §3.4 ledger: per chunk one (b, d_inner, d_state) state,
    393216 elements, 1.5 MB in float32, 12.6 MB for 8 chunks, and 8.05e8
    elements / 3.2 GB if every step's state were kept.  Checked against the
    shape of the oracle's chunk-boundary output on the same workload's
    (b, d, n) at a short L (K+1 boundary slots, first one h_0)."""
    with open(os.path.join(GOLDEN, "chunk_state_sizes.json")) as f:
        g = json.load(f)
    w, p = g["workload"], g["printed"]
    assert w["d_model"] * w["expand"] == w["d_inner"]
    K = w["seq_len"] // w["chunk"]
    per_chunk = w["batch"] * w["d_inner"] * w["d_state"]
    assert K == p["chunks"] and per_chunk == p["elements_per_chunk_state"]
    assert per_chunk * 4 / 2**20 == p["mb_per_chunk_state_fp32"]
    assert round(K * per_chunk * 4 / 1e6, 1) == p["mb_all_chunk_states_fp32"]
    assert float(f"{per_chunk * w['seq_len']:.2e}") == p["elements_all_states"]
    assert round(per_chunk * w["seq_len"] * 4 / 1e9, 1) == p["gb_all_states_fp32"]
    # the oracle keeps exactly one state per chunk boundary
    rng = np.random.default_rng(13)
    bsz, d, n, L, ch = 2, 5, w["d_state"], 64, 8
    u = rng.normal(size=(bsz, d, L)); dl = rng.normal(size=(bsz, d, L))
    _, _, bnd = ref.selective_scan_fwd(u, dl, -np.ones((d, n)), rng.normal(size=(bsz, n, L)),
                                       rng.normal(size=(bsz, n, L)), delta_softplus=True, chunk=ch)
    assert bnd.shape == (bsz, d, n, L // ch + 1)


# ---------------------------------------------------------------- start state

def test_start_state_decays_in_closed_form():
    """With no input (B = 0) the state only decays: h_t = exp(A * sum_{s<=t}
    Delta_s) * h_0, the h_t = A_t h_0 + B_t form of [Scan page] §2.1 with
    B_t = 0, written here as one exponential of the running sum; y follows as
    C_t . h_t + D u_t."""
    rng = np.random.default_rng(21)
    bsz, d, n, L = 2, 3, 4, 40
    u = rng.normal(size=(bsz, d, L))
    dl = rng.normal(size=(bsz, d, L))
    A = -np.exp(rng.normal(size=(d, n)))
    C = rng.normal(size=(bsz, n, L))
    D = rng.normal(size=d)
    h0 = rng.normal(size=(bsz, d, n))
    y, last = ref.selective_scan_fwd(u, dl, A, np.zeros((bsz, n, L)), C, D=D, delta_softplus=True, h0=h0)
    dt = ref.softplus(dl)
    cum = np.cumsum(dt, axis=-1)                                        # [b, d, L]
    h = np.exp(cum[:, :, None, :] * A[None, :, :, None]) * h0[..., None]  # [b, d, n, L]
    y_cf = np.einsum("bdnt,bnt->bdt", h, C) + D[None, :, None] * u
    assert np.max(np.abs(y - y_cf)) <= 1e-12 * np.max(np.abs(y_cf))
    assert np.max(np.abs(last - h[..., -1])) <= 1e-12 * np.max(np.abs(h[..., -1]))


def test_start_state_split_invariance():
    """Running steps [0, t1) and then [t1, L) from the state reached gives the
    whole run: the recurrence composes (h_t = A_t h_0 + B_t for any h_0,
    [Scan page] §2.1).  A dropped or misplaced h0 term fails this."""
    rng = np.random.default_rng(22)
    bsz, d, n, L, t1 = 2, 3, 5, 30, 11
    u = rng.normal(size=(bsz, d, L)); dl = rng.normal(size=(bsz, d, L)); z = rng.normal(size=(bsz, d, L))
    A = -np.exp(rng.normal(size=(d, n)))
    B = rng.normal(size=(bsz, n, L)); C = rng.normal(size=(bsz, n, L))
    D = rng.normal(size=d); bias = rng.normal(size=d)
    h0 = rng.normal(size=(bsz, d, n))
    kw = dict(D=D, delta_bias=bias, delta_softplus=True)
    y, last = ref.selective_scan_fwd(u, dl, A, B, C, z=z, h0=h0, **kw)
    y1, h1 = ref.selective_scan_fwd(u[..., :t1], dl[..., :t1], A, B[..., :t1], C[..., :t1], z=z[..., :t1],
                                    h0=h0, **kw)
    y2, h2 = ref.selective_scan_fwd(u[..., t1:], dl[..., t1:], A, B[..., t1:], C[..., t1:], z=z[..., t1:],
                                    h0=h1, **kw)
    assert np.max(np.abs(np.concatenate([y1, y2], axis=-1) - y)) <= 1e-13 * np.max(np.abs(y))
    assert np.max(np.abs(h2 - last)) <= 1e-13 * np.max(np.abs(last))


# ---------------------------------------------------------------- causal conv1d

def test_causal_conv1d_matches_numpy_convolve():
    """Each channel's causal convolution is the first L terms of the full
    discrete convolution np.convolve(x, w[::-1]): with w[K-1] on the current
    step, the tap on x[t - j] is w[K-1-j], i.e. the reversed taps."""
    rng = np.random.default_rng(11)
    for K in (1, 2, 3, 4):
        x = rng.normal(size=(2, 3, 37))
        w = rng.normal(size=(3, K))
        b = rng.normal(size=3)
        got = ref.causal_conv1d(x, w, b, activation=None)
        for bi in range(2):
            for d in range(3):
                want = np.convolve(x[bi, d], w[d, ::-1])[:37] + b[d]
                np.testing.assert_allclose(got[bi, d], want, rtol=1e-13, atol=1e-13)


def test_causal_conv1d_matches_torch_grouped_conv():
    """torch.nn.functional.conv1d with groups = channels and K-1 steps of
    left padding (cross-correlation, w[K-1] on the current step) then SiLU."""
    rng = np.random.default_rng(12)
    x = rng.normal(size=(2, 5, 50))
    w = rng.normal(size=(5, 4))
    b = rng.normal(size=5)
    got = ref.causal_conv1d(x, w, b)
    xt = torch.tensor(x)
    pre = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (3, 0)), torch.tensor(w)[:, None, :],
                                     torch.tensor(b), groups=5)
    want = torch.nn.functional.silu(pre).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_causal_conv1d_single_tap_is_pointwise():
    rng = np.random.default_rng(13)
    x = rng.normal(size=(1, 4, 9))
    w = rng.normal(size=(4, 1))
    got = ref.causal_conv1d(x, w, None, activation=None)
    np.testing.assert_allclose(got, x * w[None, :, :], rtol=0, atol=0)


# ------------------------------------------------------------ out projection

def test_out_proj_matches_bruteforce_in_exact_arithmetic():
    """out[b, t, m] = sum_k W[m, k] y[b, k, t], summed term by term in exact
    rationals over small integers (so the float64 product is exact too).
    Non-square W and distinct b, d_inner, L, d_model catch a transposed
    operand or a swapped index."""
    rng = random.Random(5)
    bsz, dk, L, dm = 2, 5, 3, 4
    y = np.array([[[rng.randint(-9, 9) for _ in range(L)] for _ in range(dk)] for _ in range(bsz)], dtype=float)
    W = np.array([[rng.randint(-9, 9) for _ in range(dk)] for _ in range(dm)], dtype=float)
    got = ref.out_proj(y, W)
    assert got.shape == (bsz, L, dm)
    for b in range(bsz):
        for t in range(L):
            for m in range(dm):
                want = sum(Fraction(int(W[m, k])) * Fraction(int(y[b, k, t])) for k in range(dk))
                assert Fraction(got[b, t, m]) == want, (b, t, m)


def test_out_proj_identity_weight_is_the_token_major_transpose():
    """W = I (d_model = d_inner): out[b, t, :] is y[b, :, t] exactly."""
    y = np.random.default_rng(1).standard_normal((3, 6, 7))
    out = ref.out_proj(y, np.eye(6))
    assert np.array_equal(out, y.transpose(0, 2, 1))


def test_out_proj_selector_rows_pick_channels():
    """A one-hot row of W copies one channel's sequence; a row of ones sums
    the channels (the column sum of y at every step)."""
    y = np.random.default_rng(2).standard_normal((2, 5, 9))
    W = np.zeros((3, 5))
    W[0, 3] = 1.0
    W[1, 0] = 1.0
    W[2, :] = 1.0
    out = ref.out_proj(y, W)
    assert np.array_equal(out[:, :, 0], y[:, 3, :])
    assert np.array_equal(out[:, :, 1], y[:, 0, :])
    np.testing.assert_allclose(out[:, :, 2], y.sum(axis=1), rtol=1e-14, atol=1e-14)


def test_out_proj_tokens_agrees_with_full_projection():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((2, 16, 11))
    W = rng.standard_normal((8, 16))
    full = ref.out_proj(y, W)
    pairs = [(0, 0), (1, 10), (0, 5), (1, 3)]
    got = ref.out_proj_tokens(y, W, pairs)
    for i, (b, t) in enumerate(pairs):
        np.testing.assert_allclose(got[i], full[b, t], rtol=1e-14, atol=1e-13)


def test_out_proj_bwd_matches_central_differences():
    """The gradients of the loss sum(out_proj(y, W) * R) by central
    differences of the forward oracle (exact for a bilinear map up to
    rounding), element by element on a tiny non-square case."""
    rng = np.random.default_rng(11)
    bsz, dk, L, dm = 2, 3, 4, 5
    y = rng.standard_normal((bsz, dk, L))
    W = rng.standard_normal((dm, dk))
    R = rng.standard_normal((bsz, L, dm))
    dy, dW = ref.out_proj_bwd(y, W, R)
    loss = lambda yy, WW: float(np.sum(ref.out_proj(yy, WW) * R))
    eps = 1e-3
    for idx in np.ndindex(y.shape):
        e = np.zeros_like(y)
        e[idx] = eps
        fd = (loss(y + e, W) - loss(y - e, W)) / (2 * eps)
        assert abs(fd - dy[idx]) <= 1e-9 * max(1.0, abs(fd)), idx
    for idx in np.ndindex(W.shape):
        e = np.zeros_like(W)
        e[idx] = eps
        fd = (loss(y, W + e) - loss(y, W - e)) / (2 * eps)
        assert abs(fd - dW[idx]) <= 1e-9 * max(1.0, abs(fd)), idx


def test_out_proj_bwd_adjoint_identities():
    """For the bilinear map out = P(y, W): <P(y, W), R> = <y, dy(R)> =
    <W, dW(R)>, exactly in rationals over small integers (a transposed
    or swapped term breaks one of them)."""
    rng = random.Random(12)
    bsz, dk, L, dm = 2, 3, 4, 5
    y = np.array([[[rng.randint(-5, 5) for _ in range(L)] for _ in range(dk)] for _ in range(bsz)], dtype=float)
    W = np.array([[rng.randint(-5, 5) for _ in range(dk)] for _ in range(dm)], dtype=float)
    R = np.array([[[rng.randint(-5, 5) for _ in range(dm)] for _ in range(L)] for _ in range(bsz)], dtype=float)
    dy, dW = ref.out_proj_bwd(y, W, R)
    lhs = int(np.sum(ref.out_proj(y, W) * R))
    assert int(np.sum(y * dy)) == lhs
    assert int(np.sum(W * dW)) == lhs
