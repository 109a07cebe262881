"""The C ABI on the host (no GPU): the library loads, exports every entry
point the public header declares, and rejects bad arguments before any HIP
call.  Fake device addresses are used only in calls that must fail
validation; none of them reaches the GPU."""
import ctypes
import os
import re

import pytest

import selective_state_space_ssm_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_entry_points():
    names = set(_declared_functions())
    assert {"ssm_scan_fwd", "ssm_scan_fwd_plan", "ssm_scan_plan_for", "affine_scan", "affine_scan_order",
            "ssm_last_error"} <= names


def test_library_exports_every_declared_symbol():
    lib = ssm.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_affine_scan_order_constants():
    o = ssm.affine_scan_order()
    assert o == {"items_per_lane": 8, "lanes": 64, "waves": 4, "chunk": 8 * 64 * 4}


# ------------------------------------------------------------ validation
F = 0x100000  # fake, 16-byte aligned "device" addresses; never dereferenced


def _fwd(**kw):
    lib = ssm.load_library()
    args = dict(u=F, delta=F * 2, A=F * 3, B=F * 4, C=F * 5, D=None, z=None, bias=None, sp=1, y=F * 8,
                last=None, b=1, d=64, n=16, L=64, dtype=0, plan=0, S=0, chunk=0)
    args.update(kw)
    P = ctypes.c_void_p
    rc = lib.ssm_scan_fwd_plan(P(args["u"]), P(args["delta"]), P(args["A"]), P(args["B"]), P(args["C"]),
                               P(args["D"]), P(args["z"]), P(args["bias"]), args["sp"], P(args["y"]),
                               P(args["last"]), args["b"], args["d"], args["n"], args["L"], args["dtype"],
                               args["plan"], args["S"], args["chunk"], None)
    return rc, lib.ssm_last_error().decode()


# Addresses are spaced so that no tensor of these sizes overlaps another;
# each case breaks exactly one rule.
BIG = 1 << 30


@pytest.mark.parametrize("kw,code", [
    (dict(u=None), ssm.SSM_EINVAL),
    (dict(y=None), ssm.SSM_EINVAL),
    (dict(b=0), ssm.SSM_EINVAL),
    (dict(L=-1), ssm.SSM_EINVAL),
    (dict(n=17), ssm.SSM_EUNSUPPORTED),
    (dict(dtype=7), ssm.SSM_EUNSUPPORTED),
    (dict(sp=2), ssm.SSM_EINVAL),
    (dict(plan=9), ssm.SSM_EINVAL),
    (dict(S=3), ssm.SSM_EINVAL),
    (dict(chunk=100), ssm.SSM_EINVAL),
    (dict(u=BIG + 4), ssm.SSM_EINVAL),          # misaligned
    (dict(L=((1 << 32) - 4096) // 64 + 1), ssm.SSM_EUNSUPPORTED),   # longest L + 1 (32-bit row offsets)
    (dict(b=65536), ssm.SSM_EUNSUPPORTED),      # batch above the grid's y range
    (dict(y=BIG), ssm.SSM_EINVAL, ),             # placeholder replaced below
])
def test_fwd_rejects_bad_arguments(kw, code):
    base = dict(u=BIG, delta=2 * BIG, A=3 * BIG, B=4 * BIG, C=5 * BIG, y=8 * BIG)
    base.update(kw)
    if kw == dict(y=BIG):
        base["y"] = base["u"] + 64  # y overlaps u
    rc, msg = _fwd(**base)
    assert rc == code, msg
    assert msg


def test_fwd_rejects_last_state_overlapping_y():
    rc, msg = _fwd(u=BIG, delta=2 * BIG, A=3 * BIG, B=4 * BIG, C=5 * BIG, y=8 * BIG, last=8 * BIG + 256)
    assert rc == ssm.SSM_EINVAL and "overlap" in msg


def test_affine_scan_rejects_bad_arguments():
    lib = ssm.load_library()
    P = ctypes.c_void_p
    assert lib.affine_scan(None, P(BIG), None, P(2 * BIG), 4, 8, None) == ssm.SSM_EINVAL
    assert lib.affine_scan(P(BIG), P(2 * BIG), None, P(3 * BIG), 0, 8, None) == ssm.SSM_EINVAL
    assert lib.affine_scan(P(BIG + 8), P(2 * BIG), None, P(3 * BIG), 4, 8, None) == ssm.SSM_EINVAL
    # out_b partially overlapping a
    assert lib.affine_scan(P(BIG), P(2 * BIG), None, P(BIG + 16), 4, 8, None) == ssm.SSM_EINVAL
    # out_a equal to b (not its own input)
    assert lib.affine_scan(P(BIG), P(2 * BIG), P(2 * BIG), P(3 * BIG), 4, 8, None) == ssm.SSM_EINVAL


def test_plan_choice():
    # many channels: carry plan over the whole length
    p = ssm.plan_for(8, 1536, 16, 2048)
    assert p["plan"] == "mixed" and p["chunk"] == 2048  # 768 groups: three per CU
    p = ssm.plan_for(8, 4096, 16, 2048, "bf16")
    assert p["plan"] == "carry" and p["states_per_lane"] == 4
    p = ssm.plan_for(16, 5120, 16, 8192, "bf16")
    assert p["plan"] == "carry"
    # below 2.5 channel groups per CU: the L-parallel plan (4 states per lane)
    p = ssm.plan_for(4, 1536, 16, 2048)
    assert p["plan"] == "lpar" and p["states_per_lane"] == 4 and p["chunk"] == 2048
    assert ssm.plan_for(1, 2048, 16, 65536)["plan"] == "lpar"
    assert ssm.plan_for(1, 1536, 16, 512)["plan"] == "lpar"
    # ... but not below 512 steps (256-step tiles)
    assert ssm.plan_for(1, 1536, 16, 511)["plan"] == "carry"
    # few channels, very long sequence: two-pass over chunks that are multiples of 64
    p = ssm.plan_for(1, 512, 16, 65536)
    assert p["plan"] == "twopass" and p["chunk"] % 64 == 0 and 2 <= -(-65536 // p["chunk"]) <= 65535
    assert ssm.plan_for(1, 16, 16, 1 << 20)["plan"] == "twopass"
    # short sequence never splits
    assert ssm.plan_for(1, 64, 16, 256)["plan"] == "carry"
    with pytest.raises(ssm.SSMError):
        ssm.plan_for(1, 64, 17, 256)


def test_states_entry_point_rejects_bad_state_chunk():
    lib = ssm.load_library()
    P = ctypes.c_void_p
    args = [P(BIG), P(2 * BIG), P(3 * BIG), P(4 * BIG), P(5 * BIG), None, None, None, 0, None, P(6 * BIG),
            P(7 * BIG), P(8 * BIG)]
    # state_chunk must be a positive multiple of 32 when chunk_states is given
    for sc in (0, 16, 33, -32):
        assert lib.ssm_scan_fwd_states(*args, sc, 1, 64, 16, 256, 0, 0, None) == ssm.SSM_EINVAL
    # chunk_states overlapping an input
    args2 = list(args)
    args2[12] = P(BIG)
    assert lib.ssm_scan_fwd_states(*args2, 64, 1, 64, 16, 256, 0, 0, None) == ssm.SSM_EINVAL


def test_lpar_plan_checks_state_chunk():
    """Under the L-parallel plan a chunk-state spacing that is not a multiple
    of 32 is SSM_EINVAL, and an unknown plan number stays invalid, both before
    any HIP call."""
    lib = ssm.load_library()
    P = ctypes.c_void_p
    args = [P(BIG), P(2 * BIG), P(3 * BIG), P(4 * BIG), P(5 * BIG), None, None, None, 0, None, P(6 * BIG),
            P(7 * BIG), P(8 * BIG)]
    assert lib.ssm_scan_fwd_states(*args, 48, 1, 64, 16, 256, 0, ssm.PLANS["lpar"], None) == ssm.SSM_EINVAL
    assert lib.ssm_scan_fwd_states(*args, 64, 1, 64, 16, 256, 0, 5, None) == ssm.SSM_EINVAL


def test_step_rejects_bad_arguments():
    lib = ssm.load_library()
    P = ctypes.c_void_p
    base = [P(BIG), P(2 * BIG), P(3 * BIG), P(4 * BIG), P(5 * BIG), None, None, None, 0, P(6 * BIG), P(6 * BIG),
            P(7 * BIG)]
    ok_sizes = (8, 64, 16, 0, None)
    bad = list(base); bad[0] = None
    assert lib.ssm_step(*bad, *ok_sizes) == ssm.SSM_EINVAL                      # null u
    assert lib.ssm_step(*base, 8, 64, 17, 0, None) == ssm.SSM_EUNSUPPORTED      # d_state > 16
    bad = list(base); bad[10] = P(6 * BIG + 16)
    assert lib.ssm_step(*bad, *ok_sizes) == ssm.SSM_EINVAL                      # partial state overlap
    bad = list(base); bad[11] = P(6 * BIG)
    assert lib.ssm_step(*bad, *ok_sizes) == ssm.SSM_EINVAL                      # y on the state
    bad = list(base); bad[8] = 3
    assert lib.ssm_step(*bad, *ok_sizes) == ssm.SSM_EINVAL                      # softplus flag


def test_bwd_rejects_bad_arguments():
    lib = ssm.load_library()
    P = ctypes.c_void_p
    # u, delta, A, B, C, D, z, delta_bias, softplus, h0, chunk_states, state_chunk, dy, dlast,
    # du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0
    base = [P(BIG), P(2 * BIG), P(3 * BIG), P(4 * BIG), P(5 * BIG), None, P(6 * BIG), None, 1, None,
            P(7 * BIG), 64, P(8 * BIG), None, P(9 * BIG), P(10 * BIG), P(11 * BIG), P(12 * BIG), P(13 * BIG),
            None, P(14 * BIG), None, None]
    sizes = [2, 64, 16, 256, 0, 0, None]   # batch, d_inner, d_state, L, dtype, states_per_lane, stream

    def call(args=None, sz=None):
        return lib.ssm_scan_bwd(*(args or base), *(sz or sizes))

    def with_(**kw):
        idx = {"u": 0, "z": 6, "h0": 9, "cs": 10, "sc": 11, "dy": 12, "du": 14, "dA": 16, "dB": 17, "dC": 18,
               "dz": 20}
        a = list(base)
        for k, v in kw.items():
            a[idx[k]] = v
        return a

    assert call(with_(cs=None)) == ssm.SSM_EINVAL                   # chunk states are required
    for sc in (0, 16, 48, 544, 1024, -32):                          # multiple of 32, at most 512
        assert call(with_(sc=sc)) == ssm.SSM_EINVAL, sc
    assert call(with_(dz=None)) == ssm.SSM_EINVAL                   # z given without dz
    assert call(with_(z=None)) == ssm.SSM_EINVAL                    # dz given without z
    assert call(with_(du=P(BIG))) == ssm.SSM_EINVAL                 # output on an input
    assert call(with_(dC=P(12 * BIG))) == ssm.SSM_EINVAL            # outputs overlap each other
    assert call(with_(dA=P(11 * BIG + 4))) == ssm.SSM_EINVAL        # misaligned
    assert call(with_(dy=None)) == ssm.SSM_EINVAL                   # null dy
    for spl in (3, 8, -1):
        s2 = list(sizes); s2[5] = spl
        assert call(sz=s2) == ssm.SSM_EINVAL, spl
    s2 = list(sizes); s2[2] = 17
    assert call(sz=s2) == ssm.SSM_EUNSUPPORTED                      # d_state > 16
    s2 = list(sizes); s2[4] = 7
    assert call(sz=s2) == ssm.SSM_EUNSUPPORTED                      # dtype
    bad = list(base); bad[8] = 2
    assert call(bad) == ssm.SSM_EINVAL                              # softplus flag


def test_step_conv_rejects_bad_arguments():
    lib = ssm.load_library()
    P = ctypes.c_void_p
    # x, conv_w, conv_b, K, cs_in, cs_out, delta, A, B, C, D, z, bias, softplus, state_in, state_out, y, u_out
    base = [P(BIG), P(2 * BIG), None, 4, P(3 * BIG), P(3 * BIG), P(4 * BIG), P(5 * BIG), P(6 * BIG), P(7 * BIG),
            None, None, None, 0, P(8 * BIG), P(8 * BIG), P(9 * BIG), None]
    sizes = (8, 64, 16, 0, None)

    def call(**kw):
        idx = {"x": 0, "w": 1, "K": 3, "csi": 4, "cso": 5, "y": 16, "u": 17}
        a = list(base)
        for k, v in kw.items():
            a[idx[k]] = v
        return lib.ssm_step_conv(*a, *sizes)

    assert call(w=None) == ssm.SSM_EINVAL                         # conv weights required
    assert call(K=0) == ssm.SSM_EUNSUPPORTED and call(K=5) == ssm.SSM_EUNSUPPORTED
    assert call(csi=None) == ssm.SSM_EINVAL                       # conv state needed for K > 1
    assert call(cso=P(3 * BIG + 16)) == ssm.SSM_EINVAL            # partial conv-state overlap
    assert call(u=P(9 * BIG)) == ssm.SSM_EINVAL                   # u_out on y
    assert call(y=P(BIG)) == ssm.SSM_EINVAL                       # y on x


def test_autograd_wrappers_refuse_host_tensors():
    """The autograd wrappers run only on the library: host tensors are
    refused, never computed on the CPU."""
    import torch
    from selective_state_space_ssm_amd.autograd import selective_scan, selective_scan_conv
    u = torch.zeros((1, 4, 8), requires_grad=True)
    A = -torch.ones((4, 2))
    B = torch.zeros((1, 2, 8))
    with pytest.raises(ValueError, match="CUDA/HIP"):
        selective_scan(u, u, A, B, B)
    with pytest.raises(ValueError, match="CUDA/HIP"):
        selective_scan_conv(u, torch.ones((4, 4)), None, u, A, B, B)


def test_out_proj_rejects_bad_arguments():
    lib = ssm.load_library()
    P = ctypes.c_void_p
    y, w, out = P(BIG), P(2 * BIG), P(3 * BIG)

    def call(y=y, w=w, out=out, b=2, k=64, m=32, L=128, dtype=ssm.SSM_BF16):
        return lib.ssm_out_proj(y, w, out, b, k, m, L, dtype, None)

    assert call(y=None) == ssm.SSM_EINVAL
    assert call(out=None) == ssm.SSM_EINVAL
    assert call(k=0) == ssm.SSM_EINVAL and call(L=-1) == ssm.SSM_EINVAL
    assert call(dtype=7) == ssm.SSM_EUNSUPPORTED
    assert call(w=P(2 * BIG + 8)) == ssm.SSM_EINVAL                   # misaligned
    assert call(out=P(BIG + 64)) == ssm.SSM_EINVAL                     # out inside y
    assert call(k=1 << 16, L=1 << 15) == ssm.SSM_EUNSUPPORTED          # a y row of 2^32 bytes
    assert call(m=1 << 20, k=1 << 11) == ssm.SSM_EUNSUPPORTED          # W of 2^32 bytes
    assert "2^31" in lib.ssm_last_error().decode()


def test_out_proj_bwd_rejects_bad_arguments():
    lib = ssm.load_library()
    P = ctypes.c_void_p
    y, w, dout, dy, dw = P(BIG), P(2 * BIG), P(3 * BIG), P(4 * BIG), P(5 * BIG)

    def call(y=y, w=w, dout=dout, dy=dy, dw=dw, b=2, k=64, m=32, L=128, dtype=ssm.SSM_BF16):
        return lib.ssm_out_proj_bwd(y, w, dout, dy, dw, b, k, m, L, dtype, None)

    assert call(dout=None) == ssm.SSM_EINVAL
    assert call(dy=None, dw=None) == ssm.SSM_EINVAL                    # nothing asked for
    assert call(m=0) == ssm.SSM_EINVAL
    assert call(dtype=5) == ssm.SSM_EUNSUPPORTED
    assert call(dy=P(4 * BIG + 4)) == ssm.SSM_EINVAL                   # misaligned
    assert call(dw=P(BIG + 256)) == ssm.SSM_EINVAL                     # dW inside y
    assert call(dw=P(4 * BIG + 64)) == ssm.SSM_EINVAL                  # dW inside dy
    assert call(m=1 << 16, k=1 << 14) == ssm.SSM_EUNSUPPORTED          # W in float32 reaches 2^32 bytes


def test_noalloc_rejects_bad_arguments_before_any_hip_call():
    """The entry point that allocates nothing validates like ssm_scan_fwd."""
    lib = ssm.load_library()
    P = ctypes.c_void_p
    cases = [  # (u, y, batch, n, code)
        (None, 8 * BIG, 1, 16, ssm.SSM_EINVAL),
        (BIG, None, 1, 16, ssm.SSM_EINVAL),
        (BIG, 8 * BIG, 0, 16, ssm.SSM_EINVAL),
        (BIG, 8 * BIG, 1, 17, ssm.SSM_EUNSUPPORTED),
        (BIG + 4, 8 * BIG, 1, 16, ssm.SSM_EINVAL),
        (BIG, BIG, 1, 16, ssm.SSM_EINVAL),          # y overlaps u
    ]
    for u, y, b, n, code in cases:
        rc = lib.ssm_scan_fwd_noalloc(P(u), P(2 * BIG), P(3 * BIG), P(4 * BIG), P(5 * BIG), None, None, None, 1,
                                      P(y), None, b, 64, n, 4096, 0, None)
        assert rc == code, (u, y, b, n, lib.ssm_last_error().decode())


@pytest.mark.parametrize("L", [2048, 4096, 65536, 1 << 20, 1 << 22, ((1 << 32) - 4096) // 64])
def test_automatic_two_pass_workspace_fits_the_noalloc_scratch(L):
    """Wherever the automatic plan splits L (fewer channel groups than CUs),
    its workspace, 3 float32 per (batch, channel, state, chunk), stays below
    the 8 MiB scratch of ssm_scan_fwd_noalloc."""
    worst = 0
    for b in (1, 2, 3, 8, 16, 255):
        for d in (1, 16, 17, 100, 255, 1024, 4080):
            for n in (1, 16):
                p = ssm.plan_for(b, d, n, L, "f32")
                if p["plan"] != "twopass":
                    continue
                K = -(-L // p["chunk"])
                worst = max(worst, 12 * b * d * n * K)
    assert worst <= 8 << 20, worst
