"""The library on several streams at once and from several host threads:
every call carries its own stream and keeps no state between calls (the
error text is per thread), so work issued concurrently gives exactly what
the same calls give one after another.  All streams have the default
priority."""
import threading

import pytest
import torch

import selective_state_space_ssm_amd as ssm
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _inputs(seed, L=400, dtype="f32"):
    w = workloads.Workload("t", 2, 96, 16, L, dtype, True, "normal", "dt_init", softplus=True)
    inp = workloads.make_inputs(w, device=DEV, seed=seed)
    inp["A"] = workloads.random_A(96, 16, device=DEV, seed=seed + 1)
    return inp


def _fwd(inp, stream):
    with torch.cuda.stream(stream):
        return ssm.ssm_scan_fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                inp["delta_bias"], delta_softplus=True)


def test_two_streams_match_sequential():
    a, b = _inputs(1), _inputs(2, L=777, dtype="bf16")
    main = torch.cuda.current_stream()
    ya, la = _fwd(a, main)
    yb, lb = _fwd(b, main)
    torch.cuda.synchronize(DEV)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    outs = []
    for _ in range(5):
        outs.append((_fwd(a, s1), _fwd(b, s2)))
    torch.cuda.synchronize(DEV)
    for (ya2, la2), (yb2, lb2) in outs:
        assert torch.equal(ya, ya2) and torch.equal(la, la2)
        assert torch.equal(yb, yb2) and torch.equal(lb, lb2)


def test_host_threads_with_own_streams_match_sequential():
    inps = [_inputs(10 + i, L=300 + 50 * i) for i in range(4)]
    main = torch.cuda.current_stream()
    want = [_fwd(x, main) for x in inps]
    torch.cuda.synchronize(DEV)
    got = [None] * len(inps)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(main)
            res = []
            for _ in range(8):
                res.append(_fwd(inps[i], s))
            s.synchronize()
            got[i] = res
        except Exception as e:          # surfaced after the join
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(inps))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for i, res in enumerate(got):
        assert res is not None, f"thread {i} did not finish"
        for y, last in res:
            assert torch.equal(y, want[i][0]) and torch.equal(last, want[i][1])


def test_error_text_is_per_thread():
    """A failing call on one host thread leaves another thread's last error
    untouched."""
    lib = ssm.load_library()
    texts = {}

    def bad():
        lib.ssm_scan_fwd(None, None, None, None, None, None, None, None, 0, None, None, 1, 1, 1, 1, 0, None)
        texts["bad"] = lib.ssm_last_error().decode()

    def good():
        inp = _inputs(30)
        _fwd(inp, torch.cuda.current_stream())
        torch.cuda.synchronize(DEV)
        texts["good"] = lib.ssm_last_error().decode()

    for fn in (bad, good):
        t = threading.Thread(target=fn)
        t.start()
        t.join(timeout=60)
    assert "NULL" in texts["bad"]
    assert texts["good"] == ""
