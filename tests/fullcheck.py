"""Whole-tensor comparison of a forward result with the C oracle, in blocks
of channels, for the full-size workloads.

The oracle runs on every (batch, channel) row; each block's float64 result
is compared with the GPU's and dropped, so only running maxima are kept:
max |gpu - oracle| and max |oracle| per output tensor.  The metric is their
ratio over the whole tensor, the same as comparing the full tensors at once.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import cpu


class MaxRatio:
    """Running max |got - want| and max |want| over blocks."""

    def __init__(self):
        self.diff = 0.0
        self.scale = 0.0
        self.nan_mismatch = 0

    def add(self, got, want):
        got = np.asarray(got, dtype=np.float64)
        want = np.asarray(want, dtype=np.float64)
        self.nan_mismatch += int(np.count_nonzero(np.isnan(got) != np.isnan(want)))
        ok = ~np.isnan(want)
        if ok.any():
            self.diff = max(self.diff, float(np.max(np.abs(got[ok] - want[ok]))))
            self.scale = max(self.scale, float(np.max(np.abs(want[ok]))))

    def value(self):
        assert self.nan_mismatch == 0, f"{self.nan_mismatch} NaN positions differ"
        return self.diff / (self.scale if self.scale > 0 else 1.0)


def _rows_f32(x, b, d0, d1):
    """Rows [b, d0:d1, :] of a host tensor as a float32 [d1-d0, L] array."""
    return None if x is None else x[b, d0:d1].to(torch.float32).numpy()


def compare_forward(inp, y, last, u_override=None, h0=None, chunk_states=None, state_chunk=0,
                    block_rows=2048, nthreads=0):
    """Compare y [b,d,L], last_state [b,d,n] (and chunk_states [b,K,d,n]) of
    the GPU with the C oracle on every row of ``inp``.  u_override replaces
    inp["u"] (the conv output in front of the scan); h0 [b,d,n] is the start
    state.  Returns a dict of metric values per tensor."""
    host = lambda t: None if t is None else t.detach().cpu()
    u = host(u_override if u_override is not None else inp["u"])
    dl, z = host(inp["delta"]), host(inp["z"])
    A, B, C = (host(inp[k]).float().numpy() for k in ("A", "B", "C"))
    D = None if inp["D"] is None else host(inp["D"]).float().numpy()
    bias = None if inp["delta_bias"] is None else host(inp["delta_bias"]).float().numpy()
    yh, lh = host(y), host(last)
    csh = host(chunk_states)
    h0h = host(h0)
    bsz, dim, L = inp["u"].shape
    n = A.shape[1]
    m = {"y": MaxRatio(), "last_state": MaxRatio()}
    if csh is not None:
        m["chunk_states"] = MaxRatio()
    for b in range(bsz):
        for d0 in range(0, dim, block_rows):
            d1 = min(dim, d0 + block_rows)
            rb = np.full(d1 - d0, b, dtype=np.int64)
            rd = np.arange(d0, d1, dtype=np.int64)
            h0_rows = None if h0h is None else h0h[b, d0:d1].double().numpy()
            res = cpu.fwd_rows(_rows_f32(u, b, d0, d1), _rows_f32(dl, b, d0, d1), _rows_f32(z, b, d0, d1), rb, rd,
                               A, B, C, D, bias, inp["delta_softplus"], bsz, dim, n, L, nthreads=nthreads,
                               h0_rows=h0_rows, chunk=state_chunk if csh is not None else 0)
            m["y"].add(yh[b, d0:d1].float().numpy(), res[0])
            m["last_state"].add(lh[b, d0:d1].numpy(), res[1])
            if csh is not None:
                m["chunk_states"].add(csh[b, :, d0:d1].numpy().transpose(1, 0, 2), res[2])
    return {k: v.value() for k, v in m.items()}
