"""Full-size parity against the C oracle, streamed in token windows.

The packed token axis is cut into windows of W tokens.  Every (sequence
piece, head) chain of a window runs through the fp64 C oracle from either the
sequence's initial state or the fp64 state the oracle reached at the end of
the previous window, so a long sequence is followed exactly across windows
while host memory stays bounded (a window of 32768 tokens x 32 heads holds
about 5 GB).  The comparison accumulates max|x - ref| and sum(ref^2) over the
whole output, so the criterion is the same as for whole tensors:
max|x - ref| / rms(ref) over all of o, and over all final states.
"""
from __future__ import annotations

import math
import time

import numpy as np
import torch

from oracle import cref


class Accum:
    """max |x - ref| and rms(ref) over chunks of one tensor."""

    def __init__(self):
        self.maxabs = 0.0
        self.sumsq = 0.0
        self.count = 0

    def add(self, x: np.ndarray, ref: np.ndarray):
        if ref.size == 0:
            return
        self.maxabs = max(self.maxabs, float(np.max(np.abs(x - ref))))
        self.sumsq += float(np.sum(ref * ref))
        self.count += ref.size

    def rel(self) -> float:
        if self.count == 0:
            return 0.0
        return self.maxabs / max(math.sqrt(self.sumsq / self.count), 1e-30)


def _host_hmajor(t: torch.Tensor) -> np.ndarray:
    """[W, H, d] device slice -> float32 host array [H, W, d] (rows h W + t)."""
    return t.to("cpu", torch.float32).permute(1, 0, 2).contiguous().numpy()


def stream_compare(x, o: torch.Tensor, final: torch.Tensor, window: int = 32768,
                   n_threads: int = 0, log=print, absolute: bool = False):
    """Compare o [1, T, H, dv] and final [N, H, dk, dv] (device tensors) of
    inputs x (synth.KDAInputs, B = 1, on the device) with the C oracle over
    every token, head and sequence.  Returns (rel_o, rel_final), the
    max|x - ref| / rms(ref) of each, or with absolute=True the max|x - ref|
    of each (the fp32-input criterion)."""
    B, T, H, dk = x.q.shape
    dv = x.v.shape[-1]
    assert B == 1
    cu = np.asarray(x.cu_seqlens if x.cu_seqlens is not None else [0, T], dtype=np.int64)
    N = len(cu) - 1
    carry = {}
    acc_o, acc_f = Accum(), Accum()
    t_oracle = 0.0
    for a in range(0, T, window):
        b = min(a + window, T)
        W = b - a
        pieces = []  # (n, s, e)
        for n in range(N):
            s, e = max(int(cu[n]), a), min(int(cu[n + 1]), b)
            if s < e:
                pieces.append((n, s, e))
        if not pieces:
            continue
        arrs = [_host_hmajor(t[0, a:b]) for t in (x.q, x.k, x.v, x.g)]
        beta = x.beta[0, a:b].to("cpu", torch.float32).t().contiguous().numpy()  # [H, W]
        starts, lens, h0s = [], [], []
        have_h0 = x.h0 is not None
        h0_host = None
        for n, s, e in pieces:
            for h in range(H):
                starts.append(h * W + (s - a))
                lens.append(e - s)
                if s == int(cu[n]):
                    if have_h0:
                        if h0_host is None:
                            h0_host = x.h0.to("cpu", torch.float64).numpy()
                        h0s.append(h0_host[n, h])
                    else:
                        h0s.append(np.zeros((dk, dv)))
                else:
                    h0s.append(carry.pop((n, h)))
        t_0 = time.perf_counter()
        o_ref, fin = cref.run_packed(starts, lens, dk, dv, x.scale,
                                     *(z.reshape(H * W, -1) for z in arrs),
                                     beta.reshape(H * W), np.stack(h0s), True, n_threads)
        t_oracle += time.perf_counter() - t_0
        o_gpu = o[0, a:b].to("cpu", torch.float64).permute(1, 0, 2).contiguous().numpy().reshape(H * W, dv)
        i = 0
        for n, s, e in pieces:
            for h in range(H):
                r0 = h * W + (s - a)
                acc_o.add(o_gpu[r0:r0 + (e - s)], o_ref[r0:r0 + (e - s)])
                if e == int(cu[n + 1]):
                    acc_f.add(final[n, h].to("cpu", torch.float64).numpy(), fin[i])
                else:
                    carry[(n, h)] = fin[i]
                i += 1
        # a sequence that ends before its first token reaches a window (empty)
        log(f"  tokens [{a}, {b}): running max|do| {acc_o.maxabs:.2e}, max|do|/rms {acc_o.rel():.2e}, "
            f"oracle {t_oracle:.1f} s")
    for n in range(N):  # empty sequences: final state = initial state
        if cu[n] == cu[n + 1]:
            for h in range(H):
                ref = x.h0[n, h].to("cpu", torch.float64).numpy() if x.h0 is not None \
                    else np.zeros((dk, dv))
                acc_f.add(final[n, h].to("cpu", torch.float64).numpy(), ref)
    assert not carry, "every sequence must end inside the token axis"
    if absolute:
        return acc_o.maxabs, acc_f.maxabs
    return acc_o.rel(), acc_f.rel()
