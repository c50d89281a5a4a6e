"""Loader for the C fp64 oracle (kda_ref.c) -- test infrastructure only.

The library is built with gcc into oracle/libkda_ref.so (`build()`); the
loader builds it when it is missing.  It shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .ref import chain_list, _np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_ref.c")
_LIB = os.path.join(_HERE, "libkda_ref.so")
_lib = None


def build(force: bool = True) -> str:
    stale = not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.kda_ref_chains.argtypes = [ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_double, P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.kda_ref_chains.restype = ctypes.c_int
        lib.kda_ref_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_ref_max_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def run_packed(start, length, dk, dv, scale, q, k, v, g, beta, h0=None, with_o=True,
               n_threads=0):
    """Chains given by row ranges of packed float32 arrays (see kda_ref.c)."""
    lib = _load()
    start = np.ascontiguousarray(start, dtype=np.int64)
    length = np.ascontiguousarray(length, dtype=np.int64)
    arrs = [np.ascontiguousarray(x, dtype=np.float32) for x in (q, k, v, g, beta)]
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    rows = arrs[0].shape[0]
    o = np.zeros((rows, dv), dtype=np.float64) if with_o else None
    fin = np.zeros((len(start), dk, dv), dtype=np.float64)
    rc = lib.kda_ref_chains(len(start), _ptr(start), _ptr(length), dk, dv, float(scale),
                            *[_ptr(a) for a in arrs], _ptr(h0), _ptr(o), _ptr(fin), int(n_threads))
    if rc != 0:
        raise RuntimeError("kda_ref_chains failed")
    return o, fin


def kda_forward_chains(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None,
                       select=None, with_o=True, n_threads=0):
    """Run the chains `select` (list of (sequence n, head h); all when None)
    of a [B, T, H, d] batch.  Returns a list of (o [L, dv] or None,
    final [dk, dv]) in fp64, one per selected chain."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    chains = chain_list(B, T, cu_seqlens)
    if select is None:
        select = [(n, h) for n in range(len(chains)) for h in range(H)]
    parts = {x: [] for x in "qkvgb"}
    h0s, starts, lens = [], [], []
    row = 0
    for n, h in select:
        b, t0, t1 = chains[n]
        for name, src in zip("qkvgb", (q, k, v, g, beta)):
            parts[name].append(_np(src[b, t0:t1, h], np.float32))
        if initial_state is not None:
            h0s.append(_np(initial_state[n, h], np.float64))
        starts.append(row)
        lens.append(t1 - t0)
        row += t1 - t0
    cat = lambda xs, shp: np.concatenate(xs) if xs else np.zeros(shp, np.float32)
    o, fin = run_packed(starts, lens, dk, dv, scale, cat(parts["q"], (0, dk)),
                        cat(parts["k"], (0, dk)), cat(parts["v"], (0, dv)),
                        cat(parts["g"], (0, dk)), cat(parts["b"], (0,)),
                        np.stack(h0s) if h0s else None, with_o, n_threads)
    out = []
    for i, (s, L) in enumerate(zip(starts, lens)):
        out.append((o[s:s + L] if o is not None else None, fin[i]))
    return out


def kda_forward(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None, n_threads=0):
    """Whole-batch form with the same outputs as ref.kda_forward (fp64)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    chains = chain_list(B, T, cu_seqlens)
    res = kda_forward_chains(q, k, v, g, beta, scale, initial_state, cu_seqlens,
                             n_threads=n_threads)
    o = np.zeros((B, T, H, dv))
    fin = np.zeros((len(chains), H, dk, dv))
    i = 0
    for n, (b, t0, t1) in enumerate(chains):
        for h in range(H):
            oc, f = res[i]
            o[b, t0:t1, h] = oc
            fin[n, h] = f
            i += 1
    return o, fin
