"""ctypes binding of libkda.so (argument marshalling only).

Every step of the operator runs in the library's HIP kernels; this module
only checks torch tensors, allocates outputs and workspace with torch, and
passes raw device pointers plus the current HIP stream across the C ABI
declared in include/kda.h.  There is no fallback: if the library is missing
the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
          4: "KDA_ERR_UNSUPPORTED", 5: "KDA_ERR_SEQLENS", 6: "KDA_ERR_ALIAS",
          7: "KDA_ERR_ALIGN", 8: "KDA_ERR_WORKSPACE", 9: "KDA_ERR_HIP"}
F32, BF16 = 0, 1
VARIANTS = {"auto": 0, "recurrent": 1, "chunk": 2, "chunk_scan": 3, "chunk64": 4, "chunk8": 5}
EXPORTS = ("kda_abi_version", "kda_status_str", "kda_chunk_fwd_workspace_size",
           "kda_chunk_fwd", "kda_decode_step", "kda_fused_recurrent_fwd",
           "kda_chunk_fwd_snapshots_workspace_size", "kda_chunk_fwd_snapshots",
           "kda_chunk_fwd_gated", "kda_fused_gate", "kda_chunk_fwd_noalloc")
NOALLOC_MAX_WORKSPACE = 32 << 20
FUSED_RECURRENT_MAX_T = 64


class KDAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m gated_delta_rule_89_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_size.argtypes = [I32] * 6 + [P, ctypes.c_int, ctypes.c_int]
    lib.kda_chunk_fwd_workspace_size.restype = SZ
    lib.kda_chunk_fwd.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P,
                                  I32, I32, I32, I32, I32, I32, ctypes.c_int, ctypes.c_int,
                                  P, P, P, SZ, ctypes.c_int, P]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [P, P, P, P, P, ctypes.c_float, P, I32, I32, I32, I32,
                                    ctypes.c_int, ctypes.c_int, P, P]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_fused_recurrent_fwd.argtypes = [P, P, P, P, P, ctypes.c_float, P, I32, I32, I32, I32,
                                            I32, ctypes.c_int, ctypes.c_int, P, P]
    lib.kda_fused_recurrent_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_snapshots_workspace_size.argtypes = [I32] * 6 + [P, ctypes.c_int, ctypes.c_int, I32]
    lib.kda_chunk_fwd_snapshots_workspace_size.restype = SZ
    lib.kda_chunk_fwd_snapshots.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P,
                                            I32, I32, I32, I32, I32, I32, ctypes.c_int, ctypes.c_int,
                                            P, P, I32, P, P, SZ, ctypes.c_int, P]
    lib.kda_chunk_fwd_snapshots.restype = ctypes.c_int
    lib.kda_chunk_fwd_gated.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P,
                                        I32, I32, I32, I32, I32, I32, ctypes.c_int, ctypes.c_int,
                                        P, P, ctypes.c_float, P, P, P, SZ, ctypes.c_int, P]
    lib.kda_chunk_fwd_gated.restype = ctypes.c_int
    lib.kda_fused_gate.argtypes = [P, P, P, P, I32, I32, I32, I32, ctypes.c_int, P, P, P]
    lib.kda_fused_gate.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, P,
                                          I32, I32, I32, I32, I32, I32, ctypes.c_int, ctypes.c_int,
                                          P, P, ctypes.c_int, P]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    return lib


lib = _load()


def status_str(code: int) -> str:
    return lib.kda_status_str(code).decode()


def abi_version() -> int:
    return int(lib.kda_abi_version())


def _check(code: int):
    if code != 0:
        raise KDAError(code, status_str(code))


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_size(B, T, H, dk, dv, N, in_dtype=torch.bfloat16, variant="auto",
                   cu_seqlens_host=None) -> int:
    """Workspace bytes for these sizes; cu_seqlens_host is an int32 CPU tensor or None."""
    ptr = None if cu_seqlens_host is None else ctypes.c_void_p(cu_seqlens_host.data_ptr())
    return int(lib.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, N, ptr, _dt(in_dtype),
                                                VARIANTS[variant]))


def snapshots_workspace_size(B, T, H, dk, dv, N, interval, in_dtype=torch.bfloat16,
                             variant="auto", cu_seqlens_host=None) -> int:
    """Workspace bytes kda_chunk_fwd_snapshots needs for these sizes."""
    ptr = None if cu_seqlens_host is None else ctypes.c_void_p(cu_seqlens_host.data_ptr())
    return int(lib.kda_chunk_fwd_snapshots_workspace_size(B, T, H, dk, dv, N, ptr, _dt(in_dtype),
                                                          VARIANTS[variant], int(interval)))


def snapshot_rows(lengths, interval: int) -> np.ndarray:
    """Row of every sequence's first snapshot and, last, the total: an
    exclusive prefix sum of floor(length / interval)."""
    cnt = np.asarray(lengths, dtype=np.int64) // int(interval)
    return np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)


def chunk_fwd_snapshots(q, k, v, g, beta, scale, snapshot_interval: int, **kw):
    """kda_chunk_fwd_snapshots: chunk_fwd that also returns the state of every
    sequence after each `snapshot_interval` tokens (a multiple of 64).
    Returns (o, final_state, snapshots [total, H, dk, dv]); sequence n's
    snapshots are rows snapshot_rows(lengths, interval)[n] onwards."""
    return chunk_fwd(q, k, v, g, beta, scale, snapshot_interval=snapshot_interval, **kw)


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, scale: float, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Union[None, torch.Tensor, np.ndarray, Sequence[int]] = None,
              output_final_state: bool = True, out_dtype: torch.dtype = torch.float32,
              variant: str = "auto", o: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None,
              cu_seqlens_host: Optional[torch.Tensor] = None,
              snapshot_interval: Optional[int] = None,
              snapshots: Optional[torch.Tensor] = None,
              out_gate: Optional[torch.Tensor] = None,
              norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
              _noalloc: bool = False):
    """kda_chunk_fwd on torch tensors.  q, k, g: [B, T, H, dk]; v: [B, T, H, dv];
    beta: [B, T, H]; initial_state [N, H, dk, dv] fp32 or None; cu_seqlens int32
    [N+1] (device tensor, CPU tensor, numpy array or list) or None.  A caller
    holding both copies passes the device tensor as cu_seqlens and an int32 CPU
    tensor as cu_seqlens_host, and no copy is made.
    Returns (o [B, T, H, dv], final_state [N, H, dk, dv] or None), and with
    snapshot_interval also the snapshots (kda_chunk_fwd_snapshots).  With
    out_gate [B, T, H, dv] (q's dtype) and norm_weight [dv] fp32, o is the gated
    RMSNorm of the read-out (kda_chunk_fwd_gated)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _dev(t, name)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    cu_dev = cu_host = None
    if cu_seqlens is not None and cu_seqlens_host is not None:
        cu_dev, cu_host = cu_seqlens, cu_seqlens_host
        _dev(cu_dev, "cu_seqlens")
        if cu_host.is_cuda or cu_host.dtype != torch.int32 or not cu_host.is_contiguous():
            raise ValueError("cu_seqlens_host must be a contiguous int32 CPU tensor")
        N = cu_host.numel() - 1
    elif cu_seqlens is not None:
        if isinstance(cu_seqlens, torch.Tensor):
            cu_host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
            cu_dev = cu_seqlens if (cu_seqlens.is_cuda and cu_seqlens.dtype == torch.int32
                                    and cu_seqlens.is_contiguous()) else cu_host.to(dev)
        else:
            cu_host = torch.as_tensor(np.asarray(cu_seqlens, dtype=np.int32))
            cu_dev = cu_host.to(dev)
        N = cu_host.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _dev(initial_state, "initial_state")
    if o is None:
        o = torch.empty(B, T, H, dv, dtype=out_dtype, device=dev)
    if output_final_state and final_state is None:
        final_state = torch.empty(N, H, dk, dv, dtype=torch.float32, device=dev)
    if not output_final_state:
        final_state = None
    if snapshot_interval is not None:
        lens = np.diff(cu_host.numpy()) if cu_host is not None else np.full(N, T)
        total = int(snapshot_rows(lens, snapshot_interval)[-1]) if snapshot_interval > 0 else 0
        if snapshots is None:
            snapshots = torch.empty(total, H, dk, dv, dtype=torch.float32, device=dev)
        cu_ptr = None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr())
        ws_bytes = snapshots_workspace_size(B, T, H, dk, dv, N, snapshot_interval, q.dtype, variant,
                                            cu_host)
        if workspace is None and ws_bytes > 0:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        code = lib.kda_chunk_fwd_snapshots(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(initial_state),
            _ptr(cu_dev), cu_ptr, B, T, H, dk, dv, N, _dt(q.dtype), _dt(o.dtype), _ptr(o),
            _ptr(final_state), int(snapshot_interval), _ptr(snapshots) if snapshots.numel() else None,
            _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
            VARIANTS[variant], _stream(dev))
        _check(code)
        return o, final_state, snapshots
    if _noalloc:
        code = lib.kda_chunk_fwd_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(initial_state),
            _ptr(cu_dev), None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr()),
            B, T, H, dk, dv, N, _dt(q.dtype), _dt(o.dtype), _ptr(o), _ptr(final_state),
            VARIANTS[variant], _stream(dev))
        _check(code)
        return o, final_state
    ws_bytes = workspace_size(B, T, H, dk, dv, N, q.dtype, variant, cu_host)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if out_gate is not None:
        _dev(out_gate, "out_gate")
        _dev(norm_weight, "norm_weight")
        code = lib.kda_chunk_fwd_gated(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(initial_state),
            _ptr(cu_dev), None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr()),
            B, T, H, dk, dv, N, _dt(q.dtype), _dt(o.dtype), _ptr(out_gate), _ptr(norm_weight),
            float(norm_eps), _ptr(o), _ptr(final_state), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            VARIANTS[variant], _stream(dev))
        _check(code)
        return o, final_state
    code = lib.kda_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(initial_state),
        _ptr(cu_dev), None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr()),
        B, T, H, dk, dv, N, _dt(q.dtype), _dt(o.dtype), _ptr(o), _ptr(final_state),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        VARIANTS[variant], _stream(dev))
    _check(code)
    return o, final_state


def chunk_fwd_noalloc(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None, **kw):
    """kda_chunk_fwd_noalloc: chunk_fwd whose workspace is the library's own
    per-GPU device array (at most NOALLOC_MAX_WORKSPACE bytes), so the C call
    allocates nothing; pass o and final_state to allocate nothing here either.
    Calls on one GPU must not overlap.  No snapshots or gated output."""
    for bad in ("workspace", "snapshot_interval", "snapshots", "out_gate", "norm_weight"):
        if kw.get(bad) is not None:
            raise ValueError(f"chunk_fwd_noalloc takes no {bad}")
    return chunk_fwd(q, k, v, g, beta, scale, initial_state, cu_seqlens, _noalloc=True, **kw)


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, scale: float, state: torch.Tensor,
                out_dtype: torch.dtype = torch.float32, o: Optional[torch.Tensor] = None):
    """kda_decode_step: q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H];
    state [N, H, dk, dv] fp32, updated in place.  Returns o [N, H, dv]."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state)):
        _dev(t, name)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty(N, H, dv, dtype=out_dtype, device=q.device)
    code = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                               _ptr(state), N, H, dk, dv, _dt(q.dtype), _dt(o.dtype), _ptr(o),
                               _stream(q.device))
    _check(code)
    return o


def fused_recurrent_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        beta: torch.Tensor, scale: float, state: torch.Tensor,
                        out_dtype: torch.dtype = torch.float32, o: Optional[torch.Tensor] = None):
    """kda_fused_recurrent_fwd: q, k, g [N, T, H, dk]; v [N, T, H, dv];
    beta [N, T, H]; state [N, H, dk, dv] fp32, updated in place after the
    run of T tokens.  Returns o [N, T, H, dv]."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state)):
        _dev(t, name)
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty(N, T, H, dv, dtype=out_dtype, device=q.device)
    code = lib.kda_fused_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                       _ptr(state), N, T, H, dk, dv, _dt(q.dtype), _dt(o.dtype),
                                       _ptr(o), _stream(q.device))
    _check(code)
    return o


def fused_gate(z: torch.Tensor, w_up: torch.Tensor, u: torch.Tensor,
               b_up: Optional[torch.Tensor] = None, H: Optional[int] = None):
    """kda_fused_gate: z [M, r] bf16, w_up [H*dk, r] bf16 (a linear layer's
    weight), u [M, H] fp32, b_up [H*dk] fp32 or None.  Returns
    (g [M, H, dk] fp32, beta [M, H] fp32) with g = -softplus(z w_up^T + b_up)
    and beta = sigmoid(u)."""
    for name, t in (("z", z), ("w_up", w_up), ("u", u)):
        _dev(t, name)
    if b_up is not None:
        _dev(b_up, "b_up")
    M, r = z.shape
    H = u.shape[1] if H is None else H
    dk = w_up.shape[0] // H
    g = torch.empty(M, H, dk, dtype=torch.float32, device=z.device)
    beta = torch.empty(M, H, dtype=torch.float32, device=z.device)
    code = lib.kda_fused_gate(_ptr(z), _ptr(w_up), _ptr(b_up), _ptr(u), M, r, H, dk, _dt(z.dtype),
                              _ptr(g), _ptr(beta), _stream(z.device))
    _check(code)
    return g, beta
