"""MI355X (gfx950) Kimi Delta Attention operator.

The compute lives in libkda.so (hand-written HIP kernels behind the C ABI in
include/kda.h); this package is a thin binding over it:

    chunk_fwd(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None)
        -> (o, final_state)          chunked prefill, varlen via cu_seqlens
    decode_step(q, k, v, g, beta, scale, state) -> o
                                     one token per sequence, state in place
    chunk_fwd_snapshots(q, k, v, g, beta, scale, interval, ...)
        -> (o, final_state, snapshots) states every `interval` tokens
    fused_gate(z, w_up, u, b_up=None) -> (g, beta)
                                     gate inputs from their projections
    fused_recurrent_fwd(q, k, v, g, beta, scale, state) -> o
                                     a short run of tokens per sequence
                                     (T <= 64), state in place
    chunk_fwd_noalloc(q, k, v, g, beta, scale, ...) -> (o, final_state)
                                     chunk_fwd with the library's own
                                     workspace (no device allocation)
"""
from ._lib import (KDAError, abi_version, chunk_fwd, chunk_fwd_noalloc, chunk_fwd_snapshots,  # noqa: F401
                   decode_step,
                   fused_gate, fused_recurrent_fwd, lib, snapshot_rows, snapshots_workspace_size, status_str,
                   workspace_size)
