"""numpy reference of the KDA recurrence (oracle, test infrastructure only).

Follows "Understanding Kimi Delta Attention", section "The KDA Recurrence"
(channel-wise update S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T)
and "kimi delta attn from first principles", section "KDA" (row-wise decay
Diag(alpha) S_{t-1}, then the delta-rule error form of the update) and
section "three gates" (read-out o_t = S_t^T q_t).

Readings of the pages adopted here:
  * decay before erase: the update multiplies Diag(alpha) onto S_{t-1} first
    and the delta-rule error is taken against the decayed state (equation of
    the first page's "The KDA Recurrence"; the step list "decay, erase,
    write" of the second page's notebook toy);
  * the gate scales rows, and rows are key channels (one forget gate per row
    of the memory matrix, third page, section "Problems with GDN"/"KDA");
  * the read-out uses the query and the updated state (third page, "three
    gates"; the first page's "o_t = S_t k_t" is read as a garbled form);
  * o is multiplied by the caller's `scale` (the pages give none);
  * alpha = exp(g): the operator takes the log-gate g;
  * a missing initial state is zero (the toy notebook "starts empty");
  * packed sequences (cu_seqlens) are independent chains with their own
    initial and final states.
"""
from __future__ import annotations

import numpy as np


def _np(x, dtype):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=dtype)


def chain_list(B, T, cu_seqlens):
    """(row, start, end) for every sequence: rows of a [B, T] batch, or the
    packed segments of cu_seqlens (then B must be 1)."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    assert B == 1 and cu[0] == 0 and cu[-1] == T
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def kda_forward(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None,
                dtype=np.float64):
    """Sequential KDA over every chain.

    q, k, g: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H];
    initial_state: [N, H, dk, dv] or None (zeros); cu_seqlens: [N+1] or None.
    Returns o [B, T, H, dv] and the final states [N, H, dk, dv] in `dtype`.
    """
    q, k, v, g, beta = (_np(x, dtype) for x in (q, k, v, g, beta))
    h0 = _np(initial_state, dtype)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    chains = chain_list(B, T, cu_seqlens)
    o = np.zeros((B, T, H, dv), dtype=dtype)
    final = np.zeros((len(chains), H, dk, dv), dtype=dtype)
    for n, (b, t0, t1) in enumerate(chains):
        S = np.zeros((H, dk, dv), dtype=dtype) if h0 is None else h0[n].copy()
        for t in range(t0, t1):
            alpha = np.exp(g[b, t])                      # [H, dk]   step 1
            S = alpha[:, :, None] * S                    # decay rows  step 2
            pred = np.einsum("hkv,hk->hv", S, k[b, t])   # S^T k
            u = beta[b, t][:, None] * (v[b, t] - pred)   # step 3
            S = S + k[b, t][:, :, None] * u[:, None, :]  # step 4
            o[b, t] = scale * np.einsum("hkv,hk->hv", S, q[b, t])  # step 5
        final[n] = S
    return o, final


def kda_decode(q, k, v, g, beta, scale, state, dtype=np.float64):
    """One token for each of N independent sequences.

    q, k, g: [N, H, dk]; v: [N, H, dv]; beta: [N, H]; state [N, H, dk, dv].
    Returns (o [N, H, dv], new_state).  This is the same recurrence with one
    token per chain, which is what the single-token (fused recurrent) mode on
    the first page computes.
    """
    q, k, v, g, beta = (_np(x, dtype) for x in (q, k, v, g, beta))
    s = _np(state, dtype)
    o, final = kda_forward(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                           scale, s, None, dtype)
    return o[:, 0], final


def kda_fused_recurrent(q, k, v, g, beta, scale, state, dtype=np.float64):
    """A run of T tokens for each of N independent sequences from a given
    state: q, k, g [N, T, H, dk]; v [N, T, H, dv]; beta [N, T, H];
    state [N, H, dk, dv].  Returns (o [N, T, H, dv], state after the run).
    Row n of the batch is one chain, so this is the sequential recurrence
    above with the rows as sequences (the fused recurrent mode of the first
    page run over several tokens)."""
    return kda_forward(q, k, v, g, beta, scale, state, None, dtype)


def kda_forward_snapshots(q, k, v, g, beta, scale, interval, initial_state=None,
                          cu_seqlens=None, dtype=np.float64):
    """kda_forward that also keeps the state of every chain after each
    `interval` tokens: states at prefix boundaries, as a KDA-aware prefix
    cache stores them (concept page "Kimi Delta Attention (KDA)", section
    "KV Caching Challenges & vLLM Contribution").

    Returns (o, final, snaps): snaps [total, H, dk, dv] holds, chain by chain
    in order and within a chain by position, the state after tokens
    0 .. (j + 1) interval - 1 of the chain for j = 0 .. floor(len / interval) - 1.
    """
    q, k, v, g, beta = (_np(x, dtype) for x in (q, k, v, g, beta))
    h0 = _np(initial_state, dtype)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    chains = chain_list(B, T, cu_seqlens)
    o = np.zeros((B, T, H, dv), dtype=dtype)
    final = np.zeros((len(chains), H, dk, dv), dtype=dtype)
    snaps = []
    for n, (b, t0, t1) in enumerate(chains):
        S = np.zeros((H, dk, dv), dtype=dtype) if h0 is None else h0[n].copy()
        for t in range(t0, t1):
            S = np.exp(g[b, t])[:, :, None] * S
            u = beta[b, t][:, None] * (v[b, t] - np.einsum("hkv,hk->hv", S, k[b, t]))
            S = S + k[b, t][:, :, None] * u[:, None, :]
            o[b, t] = scale * np.einsum("hkv,hk->hv", S, q[b, t])
            if (t + 1 - t0) % interval == 0:   # a prefix boundary
                snaps.append(S.copy())
        final[n] = S
    snaps = np.stack(snaps) if snaps else np.zeros((0, H, dk, dv), dtype=dtype)
    return o, final, snaps


def rms_norm_gate(o, gate, weight, eps, dtype=np.float64):
    """The output path after the read-out ("kimi delta attn from first
    principles", section "three gates": RMSNorm is applied to o_t = S_t^T q_t,
    then the result is multiplied elementwise by the output gate).

    o, gate: [..., dv] (one vector per token and head); weight: [dv]; returns
    gate * weight * o / sqrt(mean(o^2) + eps), the mean over the dv channels of
    one (token, head).  Readings: the RMSNorm has a per-channel weight shared
    by all heads and an eps inside the root (the pages name RMSNorm without
    its parameters); the gate arrives already activated (the pages give the
    gate a low-rank projection but not its activation).
    """
    o, gate = _np(o, dtype), _np(gate, dtype)
    w = _np(weight, dtype)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return gate * w * o / np.sqrt(ms + eps)


def fused_gate(z, w_up, u, b_up=None, H=None, dtype=np.float64):
    """The gate inputs from their projections ("kimi delta attn from first
    principles", section "three gates": a low-rank projection -- down, then
    up to the key channels -- gives the forget gate; a sigmoid of its
    projection gives the update gate beta).

    z [M, r], w_up [H dk, r] (one row per output channel), u [M, H],
    b_up [H dk] or None.  Returns g [M, H, dk] = -softplus(z w_up^T + b_up)
    (the log-decay, <= 0) and
    beta [M, H] = sigmoid(u).  Reading: the pages do not give the activation
    that turns the up-projection into a log-decay; -softplus is the one
    adopted here (alpha = exp(g) = sigmoid(-(z w_up^T + b)) lies in (0, 1)).
    """
    z, w, u = _np(z, dtype), _np(w_up, dtype), _np(u, dtype)
    M = z.shape[0]
    H = u.shape[1] if H is None else H
    a = z @ w.T
    if b_up is not None:
        a = a + _np(b_up, dtype)
    g = -np.logaddexp(0.0, a)
    beta = 1.0 / (1.0 + np.exp(-u))
    return g.reshape(M, H, -1), beta
