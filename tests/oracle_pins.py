"""Pins for the oracle: checks against what the pages and the mathematics fix,
independent of the oracle's own step-by-step code.

Each check takes an implementation `fn(q, k, v, g, beta, scale, h0, cu)` that
returns (o [B,T,H,dv], final [N,H,dk,dv]) as numpy fp64 and raises
AssertionError when the implementation disagrees with the pinned result.
The same checks run on the numpy oracle, the C oracle and on planted-mistake
mutants of the oracle (which must each fail at least one check).

Page references use the page titles:
  [P1] "Understanding Kimi Delta Attention"
  [P2] "kimi-k3 / KDA scales" (the notebook toy)
  [P3] "kimi delta attn from first principles"
"""
from __future__ import annotations

import numpy as np

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(x):
    """Inputs are drawn as float32-representable values so that implementations
    taking float32 inputs (the C oracle, the GPU path) see the exact same numbers."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _unit_keys(rng, shape):
    """Keys of exactly unit norm in binary floating point: +-1/2 on four channels."""
    *lead, dk = shape
    k = np.zeros(shape)
    flat = k.reshape(-1, dk)
    for r in range(flat.shape[0]):
        ch = rng.choice(dk, size=4, replace=False)
        flat[r, ch] = 0.5 * rng.choice([-1.0, 1.0], size=4)
    return k


def _batch(rng, B=1, T=12, H=2, dk=6, dv=5, unit_k=False, beta_hi=1.0, g_scale=0.7):
    q = _f32(rng.standard_normal((B, T, H, dk)))
    k = _unit_keys(rng, (B, T, H, dk)) if unit_k else _f32(rng.standard_normal((B, T, H, dk)))
    v = _f32(rng.standard_normal((B, T, H, dv)))
    g = _f32(-g_scale * rng.random((B, T, H, dk)) * 2.0)
    beta = _f32(beta_hi * rng.random((B, T, H)))
    return q, k, v, g, beta


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol * max(1.0, np.max(np.abs(b)) if b.size else 1.0), f"{what}: max err {err:g}"


# --- P1: brute-force products of the per-step transition matrices -----------------------
def transition_products(q, k, v, g, beta, scale, h0):
    """S_t = M_t S_{t-1} + b_t with explicit M_t = (I - beta k k^T) Diag(exp g) and
    b_t = beta k v^T ([P1] "The KDA Recurrence"), evaluated as the closed sum
    S_t = (prod_{s<=t} M_s) S_0 + sum_{i<=t} (prod_{i<s<=t} M_s) b_i for every t."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    fin = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            M = [(np.eye(dk) - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h]))
                 @ np.diag(np.exp(g[b, t, h])) for t in range(T)]
            bt = [beta[b, t, h] * np.outer(k[b, t, h], v[b, t, h]) for t in range(T)]
            S0 = np.zeros((dk, dv)) if h0 is None else h0[b, h]
            for t in range(T):
                P = np.eye(dk)
                for s in range(t + 1):
                    P = M[s] @ P
                St = P @ S0
                for i in range(t + 1):
                    Pi = np.eye(dk)
                    for s in range(i + 1, t + 1):
                        Pi = M[s] @ Pi
                    St = St + Pi @ bt[i]
                o[b, t, h] = scale * St.T @ q[b, t, h]
                if t == T - 1:
                    fin[b, h] = St
    return o, fin


def pin_bruteforce(fn, seed=11):
    rng = _rng(seed)
    q, k, v, g, beta = _batch(rng, B=2, T=9, H=2, dk=5, dv=4, beta_hi=1.5)
    h0 = _f32(rng.standard_normal((2, 2, 5, 4)))
    o, f = fn(q, k, v, g, beta, 0.37, h0, None)
    ob, fb = transition_products(q, k, v, g, beta, 0.37, h0)
    _close(o, ob, what="P1 o")
    _close(f, fb, what="P1 final")


# --- P2: scalar gate => Gated DeltaNet --------------------------------------------------
def pin_scalar_gate(fn, seed=12):
    """g_t equal on every channel reduces KDA to Gated DeltaNet,
    S_t = a_t (I - beta k k^T) S_{t-1} + beta k v^T ([P1] "The KDA Recurrence";
    [P3] "Gated DeltaNet"), here evaluated as plain matrix products."""
    rng = _rng(seed)
    q, k, v, g, beta = _batch(rng, T=14, H=2, dk=6, dv=7)
    gam = _f32(-rng.random((1, 14, 2)))
    g = np.repeat(gam[..., None], 6, axis=-1)
    h0 = _f32(rng.standard_normal((1, 2, 6, 7)))
    o, f = fn(q, k, v, g, beta, 0.5, h0, None)
    for h in range(2):
        S = h0[0, h].copy()
        for t in range(14):
            kk = k[0, t, h]
            S = np.exp(gam[0, t, h]) * (np.eye(6) - beta[0, t, h] * np.outer(kk, kk)) @ S \
                + beta[0, t, h] * np.outer(kk, v[0, t, h])
            _close(o[0, t, h], 0.5 * S.T @ q[0, t, h], what="P2 o")
        _close(f[0, h], S, what="P2 final")


# --- P3: alpha = 1, orthonormal keys => causal linear attention -------------------------
def pin_linear_attention(fn, seed=13):
    """With alpha = 1, S_0 = 0 and orthonormal keys the erase term vanishes and
    o_t = scale * sum_{i<=t} beta_i (k_i . q_t) v_i: causal linear attention with
    beta-weighted values ([P3] "Linear Attention", "So what's wrong with Linear
    attention?").  Evaluated as a masked (Q K^T) diag(beta) V product."""
    rng = _rng(seed)
    T, dk, dv = 10, 16, 6
    Hd = np.array([[1.0]])
    while Hd.shape[0] < dk:                           # Sylvester Hadamard, rows / 4 are
        Hd = np.block([[Hd, Hd], [Hd, -Hd]])          # exactly orthonormal in binary
    Hd = Hd[rng.permutation(dk)] * (rng.choice([-1.0, 1.0], size=dk)[None, :]) / 4.0
    k = Hd[:T][None, :, None, :]                     # orthonormal rows
    q = _f32(rng.standard_normal((1, T, 1, dk)))
    v = _f32(rng.standard_normal((1, T, 1, dv)))
    beta = _f32(rng.random((1, T, 1)) + 0.2)
    g = np.zeros((1, T, 1, dk))
    o, f = fn(q, k, v, g, beta, 0.3, None, None)
    A = np.tril(q[0, :, 0] @ k[0, :, 0].T)           # [T, T] causal scores
    ref = 0.3 * A @ (beta[0, :, 0][:, None] * v[0, :, 0])
    _close(o[0, :, 0], ref, what="P3 o")
    _close(f[0, 0], (beta[0, :, 0][:, None] * k[0, :, 0]).T @ v[0, :, 0], what="P3 final")


# --- P4: alpha = 1 => DeltaNet ----------------------------------------------------------
def pin_deltanet(fn, seed=14):
    """g = 0 gives the plain delta rule, written in its factored form
    S_t = (I - beta k k^T) S_{t-1} + beta k v^T ([P3] "KDA", expansion of the
    DeltaNet update)."""
    rng = _rng(seed)
    q, k, v, g, beta = _batch(rng, T=11, H=1, dk=4, dv=6, beta_hi=1.8)
    g[:] = 0.0
    h0 = _f32(rng.standard_normal((1, 1, 4, 6)))
    o, f = fn(q, k, v, g, beta, 1.0, h0, None)
    S = h0[0, 0].copy()
    for t in range(11):
        kk = k[0, t, 0]
        S = (np.eye(4) - beta[0, t, 0] * np.outer(kk, kk)) @ S + beta[0, t, 0] * np.outer(kk, v[0, t, 0])
        _close(o[0, t, 0], S.T @ q[0, t, 0], what="P4 o")
    _close(f[0, 0], S, what="P4 final")


# --- P5: rank-1 overwrite ---------------------------------------------------------------
def pin_overwrite(fn, seed=15):
    """beta = 1 and unit k: the write first erases the (decayed) memory's
    projection on k, so the updated state returns exactly v for k:
    S_t^T k_t = v_t ([P1] "The role of beta"; [P3] "DeltaNet").  Read with q = k."""
    rng = _rng(seed)
    q, k, v, g, beta = _batch(rng, T=16, H=3, dk=7, dv=5, unit_k=True)
    beta[:] = 1.0
    h0 = _f32(rng.standard_normal((1, 3, 7, 5)))
    o, _ = fn(k.copy(), k, v, g, beta, 1.0, h0, None)
    _close(o, v, what="P5 S^T k = v")


# --- P6: one-hot keys => independent per-row EMAs --------------------------------------
def pin_one_hot(fn, seed=16):
    """With k_t = e_c every row decays by its own gate and only row c is
    rewritten: row c <- (1 - beta) alpha_c row c + beta v, other rows
    <- alpha row ([P3] "KDA": one forget gate per row; [P2] notebook toy:
    decay, erase, write).  Evaluated row by row with scalar loops."""
    rng = _rng(seed)
    T, dk, dv = 20, 5, 3
    idx = rng.integers(0, dk, size=T)
    k = np.zeros((1, T, 1, dk))
    k[0, np.arange(T), 0, idx] = 1.0
    q = _f32(rng.standard_normal((1, T, 1, dk)))
    v = _f32(rng.standard_normal((1, T, 1, dv)))
    g = _f32(-rng.random((1, T, 1, dk)) * 1.5)
    beta = _f32(rng.random((1, T, 1)))
    h0 = _f32(rng.standard_normal((1, 1, dk, dv)))
    o, f = fn(q, k, v, g, beta, 1.0, h0, None)
    rows = [list(h0[0, 0, c]) for c in range(dk)]
    bound = max(np.abs(h0).max(), np.abs(v).max())
    for t in range(T):
        for c in range(dk):
            a = float(np.exp(g[0, t, 0, c]))
            for j in range(dv):
                rows[c][j] *= a
        c = idx[t]
        b = float(beta[0, t, 0])
        for j in range(dv):
            rows[c][j] = (1.0 - b) * rows[c][j] + b * float(v[0, t, 0, j])
        ot = [sum(rows[cc][j] * q[0, t, 0, cc] for cc in range(dk)) for j in range(dv)]
        _close(o[0, t, 0], ot, what="P6 o")
    _close(f[0, 0], np.array(rows), what="P6 final")
    assert np.abs(f).max() <= bound + 1e-12, "P6 fixed budget"


# --- P7: state passing ------------------------------------------------------------------
def pin_state_passing(fn, seed=17):
    """The recurrence is a left-to-right scan: a split call resumed from the
    first half's final state equals the whole call, and packed sequences
    equal separate calls ([P1] chunkwise mode "equivalent to the sequential
    recurrence"; prefix states of [P4] "KV Caching")."""
    rng = _rng(seed)
    q, k, v, g, beta = _batch(rng, T=13, H=2, dk=4, dv=3)
    h0 = _f32(rng.standard_normal((1, 2, 4, 3)))
    o, f = fn(q, k, v, g, beta, 0.7, h0, None)
    o1, f1 = fn(q[:, :5], k[:, :5], v[:, :5], g[:, :5], beta[:, :5], 0.7, h0, None)
    o2, f2 = fn(q[:, 5:], k[:, 5:], v[:, 5:], g[:, 5:], beta[:, 5:], 0.7, f1, None)
    _close(np.concatenate([o1, o2], axis=1), o, what="P7 split o")
    _close(f2, f, what="P7 split final")
    # packed varlen == separate calls, including an empty sequence
    lens = [3, 0, 6, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    hs = _f32(rng.standard_normal((4, 2, 4, 3)))
    op, fp = fn(q, k, v, g, beta, 0.7, hs, cu)
    for n in range(4):
        a, b_ = cu[n], cu[n + 1]
        on, fnn = fn(q[:, a:b_], k[:, a:b_], v[:, a:b_], g[:, a:b_], beta[:, a:b_], 0.7,
                     hs[n:n + 1], None)
        _close(op[:, a:b_], on, what="P7 varlen o")
        _close(fp[n], fnn[0], what="P7 varlen final")
    _close(fp[1], hs[1], what="P7 empty sequence keeps its state")


# --- P8: beta = 0 closed form -----------------------------------------------------------
def pin_beta_zero(fn, seed=18):
    """beta = 0 writes nothing, so the state is the initial one decayed by the
    accumulated gates: S_t = Diag(exp(sum_{s<=t} g_s)) S_0 ([P1] "The KDA
    Recurrence")."""
    rng = _rng(seed)
    q, k, v, g, beta = _batch(rng, T=10, H=2, dk=6, dv=3)
    beta[:] = 0.0
    h0 = _f32(rng.standard_normal((1, 2, 6, 3)))
    o, f = fn(q, k, v, g, beta, 0.9, h0, None)
    G = np.cumsum(g, axis=1)  # [1, T, H, dk]
    St = np.exp(G)[0][:, :, :, None] * h0[0][None]  # [T, H, dk, dv]
    _close(o[0], 0.9 * np.einsum("thkv,thk->thv", St, q[0]), what="P8 o")
    _close(f[0], St[-1], what="P8 final")


ALL_PINS = [pin_bruteforce, pin_scalar_gate, pin_linear_attention, pin_deltanet,
            pin_overwrite, pin_one_hot, pin_state_passing, pin_beta_zero]
