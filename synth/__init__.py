"""Seeded synthetic inputs for the KDA operator.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It draws random tensors of the shapes and distributions of the
six workloads below and holds none of the operator's arithmetic: the L2
normalisation of q/k, the sigmoid for beta and the softplus for the log-gate
are the upstream projections that feed the operator (q/k normalisation and the
sigmoid update gate: "kimi delta attn from first principles", sections "three
gates" and "KDA Architecture"), not part of the recurrence.

Workloads (names used everywhere in the repository):

  tiny    B=1, T=64, H=1, d=16, all fp32, g=-softplus(N(0,1)), zero h0
  prefill B=1, T=4096, H=8, d=128, bf16 q/k/v, g=-softplus(N(0,2)-2),
          h0 ~ N(0, 0.02)
  decode  256 sequences x H=32, one token each, d=128, state ~ N(0, 0.02)
  verify  256 sequences x H=32, a run of 8 tokens each (a speculative draft
          checked against a cached state), d=128, state ~ N(0, 0.02)
  varlen  64 packed sequences, lengths log-uniform in [512, 32768] with an
          exact total of 262144 tokens, H=32, per-sequence h0 ~ N(0, 0.02)
  long    B=1, T=1048576, H=32, g=-softplus(N(0,2)-3), zero h0

N(mu, s) means mean mu and standard deviation s.

Generation rule.  Tokens are drawn in blocks of 65536 along the packed token
axis; block b of seed s uses a generator seeded with 1_000_003*s + b and draws
q, k, v, beta, g in that order.  The initial state uses seed 1_000_003*s - 1.
A torch generator on the requested device is used, so CPU and GPU draws
differ, but each is deterministic; parity tests hand the very same tensors to
both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch
import torch.nn.functional as F

BLOCK_TOKENS = 65536
SEED_STRIDE = 1_000_003


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    dk: int
    dv: int
    T: int                 # packed tokens (or decode sequences)
    in_dtype: torch.dtype  # dtype of q/k/v
    g_mu: float
    g_sigma: float
    h0_std: float          # 0 => zero initial state
    seed: int
    n_seqs: int = 1
    decode: bool = False
    steps: int = 1         # tokens per sequence of a state-in-place run

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)


WORKLOADS = {
    "tiny": Workload("tiny", H=1, dk=16, dv=16, T=64, in_dtype=torch.float32,
                     g_mu=0.0, g_sigma=1.0, h0_std=0.0, seed=1),
    "prefill": Workload("prefill", H=8, dk=128, dv=128, T=4096, in_dtype=torch.bfloat16,
                        g_mu=-2.0, g_sigma=2.0, h0_std=0.02, seed=2),
    "decode": Workload("decode", H=32, dk=128, dv=128, T=256, in_dtype=torch.bfloat16,
                       g_mu=-2.0, g_sigma=2.0, h0_std=0.02, seed=3, n_seqs=256, decode=True),
    "verify": Workload("verify", H=32, dk=128, dv=128, T=256, in_dtype=torch.bfloat16,
                       g_mu=-2.0, g_sigma=2.0, h0_std=0.02, seed=6, n_seqs=256, decode=True,
                       steps=8),
    "varlen": Workload("varlen", H=32, dk=128, dv=128, T=262144, in_dtype=torch.bfloat16,
                       g_mu=-2.0, g_sigma=2.0, h0_std=0.02, seed=4, n_seqs=64),
    "long": Workload("long", H=32, dk=128, dv=128, T=1048576, in_dtype=torch.bfloat16,
                     g_mu=-3.0, g_sigma=2.0, h0_std=0.0, seed=5),
    # the varlen workload's distributions with fp32 q/k/v (full mantissas)
    "varlen_f32": Workload("varlen_f32", H=32, dk=128, dv=128, T=262144, in_dtype=torch.float32,
                           g_mu=-2.0, g_sigma=2.0, h0_std=0.02, seed=8, n_seqs=64),
}


def varlen_lengths(n_seqs: int = 64, total: int = 262144, lo: int = 512, hi: int = 32768,
                   seed: int = 4) -> np.ndarray:
    """Sequence lengths for the packed prefill workload.

    A free log-uniform draw on [lo, hi] has a mean far above total/n_seqs, so
    the draw is pinned at both ends (one sequence of length hi, one of length
    lo), the other n_seqs-2 lengths are drawn log-uniformly and rescaled with
    clipping until they sum to the remaining total, then rounded with the
    largest-remainder rule and shuffled.
    """
    rng = np.random.default_rng(seed)
    rest = total - hi - lo
    L = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n_seqs - 2))
    for _ in range(200):
        L = np.clip(L * rest / L.sum(), lo, hi)
    base = np.floor(L).astype(np.int64)
    short = rest - int(base.sum())
    frac = L - base
    order = np.argsort(-frac, kind="stable")
    base[order[:short]] += 1
    lens = np.concatenate([[hi, lo], base]).astype(np.int64)
    lens = lens[rng.permutation(n_seqs)]
    assert int(lens.sum()) == total
    return lens


def cu_seqlens_from_lengths(lens) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


@dataclass
class KDAInputs:
    """One batch of operator inputs.  q/k/v/g/beta are [B, T, H, d] ([B, T, H]
    for beta); for decode and verify B is the number of sequences and T the
    tokens per sequence (1 for decode)."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    scale: float
    h0: Optional[torch.Tensor]                 # [N, H, dk, dv] fp32 or None
    cu_seqlens: Optional[np.ndarray] = None    # int32 [N+1] or None
    meta: dict = field(default_factory=dict)

    def to(self, device) -> "KDAInputs":
        mv = lambda t: None if t is None else t.to(device)
        return KDAInputs(mv(self.q), mv(self.k), mv(self.v), mv(self.g), mv(self.beta),
                         self.scale, mv(self.h0), self.cu_seqlens, dict(self.meta))


def _draw_block(gen, n, H, dk, dv, in_dtype, g_mu, g_sigma, device, unit_qk=True):
    q = torch.randn(n, H, dk, generator=gen, device=device, dtype=torch.float32)
    k = torch.randn(n, H, dk, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(n, H, dv, generator=gen, device=device, dtype=torch.float32)
    b = torch.randn(n, H, generator=gen, device=device, dtype=torch.float32)
    g = torch.randn(n, H, dk, generator=gen, device=device, dtype=torch.float32)
    if unit_qk:
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
    beta = torch.sigmoid(b)
    g = -F.softplus(g_sigma * g + g_mu)
    return q.to(in_dtype), k.to(in_dtype), v.to(in_dtype), beta, g


def draw_tokens(n_tokens, H, dk, dv, in_dtype, g_mu, g_sigma, seed, device="cpu",
                unit_qk=True):
    """Draw [n_tokens, H, *] tensors block by block (see the module rule)."""
    outs = [torch.empty(n_tokens, H, dk, dtype=in_dtype, device=device),
            torch.empty(n_tokens, H, dk, dtype=in_dtype, device=device),
            torch.empty(n_tokens, H, dv, dtype=in_dtype, device=device),
            torch.empty(n_tokens, H, dtype=torch.float32, device=device),
            torch.empty(n_tokens, H, dk, dtype=torch.float32, device=device)]
    for b0 in range(0, n_tokens, BLOCK_TOKENS):
        n = min(BLOCK_TOKENS, n_tokens - b0)
        gen = torch.Generator(device=device)
        gen.manual_seed(SEED_STRIDE * seed + b0 // BLOCK_TOKENS)
        blk = _draw_block(gen, n, H, dk, dv, in_dtype, g_mu, g_sigma, device, unit_qk)
        for dst, src in zip(outs, blk):
            dst[b0:b0 + n] = src
    return outs


def draw_state(N, H, dk, dv, std, seed, device="cpu"):
    if std == 0.0:
        return None
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED_STRIDE * seed - 1)
    return std * torch.randn(N, H, dk, dv, generator=gen, device=device, dtype=torch.float32)


def make_inputs(name: str, device="cpu", T: Optional[int] = None, H: Optional[int] = None,
                n_seqs: Optional[int] = None, lens=None, seed: Optional[int] = None,
                zero_h0: bool = False) -> KDAInputs:
    """Inputs of workload `name`, optionally shrunk (T, H, sequence count or an
    explicit list of varlen lengths) for parity runs the oracle finishes fast."""
    w = WORKLOADS[name]
    H = w.H if H is None else H
    seed = w.seed if seed is None else seed
    if w.decode:
        N = w.n_seqs if n_seqs is None else n_seqs
        S = w.steps if T is None else T  # tokens per sequence
        q, k, v, beta, g = draw_tokens(N * S, H, w.dk, w.dv, w.in_dtype, w.g_mu, w.g_sigma, seed,
                                       device)
        h0 = draw_state(N, H, w.dk, w.dv, w.h0_std, seed, device)
        q, k, v, g = (x.view(N, S, H, x.shape[-1]) for x in (q, k, v, g))
        return KDAInputs(q, k, v, g, beta.view(N, S, H), w.scale, h0, None,
                         {"workload": name, "N": N, "T": S, "H": H})
    cu = None
    if lens is not None:
        cu = cu_seqlens_from_lengths(lens)
    elif name in ("varlen", "varlen_f32"):
        if T is None and n_seqs is None:
            cu = cu_seqlens_from_lengths(varlen_lengths())
        else:
            ns = n_seqs or w.n_seqs
            tot = T or w.T
            lens_ = varlen_lengths(ns, tot, lo=max(1, tot // (ns * 8)), hi=max(2, tot // 4)) \
                if ns > 2 else np.array([tot - tot // 2, tot // 2][:ns])
            cu = cu_seqlens_from_lengths(lens_)
    if cu is not None:
        Ttot = int(cu[-1])
        N = len(cu) - 1
    else:
        Ttot = w.T if T is None else T
        N = 1
    q, k, v, beta, g = draw_tokens(Ttot, H, w.dk, w.dv, w.in_dtype, w.g_mu, w.g_sigma, seed, device)
    h0 = None if zero_h0 else draw_state(N, H, w.dk, w.dv, w.h0_std, seed, device)
    return KDAInputs(q[None], k[None], v[None], g[None], beta[None], w.scale, h0, cu,
                     {"workload": name, "T": Ttot, "H": H, "N": N})
