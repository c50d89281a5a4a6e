"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Inputs come from the seeded generator in `synth`; the oracle receives the
very same values (bf16 widened exactly).  Criteria: tests/parity.py.
"""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import cref, ref
from tests.parity import TOL_BF16_REL, assert_parity, max_abs, rel_rms
from tests.stream_oracle import stream_compare

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


def _kda():
    import gated_delta_rule_89_amd as kda
    return kda


def say(msg):
    print(f"[case] {msg}", flush=True)


def oracle_prefill(x, select=None):
    return cref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens,
                            n_threads=THREADS)


def run_prefill(x, variant="auto", **kw):
    dev = torch.device("cuda")
    xd = x.to(dev)
    o, f = _kda().chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens,
                            variant=variant, **kw)
    torch.cuda.synchronize()
    return o, f


VARIANTS = ["auto", "recurrent", "chunk", "chunk_scan", "chunk64", "chunk8"]
CHUNKED = ["chunk", "chunk64"]  # the two chunkwise kernels (32- and 64-token chunks)


@pytest.mark.parametrize("variant", ["auto", "recurrent", "chunk8"])
def test_tiny_fp32(variant):
    say(f"tiny fp32 T=64 d=16 variant={variant}")
    x = synth.make_inputs("tiny")
    o, f = run_prefill(x, variant)
    o_ref, f_ref = ref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0)
    assert_parity(o, o_ref, torch.float32, "o")
    assert_parity(f, f_ref, torch.float32, "final")


@pytest.mark.parametrize("variant", VARIANTS)
def test_prefill_workload_full(variant):
    say(f"prefill B=1 T=4096 H=8 d=128 bf16 variant={variant}")
    x = synth.make_inputs("prefill")
    o, f = run_prefill(x, variant)
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.bfloat16, "o")
    ef = assert_parity(f, f_ref, torch.bfloat16, "final")
    say(f"  o {eo:.2e} final {ef:.2e}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_varlen_ragged(variant):
    lens = [1000, 0, 77, 2500, 64, 1, 130]
    say(f"varlen lens={lens} H=4 bf16 variant={variant}")
    x = synth.make_inputs("varlen", lens=lens, H=4)
    o, f = run_prefill(x, variant)
    o_ref, f_ref = oracle_prefill(x)
    assert_parity(o, o_ref, torch.bfloat16, "o")
    assert_parity(f, f_ref, torch.bfloat16, "final")
    # the empty sequence keeps its initial state exactly
    assert torch.equal(f[1].cpu(), x.h0[1])


@pytest.mark.parametrize("variant", ["recurrent", "chunk8"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (128, 128),
                                   (64, 64), (32, 32), (128, 64), (64, 128)])
def test_head_sizes_fp32(dk, dv, variant):
    say(f"{variant} fp32 dk={dk} dv={dv} B=2 T=37 H=2")
    rng = np.random.default_rng(dk * 1000 + dv)
    B, T, H = 2, 37, 2
    q = torch.tensor(rng.standard_normal((B, T, H, dk)), dtype=torch.float32)
    k = torch.nn.functional.normalize(torch.tensor(rng.standard_normal((B, T, H, dk)),
                                                   dtype=torch.float32), dim=-1)
    v = torch.tensor(rng.standard_normal((B, T, H, dv)), dtype=torch.float32)
    g = -torch.nn.functional.softplus(torch.tensor(rng.standard_normal((B, T, H, dk)),
                                                   dtype=torch.float32))
    beta = torch.sigmoid(torch.tensor(rng.standard_normal((B, T, H)), dtype=torch.float32))
    h0 = torch.tensor(0.1 * rng.standard_normal((B, H, dk, dv)), dtype=torch.float32)
    dev = torch.device("cuda")
    o, f = _kda().chunk_fwd(q.to(dev), k.to(dev), v.to(dev), g.to(dev), beta.to(dev), 0.3,
                            h0.to(dev), variant=variant)
    o_ref, f_ref = ref.kda_forward(q, k, v, g, beta, 0.3, h0)
    assert_parity(o, o_ref, torch.float32, "o")
    assert_parity(f, f_ref, torch.float32, "final")


def test_decode_workload_full():
    say("decode N=256 H=32 d=128 bf16")
    x = synth.make_inputs("decode")
    dev = torch.device("cuda")
    xd = x.to(dev)
    st = xd.h0.clone()
    o = _kda().decode_step(xd.q[:, 0], xd.k[:, 0], xd.v[:, 0], xd.g[:, 0], xd.beta[:, 0],
                           x.scale, st)
    torch.cuda.synchronize()
    res = cref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, None, n_threads=THREADS)
    o_ref, s_ref = res
    e1 = max_abs(o[:, None], o_ref)
    e2 = max_abs(st, s_ref)
    say(f"  o max-abs {e1:.2e}  state max-abs {e2:.2e}")
    # fp32 arithmetic on exact inputs: the fp32 bound applies
    assert e1 <= 1e-4 and e2 <= 1e-4


@pytest.mark.parametrize("dk,dv,ind", [(16, 16, torch.float32), (64, 128, torch.bfloat16),
                                        (128, 32, torch.float32), (32, 16, torch.bfloat16)])
def test_decode_head_sizes(dk, dv, ind):
    say(f"decode dk={dk} dv={dv} {ind}")
    rng = np.random.default_rng(dk + dv)
    N, H = 5, 3
    q = torch.tensor(rng.standard_normal((N, H, dk)), dtype=torch.float32).to(ind)
    k = torch.nn.functional.normalize(torch.tensor(rng.standard_normal((N, H, dk))), dim=-1).to(ind)
    v = torch.tensor(rng.standard_normal((N, H, dv)), dtype=torch.float32).to(ind)
    g = -torch.rand(N, H, dk, generator=torch.Generator().manual_seed(1))
    beta = torch.rand(N, H, generator=torch.Generator().manual_seed(2))
    s0 = torch.randn(N, H, dk, dv, generator=torch.Generator().manual_seed(3))
    dev = torch.device("cuda")
    st = s0.to(dev)
    o = _kda().decode_step(q.to(dev), k.to(dev), v.to(dev), g.to(dev), beta.to(dev), 0.7, st)
    o_ref, s_ref = ref.kda_decode(q, k, v, g, beta, 0.7, s0)
    assert max_abs(o, o_ref) <= 1e-4 and max_abs(st, s_ref) <= 1e-4


def test_fused_recurrent_verify_workload_full():
    say("fused recurrent N=256 T=8 H=32 d=128 bf16 (verify workload)")
    x = synth.make_inputs("verify")
    dev = torch.device("cuda")
    xd = x.to(dev)
    st = xd.h0.clone()
    o = _kda().fused_recurrent_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, st)
    torch.cuda.synchronize()
    o_ref, s_ref = cref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, None,
                                    n_threads=THREADS)
    e1, e2 = max_abs(o, o_ref), max_abs(st, s_ref)
    say(f"  o max-abs {e1:.2e}  state max-abs {e2:.2e}")
    assert e1 <= 1e-4 and e2 <= 1e-4   # fp32 arithmetic on exact inputs


@pytest.mark.parametrize("dk,dv,ind,T", [(16, 16, torch.float32, 1), (64, 128, torch.bfloat16, 5),
                                          (128, 32, torch.float32, 64), (32, 64, torch.bfloat16, 17),
                                          (128, 128, torch.bfloat16, 3),
                                          # d = 128 runs in 8-token sub-chunks: several, and a ragged last one
                                          (128, 128, torch.float32, 64), (128, 128, torch.bfloat16, 17),
                                          (128, 128, torch.float32, 9)])
def test_fused_recurrent_shapes(dk, dv, ind, T):
    say(f"fused recurrent dk={dk} dv={dv} {ind} T={T}")
    rng = np.random.default_rng(dk + dv + T)
    N, H = 5, 3
    q = torch.tensor(rng.standard_normal((N, T, H, dk)), dtype=torch.float32).to(ind)
    k = torch.nn.functional.normalize(torch.tensor(rng.standard_normal((N, T, H, dk))),
                                      dim=-1).to(ind)
    v = torch.tensor(rng.standard_normal((N, T, H, dv)), dtype=torch.float32).to(ind)
    g = -torch.rand(N, T, H, dk, generator=torch.Generator().manual_seed(1))
    beta = torch.rand(N, T, H, generator=torch.Generator().manual_seed(2))
    s0 = torch.randn(N, H, dk, dv, generator=torch.Generator().manual_seed(3))
    dev = torch.device("cuda")
    st = s0.to(dev)
    o = _kda().fused_recurrent_fwd(q.to(dev), k.to(dev), v.to(dev), g.to(dev), beta.to(dev),
                                   0.7, st, out_dtype=ind)
    torch.cuda.synchronize()
    o_ref, s_ref = ref.kda_fused_recurrent(q, k, v, g, beta, 0.7, s0)
    assert max_abs(st, s_ref) <= 1e-4
    if ind == torch.float32:
        assert max_abs(o, o_ref) <= 1e-4
    else:  # bf16 output: fp32 arithmetic, then one rounding of each value (half an ulp, 2^-9)
        err = np.abs(o.float().cpu().numpy() - np.asarray(o_ref, dtype=np.float64))
        bound = 2.0 ** -8 * np.abs(np.asarray(o_ref, dtype=np.float64)) + 1e-4
        assert bool(np.all(err <= bound)), float(np.max(err / bound))


def test_fused_recurrent_equals_decode_steps():
    say("fused recurrent T=6 == six decode steps (N=64, H=4, d=128, bf16)")
    x = synth.make_inputs("verify", n_seqs=64, H=4, T=6)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    s1 = xd.h0.clone()
    o = kda.fused_recurrent_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, s1)
    s2 = xd.h0.clone()
    od = [kda.decode_step(xd.q[:, t].contiguous(), xd.k[:, t].contiguous(), xd.v[:, t].contiguous(),
                          xd.g[:, t].contiguous(), xd.beta[:, t].contiguous(), x.scale, s2)
          for t in range(6)]
    torch.cuda.synchronize()
    assert max_abs(o, torch.stack(od, 1)) <= 1e-5 and max_abs(s1, s2) <= 1e-5


def test_fused_recurrent_empty_and_rejects_long_runs():
    say("fused recurrent T=0 no-op; T=65 rejected")
    kda = _kda()
    dev = torch.device("cuda")
    st = torch.ones(2, 1, 16, 16, device=dev)
    z = torch.zeros(2, 0, 1, 16, device=dev)
    o = kda.fused_recurrent_fwd(z, z, z, z, torch.zeros(2, 0, 1, device=dev), 1.0, st)
    assert o.shape == (2, 0, 1, 16) and bool((st == 1).all())
    x = torch.zeros(2, 65, 1, 16, device=dev)
    with pytest.raises(kda.KDAError):
        kda.fused_recurrent_fwd(x, x, x, x, torch.zeros(2, 65, 1, device=dev), 1.0, st)


@pytest.mark.parametrize("variant,interval", [("chunk", 64), ("chunk", 192), ("chunk64", 128),
                                              ("recurrent", 64), ("chunk_scan", 256), ("chunk8", 64),
                                              ("chunk8", 192)])
def test_snapshots_varlen(variant, interval):
    say(f"snapshots variant={variant} interval={interval} (ragged varlen, H=2)")
    lens = [1, 63, 64, 65, 200, 384, 700, 1030] if variant != "chunk_scan" else [64, 2500, 4096, 130]
    x = synth.make_inputs("varlen", lens=lens, H=2)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    o, f, sn = kda.chunk_fwd_snapshots(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, interval,
                                       initial_state=xd.h0, cu_seqlens=x.cu_seqlens, variant=variant)
    o2, f2 = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens,
                           variant=variant)
    torch.cuda.synchronize()
    # the snapshot instantiation does the same arithmetic as the plain one
    assert torch.equal(o, o2) and torch.equal(f, f2)
    o_ref, f_ref, s_ref = ref.kda_forward_snapshots(x.q, x.k, x.v, x.g, x.beta, x.scale, interval,
                                                    x.h0, x.cu_seqlens)
    assert tuple(sn.shape) == s_ref.shape and s_ref.shape[0] == sum(L // interval for L in lens)
    rows = kda.snapshot_rows(lens, interval)
    for n, L in enumerate(lens):  # per sequence, so an error names its rows
        a, b = rows[n], rows[n + 1]
        if b > a:
            assert_parity(sn[a:b], s_ref[a:b], x.q.dtype, f"snapshots of sequence {n}")
    assert_parity(f, f_ref, x.q.dtype, "final")


def test_snapshot_resume_equals_full_run():
    say("resume from a snapshot == the uninterrupted run (prefix caching), T=1500 H=4")
    x = synth.make_inputs("prefill", T=1500, H=4)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    o, f, sn = kda.chunk_fwd_snapshots(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, 512,
                                       initial_state=xd.h0)
    assert sn.shape[0] == 2
    p = 1024  # resume after the second snapshot
    sl = lambda t: t[:, p:].contiguous()
    o_r, f_r = kda.chunk_fwd(sl(xd.q), sl(xd.k), sl(xd.v), sl(xd.g), sl(xd.beta), x.scale,
                             sn[1:2].contiguous())
    torch.cuda.synchronize()
    assert rel_rms(o_r, o[:, p:]) <= 2e-2 and rel_rms(f_r, f) <= 2e-2


def test_snapshots_varlen_workload_full_size_sampled():
    say("snapshots on the varlen workload (262144 tokens, H=32), interval 4096, sampled chains")
    x = synth.make_inputs("varlen")
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    lens = np.diff(x.cu_seqlens)
    o, f, sn = kda.chunk_fwd_snapshots(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, 4096,
                                       initial_state=xd.h0, cu_seqlens=x.cu_seqlens)
    o2, f2 = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(f, f2)
    rows = kda.snapshot_rows(lens, 4096)
    assert sn.shape[0] == rows[-1]
    longest = int(np.argmax(lens))
    # the snapshot after p tokens is the final state of the oracle run on the first p tokens
    for n, j in ((longest, 0), (longest, int(lens[longest] // 4096) - 1), (int(np.argmax(lens >= 8192)), 1)):
        p = (j + 1) * 4096
        a = int(x.cu_seqlens[n])
        sl = slice(a, a + p)
        heads = [0, 17, 31]
        _, fr = cref.kda_forward(x.q[:, sl, heads], x.k[:, sl, heads], x.v[:, sl, heads],
                                 x.g[:, sl, heads], x.beta[:, sl, heads], x.scale,
                                 x.h0[n:n + 1, heads], None, n_threads=THREADS)
        say(f"  sequence {n} snapshot {j} (after {p} tokens), heads {heads}")
        assert_parity(sn[rows[n] + j][heads], fr[0], x.q.dtype, f"snapshot {j} of sequence {n}")


def _gate_inputs(x, seed=7):
    gen = torch.Generator().manual_seed(seed)
    B, T, H, _ = x.q.shape
    dv = x.v.shape[-1]
    gate = torch.sigmoid(torch.randn(B, T, H, dv, generator=gen)).to(x.q.dtype)
    w = 1.0 + 0.5 * torch.randn(dv, generator=gen)
    return gate, w


@pytest.mark.parametrize("variant", ["chunk", "chunk_scan", "chunk64", "recurrent", "chunk8"])
def test_gated_rmsnorm_output(variant):
    say(f"gated RMSNorm output variant={variant} (ragged varlen, H=2)")
    lens = [1, 31, 33, 64, 200, 700] if variant != "chunk_scan" else [64, 2500, 130]
    x = synth.make_inputs("varlen", lens=lens, H=2)
    gate, w = _gate_inputs(x)
    dev = torch.device("cuda")
    xd = x.to(dev)
    y, f = _kda().chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens,
                            variant=variant, out_gate=gate.to(dev), norm_weight=w.to(dev),
                            norm_eps=1e-5)
    torch.cuda.synchronize()
    o_ref, f_ref = ref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens)
    y_ref = ref.rms_norm_gate(o_ref, gate, w, 1e-5)
    assert_parity(y, y_ref, x.q.dtype, "gated o")
    assert_parity(f, f_ref, x.q.dtype, "final")


@pytest.mark.parametrize("variant", ["recurrent", "chunk8"])
def test_gated_rmsnorm_fp32_and_bf16_out(variant):
    say(f"gated RMSNorm, fp32 inputs ({variant}, d=32/64), fp32 and bf16 outputs")
    rng = np.random.default_rng(3)
    B, T, H, dk, dv = 2, 40, 3, 32, 64
    q = torch.tensor(rng.standard_normal((B, T, H, dk)), dtype=torch.float32)
    k = torch.nn.functional.normalize(torch.tensor(rng.standard_normal((B, T, H, dk))), dim=-1).float()
    v = torch.tensor(rng.standard_normal((B, T, H, dv)), dtype=torch.float32)
    g = -torch.rand(B, T, H, dk, generator=torch.Generator().manual_seed(1))
    beta = torch.rand(B, T, H, generator=torch.Generator().manual_seed(2))
    gate = torch.rand(B, T, H, dv, generator=torch.Generator().manual_seed(4))
    w = torch.randn(dv, generator=torch.Generator().manual_seed(5))
    dev = torch.device("cuda")
    args = [t.to(dev) for t in (q, k, v, g, beta)]
    o_ref, _ = ref.kda_forward(q, k, v, g, beta, 0.3)
    y_ref = ref.rms_norm_gate(o_ref, gate, w, 1e-6)
    y, _ = _kda().chunk_fwd(*args, 0.3, out_gate=gate.to(dev), norm_weight=w.to(dev), norm_eps=1e-6,
                            variant=variant)
    yb, _ = _kda().chunk_fwd(*args, 0.3, out_gate=gate.to(dev), norm_weight=w.to(dev), norm_eps=1e-6,
                             out_dtype=torch.bfloat16, variant=variant)
    torch.cuda.synchronize()
    assert max_abs(y, y_ref) <= 1e-4
    # bf16 output: o is written in bf16 and rewritten in place, so each value
    # carries at most two bf16 roundings plus the rms's: within 2^-7 of itself.
    yr = np.asarray(y_ref)
    err = np.abs(yb.float().cpu().numpy() - yr)
    assert np.all(err <= 2.0 ** -7 * np.abs(yr) + 1e-6), float(np.max(err / (np.abs(yr) + 1e-6)))


def test_gated_varlen_workload_full_size():
    say("gated RMSNorm on the varlen workload (262144 tokens, H=32): fused == plain o then the formula")
    x = synth.make_inputs("varlen")
    dev = torch.device("cuda")
    xd = x.to(dev)
    gen = torch.Generator(device=dev).manual_seed(11)
    gate = torch.sigmoid(torch.randn(xd.v.shape, generator=gen, device=dev)).to(torch.bfloat16)
    w = 1.0 + 0.5 * torch.randn(128, generator=gen, device=dev)
    kda = _kda()
    y, f = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens,
                         out_gate=gate, norm_weight=w, norm_eps=1e-6)
    o, f2 = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens)
    torch.cuda.synchronize()
    assert torch.equal(f, f2)
    y2 = gate.float() * w * o * torch.rsqrt(o.pow(2).mean(-1, keepdim=True) + 1e-6)
    e = float(((y - y2).abs().max() / y2.pow(2).mean().sqrt()).item())
    say(f"  fused vs formula on the plain output: max|d|/rms {e:.2e}")
    assert e <= 1e-4


def _gate_proj(M, r, H, seed, dev=None):
    gen = torch.Generator().manual_seed(seed)
    z = (torch.randn(M, r, generator=gen) * 0.5).to(torch.bfloat16)
    w = (torch.randn(H * 128, r, generator=gen) / np.sqrt(r)).to(torch.bfloat16)
    b = torch.randn(H * 128, generator=gen) - 2.0
    u = torch.randn(M, H, generator=gen) * 2.0
    return z, w, b, u


@pytest.mark.parametrize("M,r,H,bias", [(1, 32, 1, True), (127, 64, 3, False), (300, 128, 2, True),
                                        (129, 256, 1, True)])
def test_fused_gate(M, r, H, bias):
    say(f"fused gate M={M} r={r} H={H} bias={bias}")
    z, w, b, u = _gate_proj(M, r, H, M + r)
    dev = torch.device("cuda")
    g, beta = _kda().fused_gate(z.to(dev), w.to(dev), u.to(dev), b.to(dev) if bias else None)
    torch.cuda.synchronize()
    g_ref, b_ref = ref.fused_gate(z, w, u, b if bias else None)
    gd = g.cpu().double().numpy()
    assert np.all(np.abs(gd - g_ref) <= 1e-5 * (1.0 + np.abs(g_ref)))
    assert max_abs(beta, b_ref) <= 1e-6


def test_fused_gate_full_size_sampled_rows():
    say("fused gate M=262144 r=128 H=32 (the varlen workload's tokens), sampled rows")
    M, r, H = 262144, 128, 32
    z, w, b, u = _gate_proj(M, r, H, 99)
    dev = torch.device("cuda")
    g, beta = _kda().fused_gate(z.to(dev), w.to(dev), u.to(dev), b.to(dev))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 4095, 131071, 200003, M - 1])
    g_ref, b_ref = ref.fused_gate(z[rows], w, u[rows], b)
    gd = g[torch.as_tensor(rows, device=dev)].cpu().double().numpy()
    assert np.all(np.abs(gd - g_ref) <= 1e-5 * (1.0 + np.abs(g_ref)))
    assert max_abs(beta[torch.as_tensor(rows, device=dev)], b_ref) <= 1e-6
    assert bool(torch.isfinite(g).all()) and bool((g < 0).all())


def test_many_sequences_beyond_ordering_limit():
    say("20000 short sequences (lengths 0..64), H=2: past the longest-first ordering limit")
    rng = np.random.default_rng(31)
    lens = rng.integers(0, 65, size=20000)
    x = synth.make_inputs("varlen", lens=lens, H=2)
    o, f = run_prefill(x)
    o_ref, f_ref = oracle_prefill(x)
    assert_parity(o, o_ref, x.q.dtype, "o")
    assert_parity(f, f_ref, x.q.dtype, "final")
    empty = np.flatnonzero(lens == 0)
    assert torch.equal(f[torch.as_tensor(empty)].cpu(), x.h0[torch.as_tensor(empty)])


def test_scan_and_snapshots_over_many_sequence_blocks():
    say("segment scan + snapshots with 300 sequences (several 256-sequence plan blocks), H=2")
    rng = np.random.default_rng(32)
    lens = rng.integers(1, 90, size=300)
    lens[[3, 150, 257, 299]] = [3000, 2100, 1500, 2600]
    x = synth.make_inputs("varlen", lens=lens, H=2)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    o, f, sn = kda.chunk_fwd_snapshots(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, 512,
                                       initial_state=xd.h0, cu_seqlens=x.cu_seqlens,
                                       variant="chunk_scan")
    torch.cuda.synchronize()
    o_ref, f_ref = oracle_prefill(x)
    assert_parity(o, o_ref, x.q.dtype, "o")
    assert_parity(f, f_ref, x.q.dtype, "final")
    rows = kda.snapshot_rows(lens, 512)
    for n in (3, 150, 257, 299):
        a = int(x.cu_seqlens[n])
        for j in range(int(rows[n + 1] - rows[n])):
            sl = slice(a, a + 512 * (j + 1))
            _, fr = cref.kda_forward(x.q[:, sl], x.k[:, sl], x.v[:, sl], x.g[:, sl], x.beta[:, sl],
                                     x.scale, x.h0[n:n + 1], None, n_threads=THREADS)
            assert_parity(sn[rows[n] + j], fr[0], x.q.dtype, f"snapshot {j} of sequence {n}")


def test_many_heads():
    say("H=96 (the largest head count the pages mention), T=300")
    x = synth.make_inputs("prefill", T=300, H=96)
    o, f = run_prefill(x)
    o_ref, f_ref = oracle_prefill(x)
    assert_parity(o, o_ref, x.q.dtype, "o")
    assert_parity(f, f_ref, x.q.dtype, "final")


@pytest.mark.parametrize("variant", ["chunk", "chunk_scan", "recurrent"])
def test_no_decay_no_write_keeps_state(variant):
    say(f"g = 0 and beta = 0: the state is untouched and o = scale S0^T q ({variant})")
    x = synth.make_inputs("prefill", T=1100, H=2)
    dev = torch.device("cuda")
    g0 = torch.zeros_like(x.g)
    b0 = torch.zeros_like(x.beta)
    o, f = _kda().chunk_fwd(x.q.to(dev), x.k.to(dev), x.v.to(dev), g0.to(dev), b0.to(dev), x.scale,
                            x.h0.to(dev), variant=variant)
    torch.cuda.synchronize()
    if variant == "chunk_scan":
        # the scan composes segment maps (identities here) in split bf16, ~16 significant bits
        assert max_abs(f, x.h0) <= 1e-5 * float(x.h0.abs().max())
    else:
        assert torch.equal(f.cpu(), x.h0)  # alpha = 1 and no write leave every value exact
    o_ref = x.scale * np.einsum("hkv,bthk->bthv", x.h0[0].double().numpy(), x.q.double().numpy())
    assert_parity(o, o_ref, x.q.dtype, "o")


def test_prefill_then_decode_equals_prefill():
    say("prefill T-1 then decode == prefill T (H=4, T=300)")
    x = synth.make_inputs("prefill", T=300, H=4)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    o_all, f_all = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0)
    _, f1 = kda.chunk_fwd(xd.q[:, :-1].contiguous(), xd.k[:, :-1].contiguous(),
                          xd.v[:, :-1].contiguous(), xd.g[:, :-1].contiguous(),
                          xd.beta[:, :-1].contiguous(), x.scale, xd.h0)
    od = kda.decode_step(xd.q[:, -1].contiguous(), xd.k[:, -1].contiguous(),
                         xd.v[:, -1].contiguous(), xd.g[:, -1].contiguous(),
                         xd.beta[:, -1].contiguous(), x.scale, f1)
    torch.cuda.synchronize()
    assert rel_rms(od, o_all[:, -1]) <= 2e-2
    assert rel_rms(f1, f_all) <= 2e-2


def test_split_call_state_passing():
    say("split call at 700 of T=1500 H=2")
    x = synth.make_inputs("prefill", T=1500, H=2)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    sl = lambda t, a, b: t[:, a:b].contiguous()
    o_all, f_all = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0)
    o1, f1 = kda.chunk_fwd(*(sl(t, 0, 700) for t in (xd.q, xd.k, xd.v, xd.g, xd.beta)),
                           x.scale, xd.h0)
    o2, f2 = kda.chunk_fwd(*(sl(t, 700, 1500) for t in (xd.q, xd.k, xd.v, xd.g, xd.beta)),
                           x.scale, f1)
    torch.cuda.synchronize()
    assert rel_rms(torch.cat([o1, o2], 1), o_all) <= 2e-2
    assert rel_rms(f2, f_all) <= 2e-2


def test_in_place_final_state_and_bf16_output():
    say("final_state is initial_state; bf16 o equals the fp32 o rounded")
    x = synth.make_inputs("prefill", T=130, H=2)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    o32, f32 = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0)
    st = xd.h0.clone()
    o16, f16 = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, st, final_state=st,
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert f16.data_ptr() == st.data_ptr()
    assert torch.equal(f16, f32)
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_empty_inputs():
    say("T=0 copies the initial state; N=0 is a no-op")
    dev = torch.device("cuda")
    kda = _kda()
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=dev)
    h0 = torch.randn(1, 2, 128, 128, device=dev)
    o, f = kda.chunk_fwd(z(1, 0, 2, 128), z(1, 0, 2, 128), z(1, 0, 2, 128),
                         z(1, 0, 2, 128, dt=torch.float32), z(1, 0, 2, dt=torch.float32),
                         0.1, h0)
    o2, f2 = kda.chunk_fwd(z(1, 0, 2, 128), z(1, 0, 2, 128), z(1, 0, 2, 128),
                           z(1, 0, 2, 128, dt=torch.float32), z(1, 0, 2, dt=torch.float32), 0.1)
    torch.cuda.synchronize()
    assert torch.equal(f, h0) and o.numel() == 0
    assert torch.count_nonzero(f2).item() == 0


def test_run_to_run_determinism():
    say("bitwise determinism, varlen H=4")
    x = synth.make_inputs("varlen", lens=[300, 17, 900], H=4)
    a = run_prefill(x)
    b = run_prefill(x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("variant", CHUNKED)
def test_chunk_rejects_fp32_and_small_heads(variant):
    say(f"{variant} variant: fp32 inputs / d=16 are unsupported")
    x = synth.make_inputs("tiny")
    with pytest.raises(_kda().KDAError) as e:
        run_prefill(x, variant)
    assert e.value.code == 4


@pytest.mark.parametrize("variant", CHUNKED)
@pytest.mark.parametrize("T", [1, 17, 31, 32, 33, 63, 64, 65, 100, 129])
def test_chunk_ragged_lengths(T, variant):
    say(f"{variant} T={T} H=3 (partial chunks)")
    x = synth.make_inputs("prefill", T=T, H=3, seed=7)
    o, f = run_prefill(x, variant)
    o_ref, f_ref = ref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0)
    assert_parity(o, o_ref, torch.bfloat16, "o")
    assert_parity(f, f_ref, torch.bfloat16, "final")


GATE_VARIANTS = ["chunk", "chunk64", "chunk_scan"]


def _gate_case_T(variant):
    # the segment scan needs sequences longer than its 512-token minimum segment
    return 3000 if variant == "chunk_scan" else 300


@pytest.mark.parametrize("variant", GATE_VARIANTS)
@pytest.mark.parametrize("mu,sigma", [(4.0, 1.0), (-4.0, 0.5), (8.0, 2.0)])
def test_chunk_gate_range(mu, sigma, variant):
    """Strong and weak decay, g = -softplus(sigma N(0,1) + mu), unclamped:
    mu = 8 puts 16-token gate sums near -130 and beyond on many channels."""
    T = _gate_case_T(variant)
    say(f"{variant} gate range g=-softplus({sigma} N + {mu}) T={T} H=2")
    x = synth.make_inputs("prefill", T=T, H=2, seed=11)
    gen = torch.Generator().manual_seed(5)
    x.g = -torch.nn.functional.softplus(sigma * torch.randn(x.g.shape, generator=gen) + mu)
    o, f = run_prefill(x, variant)
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.bfloat16, "o")
    ef = assert_parity(f, f_ref, torch.bfloat16, "final")
    say(f"  o {eo:.2e} final {ef:.2e}")


def strong_forget_gates(shape, seed):
    """Per-channel log-gates over the whole forget range of the recurrence
    ("Understanding Kimi Delta Attention", section "Understanding the
    Recurrence": every channel keeps anything from all to nothing of the
    previous state): channels 0-31 lose e^-20 per token, 32-63 e^-60, 64-95
    almost nothing (g = -1e-3), 96-127 the workload draw; token 777 forgets
    everything on every channel (g = -1e4: alpha is 0 in fp32 and fp64) and
    token 2000 with g = -1e30."""
    gen = torch.Generator().manual_seed(seed)
    g = -torch.nn.functional.softplus(2.0 * torch.randn(shape, generator=gen) - 2.0)
    g[..., 0:32] = -20.0
    g[..., 32:64] = -60.0
    g[..., 64:96] = -1e-3
    T = shape[1]
    if T > 777:
        g[:, 777] = -1e4
    if T > 2000:
        g[:, 2000] = -1e30
    return g


@pytest.mark.parametrize("variant", GATE_VARIANTS + ["auto", "recurrent", "chunk8"])
def test_chunk_strong_forget(variant):
    """Full forgetting on some channels and tokens, none on others, compared
    with the oracle; a random initial state shows whether it is wiped."""
    T = _gate_case_T(variant) if variant != "auto" else 3000
    T = max(T, 801)
    say(f"{variant} strong-forget gates (g=-20/-60/-1e-3/drawn, alpha=0 tokens) T={T} H=2")
    x = synth.make_inputs("prefill", T=T, H=2, seed=13)
    x.g = strong_forget_gates(x.g.shape, 17)
    o, f = run_prefill(x, variant)
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.bfloat16, "o")
    ef = assert_parity(f, f_ref, torch.bfloat16, "final")
    say(f"  o {eo:.2e} final {ef:.2e}")


def test_strong_forget_varlen_and_steps():
    """The same gates through packed sequences (several chains per call) and
    through the single-token and short-run entry points (fp32 agreement)."""
    lens = [900, 33, 2100, 64]
    say(f"strong-forget varlen lens={lens} H=3, decode and short runs")
    x = synth.make_inputs("varlen", lens=lens, H=3, seed=19)
    x.g = strong_forget_gates(x.g.shape, 23)
    o, f = run_prefill(x)
    o_ref, f_ref = oracle_prefill(x)
    assert_parity(o, o_ref, torch.bfloat16, "o")
    assert_parity(f, f_ref, torch.bfloat16, "final")
    d = synth.make_inputs("verify", n_seqs=4, H=3, T=8)
    d.g = strong_forget_gates(d.g.reshape(1, 32, 3, 128).shape, 29).reshape(d.g.shape)
    d.g[1, 3] = -1e4
    dev = torch.device("cuda")
    dd = d.to(dev)
    st = dd.h0.clone()
    od = _kda().fused_recurrent_fwd(dd.q, dd.k, dd.v, dd.g, dd.beta, d.scale, st)
    st1 = dd.h0.clone()
    o1 = _kda().decode_step(dd.q[:, 0].contiguous(), dd.k[:, 0].contiguous(), dd.v[:, 0].contiguous(),
                            dd.g[:, 0].contiguous(), dd.beta[:, 0].contiguous(), d.scale, st1)
    torch.cuda.synchronize()
    od_ref, s_ref = ref.kda_fused_recurrent(d.q, d.k, d.v, d.g, d.beta, d.scale, d.h0)
    o1_ref, s1_ref = ref.kda_decode(d.q[:, 0], d.k[:, 0], d.v[:, 0], d.g[:, 0], d.beta[:, 0],
                                    d.scale, d.h0)
    assert max_abs(od, od_ref) <= 1e-4 and max_abs(st, s_ref) <= 1e-4
    assert max_abs(o1, o1_ref) <= 1e-4 and max_abs(st1, s1_ref) <= 1e-4


def test_chunk_matches_recurrent_varlen():
    lens = [513, 31, 2000, 64, 7]
    say(f"chunk vs recurrent on the GPU, lens={lens} H=4")
    x = synth.make_inputs("varlen", lens=lens, H=4)
    oc, fc = run_prefill(x, "chunk")
    orc, frc = run_prefill(x, "recurrent")
    assert rel_rms(oc, orc) <= 2e-2 and rel_rms(fc, frc) <= 2e-2


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (16, 16), (32, 128), (128, 32), (64, 16)])
def test_chunk8_varlen_fp32(dk, dv):
    """fp32 inputs with full mantissas through packed sequences (empty, one
    token, ragged 8-token tails, several thousand tokens) on the fp32 chunk
    kernel: o and the final states within the fp32 bound, the empty
    sequence's state copied exactly."""
    lens = [300, 0, 77, 2500, 64, 1, 130, 9]
    say(f"chunk8 fp32 varlen lens={lens} H=3 dk={dk} dv={dv}")
    x = synth.make_inputs("varlen_f32", lens=lens, H=3)
    if (dk, dv) != (128, 128):
        w = synth.WORKLOADS["varlen_f32"]
        n = int(x.cu_seqlens[-1])
        q, k, v, beta, g = synth.draw_tokens(n, 3, dk, dv, torch.float32, w.g_mu, w.g_sigma, 41)
        x = synth.KDAInputs(q[None], k[None], v[None], g[None], beta[None], dk ** -0.5,
                            synth.draw_state(len(lens), 3, dk, dv, w.h0_std, 41), x.cu_seqlens)
    o, f = run_prefill(x, "chunk8")
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.float32, "o")
    ef = assert_parity(f, f_ref, torch.float32, "final")
    say(f"  o max-abs {eo:.2e} final max-abs {ef:.2e}")
    assert torch.equal(f[1].cpu(), x.h0[1])


@pytest.mark.parametrize("dk,dv", [(64, 64), (32, 128), (128, 16)])
def test_chunk8_bf16_inputs_other_head_sizes(dk, dv):
    """bf16 q/k/v at head sizes the fp16 kernel does not take: AUTO runs the
    fp32 chunk kernel.  Its arithmetic is fp32, so o (fp32) meets the fp32
    bound of the oracle on the same widened inputs, and a bf16 o is each
    value rounded once: within 2^-8 of the oracle's (plus 1e-6)."""
    lens = [700, 1, 64, 129]
    say(f"AUTO bf16 in dk={dk} dv={dv} lens={lens} H=2, fp32 and bf16 o")
    w = synth.WORKLOADS["varlen"]
    cu = synth.cu_seqlens_from_lengths(lens)
    q, k, v, beta, g = synth.draw_tokens(int(cu[-1]), 2, dk, dv, torch.bfloat16, w.g_mu, w.g_sigma, 53)
    x = synth.KDAInputs(q[None], k[None], v[None], g[None], beta[None], dk ** -0.5,
                        synth.draw_state(len(lens), 2, dk, dv, w.h0_std, 53), cu)
    o, f = run_prefill(x)
    ob, fb = run_prefill(x, out_dtype=torch.bfloat16)
    o_ref, f_ref = oracle_prefill(x)
    assert max_abs(o, o_ref) <= 1e-4 and max_abs(f, f_ref) <= 1e-4
    assert torch.equal(fb, f)
    err = np.abs(ob.float().cpu().numpy() - np.asarray(o_ref))
    assert bool(np.all(err <= 2.0 ** -8 * np.abs(np.asarray(o_ref)) + 1e-6)), float(np.max(err))


def test_chunk8_prefill_shape_fp32():
    """The single-sequence prefill shape (T = 4096, H = 8, d = 128, random
    initial state) with fp32 q/k/v through AUTO: eight chains of 512
    sub-chunks each on the fp32 chunk kernel, o and final states within the
    fp32 bound of the oracle."""
    say("AUTO fp32 prefill T=4096 H=8 d=128")
    w = synth.WORKLOADS["prefill"]
    q, k, v, beta, g = synth.draw_tokens(4096, 8, 128, 128, torch.float32, w.g_mu, w.g_sigma, 59)
    x = synth.KDAInputs(q[None], k[None], v[None], g[None], beta[None], w.scale,
                        synth.draw_state(1, 8, 128, 128, w.h0_std, 59), None)
    o, f = run_prefill(x)
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.float32, "o")
    ef = assert_parity(f, f_ref, torch.float32, "final")
    say(f"  o max-abs {eo:.2e} final max-abs {ef:.2e}")


def test_chunk8_strong_forget_fp32():
    """The strong-forget gates (alpha = 0 tokens, e^-20 and e^-60 channels,
    g = -1e30) on fp32 inputs: the entry-by-entry Gram path keeps the fp32
    bound."""
    lens = [900, 33, 2100, 64]
    say(f"chunk8 fp32 strong-forget varlen lens={lens} H=2")
    x = synth.make_inputs("varlen_f32", lens=lens, H=2, seed=43)
    x.g = strong_forget_gates(x.g.shape, 47)
    o, f = run_prefill(x, "chunk8")
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.float32, "o")
    ef = assert_parity(f, f_ref, torch.float32, "final")
    say(f"  o max-abs {eo:.2e} final max-abs {ef:.2e}")


def test_chunk8_in_place_and_short_runs():
    """The final state written over the initial one, and agreement with the
    short-run entry point (same sub-chunk arithmetic, state in place)."""
    say("chunk8 in place; equals fused_recurrent_fwd on 8-token runs")
    x = synth.make_inputs("verify", n_seqs=6, H=4, T=8)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    st = xd.h0.clone()
    o1 = kda.fused_recurrent_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, st)
    st2 = xd.h0.clone()
    o2, f2 = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, st2, final_state=st2,
                           variant="chunk8")
    torch.cuda.synchronize()
    assert f2.data_ptr() == st2.data_ptr()
    assert max_abs(o2, o1) <= 1e-5 and max_abs(st2, st) <= 1e-5
    o_ref, s_ref = ref.kda_fused_recurrent(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0)
    assert max_abs(o2, o_ref) <= 1e-4 and max_abs(st2, s_ref) <= 1e-4


def test_chunk8_fp32_workload_sized():
    """fp32 varlen over 16 sequences (65536 tokens, H=4, log-uniform lengths
    from 256 to 16384), compared whole with the oracle."""
    lens = synth.varlen_lengths(16, 65536, lo=256, hi=16384)
    say(f"chunk8 fp32 varlen 16 sequences, 65536 tokens, H=4")
    x = synth.make_inputs("varlen_f32", lens=lens, H=4)
    o, f = run_prefill(x)  # AUTO takes the fp32 chunk kernel
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.float32, "o")
    ef = assert_parity(f, f_ref, torch.float32, "final")
    say(f"  o max-abs {eo:.2e} final max-abs {ef:.2e}")


@pytest.mark.parametrize("T,H", [(20000, 2), (1500, 3)])
def test_scan_long_sequence(T, H):
    """A long sequence cut into segments: maps, scan and segment pass against
    the sequential oracle, with a random initial state."""
    say(f"chunk_scan one sequence T={T} H={H}")
    x = synth.make_inputs("long", T=T, H=H, seed=9)
    x.h0 = 0.02 * torch.randn(1, H, 128, 128, generator=torch.Generator().manual_seed(3))
    o, f = run_prefill(x, "chunk_scan")
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.bfloat16, "o")
    ef = assert_parity(f, f_ref, torch.bfloat16, "final")
    say(f"  o {eo:.2e} final {ef:.2e}")


@pytest.mark.timeout(600)
def test_scan_maps_and_corrections_stop_early():
    """Segments of 2048 tokens (T=65536, H=32) under the long workload's gates:
    the influence of a segment's initial state vanishes in fp16 well inside
    the segment, so the map and correction passes stop early; every token and
    head against the oracle."""
    T, H = 65536, 32
    say(f"chunk_scan early stop T={T} H={H}, every chain against the oracle")
    dev = torch.device("cuda")
    x = synth.make_inputs("long", T=T, H=H, seed=21, device=dev)
    x.h0 = 0.02 * torch.randn(1, H, 128, 128, generator=torch.Generator(device=dev).manual_seed(4),
                              device=dev)
    o, f = _kda().chunk_fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, variant="chunk_scan")
    torch.cuda.synchronize()
    eo, ef = stream_compare(x, o, f, n_threads=THREADS, log=lambda m: None)
    say(f"  o {eo:.2e} final {ef:.2e}")
    assert eo <= TOL_BF16_REL and ef <= TOL_BF16_REL


@pytest.mark.parametrize("T,H", [(3000, 2), (9000, 1)])
def test_scan_slow_decay(T, H):
    """Almost no forgetting (g = -1e-3) and small update gates: segment maps and
    initial-state corrections never vanish, so the scan composes full maps
    and the corrections run over whole segments."""
    say(f"chunk_scan slow decay T={T} H={H}")
    x = synth.make_inputs("prefill", T=T, H=H, seed=23)
    gen = torch.Generator().manual_seed(29)
    x.g = torch.full_like(x.g, -1e-3)
    x.beta = torch.sigmoid(torch.randn(x.beta.shape, generator=gen) - 4.0)
    o, f = run_prefill(x, "chunk_scan")
    o_ref, f_ref = oracle_prefill(x)
    eo = assert_parity(o, o_ref, torch.bfloat16, "o")
    ef = assert_parity(f, f_ref, torch.bfloat16, "final")
    say(f"  o {eo:.2e} final {ef:.2e}")


def test_scan_in_place_state_and_agreement():
    """Segment scan with final_state == initial_state, compared with the
    one-workgroup-per-sequence chunked path on the GPU."""
    lens = [6000, 40, 0, 3000]
    say(f"chunk_scan in place, lens={lens} H=2")
    x = synth.make_inputs("varlen", lens=lens, H=2)
    dev = torch.device("cuda")
    xd = x.to(dev)
    kda = _kda()
    oc, fc = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens,
                           variant="chunk")
    st = xd.h0.clone()
    os_, fs = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, st, x.cu_seqlens,
                            variant="chunk_scan", final_state=st)
    torch.cuda.synchronize()
    assert fs.data_ptr() == st.data_ptr()
    assert rel_rms(os_, oc) <= 2e-2 and rel_rms(fs, fc) <= 2e-2
    assert torch.equal(fs[2], xd.h0[2])  # empty sequence keeps its state


@pytest.mark.timeout(900)
def test_varlen_workload_full_size():
    """The full packed varlen workload (64 sequences, 262144 tokens, H=32) in the
    launch configuration the benchmark times (AUTO), against the C oracle on
    every (sequence, head) chain: o over all tokens and all 2048 final states."""
    say("varlen full size 262144 tokens H=32, every chain against the oracle")
    dev = torch.device("cuda")
    x = synth.make_inputs("varlen", device=dev)
    o, f = _kda().chunk_fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens)
    torch.cuda.synchronize()
    eo, ef = stream_compare(x, o, f, n_threads=THREADS, log=say)
    say(f"  varlen full size: max|do|/rms(o) {eo:.2e}  max|dS|/rms(S) {ef:.2e}")
    assert eo <= TOL_BF16_REL and ef <= TOL_BF16_REL


@pytest.mark.timeout(900)
def test_varlen_f32_workload_full_size():
    """The varlen shape with fp32 q/k/v (64 sequences, 262144 tokens, H=32)
    through AUTO, which takes the fp32 chunk kernel, against the C oracle on
    every chain at the fp32 bound: max-abs over all of o and all 2048 final
    states."""
    say("varlen fp32 full size 262144 tokens H=32 (fp32 chunk kernel), every chain against the oracle")
    dev = torch.device("cuda")
    x = synth.make_inputs("varlen_f32", device=dev)
    o, f = _kda().chunk_fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens)
    torch.cuda.synchronize()
    eo, ef = stream_compare(x, o, f, n_threads=THREADS, log=say, absolute=True)
    say(f"  varlen fp32 full size: max|do| {eo:.2e}  max|dS| {ef:.2e}")
    assert eo <= 1e-4 and ef <= 1e-4


@pytest.mark.timeout(900)
def test_long_workload_full_size():
    """The full long workload (one sequence of 1,048,576 tokens, H=32) through
    AUTO (the segment scan), against the C oracle on every token and head: the
    oracle runs in 32768-token windows and carries its fp64 state across them,
    so o over all 1M tokens and the final states of all 32 heads are checked."""
    say("long full size 1048576 tokens H=32, every token and head against the oracle")
    dev = torch.device("cuda")
    x = synth.make_inputs("long", device=dev)
    kda = _kda()
    o, f = kda.chunk_fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, None)
    torch.cuda.synchronize()
    eo, ef = stream_compare(x, o, f, n_threads=THREADS, log=say)
    say(f"  long full size: max|do|/rms(o) {eo:.2e}  max|dS|/rms(S) {ef:.2e}")
    assert eo <= TOL_BF16_REL and ef <= TOL_BF16_REL
    # State passing on the GPU: a call split at a chunk-unaligned point agrees
    # with the whole call.
    cut = 500001
    sl = lambda t, a, b: t[:, a:b].contiguous()
    o1, f1 = kda.chunk_fwd(*(sl(t, 0, cut) for t in (x.q, x.k, x.v, x.g, x.beta)), x.scale, None)
    del o1
    o2, f2 = kda.chunk_fwd(*(sl(t, cut, None) for t in (x.q, x.k, x.v, x.g, x.beta)), x.scale, f1)
    torch.cuda.synchronize()
    assert rel_rms(o2[:, -4096:], o[:, cut:][:, -4096:]) <= 2e-2
    assert rel_rms(f2, f) <= 2e-2
