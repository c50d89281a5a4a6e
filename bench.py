"""Benchmark of the KDA operator on one MI355X.

One step = one pass of the hot path over one batch of synthetic input:
  * chunked prefill of the packed varlen workload (64 sequences, 262144
    tokens, H=32, d=128, bf16 q/k/v, fp32 g/beta/states, per-sequence
    initial and final states), and
  * one decode step of 256 sequences x 32 heads (state updated in place).

`value` is prefill tokens/s (tokens counted once across heads) over the
prefill launches of the timed steps; the decode step is reported beside it
as state/total HBM GB/s.  Inputs are generated on the device before the
timed region.  The roofline entry is for the prefill kernel: algorithmic
bytes per launch / average launch time from HIP events on the launch stream.
The CPU baseline is the C oracle on a bounded sample of the same workload.
After the steps, the long-context workload (one sequence of 1,048,576
tokens, H=32) is timed through the same entry point and reported under
"long"; entry points outside the hot path (short runs, gated output,
snapshots, the fused gate) are timed after the steps and reported under
"extras".

    python bench.py [--steps K] [--warmup W] [--workload varlen|long|prefill]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP32_PEAK_TFLOPS = 157.3


def prefill_alg_bytes(tokens, H, dk, dv, N, in_bytes=2, out_bytes=4, h0=True, final=True):
    """Bytes the prefill must move at least once: q, k, v, g, beta, o per token
    and head, plus the initial and final states per sequence and head."""
    per_th = (2 * dk + dv) * in_bytes + dk * 4 + 4 + dv * out_bytes
    st = N * H * dk * dv * 4 * (int(h0) + int(final))
    return tokens * H * per_th + st


def prefill_alg_flops(tokens, H, dk, dv, C=64):
    """Chunk-form FLOPs per token and head with triangles counted once:
    2[(C/2)(3 dk + 2 dv) + 3 dk dv]."""
    return tokens * H * 2 * ((C / 2) * (3 * dk + 2 * dv) + 3 * dk * dv)


def decode_alg_bytes(N, H, dk, dv, in_bytes=2, out_bytes=4):
    state = N * H * dk * dv * 4 * 2
    other = N * H * ((2 * dk + dv) * in_bytes + dk * 4 + 4 + dv * out_bytes)
    return state, state + other


def steps_alg_bytes(N, T, H, dk, dv, in_bytes=2, out_bytes=4):
    """A run of T tokens per sequence with the state in place: the state is
    read and written once, the per-token vectors once."""
    state = N * H * dk * dv * 4 * 2
    return state + N * T * H * ((2 * dk + dv) * in_bytes + dk * 4 + 4 + dv * out_bytes)


def time_launches(fn, stream, reps, warmup=2):
    """Average milliseconds of fn() between HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def code_sha256(path):
    """sha256 of a C/HIP source and the headers it includes from its own
    directory (recursively, each once), with comments and whitespace removed,
    so that only changes to the code itself count as a change of the kernel."""
    import hashlib
    import re
    h = hashlib.sha256()
    todo, seen = [os.path.abspath(path)], set()
    while todo:
        p = todo.pop(0)
        if p in seen or not os.path.exists(p):
            continue
        seen.add(p)
        src = open(p, encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update(re.sub(r"\s+", "", src).encode())
        todo += [os.path.join(os.path.dirname(p), f) for f in re.findall(r'#include\s+"([^"]+)"', src)]
    return h.hexdigest()


def measured_traffic(key, workload_label):
    """HBM bytes per launch from the committed rocprofv3 counter record
    (profiles/hbm_traffic.json), or None when the kernel code has changed
    since the counters were taken or the workload differs."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))["kernels"][key]
        digest = code_sha256(os.path.join(ROOT, rec["source"]))
    except (OSError, KeyError, ValueError):
        return None
    if digest != rec["code_sha256"] or rec["workload"] != workload_label:
        return None
    return rec["traffic_bytes"]


def cpu_baseline(x, budget_s=12.0):
    """The C oracle (fp64, OpenMP over chains) on a sample of the workload's
    (sequence, head) chains, each cut to a prefix so that the sample takes
    about `budget_s` of CPU time."""
    import numpy as np
    import torch
    from oracle import cref
    from oracle.ref import chain_list

    threads = cref.max_threads()
    B, T, H, dk = x.q.shape
    dv = x.v.shape[-1]
    chains = chain_list(B, T, x.cu_seqlens)

    def run(sel, lo, hi):
        """Oracle over tokens [lo, hi) of each selected chain (from the chain's
        initial state: a timing sample, not a continuation)."""
        parts = [[], [], [], [], []]
        h0s, starts, lens = [], [], []
        row = 0
        for n, h in sel:
            b, t0, t1 = chains[n]
            a0, a1 = min(t0 + lo, t1), min(t0 + hi, t1)
            if a1 <= a0:
                continue
            for i, src in enumerate((x.q, x.k, x.v, x.g, x.beta)):
                parts[i].append(src[b, a0:a1, h].to("cpu", torch.float32).numpy())
            if x.h0 is not None:
                h0s.append(x.h0[n, h].to("cpu", torch.float64).numpy())
            starts.append(row)
            lens.append(a1 - a0)
            row += a1 - a0
        if not row:
            return 0, 0.0
        arrs = [np.concatenate(p) for p in parts]
        t_0 = time.perf_counter()
        cref.run_packed(starts, lens, dk, dv, x.scale, *arrs,
                        np.stack(h0s) if h0s else None, True, threads)
        return row, time.perf_counter() - t_0

    # Batches of (sequence, head) chains in order, each over a 4096-token
    # window (about 1M head-tokens of host arrays per batch, one OpenMP run
    # each), until the runs add up to the budget; after the first window of
    # every chain, later windows of the same chains follow.
    order = [(n, h) for n in range(len(chains)) for h in range(H)]
    longest = max(t1 - t0 for _, t0, t1 in chains)
    win, per_batch = 4096, 16 * max(threads, 1)
    ht, dt, batches = 0, 0.0, 0
    for lo in range(0, max(longest, 1), win):
        for i in range(0, len(order), per_batch):
            if dt >= budget_s:
                break
            n_ht, n_dt = run(order[i:i + per_batch], lo, lo + win)
            ht += n_ht
            dt += n_dt
            batches += n_ht > 0
        if dt >= budget_s:
            break
    return {"value": ht / dt / H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{batches} batches of up to {per_batch} (sequence, head) chains over {win}-token "
                      f"windows ({ht} head-tokens, {dt:.1f} s); fp64 C recurrence, OpenMP over chains; "
                      f"tokens/s = head-tokens/s / H"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="varlen", choices=["varlen", "long", "prefill"])
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the entry points outside the timed step (short runs)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context workload timed after the varlen steps")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one 1 GiB device copy first (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(heads and sequences would shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_89_amd as kda
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    print(f"bench: generating {args.workload} inputs on the device", file=sys.stderr, flush=True)
    x = synth.make_inputs(args.workload, device=dev)
    B, T, H, dk = x.q.shape
    dv = x.v.shape[-1]
    N = len(x.cu_seqlens) - 1 if x.cu_seqlens is not None else B
    tokens = B * T
    cu_dev = torch.as_tensor(x.cu_seqlens, dtype=torch.int32).to(dev) if x.cu_seqlens is not None else None
    o = torch.empty(B, T, H, dv, device=dev, dtype=torch.float32)
    fin = torch.empty(N, H, dk, dv, device=dev, dtype=torch.float32)
    cu_host = None if x.cu_seqlens is None else torch.as_tensor(x.cu_seqlens, dtype=torch.int32)
    ws_bytes = kda.workspace_size(B, T, H, dk, dv, N, x.q.dtype, args.variant, cu_host)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def prefill():
        kda.chunk_fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, cu_dev, o=o, final_state=fin,
                      workspace=ws, variant=args.variant, cu_seqlens_host=cu_host)

    dec = None
    if not args.no_decode:
        d = synth.make_inputs("decode", device=dev)
        dq, dk_, dvv, dg, db = (t[:, 0].contiguous() for t in (d.q, d.k, d.v, d.g, d.beta))
        dstate = d.h0.clone()
        dout = torch.empty(dq.shape[0], dq.shape[1], dv, device=dev)
        dec = (dq, dk_, dvv, dg, db, dstate, dout, d.scale)

    def decode():
        dq, dk_, dvv, dg, db, dstate, dout, sc = dec
        kda.decode_step(dq, dk_, dvv, dg, db, sc, dstate, o=dout)

    if args.copy_probe:
        src = torch.ones(1 << 28, device=dev)  # 1 GiB of fp32
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        prefill()
        if dec:
            decode()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        if dec:
            decode()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [a.elapsed_time(b) for a, b, _ in ev]
    dec_ms = [b.elapsed_time(c) for _, b, c in ev]
    pre_avg = sum(pre_ms) / len(pre_ms)

    alg_b = prefill_alg_bytes(tokens, H, dk, dv, N, h0=x.h0 is not None)
    traffic = None
    if args.workload == "varlen" and args.variant == "auto":
        t = measured_traffic("chunk", "packed varlen prefill: 64 sequences, 262144 tokens, H=32, d=128")
        traffic = None if t is None else t / 1e9
    alg_f = prefill_alg_flops(tokens, H, dk, dv)
    achieved = alg_b / (pre_avg * 1e-3) / 1e9
    value = tokens / (pre_avg * 1e-3)
    line = {
        "metric": "KDA prefill tokens/s (H=32,d=128) + decode state HBM GB/s; % of roofline",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in; fp16 MFMA operands, fp32 accumulate, fp32 state and o",
        "data": "synthetic (seeded, generated on the device)",
        "config": {"workload": f"{args.workload}: {N} sequences, {tokens} tokens, H={H}, "
                               f"d_k=d_v={dk}, bf16 q/k/v, fp32 g/beta/state/o",
                   "global_batch": N, "seq_len": tokens, "parallelism": "none (1 GPU)"},
        "prefill_ms": pre_avg, "prefill_ms_min": min(pre_ms),
        "mfma_peak_equiv_frac": alg_f / (pre_avg * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "traffic_unit": "GB per launch",
                     "kernel": f"prefill ({args.variant})", "alg_bytes_per_launch": alg_b},
    }
    if dec:
        N3, H3 = dec[0].shape[0], dec[0].shape[1]
        sb, tb = decode_alg_bytes(N3, H3, 128, 128)
        dm = sum(dec_ms) / len(dec_ms)
        td = measured_traffic("decode", "decode step: 256 sequences x 32 heads, d=128, state in place")
        line["decode"] = {"us_per_step": dm * 1e3, "state_gbs": sb / (dm * 1e-3) / 1e9,
                          "traffic_gb": None if td is None else td / 1e9,
                          "total_gbs": tb / (dm * 1e-3) / 1e9,
                          "frac": tb / (dm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "config": f"{N3} sequences x {H3} heads, d=128"}
    if not args.no_extras:
        # A measured streaming rate beside the spec peak: an elementwise kernel
        # reading 1 GiB and writing 1 GiB (torch.neg; the runtime's own
        # device-to-device copy is slower), timed after the steps.
        csrc = torch.ones(1 << 28, device=dev)
        cdst = torch.empty_like(csrc)
        cm = time_launches(lambda: torch.neg(csrc, out=cdst), stream, 5)
        stream_gbs = 2 * csrc.numel() * 4 / (cm * 1e-3) / 1e9
        # and a write-only one (torch.fill_ over 1 GiB), the ceiling of a
        # kernel whose traffic is almost all writes
        wm = time_launches(lambda: cdst.fill_(0.5), stream, 5)
        write_gbs = cdst.numel() * 4 / (wm * 1e-3) / 1e9
        del csrc, cdst
        line["measured_stream_gbs"] = stream_gbs
        line["measured_write_gbs"] = write_gbs
        line["roofline"]["frac_of_measured_stream"] = achieved / stream_gbs
        # A measured dense bf16 matrix rate beside the spec MFMA peak: one
        # 8192^3 bf16 GEMM through torch (the vendor BLAS).
        ga = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        gb_ = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        gm_ms = time_launches(lambda: torch.mm(ga, gb_), stream, 5)
        gemm_tflops = 2.0 * 8192 ** 3 / (gm_ms * 1e-3) / 1e12
        del ga, gb_
        line["measured_bf16_gemm_tflops"] = gemm_tflops
        line["mfma_frac_of_measured_gemm"] = alg_f / (pre_avg * 1e-3) / (gemm_tflops * 1e12)
        if dec:
            line["decode"]["frac_of_measured_stream"] = line["decode"]["total_gbs"] / stream_gbs
        # Outside the timed step: a short run of 8 tokens per sequence with the
        # state in place (speculative verification), through kda_fused_recurrent_fwd.
        vx = synth.make_inputs("verify", device=dev)
        Nv, Tv, Hv, dkv = vx.q.shape
        vst = vx.h0.clone()
        vo = torch.empty(Nv, Tv, Hv, vx.v.shape[-1], device=dev)
        vm = time_launches(lambda: kda.fused_recurrent_fwd(vx.q, vx.k, vx.v, vx.g, vx.beta,
                                                           vx.scale, vst, o=vo), stream, 10)
        vb = steps_alg_bytes(Nv, Tv, Hv, dkv, vx.v.shape[-1])
        vt = measured_traffic("steps", "short runs: 256 sequences x 8 tokens x 32 heads, d=128, state in place")
        line["extras"] = {"fused_recurrent": {
            "us_per_launch": vm * 1e3, "gbs": vb / (vm * 1e-3) / 1e9,
            "frac": vb / (vm * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes": vb,
            "traffic_gb": None if vt is None else vt / 1e9,
            "frac_of_measured_stream": vb / (vm * 1e-3) / 1e9 / stream_gbs,
            "config": f"{Nv} sequences x {Tv} tokens x {Hv} heads, d={dkv}, state in place"}}
        # The gate inputs from their projections for every token of the workload
        # (kda_fused_gate, bf16 MFMA up-projection of rank 128).
        rk = 128
        gen0 = torch.Generator(device=dev).manual_seed(13)
        zq = (0.5 * torch.randn(tokens, rk, generator=gen0, device=dev)).to(torch.bfloat16)
        wq = (torch.randn(H * dk, rk, generator=gen0, device=dev) / rk ** 0.5).to(torch.bfloat16)
        bq = torch.randn(H * dk, generator=gen0, device=dev) - 2.0
        uq = torch.randn(tokens, H, generator=gen0, device=dev)
        fm = time_launches(lambda: kda.fused_gate(zq, wq, uq, bq), stream, 5)
        fb = tokens * rk * 2 + rk * H * dk * 2 + H * dk * 4 + tokens * H * 4 * 2 + tokens * H * dk * 4
        ff = 2.0 * tokens * rk * H * dk
        line["extras"]["fused_gate"] = {
            "ms_per_launch": fm, "gbs": fb / (fm * 1e-3) / 1e9,
            "frac": fb / (fm * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes": fb,
            "tflops": ff / (fm * 1e-3) / 1e12,
            "frac_of_measured_write": fb / (fm * 1e-3) / 1e9 / write_gbs,
            "traffic_gb": (lambda t: None if t is None else t / 1e9)(measured_traffic(
                "gate", f"fused gate: {tokens} tokens, rank {rk}, H={H}, d_k={dk}")),
            "config": f"{tokens} tokens, rank {rk} up to {H} x {dk} log-gates (fp32) + beta"}
        del zq, uq
        if args.workload == "varlen":
            # The same prefill with the state of every sequence kept each 4096 tokens
            # (kda_chunk_fwd_snapshots), against the plain prefill timed above.
            iv = 4096
            lens = [T] * N if x.cu_seqlens is None else list(int(a) for a in
                                                             (x.cu_seqlens[1:] - x.cu_seqlens[:-1]))
            nsn = int(kda.snapshot_rows(lens, iv)[-1])
            snb = torch.empty(nsn, H, dk, dv, device=dev)
            sws = torch.empty(max(1, kda.snapshots_workspace_size(B, T, H, dk, dv, N, iv, x.q.dtype,
                                                                  args.variant, cu_host)),
                              dtype=torch.uint8, device=dev)
            sm = time_launches(lambda: kda.chunk_fwd_snapshots(
                x.q, x.k, x.v, x.g, x.beta, x.scale, iv, initial_state=x.h0, cu_seqlens=cu_dev,
                cu_seqlens_host=cu_host, o=o, final_state=fin, snapshots=snb, workspace=sws,
                variant=args.variant),
                stream, 5)
            sb = alg_b + nsn * H * dk * dv * 4
            # The same prefill with the output gate and RMSNorm applied in the o store
            # (kda_chunk_fwd_gated): reads a bf16 gate per token and head besides.
            gen = torch.Generator(device=dev).manual_seed(12)
            ogt = torch.sigmoid(torch.randn(x.v.shape, generator=gen, device=dev)).to(x.q.dtype)
            nw = 1.0 + 0.1 * torch.randn(dv, generator=gen, device=dev)
            gm = time_launches(lambda: kda.chunk_fwd(
                x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, cu_dev, o=o, final_state=fin,
                workspace=ws, variant=args.variant, cu_seqlens_host=cu_host, out_gate=ogt,
                norm_weight=nw, norm_eps=1e-6), stream, 5)
            gb = alg_b + tokens * H * dv * x.q.element_size()
            line["extras"]["gated_rmsnorm"] = {
                "ms_per_launch": gm, "plain_ms": pre_avg, "overhead": gm / pre_avg - 1.0,
                "gbs": gb / (gm * 1e-3) / 1e9, "frac": gb / (gm * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "alg_bytes": gb, "config": f"{args.workload} prefill, o = gate * RMSNorm(o) in the store"}
            line["extras"]["snapshots"] = {
                "ms_per_launch": sm, "plain_ms": pre_avg, "overhead": sm / pre_avg - 1.0,
                "snapshots": nsn, "gbs": sb / (sm * 1e-3) / 1e9,
                "frac": sb / (sm * 1e-3) / 1e9 / HBM_PEAK_GBS, "alg_bytes": sb,
                "config": f"{args.workload} prefill with the state every {iv} tokens"}
    if args.workload == "varlen" and not args.no_extras:
        # fp32 inputs of the same shape (full mantissas) through AUTO, which
        # takes the fp32 chunk kernel (8-token sub-chunks on fp32 MFMA).  Its
        # figure of merit is the fp32 matrix rate: the chunk form's 6 d_k d_v
        # FLOPs per token and head ([K~; Q~] S and the state update) against
        # the fp32 MFMA peak.
        fx = synth.make_inputs("varlen_f32", device=dev)
        fo = torch.empty(B, T, H, dv, device=dev, dtype=torch.float32)
        fws = torch.empty(max(1, kda.workspace_size(B, T, H, dk, dv, N, fx.q.dtype, "auto", cu_host)),
                          dtype=torch.uint8, device=dev)
        fm32 = time_launches(lambda: kda.chunk_fwd(fx.q, fx.k, fx.v, fx.g, fx.beta, fx.scale, fx.h0, cu_dev,
                                                   o=fo, final_state=fin, workspace=fws,
                                                   cu_seqlens_host=cu_host), stream, 5)
        f32b = prefill_alg_bytes(tokens, H, dk, dv, N, in_bytes=4)
        f32f = 6.0 * tokens * H * dk * dv
        line["extras"]["chunk_fp32"] = {
            "ms_per_launch": fm32, "tokens_per_s": tokens / (fm32 * 1e-3),
            "tflops": f32f / (fm32 * 1e-3) / 1e12,
            "frac_of_fp32_mfma_peak": f32f / (fm32 * 1e-3) / (MFMA_FP32_PEAK_TFLOPS * 1e12),
            "gbs": f32b / (fm32 * 1e-3) / 1e9, "frac": f32b / (fm32 * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alg_bytes": f32b, "alg_flops": f32f,
            "traffic_gb": (lambda t: None if t is None else t / 1e9)(measured_traffic(
                "chunk8", f"fp32 chunk kernel: varlen shape with fp32 q/k/v, {N} sequences, {tokens} tokens, "
                          f"H={H}, d={dk}")),
            "config": f"varlen shape with fp32 q/k/v: {N} sequences, {tokens} tokens, H={H}, "
                      f"d_k=d_v={dk}, fp32 o and states (AUTO: fp32 chunk kernel)"}
        del fx, fo, fws
    if args.workload == "varlen" and not args.no_long:
        # The long-context workload (one sequence of 1,048,576 tokens, H=32)
        # through the same entry point (AUTO: the segment scan), timed like the
        # prefill above and reported beside it.
        print("bench: generating long inputs on the device", file=sys.stderr, flush=True)
        lx = synth.make_inputs("long", device=dev)
        _, LT, LH, ldk = lx.q.shape
        lo = torch.empty(1, LT, LH, lx.v.shape[-1], device=dev)
        lf = torch.empty(1, LH, ldk, lx.v.shape[-1], device=dev)
        lws = torch.empty(max(1, kda.workspace_size(1, LT, LH, ldk, ldk, 1, lx.q.dtype, "auto")),
                          dtype=torch.uint8, device=dev)
        lm = time_launches(lambda: kda.chunk_fwd(lx.q, lx.k, lx.v, lx.g, lx.beta, lx.scale, None,
                                                 o=lo, final_state=lf, workspace=lws),
                           stream, 5, warmup=1)
        lb = prefill_alg_bytes(LT, LH, ldk, ldk, 1, h0=False)
        lt = measured_traffic("long", "long prefill: 1 sequence, 1048576 tokens, H=32, d=128")
        lach = lb / (lm * 1e-3) / 1e9
        line["long"] = {
            "ms_per_launch": lm, "tokens_per_s": LT / (lm * 1e-3), "alg_bytes": lb,
            "mfma_peak_equiv_frac": prefill_alg_flops(LT, LH, ldk, ldk) / (lm * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
            "roofline": {"bound": "hbm", "achieved": lach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": lach / HBM_PEAK_GBS,
                         "traffic": None if lt is None else lt / 1e9, "traffic_unit": "GB per launch",
                         "kernel": "prefill (auto: segment maps, scan, segment pass)"},
            "config": f"long: 1 sequence, {LT} tokens, H={LH}, d_k=d_v={ldk}, bf16 q/k/v, "
                      f"fp32 g/beta/o, zero initial state"}
        del lx, lo, lf, lws
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
