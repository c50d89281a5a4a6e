"""kda_chunk_fwd_noalloc, the allocation-free entry point, on the GPU: through
the C ABI it must give what kda_chunk_fwd gives with a workspace of its own,
on consecutive calls that share the library's device array (the second
smaller than the first, so stale contents of the first call are present),
and both must meet the oracle's bar."""
import os

import pytest
import torch

import synth
from oracle import cref
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


def _kda():
    import gated_delta_rule_89_amd as kda
    return kda


def say(msg):
    print(f"[case] {msg}", flush=True)


def _both(x, variant, ref_variant=None):
    kda = _kda()
    dev = torch.device("cuda")
    xd = x.to(dev)
    o_ref, f_ref = kda.chunk_fwd(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens,
                                 variant=ref_variant or variant)
    o = torch.full_like(o_ref, float("nan"))
    f = torch.full_like(f_ref, float("nan"))
    o2, f2 = kda.chunk_fwd_noalloc(xd.q, xd.k, xd.v, xd.g, xd.beta, x.scale, xd.h0, x.cu_seqlens,
                                   variant=variant, o=o, final_state=f)
    torch.cuda.synchronize()
    assert o2.data_ptr() == o.data_ptr() and f2.data_ptr() == f.data_ptr()
    return o, f, o_ref, f_ref


@pytest.mark.parametrize("variant", ["auto", "chunk", "chunk_scan", "chunk64", "recurrent", "chunk8"])
def test_noalloc_matches_chunk_fwd_on_two_calls(variant):
    cases = [("varlen", dict(lens=[3000, 77, 1500, 0, 640], H=4, seed=31)),
             ("varlen", dict(lens=[700, 33], H=2, seed=37))]
    for name, kw in cases:
        say(f"noalloc {variant} {name} {kw}")
        x = synth.make_inputs(name, **kw)
        o, f, o_ref, f_ref = _both(x, variant)
        assert torch.equal(o, o_ref) and torch.equal(f, f_ref)
        oo, ff = cref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens,
                                  n_threads=THREADS)
        assert_parity(o, oo, torch.bfloat16, "o")
        assert_parity(f, ff, torch.bfloat16, "final")


def test_noalloc_fp32_inputs_on_two_calls():
    """fp32 inputs (AUTO takes the fp32 chunk kernel, whose item list lives
    in the library's array): equal to kda_chunk_fwd and within the fp32 bound
    of the oracle on two consecutive calls, the second smaller."""
    for kw in (dict(lens=[2000, 9, 513, 0], H=3, seed=43), dict(lens=[300], H=2, seed=47)):
        say(f"noalloc fp32 auto {kw}")
        x = synth.make_inputs("varlen_f32", **kw)
        o, f, o_ref, f_ref = _both(x, "auto")
        assert torch.equal(o, o_ref) and torch.equal(f, f_ref)
        oo, ff = cref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens,
                                  n_threads=THREADS)
        assert_parity(o, oo, torch.float32, "o")
        assert_parity(f, ff, torch.float32, "final")


def test_noalloc_auto_falls_back_when_the_scan_does_not_fit():
    """A sequence long enough that AUTO picks the segment scan, whose maps
    (about 127 MB here) exceed the 32 MiB array: the plain chunked kernel
    runs instead, and an explicit segment-scan request is refused."""
    kda = _kda()
    T, H = 70000, 32
    say(f"noalloc AUTO fallback T={T} H={H}")
    assert kda.workspace_size(1, T, H, 128, 128, 1, torch.bfloat16, "auto") > kda._lib.NOALLOC_MAX_WORKSPACE
    x = synth.make_inputs("long", T=T, H=H, seed=41)
    o, f, o_ref, f_ref = _both(x, "auto", ref_variant="chunk")
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)
    with pytest.raises(kda.KDAError) as e:
        _both(x, "chunk_scan")
    assert e.value.code == 8  # KDA_ERR_WORKSPACE
