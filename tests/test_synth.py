"""The seeded input generator (CPU only): determinism, shapes and the varlen recipe."""
import numpy as np
import torch

import synth


def test_varlen_lengths_recipe():
    lens = synth.varlen_lengths()
    assert len(lens) == 64 and int(lens.sum()) == 262144
    assert lens.min() == 512 and lens.max() == 32768
    chunks = int(np.sum((lens + 63) // 64))
    partial = int(np.sum(lens % 64 != 0))
    assert 3000 < chunks < 5000 and partial > 30
    assert np.array_equal(lens, synth.varlen_lengths())  # deterministic


def test_cu_seqlens():
    cu = synth.cu_seqlens_from_lengths([3, 0, 5])
    assert cu.dtype == np.int32 and list(cu) == [0, 3, 3, 8]


def test_determinism_and_block_seeding():
    a = synth.draw_tokens(70000, 1, 4, 4, torch.bfloat16, -2.0, 2.0, seed=7)
    b = synth.draw_tokens(70000, 1, 4, 4, torch.bfloat16, -2.0, 2.0, seed=7)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # the second block restarts from its own seed: drawing only 65536 tokens
    # reproduces the first block bit for bit
    c = synth.draw_tokens(65536, 1, 4, 4, torch.bfloat16, -2.0, 2.0, seed=7)
    for x, y in zip(a, c):
        assert torch.equal(x[:65536], y)


def test_workload_shapes_and_ranges():
    x = synth.make_inputs("prefill", T=256, H=2)
    assert x.q.shape == (1, 256, 2, 128) and x.q.dtype == torch.bfloat16
    assert x.g.dtype == torch.float32 and x.beta.shape == (1, 256, 2)
    assert x.h0.shape == (1, 2, 128, 128)
    assert abs(x.h0.std().item() - 0.02) < 2e-3
    assert (x.g <= 0).all() and (x.beta > 0).all() and (x.beta < 1).all()
    n = x.k.float().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    t = synth.make_inputs("tiny")
    assert t.q.dtype == torch.float32 and t.q.shape == (1, 64, 1, 16) and t.h0 is None
    assert abs(t.scale - 0.25) < 1e-12
    d = synth.make_inputs("decode", n_seqs=4, H=2)
    assert d.q.shape == (4, 1, 2, 128) and d.h0.shape == (4, 2, 128, 128)
    v = synth.make_inputs("varlen", lens=[100, 0, 37])
    assert list(v.cu_seqlens) == [0, 100, 100, 137] and v.h0.shape == (3, 32, 128, 128)
