"""The streamed full-size comparison (tests/stream_oracle.py) on the CPU.

It must reproduce the whole-batch oracle when the token axis is cut into
windows that split sequences (the fp64 state carried across windows), and it
must see a single wrong value of o or of a final state anywhere.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import ref
from tests.stream_oracle import Accum, stream_compare


def _whole(x):
    o, f = ref.kda_forward(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens)
    return torch.tensor(o, dtype=torch.float64), torch.tensor(f, dtype=torch.float64)


@pytest.mark.parametrize("window", [64, 100, 1000])
def test_windows_reproduce_whole_batch(window):
    x = synth.make_inputs("varlen", lens=[150, 0, 37, 260, 1], H=3, seed=3)
    o, f = _whole(x)
    eo, ef = stream_compare(x, o, f, window=window, log=lambda m: None)
    assert eo < 1e-12 and ef < 1e-12


def test_long_sequence_carried_across_windows():
    x = synth.make_inputs("long", T=700, H=2, seed=5)
    o, f = _whole(x)
    eo, ef = stream_compare(x, o, f, window=128, log=lambda m: None)
    assert eo < 1e-12 and ef < 1e-12


@pytest.mark.parametrize("where", ["o_early", "o_late", "final_split", "final_empty"])
def test_single_wrong_value_is_seen(where):
    x = synth.make_inputs("varlen", lens=[150, 0, 37, 260], H=3, seed=4)
    o, f = _whole(x)
    rms_o = float(o.pow(2).mean().sqrt())
    rms_f = float(f.pow(2).mean().sqrt())
    if where == "o_early":
        o[0, 3, 1, 5] += 0.05 * rms_o
    elif where == "o_late":
        o[0, 440, 2, 127] -= 0.05 * rms_o
    elif where == "final_split":  # sequence 3 spans several windows
        f[3, 2, 100, 7] += 0.05 * rms_f
    else:  # the empty sequence keeps its initial state
        f[1, 0, 0, 0] += 0.05 * rms_f
    eo, ef = stream_compare(x, o, f, window=64, log=lambda m: None)
    ao, af = stream_compare(x, o, f, window=64, log=lambda m: None, absolute=True)
    if where.startswith("o"):
        assert 0.04 < eo < 0.06 and ef < 1e-12
        assert abs(ao - 0.05 * rms_o) < 1e-12 * rms_o and af < 1e-12
    else:
        assert eo < 1e-12 and 0.04 < ef < 0.06
        assert ao < 1e-12 and abs(af - 0.05 * rms_f) < 1e-12 * rms_f


def test_accum_matches_whole_tensor_criterion():
    rng = np.random.default_rng(0)
    ref_ = rng.standard_normal((50, 8))
    x = ref_ + 1e-3 * rng.standard_normal((50, 8))
    acc = Accum()
    for i in range(0, 50, 7):
        acc.add(x[i:i + 7], ref_[i:i + 7])
    expect = np.max(np.abs(x - ref_)) / np.sqrt(np.mean(ref_ ** 2))
    assert abs(acc.rel() - expect) < 1e-15
