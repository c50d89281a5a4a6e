"""The oracle pinned to what the pages and the mathematics fix (CPU only).

* every pin of tests/oracle_pins.py on the numpy oracle and on the C oracle;
* planted mistakes: source-level mutants of oracle/ref.py must each fail a pin;
* an exact-rational golden chain (tests/golden/exact_tiny.json, written by
  tests/golden/make_golden.py from oracle/exact.py) agrees with the
  brute-force transition products in exact arithmetic and with both fp64
  oracles to rounding;
* the C and numpy oracles agree on random batches, varlen included.
"""
import json
import math
import os
import types
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle.ref as ref
from oracle import cref
from oracle.exact import kda_chain_exact
from tests.oracle_pins import ALL_PINS

HERE = os.path.dirname(os.path.abspath(__file__))
REF_SRC = os.path.join(HERE, "..", "oracle", "ref.py")


def numpy_oracle(q, k, v, g, beta, scale, h0, cu):
    return ref.kda_forward(q, k, v, g, beta, scale, h0, cu)


def c_oracle(q, k, v, g, beta, scale, h0, cu):
    return cref.kda_forward(q, k, v, g, beta, scale, h0, cu, n_threads=2)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin_numpy(pin):
    pin(numpy_oracle)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin_c(pin):
    pin(c_oracle)


# Planted mistakes: (what, original text in oracle/ref.py, replacement).
MUTANTS = [
    ("erase before decay",
     "S = alpha[:, :, None] * S                    # decay rows  step 2",
     "S_und = S"),
    ("column gate", "S = alpha[:, :, None] * S", "S = alpha[:, None, :] * S"),
    ("read-out before the write",
     'o[b, t] = scale * np.einsum("hkv,hk->hv", S, q[b, t])',
     'o[b, t] = scale * np.einsum("hkv,hk->hv", S - k[b, t][:, :, None] * u[:, None, :], q[b, t])'),
    ("read-out with the key", 'np.einsum("hkv,hk->hv", S, q[b, t])', 'np.einsum("hkv,hk->hv", S, k[b, t])'),
    ("wrong sign of the prediction", "(v[b, t] - pred)", "(v[b, t] + pred)"),
    ("dropped beta", "u = beta[b, t][:, None] * (v[b, t] - pred)", "u = (v[b, t] - pred)"),
    ("gate not exponentiated", "alpha = np.exp(g[b, t])", "alpha = 1.0 + g[b, t]"),
    ("gate of the previous token", "alpha = np.exp(g[b, t])", "alpha = np.exp(g[b, max(t - 1, t0)])"),
    ("dropped scale", 'o[b, t] = scale * np.einsum', 'o[b, t] = np.einsum'),
    ("prediction with the query", 'pred = np.einsum("hkv,hk->hv", S, k[b, t])',
     'pred = np.einsum("hkv,hk->hv", S, q[b, t])'),
    ("write along the query", "S = S + k[b, t][:, :, None] * u[:, None, :]",
     "S = S + q[b, t][:, :, None] * u[:, None, :]"),
    ("initial state ignored", "else h0[n].copy()", "else 0.0 * h0[n]"),
    ("state not reset per sequence", "else h0[n].copy()", "else h0[0].copy()"),
]


def _mutant(orig, repl, extra=None):
    src = open(REF_SRC).read()
    assert orig in src, f"mutation anchor not found: {orig!r}"
    src = src.replace(orig, repl, 1)
    if extra:
        src = src.replace(*extra)
    mod = types.ModuleType("ref_mutant")
    exec(compile(src, "ref_mutant.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("what,orig,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(what, orig, repl):
    extra = None
    if what == "erase before decay":
        # erase with the undecayed state, then decay, then write
        extra = ("S = S + k[b, t][:, :, None] * u[:, None, :]  # step 4",
                 "S = alpha[:, :, None] * (S - beta[b, t][:, None, None] * k[b, t][:, :, None] * "
                 "pred[:, None, :]) + beta[b, t][:, None, None] * k[b, t][:, :, None] * v[b, t][:, None, :]")
    mod = _mutant(orig, repl, extra)

    def fn(q, k, v, g, beta, scale, h0, cu):
        return mod.kda_forward(q, k, v, g, beta, scale, h0, cu)

    caught = []
    for pin in ALL_PINS:
        try:
            pin(fn)
        except Exception as e:  # AssertionError or a shape error: the pin rejects it
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches the planted mistake: {what}"


def _load_golden():
    with open(os.path.join(HERE, "golden", "exact_tiny.json")) as f:
        d = json.load(f)
    F = lambda m: [[Fr(x) for x in row] for row in m]
    return d, F


def test_golden_exact_matches_transition_products():
    """The golden chain equals the matrix form S_t = M_t S_{t-1} + beta k v^T with
    M_t = (I - beta k k^T) Diag(alpha), evaluated in exact rationals."""
    d, F = _load_golden()
    q, k, v, al, S0 = F(d["q"]), F(d["k"]), F(d["v"]), F(d["alpha"]), F(d["S0"])
    beta = [Fr(b) for b in d["beta"]]
    scale = Fr(d["scale"])
    T, dk, dv = d["T"], d["dk"], d["dv"]
    S = S0
    for t in range(T):
        M = [[(Fr(int(r == c)) - beta[t] * k[t][r] * k[t][c]) * al[t][c] for c in range(dk)]
             for r in range(dk)]
        S = [[sum(M[r][c] * S[c][j] for c in range(dk)) + beta[t] * k[t][r] * v[t][j]
              for j in range(dv)] for r in range(dk)]
        o_t = [scale * sum(S[c][j] * q[t][c] for c in range(dk)) for j in range(dv)]
        assert o_t == F(d["o"])[t]
    assert S == F(d["S_final"])
    # and the oracle's own exact path reproduces the file
    o2, S2 = kda_chain_exact(q, k, v, al, beta, scale, S0)
    assert o2 == F(d["o"]) and S2 == F(d["S_final"])


@pytest.mark.parametrize("impl", ["numpy", "c"])
def test_golden_exact_vs_fp64(impl):
    d, F = _load_golden()
    fl = lambda m: np.array([[float(x) for x in row] for row in F(m)])
    T, dk, dv = d["T"], d["dk"], d["dv"]
    q = fl(d["q"]).reshape(1, T, 1, dk)
    k = fl(d["k"]).reshape(1, T, 1, dk)
    v = fl(d["v"]).reshape(1, T, 1, dv)
    g = np.log(fl(d["alpha"])).reshape(1, T, 1, dk)
    beta = np.array([float(Fr(b)) for b in d["beta"]]).reshape(1, T, 1)
    S0 = fl(d["S0"]).reshape(1, 1, dk, dv)
    fn = numpy_oracle if impl == "numpy" else c_oracle
    if impl == "c":  # the C oracle takes float32 inputs: these rationals are not all exact there
        q, k, v, g, beta, S0 = (x.astype(np.float32) for x in (q, k, v, g, beta, S0))
    o, f = fn(q, k, v, g, beta, float(Fr(d["scale"])), S0, None)
    tol = 1e-14 if impl == "numpy" else 2e-6
    assert np.max(np.abs(o[0, :, 0] - fl(d["o"]))) <= tol
    assert np.max(np.abs(f[0, 0] - fl(d["S_final"]))) <= tol


def test_c_matches_numpy_random_varlen():
    rng = np.random.default_rng(3)
    T, H, dk, dv = 97, 3, 16, 8
    q = rng.standard_normal((1, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((1, T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, H, dv)).astype(np.float32)
    g = (-rng.random((1, T, H, dk)) * 3).astype(np.float32)
    beta = rng.random((1, T, H)).astype(np.float32)
    cu = np.array([0, 40, 40, 90, 97], dtype=np.int32)
    h0 = rng.standard_normal((4, H, dk, dv)).astype(np.float32)
    o1, f1 = ref.kda_forward(q, k, v, g, beta, 0.25, h0, cu)
    o2, f2 = cref.kda_forward(q, k, v, g, beta, 0.25, h0, cu, n_threads=3)
    assert np.max(np.abs(o1 - o2)) <= 1e-13 * max(1, np.abs(o1).max())
    assert np.max(np.abs(f1 - f2)) <= 1e-13 * max(1, np.abs(f1).max())


def test_fp32_twin_drift_small():
    """The fp32 twin of the oracle stays within 1e-5 of fp64 on the tiny workload shape."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 64, 1, 16))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((1, 64, 1, 16))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, 64, 1, 16))
    g = -np.log1p(np.exp(rng.standard_normal((1, 64, 1, 16))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, 64, 1))))
    o64, f64 = ref.kda_forward(q, k, v, g, beta, 0.25)
    o32, f32 = ref.kda_forward(q, k, v, g, beta, 0.25, dtype=np.float32)
    assert np.max(np.abs(o64 - o32)) < 1e-5 and np.max(np.abs(f64 - f32)) < 1e-5


def test_decode_is_one_step_of_forward():
    """Prefill of T-1 tokens then one decode step equals prefill of T tokens."""
    rng = np.random.default_rng(8)
    T, H, dk, dv = 9, 2, 6, 4
    q, k, v = (rng.standard_normal((1, T, H, d)) for d in (dk, dk, dv))
    g = -rng.random((1, T, H, dk))
    beta = rng.random((1, T, H))
    h0 = rng.standard_normal((1, H, dk, dv))
    o, f = ref.kda_forward(q, k, v, g, beta, 0.5, h0)
    _, f1 = ref.kda_forward(q[:, :-1], k[:, :-1], v[:, :-1], g[:, :-1], beta[:, :-1], 0.5, h0)
    od, fd = ref.kda_decode(q[:, -1], k[:, -1], v[:, -1], g[:, -1], beta[:, -1], 0.5, f1)
    assert np.max(np.abs(od[0] - o[0, -1])) < 1e-13
    assert np.max(np.abs(fd - f)) < 1e-13


def test_fused_recurrent_is_successive_decode_steps():
    """A run of T tokens from a state equals T single-token steps in order,
    with each row of the batch its own chain (rows must not mix)."""
    rng = np.random.default_rng(9)
    N, T, H, dk, dv = 3, 5, 2, 6, 4
    q, k, v = (rng.standard_normal((N, T, H, d)) for d in (dk, dk, dv))
    g = -rng.random((N, T, H, dk))
    beta = rng.random((N, T, H))
    s0 = rng.standard_normal((N, H, dk, dv))
    o, f = ref.kda_fused_recurrent(q, k, v, g, beta, 0.5, s0)
    s = s0.copy()
    for t in range(T):
        od, s = ref.kda_decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], 0.5, s)
        assert np.max(np.abs(od - o[:, t])) < 1e-13
    assert np.max(np.abs(s - f)) < 1e-13
    # each row from its own state: row 1 alone gives the same result
    o1, f1 = ref.kda_fused_recurrent(q[1:2], k[1:2], v[1:2], g[1:2], beta[1:2], 0.5, s0[1:2])
    assert np.max(np.abs(o1[0] - o[1])) < 1e-13 and np.max(np.abs(f1[0] - f[1])) < 1e-13


def test_snapshots_are_prefix_final_states():
    """Snapshot j of a chain is the final state of the recurrence run on the
    chain's first (j + 1) * interval tokens; rows run chain by chain; o and the
    final states are those of kda_forward."""
    rng = np.random.default_rng(10)
    lens = [13, 8, 0, 20, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv, iv = int(cu[-1]), 2, 5, 3, 4
    q, k, v = (rng.standard_normal((1, T, H, d)) for d in (dk, dk, dv))
    g = -rng.random((1, T, H, dk))
    beta = rng.random((1, T, H))
    h0 = rng.standard_normal((len(lens), H, dk, dv))
    o, f, sn = ref.kda_forward_snapshots(q, k, v, g, beta, 0.5, iv, h0, cu)
    o2, f2 = ref.kda_forward(q, k, v, g, beta, 0.5, h0, cu)
    assert np.array_equal(o, o2) and np.array_equal(f, f2)
    assert sn.shape[0] == sum(L // iv for L in lens)
    row = 0
    for n, L in enumerate(lens):
        a = cu[n]
        for j in range(L // iv):
            p = (j + 1) * iv
            sl = slice(a, a + p)
            _, fp = ref.kda_forward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], 0.5,
                                    h0[n:n + 1])
            assert np.max(np.abs(sn[row] - fp[0])) < 1e-13, (n, j)
            row += 1
    # a chain whose length is a multiple of the interval ends on a snapshot
    assert np.max(np.abs(sn[sum(L // iv for L in lens[:2]) - 1] - f[1])) < 1e-13


def test_rms_norm_gate_pins():
    """RMSNorm then the output gate, against values fixed by the definition."""
    # hand-computed: o = (3, 4): mean square 12.5, so y = o / sqrt(12.5)
    y = ref.rms_norm_gate(np.array([3.0, 4.0]), np.ones(2), np.ones(2), 0.0)
    assert np.max(np.abs(y - np.array([3.0, 4.0]) / np.sqrt(12.5))) < 1e-15
    rng = np.random.default_rng(21)
    o = rng.standard_normal((3, 5, 16))
    one = np.ones(16)
    # unit RMS with unit gate and weight, no eps
    y = ref.rms_norm_gate(o, np.ones_like(o), one, 0.0)
    assert np.max(np.abs(np.sqrt(np.mean(y * y, axis=-1)) - 1.0)) < 1e-13
    # scale invariance per vector (positive factors), sign follows o
    lam = rng.uniform(0.1, 10.0, size=(3, 5, 1))
    assert np.max(np.abs(ref.rms_norm_gate(lam * o, np.ones_like(o), one, 0.0) - y)) < 1e-12
    # a constant vector maps to ones
    assert np.max(np.abs(ref.rms_norm_gate(np.full(16, 7.5), np.ones(16), one, 0.0) - 1.0)) < 1e-15
    # gate and weight multiply elementwise; eps only shrinks; zero stays zero
    gt, w = rng.uniform(0, 1, o.shape), rng.standard_normal(16)
    assert np.max(np.abs(ref.rms_norm_gate(o, gt, w, 0.0) - gt * w * y)) < 1e-12
    ye = ref.rms_norm_gate(o, np.ones_like(o), one, 0.5)
    assert np.all(np.abs(ye) <= np.abs(y) + 1e-15)
    # eps inside the root: a vector of ones with eps = 3 maps to 1 / sqrt(1 + 3) = 1/2
    assert np.all(ref.rms_norm_gate(np.ones(16), np.ones(16), one, 3.0) == 0.5)
    assert np.all(ref.rms_norm_gate(np.zeros(16), np.ones(16), one, 1e-6) == 0.0)


def test_fused_gate_pins():
    """g = -softplus(z w + b) and beta = sigmoid(u), against closed forms, an
    explicit triple loop for the contraction, and a one-hot layout check."""
    # closed forms: softplus(0) = ln 2; softplus(a) -> a for large a, -> e^a for very negative a
    z0 = np.zeros((1, 4))
    w0 = np.zeros((2 * 3, 4))
    g, b = ref.fused_gate(z0, w0, np.zeros((1, 2)))
    assert g.shape == (1, 2, 3) and np.all(np.abs(g + np.log(2.0)) < 1e-15) and np.all(b == 0.5)
    g, _ = ref.fused_gate(z0, w0, np.zeros((1, 2)), b_up=np.full(6, 40.0))
    assert np.all(np.abs(g + 40.0) < 1e-15)
    g, _ = ref.fused_gate(z0, w0, np.zeros((1, 2)), b_up=np.full(6, -40.0))
    assert np.all(np.abs(g + np.exp(-40.0)) < 1e-30) and np.all(g < 0)
    _, b = ref.fused_gate(z0, w0, np.array([[40.0, -40.0]]))
    assert abs(b[0, 0] - 1.0) < 1e-15 and abs(b[0, 1] - np.exp(-40.0)) < 1e-30
    # the contraction against explicit loops, with the head/channel layout
    rng = np.random.default_rng(22)
    M, r, H, dk = 3, 5, 2, 4
    z, w = rng.standard_normal((M, r)), rng.standard_normal((H * dk, r))
    bias, u = rng.standard_normal(H * dk), rng.standard_normal((M, H))
    g, b = ref.fused_gate(z, w, u, b_up=bias)
    for m in range(M):
        for h in range(H):
            for c in range(dk):
                a = bias[h * dk + c] + sum(z[m, j] * w[h * dk + c, j] for j in range(r))
                sp = a + np.log1p(np.exp(-a)) if a > 0 else np.log1p(np.exp(a))
                assert abs(g[m, h, c] + sp) < 1e-12
            assert abs(b[m, h] - 1.0 / (1.0 + np.exp(-u[m, h]))) < 1e-15
    # one hot: a single nonzero weight moves only its (head, channel)
    w1 = np.zeros((H * dk, r))
    w1[1 * dk + 3, 2] = 5.0
    z1 = np.zeros((M, r))
    z1[1, 2] = 1.0
    g, _ = ref.fused_gate(z1, w1, u)
    moved = np.argwhere(np.abs(g + np.log(2.0)) > 1e-12)
    assert moved.tolist() == [[1, 1, 3]] and abs(g[1, 1, 3] + np.logaddexp(0.0, 5.0)) < 1e-15
