"""CPU oracle for the Kimi Delta Attention operator -- TEST INFRASTRUCTURE ONLY.

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import, call, link or run anything in this directory.  The GPU product path
never reaches it, and this directory imports nothing from the product package
(the two share no code: no kernels, headers, helpers or constants).

What is computed (sources: "Understanding Kimi Delta Attention", section
"The KDA Recurrence: Scalar Gate vs Channel-wise Gate" and "Understanding the
Recurrence"; "kimi delta attn from first principles", sections "DeltaNet",
"KDA" and "three gates"):

For every chain (one sequence, one head) with state S of shape d_k x d_v
(rows indexed by key channels), for each token t in order:

  1. alpha = exp(g_t), one factor per key channel (the channel-wise gate);
  2. S <- Diag(alpha) S            (decay each row by its own gate, first);
  3. u = beta_t (v_t - S^T k_t)    (the delta-rule error on the decayed memory);
  4. S <- S + k_t u^T              (so S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T);
  5. o_t = scale * S^T q_t         (read the updated state with the query).

Readings taken where the pages are silent or disagree are listed with each
function.  Modules:

  ref.py    numpy reference in fp64 (and an fp32 twin) -- the primary oracle
  exact.py  the same recurrence over exact rationals (tiny cases)
  cref.py   loader for kda_ref.c, a plain C fp64 recurrence with OpenMP over
            independent chains, used for the large workloads

Parity status: every function here is pinned by the tests in
tests/test_oracle_pins.py (brute-force transition products, exact rationals,
reductions to linear attention / DeltaNet / scalar-gated DeltaNet, rank-1
overwrite, one-hot keys, beta = 0 closed form, state passing).
"""
from .ref import kda_forward, kda_decode, chain_list  # noqa: F401
