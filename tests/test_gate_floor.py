"""The gate floor's effect on the outputs, on the CPU with the fp64 oracle.

The kernels take a per-token log alpha below -15 ln 2 as -15 ln 2, so that the
gated operands of their log-space chunk form stay inside the fp32/bf16 exponent
range ("Lizard: An Efficient Linearization Framework for Large Language
Models", gist.science summary, section 2(c): the cumulative gate is absorbed
into q and k in log space).  The state update of section 2(a) is row-wise
(diag(alpha_t) scales key channel c's row of S by alpha_tc), so with
alpha' = max(alpha, 2^-15) the difference E_t = S'_t - S_t obeys, row by row,

    E_t[c] = (alpha'_tc - alpha_tc) S'_{t-1}[c] + alpha_tc E_{t-1}[c],

where 0 <= alpha'_tc - alpha_tc <= 2^-15, and it is non-zero only where the
floor acted (then alpha_tc < 2^-15 as well).  Hence max|E_t| <= 2^-15 M /
(1 - 2^-15) with M the largest |S'_s| entry before t, and
|o'_t - o_t| <= ||q_t||_1 max|E_t|.  The window branch does not read the gate,
so the hybrid output moves by exactly the gated branch's change.
"""
import math

import numpy as np
import pytest

import oracle

FLOOR = -15.0 * math.log(2.0)


def draw(T, d, kind, seed):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((2, 1, 1, T, d)) / math.sqrt(d)
    v = rng.standard_normal((1, 1, T, d))
    h0 = rng.standard_normal((1, 1, d, d))
    if kind == "extreme":        # every gate far below the floor
        la = -30.0 + rng.standard_normal((1, 1, T, d))
    elif kind == "half":         # half the channels extreme, half moderate
        la = -30.0 + rng.standard_normal((1, 1, T, d))
        la[..., d // 2:] = oracle.log_sigmoid(2.0 + rng.standard_normal((1, 1, T, d - d // 2)))
    else:                        # per token either side of the floor
        la = -rng.uniform(0.0, 25.0, (1, 1, T, d))
    return q, k, v, la, h0


@pytest.mark.parametrize("kind", ["extreme", "half", "straddle"])
def test_floor_moves_outputs_within_bound(kind):
    T, d, w, M = 40, 8, 6, 2
    q, k, v, la, h0 = draw(T, d, kind, seed={"extreme": 1, "half": 2, "straddle": 3}[kind])
    laf = np.maximum(la, FLOOR)
    assert (laf != la).any()
    o, _ = oracle.gla_forward(q, k, v, la, h0=h0)
    of, _ = oracle.gla_forward(q, k, v, laf, h0=h0)
    # largest state entry of the floored run before each token (prefix runs)
    Mx = np.empty(T)
    run = np.abs(h0).max()
    for t in range(T):
        Mx[t] = run
        _, St = oracle.gla_forward(q[:, :, :t + 1], k[:, :, :t + 1], v[:, :, :t + 1], laf[:, :, :t + 1], h0=h0)
        run = max(run, np.abs(St).max())
    u = 2.0 ** -15
    bound = np.abs(q[0, 0]).sum(-1) * u * Mx / (1.0 - u)  # per token
    err = np.abs(of - o)[0, 0].max(-1)
    assert (err <= bound * (1 + 1e-9) + 1e-300).all(), (err / bound).max()
    assert err.max() > 0.0
    # measured against the output's scale the change is within the fp32 parity
    # bar (1e-4 normwise) and far inside the bf16 one (2e-2)
    assert err.max() <= 1e-4 * np.abs(o).max()
    # only the gated branch reads the gate: the hybrid output moves by the same amount
    rng = np.random.default_rng(7)
    mk, mv = rng.standard_normal((2, 1, M, d))
    s = 1.0 / math.sqrt(d)
    hy = oracle.hybrid_forward(q, k, v, la, mk, mv, w, s, mix=0.7, h0=h0)
    hyf = oracle.hybrid_forward(q, k, v, laf, mk, mv, w, s, mix=0.7, h0=h0)
    np.testing.assert_allclose(hyf["o"] - hy["o"], of - o, rtol=0, atol=1e-12 * np.abs(hy["o"]).max())
    np.testing.assert_array_equal(hyf["o_swa"], hy["o_swa"])

