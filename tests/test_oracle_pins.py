"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

The pages print no worked numbers, so each pin is a closed form, a library
routine, an invariant or brute force on tiny inputs.  Together they are chosen
so that a plausible slip anywhere in the oracle (a dropped term, a wrong sign or
index, a transposed operand, an off-by-one window) breaks at least one of them;
tests/test_oracle_mutants.py plants such slips and checks that they are caught.

Cited passages: "Lizard: An Efficient Linearization Framework for Large Language
Models" (gist.science technical summary), section 2(a) hybrid attention (state
update, anchor window with meta-memory sinks, weighted sum) and section 4
efficiency (constant-memory inference).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs, to_f64_numpy

RNG = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def logsig(x):
    return -np.logaddexp(0.0, -x)


# ---------------------------------------------------------------- GLA branch
def pairwise_gla(q, k, v, la, h0=None):
    """Unrolled closed form of the state recurrence: with B_t the running sum
    of log_alpha over tokens 0..t, o_t = sum_{s<=t} sum_c q_tc k_sc e^{B_tc-B_sc} v_s
    + (q_t * e^{B_t}) h0.  The difference is taken before exp, so it is exact for
    any gates."""
    Bc = np.cumsum(la, axis=2)
    T = q.shape[2]
    o = np.zeros(q.shape[:3] + (v.shape[-1],))
    for t in range(T):
        w = np.exp(Bc[:, :, t:t + 1, :] - Bc[:, :, :t + 1, :])        # [B,H,t+1,dk]
        scores = np.einsum("bhc,bhsc->bhs", q[:, :, t], k[:, :, :t + 1] * w)
        o[:, :, t] = np.einsum("bhs,bhsj->bhj", scores, v[:, :, :t + 1])
        if h0 is not None:
            o[:, :, t] += np.einsum("bhc,bhcj->bhj", q[:, :, t] * np.exp(Bc[:, :, t]), h0)
    return o


def test_I1_alpha_one_is_masked_linear_attention():
    q, k, v = rand(2, 3, 17, 5), rand(2, 3, 17, 5), rand(2, 3, 17, 4)
    o, hT = oracle.gla_forward(q, k, v, np.zeros_like(q))
    mask = np.tril(np.ones((17, 17)))                     # diagonal included
    ref = (np.matmul(q, np.swapaxes(k, -1, -2)) * mask) @ v
    assert rel(o, ref) < 1e-13
    assert rel(hT, np.swapaxes(k, -1, -2) @ v) < 1e-13


def test_I2_scalar_decay_is_retention_parallel_form():
    gamma = 0.83
    q, k, v = rand(1, 2, 23, 6), rand(1, 2, 23, 6), rand(1, 2, 23, 3)
    o, _ = oracle.gla_forward(q, k, v, np.full(q.shape, np.log(gamma)))
    t = np.arange(23)
    D = np.where(t[:, None] >= t[None, :], gamma ** (t[:, None] - t[None, :]), 0.0)
    ref = (np.matmul(q, np.swapaxes(k, -1, -2)) * D) @ v    # gamma^(t-s), not ^(t-s+1)
    assert rel(o, ref) < 1e-13


def test_I3_recurrence_equals_pairwise_form_with_h0():
    q, k, v = rand(2, 2, 40, 6), rand(2, 2, 40, 6), rand(2, 2, 40, 5)
    la = logsig(rand(2, 2, 40, 6) + 2.0)
    h0 = rand(2, 2, 6, 5)
    o, hT = oracle.gla_forward(q, k, v, la, h0)
    assert rel(o, pairwise_gla(q, k, v, la, h0)) < 1e-12
    Bc = np.cumsum(la, axis=2)
    hT_ref = np.einsum("bhsc,bhsj->bhcj", k * np.exp(Bc[:, :, -1:] - Bc), v) \
        + np.exp(Bc[:, :, -1])[..., None] * h0
    assert rel(hT, hT_ref) < 1e-12


def test_I13_extreme_gates_match_pairwise_exactly():
    # cumulative log-decay of about -200 per 64 tokens: exp(-B) alone would overflow
    q, k, v = rand(1, 2, 96, 8), rand(1, 2, 96, 8), rand(1, 2, 96, 8)
    la = logsig(rand(1, 2, 96, 8) - 3.0)
    o, _ = oracle.gla_forward(q, k, v, la)
    assert np.all(np.isfinite(o))
    assert rel(o, pairwise_gla(q, k, v, la)) < 1e-12


def test_closed_form_halving_scalar_state():
    # d=1, q=k=v=1, alpha=1/2: S_t = S_{t-1}/2 + 1 so o_t = 2 - 2^-t
    T = 30
    one = np.ones((1, 1, T, 1))
    o, hT = oracle.gla_forward(one, one, one, np.full((1, 1, T, 1), np.log(0.5)))
    assert np.allclose(o[0, 0, :, 0], 2.0 - 2.0 ** -np.arange(T), rtol=0, atol=1e-15)


def test_I11_zero_query_and_zero_mix():
    q, k, v = rand(1, 2, 9, 4), rand(1, 2, 9, 4), rand(1, 2, 9, 4)
    la = logsig(rand(1, 2, 9, 4) + 2)
    o, _ = oracle.gla_forward(np.zeros_like(q), k, v, la)
    assert np.all(o == 0)
    mk, mv = rand(2, 3, 4), rand(2, 3, 4)
    r = oracle.hybrid_forward(q, k, v, la, mk, mv, 4, 0.5, mix=0.0)
    assert np.array_equal(r["o"], r["o_gla"])


def test_I12_norm_bound():
    q, k, v = rand(1, 2, 50, 7), rand(1, 2, 50, 7), rand(1, 2, 50, 5)
    la = logsig(rand(1, 2, 50, 7) + 1.0)
    o, _ = oracle.gla_forward(q, k, v, la)
    kv = np.cumsum(np.linalg.norm(k, axis=-1) * np.linalg.norm(v, axis=-1), axis=2)
    assert np.all(np.linalg.norm(o, axis=-1) <= np.linalg.norm(q, axis=-1) * kv * (1 + 1e-12))


# ------------------------------------------------------------- window branch
def test_I4_full_window_no_meta_is_causal_softmax_attention():
    T, s = 33, 0.37
    q, k, v = rand(2, 2, T, 8), rand(2, 2, T, 8), rand(2, 2, T, 6)
    o, lse = oracle.window_meta_attention(q, k, v, np.zeros((2, 0, 8)), np.zeros((2, 0, 6)),
                                          window=T + 5, scale=s)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=True, scale=s).numpy()
    assert rel(o, ref) < 1e-13
    L = s * q @ np.swapaxes(k, -1, -2)
    L = np.where(np.tril(np.ones((T, T), bool)), L, -np.inf)
    assert np.max(np.abs(lse - np.log(np.exp(L).sum(-1)))) < 1e-12


def test_I5_window_one_no_meta_returns_v():
    q, k, v = rand(1, 3, 12, 5), rand(1, 3, 12, 5), rand(1, 3, 12, 7)
    o, lse = oracle.window_meta_attention(q, k, v, np.zeros((3, 0, 5)), np.zeros((3, 0, 7)),
                                          window=1, scale=0.9)
    assert rel(o, v) < 1e-15
    assert np.max(np.abs(lse - 0.9 * (q * k).sum(-1))) < 1e-13


def test_I6_banded_matrix_form_including_window_edges():
    T, w, M, s = 21, 5, 3, 0.6
    q, k, v = rand(1, 2, T, 4), rand(1, 2, T, 4), rand(1, 2, T, 3)
    mk, mv = rand(2, M, 4), rand(2, M, 3)
    o, _ = oracle.window_meta_attention(q, k, v, mk, mv, w, s)
    t = np.arange(T)
    band = (t[None, :] <= t[:, None]) & (t[None, :] >= t[:, None] - w + 1)  # w keys incl. self
    assert band.sum(1).max() == w and band[0].sum() == 1
    keys = np.concatenate([k, np.broadcast_to(mk[None], (1, 2, M, 4))], 2)
    vals = np.concatenate([v, np.broadcast_to(mv[None], (1, 2, M, 3))], 2)
    L = s * q @ np.swapaxes(keys, -1, -2)
    L[..., :T] = np.where(band, L[..., :T], -np.inf)
    P = np.exp(L - L.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    assert rel(o, P @ vals) < 1e-13


def test_closed_form_uniform_weights():
    # q = 0 makes every logit 0: the output is the plain mean of the visible values
    T, w, M = 9, 4, 2
    q = np.zeros((1, 1, T, 3))
    k, v = rand(1, 1, T, 3), rand(1, 1, T, 2)
    mk, mv = rand(1, M, 3), rand(1, M, 2)
    o, lse = oracle.window_meta_attention(q, k, v, mk, mv, w, 1.0)
    for t in range(T):
        lo = max(0, t - w + 1)
        n = t + 1 - lo + M
        ref = (v[0, 0, lo:t + 1].sum(0) + mv[0].sum(0)) / n
        assert np.allclose(o[0, 0, t], ref, atol=1e-15)
        assert abs(lse[0, 0, t] - np.log(n)) < 1e-14


def test_I7_meta_slots_are_sinks_when_meta_v_is_zero():
    T, w, M, s = 19, 6, 4, 0.8
    q, k, v = rand(2, 2, T, 5), rand(2, 2, T, 5), rand(2, 2, T, 4)
    mk = rand(2, M, 5)
    o, lse = oracle.window_meta_attention(q, k, v, mk, np.zeros((2, M, 4)), w, s)
    o0, lse0 = oracle.window_meta_attention(q, k, v, np.zeros((2, 0, 5)), np.zeros((2, 0, 4)), w, s)
    # meta only enlarges the denominator: o = o_(M=0) * Z_window / (Z_window + Z_meta)
    assert rel(o, o0 * np.exp(lse0 - lse)[..., None]) < 1e-12
    meta_logits = s * np.einsum("bhtc,hmc->bhtm", q, mk)
    # relative: the partition functions reach ~1e2 with these logits
    Z, Z0, Zm = np.exp(lse), np.exp(lse0), np.exp(meta_logits).sum(-1)
    assert np.max(np.abs(Z - Z0 - Zm) / Z) < 1e-13


def test_I10_linear_in_values():
    T, w, M, s = 15, 4, 2, 0.5
    q, k = rand(1, 2, T, 4), rand(1, 2, T, 4)
    la = logsig(rand(1, 2, T, 4) + 2)
    mk = rand(2, M, 4)
    v1, v2, m1, m2 = rand(1, 2, T, 3), rand(1, 2, T, 3), rand(2, M, 3), rand(2, M, 3)
    f = lambda v, mv: oracle.hybrid_forward(q, k, v, la, mk, mv, w, s, mix=0.7)["o"]
    assert rel(f(2 * v1 - 3 * v2, 2 * m1 - 3 * m2), 2 * f(v1, m1) - 3 * f(v2, m2)) < 1e-12
    assert np.all(f(np.zeros_like(v1), np.zeros_like(m1)) == 0)


# ------------------------------------------------------------ decode + handoff
def test_I8_decode_reproduces_prefill_and_handoff():
    B, H, T0, n, d, w, M, s = 2, 2, 11, 9, 4, 5, 2, 0.6
    q, k, v = rand(B, H, T0 + n, d), rand(B, H, T0 + n, d), rand(B, H, T0 + n, d)
    la = logsig(rand(B, H, T0 + n, d) + 2)
    mk, mv = rand(H, M, d), rand(H, M, d)
    full = oracle.hybrid_forward(q, k, v, la, mk, mv, w, s, mix=0.9)
    pre = oracle.hybrid_forward(q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], la[:, :, :T0],
                                mk, mv, w, s, mix=0.9)
    o_ref, hT_ref = oracle.gla_forward(q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], la[:, :, :T0])
    assert np.array_equal(pre["hT"], hT_ref)
    S, rk, rv, pos = pre["hT"], pre["ring_k"], pre["ring_v"], np.full(B, T0)
    for i in range(n):
        t = T0 + i
        o, S, rk, rv, pos = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], la[:, :, t],
                                               S, rk, rv, pos, mk, mv, w, s, mix=0.9)
        assert rel(o, full["o"][:, :, t]) < 1e-12
    assert np.all(pos == T0 + n)
    assert rel(S, full["hT"]) < 1e-12
    assert np.array_equal(rk, full["ring_k"]) and np.array_equal(rv, full["ring_v"])


def test_decode_from_empty_state_and_short_history():
    # starting at pos 0 with a zero state and empty ring equals a prefill from scratch
    B, H, n, d, w, M, s = 1, 2, 7, 3, 4, 1, 1.0
    q, k, v = rand(B, H, n, d), rand(B, H, n, d), rand(B, H, n, d)
    la = logsig(rand(B, H, n, d))
    mk, mv = rand(H, M, d), rand(H, M, d)
    full = oracle.hybrid_forward(q, k, v, la, mk, mv, w, s)
    S, rk, rv = np.zeros((B, H, d, d)), np.zeros((B, H, w, d)), np.zeros((B, H, w, d))
    pos = np.zeros(B, dtype=np.int64)
    for t in range(n):
        o, S, rk, rv, pos = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], la[:, :, t],
                                               S, rk, rv, pos, mk, mv, w, s)
        assert rel(o, full["o"][:, :, t]) < 1e-12


def test_decode_independent_of_ring_slot_order():
    # softmax is a set function: rotating the filled ring (with pos) changes nothing
    B, H, d, w, M = 1, 1, 4, 6, 2
    S = rand(B, H, d, d)
    rk, rv = rand(B, H, w, d), rand(B, H, w, d)
    mk, mv = rand(H, M, d), rand(H, M, d)
    x = [rand(B, H, d) for _ in range(3)] + [logsig(rand(B, H, d))]
    o1, *_ = oracle.decode_step(*x, S, rk, rv, np.array([20]), mk, mv, w, 0.5)
    rk2, rv2 = np.roll(rk, 1, axis=2), np.roll(rv, 1, axis=2)
    o2, *_ = oracle.decode_step(*x, S, rk2, rv2, np.array([21]), mk, mv, w, 0.5)
    # slot 20%6=2 is overwritten in the first call; in the rolled ring the same
    # token sits in slot 3 = 21%6, so both calls see the same key/value set
    assert rel(o1, o2) < 1e-13


# -------------------------------------------------------------------- backward
def _loss(dO, **kw):
    return float((oracle.hybrid_forward(**kw)["o"] * dO).sum())


@pytest.mark.parametrize("mix", [1.0, 0.6])
def test_I9_gradients_match_central_differences(mix):
    B, H, T, d, w, M, s = 1, 1, 13, 5, 3, 2, 0.7
    args = dict(q=rand(B, H, T, d), k=rand(B, H, T, d), v=rand(B, H, T, d),
                log_alpha=logsig(rand(B, H, T, d) + 1.0), meta_k=rand(H, M, d),
                meta_v=rand(H, M, d), h0=rand(B, H, d, d))
    dO = rand(B, H, T, d)
    g = oracle.hybrid_backward(args["q"], args["k"], args["v"], args["log_alpha"], args["meta_k"],
                               args["meta_v"], w, s, dO, mix=mix, h0=args["h0"])
    names = dict(q="dq", k="dk", v="dv", log_alpha="dlog_alpha", meta_k="dmeta_k",
                 meta_v="dmeta_v", h0="dh0")
    h = 1e-6
    for arg, gname in names.items():
        x = args[arg]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(dO, window=w, scale=s, mix=mix, **args)
            x[idx] = keep - h
            lm = _loss(dO, window=w, scale=s, mix=mix, **args)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        assert rel(g[gname], fd) < 1e-6, arg
    # the mix weight
    h = 1e-6
    fd_mix = (_loss(dO, window=w, scale=s, mix=mix + h, **args)
              - _loss(dO, window=w, scale=s, mix=mix - h, **args)) / (2 * h)
    assert abs(g["dmix"] - fd_mix) < 1e-7 * max(1.0, abs(fd_mix))


def test_separate_window_inputs_gradients_match_central_differences():
    # the window branch reads its own q_w, k_w; the GLA branch q, k
    B, H, T, d, w, M, s = 1, 1, 12, 4, 4, 2, 0.6
    args = dict(q=rand(B, H, T, d), k=rand(B, H, T, d), v=rand(B, H, T, d),
                log_alpha=logsig(rand(B, H, T, d) + 1.0), meta_k=rand(H, M, d),
                meta_v=rand(H, M, d), q_w=rand(B, H, T, d), k_w=rand(B, H, T, d))
    dO = rand(B, H, T, d)
    g = oracle.hybrid_backward(args["q"], args["k"], args["v"], args["log_alpha"], args["meta_k"],
                               args["meta_v"], w, s, dO, mix=0.8, q_w=args["q_w"], k_w=args["k_w"])
    h = 1e-6
    for arg, gname in dict(q="dq", k="dk", q_w="dq_w", k_w="dk_w", v="dv", meta_k="dmeta_k").items():
        x = args[arg]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = _loss(dO, window=w, scale=s, mix=0.8, **args)
            x[idx] = keep - h
            lm = _loss(dO, window=w, scale=s, mix=0.8, **args)
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        assert rel(g[gname], fd) < 1e-6, arg


def test_separate_window_inputs_decode_reproduces_prefill():
    # decode steps with separate window inputs continue a prefill exactly; the
    # window cache holds the window keys
    B, H, T, d, w, M, s = 2, 2, 20, 3, 6, 2, 0.9
    q, k, v, qw, kw = (rand(B, H, T, d) for _ in range(5))
    la, mk, mv = logsig(rand(B, H, T, d) + 1), rand(H, M, d), rand(H, M, d)
    full = oracle.hybrid_forward(q, k, v, la, mk, mv, w, s, mix=0.7, q_w=qw, k_w=kw)
    T0 = 13
    pre = oracle.hybrid_forward(q[:, :, :T0], k[:, :, :T0], v[:, :, :T0], la[:, :, :T0], mk, mv,
                                w, s, mix=0.7, q_w=qw[:, :, :T0], k_w=kw[:, :, :T0])
    S, rk, rv, pos = pre["hT"], pre["ring_k"], pre["ring_v"], np.full(B, T0)
    for t in range(T0, T):
        o, S, rk, rv, pos = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], la[:, :, t], S,
                                               rk, rv, pos, mk, mv, w, s, mix=0.7,
                                               q_w=qw[:, :, t], k_w=kw[:, :, t])
        assert rel(o, full["o"][:, :, t]) < 1e-12
    assert rel(S, full["hT"]) < 1e-12 and rel(rk, full["ring_k"]) < 1e-13


def test_state_gradient_matches_central_differences():
    # loss with a term through the final state: L = sum(dO * o) + sum(dhT * hT)
    B, H, T, d, w, M, s = 1, 1, 11, 4, 3, 2, 0.8
    args = dict(q=rand(B, H, T, d), k=rand(B, H, T, d), v=rand(B, H, T, d),
                log_alpha=logsig(rand(B, H, T, d) + 0.5), meta_k=rand(H, M, d),
                meta_v=rand(H, M, d), h0=rand(B, H, d, d))
    dO, dhT = rand(B, H, T, d), rand(B, H, d, d)

    def loss():
        r = oracle.hybrid_forward(window=w, scale=s, mix=0.9, **args)
        return float((r["o"] * dO).sum() + (r["hT"] * dhT).sum())

    g = oracle.hybrid_backward(args["q"], args["k"], args["v"], args["log_alpha"], args["meta_k"],
                               args["meta_v"], w, s, dO, mix=0.9, h0=args["h0"], dhT=dhT)
    h = 1e-6
    for arg, gname in dict(q="dq", k="dk", v="dv", log_alpha="dlog_alpha", h0="dh0").items():
        x = args[arg]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = loss()
            x[idx] = keep - h
            lm = loss()
            x[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        assert rel(g[gname], fd) < 1e-6, arg


def test_state_gradient_chains_over_segments():
    # a sequence run as two segments (hT of the first as h0 of the second) has
    # the same outputs, and chaining dh0 of the second segment into dhT of the
    # first gives the whole sequence's gradients
    B, H, T, T1, d = 2, 1, 90, 37, 5
    q, k, v = rand(B, H, T, d), rand(B, H, T, d), rand(B, H, T, 3)
    la, dO, h0 = logsig(rand(B, H, T, d) + 1.5), rand(B, H, T, 3), rand(B, H, d, 3)
    full = oracle.gla_backward(q, k, v, la, dO, h0=h0)
    a, b = slice(0, T1), slice(T1, T)
    o1, h1 = oracle.gla_forward(q[:, :, a], k[:, :, a], v[:, :, a], la[:, :, a], h0)
    o2, _ = oracle.gla_forward(q[:, :, b], k[:, :, b], v[:, :, b], la[:, :, b], h1)
    o_full, _ = oracle.gla_forward(q, k, v, la, h0)
    assert rel(np.concatenate([o1, o2], axis=2), o_full) < 1e-13
    g2 = oracle.gla_backward(q[:, :, b], k[:, :, b], v[:, :, b], la[:, :, b], dO[:, :, b], h0=h1)
    g1 = oracle.gla_backward(q[:, :, a], k[:, :, a], v[:, :, a], la[:, :, a], dO[:, :, a], h0=h0,
                             dhT=g2["dh0"])
    for key in ("dq", "dk", "dv", "dlog_alpha"):
        assert rel(np.concatenate([g1[key], g2[key]], axis=2), full[key]) < 1e-12, key
    assert rel(g1["dh0"], full["dh0"]) < 1e-12


# ------------------------------------------------------------ logit gates
def test_log_sigmoid_special_values_and_symmetry():
    # sigma(0) = 1/2; sigma(x) + sigma(-x) = 1, so log sigma(x) - log sigma(-x) = x
    assert oracle.log_sigmoid(np.array(0.0)) == -np.log(2.0)
    x = np.concatenate([rand(200) * 6, [-700.0, -40.0, -1e-9, 1e-9, 40.0, 700.0]])
    ls, lm = oracle.log_sigmoid(x), oracle.log_sigmoid(-x)
    assert np.max(np.abs(ls - lm - x) / np.maximum(1.0, np.abs(x))) < 1e-15
    assert np.max(np.abs(np.exp(ls) + np.exp(lm) - 1.0)) < 1e-15
    assert np.all(ls <= 0.0)
    # asymptotes: log sigma(x) -> x for x -> -inf, -e^{-x} for x -> +inf
    assert oracle.log_sigmoid(np.array(-40.0)) == -40.0 - np.exp(-40.0)
    assert abs(oracle.log_sigmoid(np.array(40.0)) + np.exp(-40.0)) < 1e-30
    # the textbook form where it is accurate (|x| moderate)
    xm = rand(100) * 4
    assert rel(np.exp(oracle.log_sigmoid(xm)), 1.0 / (1.0 + np.exp(-xm))) < 1e-15


def test_log_sigmoid_gradient_matches_central_differences():
    x = np.concatenate([rand(50) * 5, [-30.0, 30.0]])
    g = rand(x.size)
    got = oracle.log_sigmoid_backward(x, g)
    h = 1e-6
    fd = g * (oracle.log_sigmoid(x + h) - oracle.log_sigmoid(x - h)) / (2 * h)
    assert np.max(np.abs(got - fd)) < 1e-8
    # sigma(-x) at the extremes, computed without cancellation
    assert oracle.log_sigmoid_backward(np.array(40.0), np.array(1.0)) == pytest.approx(
        np.exp(-40.0), rel=1e-14)
    assert oracle.log_sigmoid_backward(np.array(-40.0), np.array(1.0)) == pytest.approx(1.0, rel=1e-15)


def test_logit_gates_drive_the_recurrence_as_sigmoid_decays():
    # the state recurrence with alpha_t = 1 / (1 + e^{-x_t}) applied directly,
    # token by token, against the oracle fed log_sigmoid(x)
    B, H, T, d = 1, 2, 23, 4
    q, k, v, x = rand(B, H, T, d), rand(B, H, T, d), rand(B, H, T, d), rand(B, H, T, d) * 3 + 1
    S = np.zeros((B, H, d, d))
    o = np.zeros((B, H, T, d))
    for t in range(T):
        alpha = 1.0 / (1.0 + np.exp(-x[:, :, t]))
        S = alpha[..., None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
        o[:, :, t] = np.einsum("bhc,bhcn->bhn", q[:, :, t], S)
    got, hT = oracle.gla_forward(q, k, v, oracle.log_sigmoid(x))
    assert rel(got, o) < 1e-13 and rel(hT, S) < 1e-13


def test_logit_gate_gradient_through_the_layer():
    # d loss / d x by central differences in x, against the chain rule through
    # the backward's d log_alpha
    B, H, T, d, w, M, s = 1, 1, 11, 3, 4, 2, 0.7
    q, k, v, dO = rand(B, H, T, d), rand(B, H, T, d), rand(B, H, T, d), rand(B, H, T, d)
    x = rand(B, H, T, d) * 2 + 1
    mk, mv = rand(H, M, d), rand(H, M, d)
    loss = lambda xx: float((oracle.hybrid_forward(q, k, v, oracle.log_sigmoid(xx), mk, mv, w, s)["o"] * dO).sum())
    g = oracle.hybrid_backward(q, k, v, oracle.log_sigmoid(x), mk, mv, w, s, dO)
    dx = oracle.log_sigmoid_backward(x, g["dlog_alpha"])
    h = 1e-6
    for idx in [(0, 0, 0, 0), (0, 0, 5, 1), (0, 0, 10, 2), (0, 0, 3, 0)]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (loss(xp) - loss(xm)) / (2 * h)
        assert abs(dx[idx] - fd) < 1e-7 * max(1.0, abs(fd))


def test_I9_dlog_alpha_identity_over_chunks():
    # GLA part only: dlog_alpha = reverse cumsum over the sequence of q*dq - k*dk
    B, H, T, d = 2, 2, 150, 6
    q, k, v = rand(B, H, T, d), rand(B, H, T, d), rand(B, H, T, 4)
    la = logsig(rand(B, H, T, d) + 2)
    dO = rand(B, H, T, 4)
    g = oracle.gla_backward(q, k, v, la, dO, h0=rand(B, H, d, 4), checkpoint=64)
    db = q * g["dq"] - k * g["dk"]
    ref = np.flip(np.cumsum(np.flip(db, 2), 2), 2)
    assert rel(g["dlog_alpha"], ref) < 1e-10


def test_backward_checkpoint_length_is_irrelevant():
    B, H, T, d = 1, 2, 70, 4
    x = [rand(B, H, T, d) for _ in range(3)] + [logsig(rand(B, H, T, d))]
    dO = rand(B, H, T, d)
    a = oracle.gla_backward(*x, dO, checkpoint=64)
    b = oracle.gla_backward(*x, dO, checkpoint=7)
    for key in a:
        assert rel(a[key], b[key]) < 1e-13


# ------------------------------------------------- inputs through the recipe
def test_workload_recipe_feeds_oracle_consistently():
    inp = make_inputs(B=1, H=2, T=70, dk=16, dv=16, n_meta=4, dtype="bf16", seed=0)
    assert inp["q"].dtype == torch.bfloat16 and inp["log_alpha"].dtype == torch.float32
    la = to_f64_numpy(inp["log_alpha"])
    assert np.all(la < 0) and abs(la.mean() + 0.18) < 0.05
    q, k, v = (to_f64_numpy(inp[n]) for n in ("q", "k", "v"))
    o, _ = oracle.gla_forward(q, k, v, la)
    assert rel(o, pairwise_gla(q, k, v, la)) < 1e-12
