"""CPU checks (fp64, no GPU) of the chunk-level rewritings the HIP kernels use,
against the oracle.  These test the algebra the kernels implement, not the
oracle itself (the oracle is pinned in test_oracle_pins.py).

1. Forward: the chunk form with 16-token sub-block midpoints R_i,
   A_ts = sum_c (q_t 2^{b_t-R_i}) (k_s 2^{R_j-b_s}) 2^{R_i-R_j}, plus the inter-chunk
   state term and the (decay, state) segment carry, reproduces the recurrence.
2. Backward: the gate gradient written with in-chunk sums only
   (q-side suffix sums, k-side intra suffix / inter prefix sums, and the
   2^{b_last} dS.S state term) equals the oracle's dlog_alpha.
"""
import numpy as np

import oracle

RNG = np.random.default_rng(7)
C = 64


def logsig(x):
    return -np.logaddexp(0.0, -x)


def chunk_forward(q, k, v, la, h0, segments):
    """One head: q, k [T,d], v [T,d], la [T,d]; sub-block factorised chunks,
    sequence cut into `segments` pieces joined by the (decay, state) carry."""
    T, d = q.shape
    nc = (T + C - 1) // C
    cps = -(-nc // segments)
    bounds = [(s * cps, min(nc, (s + 1) * cps)) for s in range(segments) if s * cps < nc]
    l2 = la / np.log(2.0)

    def run(c0, c1, S, out):
        for c in range(c0, c1):
            t0, t1 = c * C, min(T, (c + 1) * C)
            n = t1 - t0
            b = np.cumsum(l2[t0:t1], axis=0)
            R = [b[min(16 * i + 7, n - 1)] for i in range(4)]
            A = np.zeros((n, n))
            for t in range(n):
                for s in range(t + 1):
                    i, j = t // 16, s // 16
                    qg = q[t0 + t] * 2.0 ** (b[t] - R[i])
                    kg = k[t0 + s] * 2.0 ** (R[j] - b[s])
                    A[t, s] = np.sum(qg * kg * 2.0 ** (R[i] - R[j]))
            if out is not None:
                out[t0:t1] = A @ v[t0:t1] + (q[t0:t1] * 2.0 ** b) @ S
            S = 2.0 ** b[-1][:, None] * S + (k[t0:t1] * 2.0 ** (b[-1] - b)).T @ v[t0:t1]
        return S

    # state pass per segment from zero, with its total log2 decay
    loc = []
    for (c0, c1) in bounds[:-1]:
        Sl = run(c0, c1, np.zeros((d, d)), None)
        gam = np.sum(l2[c0 * C:min(T, c1 * C)], axis=0)
        loc.append((Sl, gam))
    out = np.zeros((T, d))
    S_in = h0.copy()
    for g, (c0, c1) in enumerate(bounds):
        S_end = run(c0, c1, S_in, out)
        if g < len(loc):
            S_in = 2.0 ** loc[g][1][:, None] * S_in + loc[g][0]
    return out, S_end


def test_forward_chunk_form_with_segments_matches_recurrence():
    T, d = 300, 8
    q, k, v = (RNG.standard_normal((T, d)) for _ in range(3))
    la = logsig(RNG.standard_normal((T, d)) + 1.0)
    h0 = RNG.standard_normal((d, d))
    ref, refT = oracle.gla_forward(q[None, None], k[None, None], v[None, None], la[None, None],
                                   h0[None, None])
    for segs in (1, 2, 3):
        o, hT = chunk_forward(q, k, v, la, h0, segs)
        assert np.max(np.abs(o - ref[0, 0])) / np.max(np.abs(ref)) < 1e-12
        assert np.max(np.abs(hT - refT[0, 0])) / np.max(np.abs(refT)) < 1e-12


def test_forward_chunk_form_extreme_gates_stays_finite():
    T, d = 128, 4
    q, k, v = (RNG.standard_normal((T, d)) for _ in range(3))
    la = logsig(RNG.standard_normal((T, d)) - 3.0)   # about -200 nats per chunk
    ref, _ = oracle.gla_forward(q[None, None], k[None, None], v[None, None], la[None, None])
    o, _ = chunk_forward(q, k, v, la, np.zeros((d, d)), 2)
    assert np.all(np.isfinite(o))
    assert np.max(np.abs(o - ref[0, 0])) / np.max(np.abs(ref)) < 1e-12


def test_gate_gradient_chunk_local_form():
    T, d = 150, 6
    q, k, v, dO = (RNG.standard_normal((T, d)) for _ in range(4))
    la = logsig(RNG.standard_normal((T, d)) + 1.0)
    h0 = RNG.standard_normal((d, d))
    ref = oracle.gla_backward(q[None, None], k[None, None], v[None, None], la[None, None],
                              dO[None, None], h0=h0[None, None])["dlog_alpha"][0, 0]
    nc = (T + C - 1) // C
    S, Sc = h0.copy(), []
    for c in range(nc):
        Sc.append(S.copy())
        for t in range(c * C, min(T, (c + 1) * C)):
            S = np.exp(la[t])[:, None] * S + np.outer(k[t], v[t])
    dS, G = [None] * nc, np.zeros((d, d))
    for c in reversed(range(nc)):
        dS[c] = G.copy()
        t0, t1 = c * C, min(T, (c + 1) * C)
        b = np.cumsum(la[t0:t1], axis=0)
        G = np.exp(b[-1])[:, None] * G + (q[t0:t1] * np.exp(b)).T @ dO[t0:t1]
    out = np.zeros((T, d))
    for c in range(nc):
        t0, t1 = c * C, min(T, (c + 1) * C)
        n = t1 - t0
        b = np.cumsum(la[t0:t1], axis=0)
        dA = dO[t0:t1] @ v[t0:t1].T
        qdq_inter = q[t0:t1] * np.exp(b) * (dO[t0:t1] @ Sc[c].T)
        kdk_inter = k[t0:t1] * np.exp(b[-1] - b) * (v[t0:t1] @ dS[c].T)
        qdq_intra, kdk_intra = np.zeros((n, d)), np.zeros((n, d))
        for t in range(n):
            for s in range(t):          # strictly s < t: the diagonal never enters
                m = dA[t, s] * q[t0 + t] * k[t0 + s] * np.exp(b[t] - b[s])
                qdq_intra[t] += m
                kdk_intra[s] += m
        state = np.exp(b[-1]) * (dS[c] * Sc[c]).sum(axis=1)
        for u in range(n):
            out[t0 + u] = ((qdq_inter[u:] + qdq_intra[u:]).sum(0) - kdk_intra[u:].sum(0)
                           + kdk_inter[:u].sum(0) + state)
    assert np.max(np.abs(out - ref)) / np.max(np.abs(ref)) < 1e-12
