"""Plain fp64 CPU oracle for Lizard-style hybrid attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code, tables or helpers with the HIP library.

Sources (cited by page title and section; the pages print no code and no worked
numbers, so every function below is the plain definition written out):

  [LZ-2a]  "Lizard: An Efficient Linearization Framework for Large Language
           Models" (gist.science technical summary), section 2 "Methodology",
           part (a) "Hybrid attention architecture": the learnable gate
           Gamma_i = sigma(W_gamma x_i), the constant-memory state update
           S_i = Gamma_i S_{i-1} + phi(k_i) v_i^T, the anchor sliding window
           with meta-memory tokens acting as sinks in the softmax denominator,
           and the final weighted sum Y = Y_gate + alpha * Y_anchor.
  [LZ-2c]  same page, section 2 part (c) "Hardware-aware algorithm": the gate
           product is absorbed into q and k in log space.  That is a way of
           computing the same numbers faster; the oracle does not use it.
  [LZ-4]   same page, section 4 "Efficiency": constant memory at inference.

Readings of points the pages leave open (each one is listed with its reason in
the design notes):
  * phi is the identity here: callers pass phi(k), phi(q) as k, q.
  * the gate is per token and per key channel; exp(log_alpha_t) scales the
    rows of S_{t-1} before k_t^T v_t is added; the read-out o_t = q_t S_t uses
    the state after the update; no normaliser and no scale on the GLA branch.
  * the window holds the w most recent tokens including the current one,
    keys j in [t-w+1, t]; meta-memory K/V slots [H, M, d] are shared across
    the batch and take part in the same softmax as the window keys (numerator
    and denominator); the sink-only reading is the special case meta_v = 0.
  * the mix weight of the window branch is a scalar `mix` (the pages call it
    alpha, which would clash with the decay).
  * the two branches may read different query/key inputs (the GLA branch its
    feature-mapped q, k; the window branch its own q_w, k_w); by default both
    read the same q, k.

All arrays are numpy, laid out [B, H, T, D]; computations run in float64.
"""
import numpy as np

__all__ = [
    "log_sigmoid",
    "log_sigmoid_backward",
    "gla_forward",
    "window_meta_attention",
    "hybrid_forward",
    "ring_from_sequence",
    "decode_step",
    "gla_backward",
    "window_meta_backward",
    "hybrid_backward",
]


def _f64(x):
    return None if x is None else np.array(x, dtype=np.float64, copy=True)


# ---------------------------------------------------------------------------
# Gate
# ---------------------------------------------------------------------------
def log_sigmoid(x):
    """log alpha of the sigmoid gate alpha = sigma(x) [LZ-2a, learnable gate
    Gamma = sigma(W_gamma x)], from the gate logits x:
    log sigma(x) = -log(1 + exp(-x)), written as min(x, 0) - log1p(exp(-|x|))
    so that no positive number is exponentiated."""
    x = _f64(x)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def log_sigmoid_backward(x, d_log_alpha):
    """Chain rule through log_sigmoid: d/dx log sigma(x) = sigma(-x), so the
    gradient with respect to the logits is d_log_alpha * sigma(-x)."""
    return _f64(d_log_alpha) * np.exp(log_sigmoid(-_f64(x)))


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------
def gla_forward(q, k, v, log_alpha, h0=None):
    """Gated linear attention, token by token [LZ-2a, state update].

    S_t = diag(exp(log_alpha_t)) S_{t-1} + k_t^T v_t,   o_t = q_t S_t.

    q, k, log_alpha: [B,H,T,dk]; v: [B,H,T,dv]; h0: [B,H,dk,dv] or None (zeros).
    Returns (o [B,H,T,dv], hT [B,H,dk,dv]).
    """
    q, k, v, la, h0 = map(_f64, (q, k, v, log_alpha, h0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if h0 is None else h0
    o = np.empty((B, H, T, dv))
    for t in range(T):
        S = np.exp(la[:, :, t, :])[..., :, None] * S \
            + k[:, :, t, :, None] * v[:, :, t, None, :]
        o[:, :, t, :] = np.matmul(q[:, :, t, None, :], S)[:, :, 0, :]
    return o, S


def window_meta_attention(q, k, v, meta_k, meta_v, window, scale):
    """Sliding-window softmax attention plus meta-memory slots [LZ-2a, anchor window].

    For query t the candidate keys are the tokens j in [max(0, t-w+1), t] and
    the M meta slots.  Logits are scale * q_t . key; one softmax runs over all
    of them; the output is the probability-weighted sum of the matching values
    (token values and meta values).  lse_t = log sum exp of the logits.

    q, k: [B,H,T,dk]; v: [B,H,T,dv]; meta_k: [H,M,dk]; meta_v: [H,M,dv].
    Returns (o_swa [B,H,T,dv], lse [B,H,T]).
    """
    q, k, v, mk, mv = map(_f64, (q, k, v, meta_k, meta_v))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    M = mk.shape[1]
    o = np.empty((B, H, T, dv))
    lse = np.empty((B, H, T))
    mkb = np.broadcast_to(mk[None], (B, H, M, dk))
    mvb = np.broadcast_to(mv[None], (B, H, M, dv))
    for t in range(T):
        lo = max(0, t - window + 1)
        keys = np.concatenate([k[:, :, lo:t + 1, :], mkb], axis=2)
        vals = np.concatenate([v[:, :, lo:t + 1, :], mvb], axis=2)
        logits = scale * np.matmul(keys, q[:, :, t, :, None])[..., 0]
        m = logits.max(axis=-1, keepdims=True)
        e = np.exp(logits - m)
        z = e.sum(axis=-1, keepdims=True)
        o[:, :, t, :] = np.matmul((e / z)[:, :, None, :], vals)[:, :, 0, :]
        lse[:, :, t] = m[..., 0] + np.log(z[..., 0])
    return o, lse


def ring_from_sequence(k, v, window):
    """Window cache left after a prefill of T tokens [LZ-4, constant memory].

    Slot (p mod w) holds token p for the last min(T, w) tokens; slots no token
    has reached are zero.  Returns (ring_k [B,H,w,dk], ring_v [B,H,w,dv]).
    """
    k, v = _f64(k), _f64(v)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    rk = np.zeros((B, H, window, dk))
    rv = np.zeros((B, H, window, dv))
    for p in range(max(0, T - window), T):
        rk[:, :, p % window, :] = k[:, :, p, :]
        rv[:, :, p % window, :] = v[:, :, p, :]
    return rk, rv


def hybrid_forward(q, k, v, log_alpha, meta_k, meta_v, window, scale, mix=1.0, h0=None,
                   q_w=None, k_w=None):
    """Hybrid layer output o = o_gla + mix * o_swa [LZ-2a, final weighted sum].

    The GLA branch reads q, k; the window branch reads q_w, k_w (default q, k)
    [LZ-2a: the gated branch takes feature-mapped queries and keys, the
    window branch its own].  Returns a dict with o, o_gla, o_swa, lse, hT,
    ring_k, ring_v (the window cache holds the window branch's keys).
    """
    q_w = q if q_w is None else q_w
    k_w = k if k_w is None else k_w
    o_gla, hT = gla_forward(q, k, v, log_alpha, h0)
    o_swa, lse = window_meta_attention(q_w, k_w, v, meta_k, meta_v, window, scale)
    rk, rv = ring_from_sequence(k_w, v, window)
    return dict(o=o_gla + mix * o_swa, o_gla=o_gla, o_swa=o_swa, lse=lse,
                hT=hT, ring_k=rk, ring_v=rv)


def decode_step(q, k, v, log_alpha, state, ring_k, ring_v, pos, meta_k, meta_v,
                window, scale, mix=1.0, q_w=None, k_w=None):
    """One constant-memory generation step [LZ-2a state update; LZ-4].

    pos[b] tokens have been seen by sequence b.  The new token (q, k, v,
    log_alpha: [B,H,d]) updates the state exactly as one step of gla_forward;
    its window key k_w (default k) is written to ring slot pos mod w, and its
    window query q_w (default q) attends over the min(pos+1, w) filled slots
    plus the meta slots.  Returns (o [B,H,dv], state', ring_k', ring_v',
    pos + 1); the inputs are not modified.
    """
    q_w = q if q_w is None else q_w
    k_w = k if k_w is None else k_w
    q, k, v, la, S, rk, rv, mk, mv, q_w, k_w = map(
        _f64, (q, k, v, log_alpha, state, ring_k, ring_v, meta_k, meta_v, q_w, k_w))
    pos = np.array(pos, dtype=np.int64, copy=True)
    B, H, dk = q.shape
    S = np.exp(la)[..., :, None] * S + k[..., :, None] * v[..., None, :]
    o_gla = np.matmul(q[..., None, :], S)[..., 0, :]
    o_swa = np.empty_like(o_gla)
    for b in range(B):
        slot = int(pos[b] % window)
        rk[b, :, slot, :] = k_w[b]
        rv[b, :, slot, :] = v[b]
        n = int(min(pos[b] + 1, window))
        keys = np.concatenate([rk[b, :, :n, :], mk], axis=1)      # [H, n+M, dk]
        vals = np.concatenate([rv[b, :, :n, :], mv], axis=1)
        logits = scale * np.matmul(keys, q_w[b, :, :, None])[..., 0]
        e = np.exp(logits - logits.max(axis=-1, keepdims=True))
        p = e / e.sum(axis=-1, keepdims=True)
        o_swa[b] = np.matmul(p[:, None, :], vals)[:, 0, :]
    return o_gla + mix * o_swa, S, rk, rv, pos + 1


# ---------------------------------------------------------------------------
# Backward (manual reverse mode of the definitions above)
# ---------------------------------------------------------------------------
def gla_backward(q, k, v, log_alpha, dO, h0=None, checkpoint=64, dhT=None):
    """Reverse mode of gla_forward for the loss L = sum(dO * o) + sum(dhT * hT).

    dhT (optional, default 0) is the gradient of L with respect to the final
    state hT: the state is the layer's constant-size memory [LZ-2a, LZ-4], so a
    long sequence can be run in segments with hT of one segment as h0 of the
    next, and the segments' backward passes are then chained the same way
    (dh0 of a segment is dhT of the one before).
    Walks t = T-1 .. 0 with G = dL/dS_t (G = dhT before the last token):
        G += q_t^T dO_t;  dq_t = S_t dO_t;  dk_t = G v_t;  dv_t = G^T k_t;
        dlog_alpha_t = alpha_t * rowsum(G * S_{t-1});  G <- diag(alpha_t) G.
    The states S_{t-1} are recomputed forward from checkpoints taken every
    `checkpoint` tokens.  Returns dict(dq, dk, dv, dlog_alpha, dh0).
    """
    q, k, v, la, dO, h0 = map(_f64, (q, k, v, log_alpha, dO, h0))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if h0 is None else h0
    alpha = np.exp(la)
    starts = list(range(0, T, checkpoint))
    entering = {}
    S = S0
    for t in range(T):
        if t % checkpoint == 0:
            entering[t] = S.copy()
        S = alpha[:, :, t, :, None] * S + k[:, :, t, :, None] * v[:, :, t, None, :]
    dq = np.zeros_like(q)
    dk_ = np.zeros_like(k)
    dv_ = np.zeros_like(v)
    dla = np.zeros_like(la)
    G = np.zeros((B, H, dk, dv)) if dhT is None else _f64(dhT).copy()
    for t0 in reversed(starts):
        t1 = min(T, t0 + checkpoint)
        states = [entering[t0]]                        # states[i] = S_{t0+i-1}
        for t in range(t0, t1):
            states.append(alpha[:, :, t, :, None] * states[-1]
                          + k[:, :, t, :, None] * v[:, :, t, None, :])
        for t in reversed(range(t0, t1)):
            S_t = states[t - t0 + 1]
            S_prev = states[t - t0]
            G = G + q[:, :, t, :, None] * dO[:, :, t, None, :]
            dq[:, :, t, :] = np.matmul(S_t, dO[:, :, t, :, None])[..., 0]
            dk_[:, :, t, :] = np.matmul(G, v[:, :, t, :, None])[..., 0]
            dv_[:, :, t, :] = np.matmul(k[:, :, t, None, :], G)[:, :, 0, :]
            dla[:, :, t, :] = alpha[:, :, t, :] * (G * S_prev).sum(axis=-1)
            G = alpha[:, :, t, :, None] * G
    return dict(dq=dq, dk=dk_, dv=dv_, dlog_alpha=dla, dh0=G)


def window_meta_backward(q, k, v, meta_k, meta_v, window, scale, dO_swa):
    """Reverse mode of window_meta_attention for L = sum(dO_swa * o_swa).

    Per query: p = softmax(logits); dp_j = dO_swa . val_j; D = sum_j p_j dp_j;
    dlogit_j = p_j (dp_j - D); dq += scale * sum_j dlogit_j key_j;
    dkey_j += scale * dlogit_j q; dval_j += p_j dO_swa.  Meta gradients are
    summed over batch and time.  Returns dict(dq, dk, dv, dmeta_k, dmeta_v).
    """
    q, k, v, mk, mv, g = map(_f64, (q, k, v, meta_k, meta_v, dO_swa))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    M = mk.shape[1]
    dq = np.zeros_like(q)
    dk_ = np.zeros_like(k)
    dv_ = np.zeros_like(v)
    dmk = np.zeros_like(mk)
    dmv = np.zeros_like(mv)
    mkb = np.broadcast_to(mk[None], (B, H, M, dk))
    mvb = np.broadcast_to(mv[None], (B, H, M, dv))
    for t in range(T):
        lo = max(0, t - window + 1)
        n = t + 1 - lo
        keys = np.concatenate([k[:, :, lo:t + 1, :], mkb], axis=2)
        vals = np.concatenate([v[:, :, lo:t + 1, :], mvb], axis=2)
        qt = q[:, :, t, :]
        gt = g[:, :, t, :]
        logits = scale * np.matmul(keys, qt[..., None])[..., 0]
        e = np.exp(logits - logits.max(axis=-1, keepdims=True))
        p = e / e.sum(axis=-1, keepdims=True)                     # [B,H,n+M]
        dp = np.matmul(vals, gt[..., None])[..., 0]
        D = (p * dp).sum(axis=-1, keepdims=True)
        dl = p * (dp - D)
        dq[:, :, t, :] += scale * np.matmul(dl[:, :, None, :], keys)[:, :, 0, :]
        dk_[:, :, lo:t + 1, :] += scale * dl[..., :n, None] * qt[:, :, None, :]
        dv_[:, :, lo:t + 1, :] += p[..., :n, None] * gt[:, :, None, :]
        dmk += scale * (dl[..., n:, None] * qt[:, :, None, :]).sum(axis=0)
        dmv += (p[..., n:, None] * gt[:, :, None, :]).sum(axis=0)
    return dict(dq=dq, dk=dk_, dv=dv_, dmeta_k=dmk, dmeta_v=dmv)


def hybrid_backward(q, k, v, log_alpha, meta_k, meta_v, window, scale, dO, mix=1.0, h0=None,
                    dhT=None, q_w=None, k_w=None):
    """Reverse mode of hybrid_forward for L = sum(dO * o) + sum(dhT * hT)
    [LZ-2a weighted sum; dhT as in gla_backward, default 0].

    dO_gla = dO and dO_swa = mix * dO; gradients of the two branches add.  The
    mix weight enters only the final sum, so dmix = sum(dO * o_swa).  With
    separate window inputs (q_w, k_w given) dq, dk are the GLA branch's and
    dq_w, dk_w the window branch's; otherwise dq, dk hold both.
    Returns dict(dq, dk, dv, dlog_alpha, dmeta_k, dmeta_v, dh0, dmix[, dq_w, dk_w]).
    """
    dO = _f64(dO)
    sep = q_w is not None or k_w is not None
    qw = q if q_w is None else q_w
    kw = k if k_w is None else k_w
    g = gla_backward(q, k, v, log_alpha, dO, h0, dhT=dhT)
    w = window_meta_backward(qw, kw, v, meta_k, meta_v, window, scale, mix * dO)
    out = dict(dv=g["dv"] + w["dv"], dlog_alpha=g["dlog_alpha"], dmeta_k=w["dmeta_k"],
               dmeta_v=w["dmeta_v"], dh0=g["dh0"],
               dmix=float((dO * window_meta_attention(qw, kw, v, meta_k, meta_v, window,
                                                      scale)[0]).sum()))
    if sep:
        out.update(dq=g["dq"], dk=g["dk"], dq_w=w["dq"], dk_w=w["dk"])
    else:
        out.update(dq=g["dq"] + w["dq"], dk=g["dk"] + w["dk"])
    return out
