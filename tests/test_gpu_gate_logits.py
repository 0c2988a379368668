"""GPU parity with bf16 gate logits (alpha = sigmoid(x), log-sigmoid taken in the
kernels) against the fp64 oracle fed log_sigmoid(x) of the same bf16 values.

Cases: the single-pass forward (d = 128) and the two-kernel forward (d = 64 and
128, saved for the backward pass) over several chunks with ragged tails, with
gates steep enough to take the sub-block form, an initial state and separate
window inputs; the GLA entry point alone; decode after a prefill; the backward,
whose gate gradient is the gradient with respect to the logits; and the
full-size prefill workload (B=2, H=32, T=4096, d=128) on sampled heads.
"""
import math

import numpy as np
import pytest
import torch

import gated_linear_attention_chunked_amd as lz
import oracle
from tests._gpu_helpers import assert_close, f64, to_dev
from workloads import WORKLOADS, make_decode_inputs, make_inputs

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def inputs(B, H, T, d, M, seed, gate_mean=2.0, **kw):
    inp = make_inputs(B, H, T, d, d, M, seed=seed, gate_mean=gate_mean, with_gate_logits=True, **kw)
    inp.pop("log_alpha")
    return inp


def ref_forward(inp, w, s, mix, sep=False):
    r = f64(inp)
    return oracle.hybrid_forward(r["q"], r["k"], r["v"], oracle.log_sigmoid(r["gate_x"]),
                                 r["meta_k"], r["meta_v"], w, s, mix=mix, h0=r.get("h0"),
                                 q_w=r.get("q_w") if sep else None,
                                 k_w=r.get("k_w") if sep else None)


@pytest.mark.parametrize("B,H,T,d,w,M,gate_mean,sep", [
    (2, 2, 300, 128, 128, 4, 2.0, False),    # single pass
    (1, 2, 2100, 128, 64, 3, 2.0, False),    # single pass, several state segments
    (2, 2, 257, 128, 100, 2, -3.0, True),    # steep gates (sub-block form), own window q, k
    (2, 2, 333, 64, 64, 4, 2.0, False),      # single pass at d = 64, three-chunk ring
    (1, 3, 200, 64, 40, 0, -3.0, False),
])
def test_forward_gate_logits(B, H, T, d, w, M, gate_mean, sep):
    print(f"[case] logit fwd B{B} H{H} T{T} d{d} w{w} M{M} gate{gate_mean} sep{sep}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.9
    inp = inputs(B, H, T, d, M, seed=T + d, gate_mean=gate_mean, with_h0=True, with_window_qk=sep)
    x = to_dev(inp)
    ref = ref_forward(inp, w, s, mix, sep)
    args = (x["q"], x["k"], x["v"], x["gate_x"], x["meta_k"], x["meta_v"], w)
    kw = dict(scale=s, mix=mix, h0=x["h0"], return_state=True, return_ring=True,
              q_w=x.get("q_w"), k_w=x.get("k_w"))
    inf = lz.hybrid_fwd(*args, **kw)
    sav = lz.hybrid_fwd(*args, save_for_backward=True, **kw)
    torch.cuda.synchronize()
    for tag, out in (("inference", inf), ("saved", sav)):
        assert_close(f"{tag}.o", out["o"], ref["o"], BF)
        assert_close(f"{tag}.hT", out["hT"], ref["hT"], BF)
        assert_close(f"{tag}.ring_k", out["ring_k"], ref["ring_k"], BF, tol=0.0)
    assert_close("saved.o_swa", sav["o_swa"], ref["o_swa"], BF)
    if not sep:
        o_gla, hT = lz.gla_fwd(x["q"], x["k"], x["v"], x["gate_x"], h0=x["h0"], return_state=True)
        torch.cuda.synchronize()
        assert_close("gla.o", o_gla, ref["o_gla"], BF)
        assert_close("gla.hT", hT, ref["hT"], BF)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_gate_logits(d):
    B, H, T0, n, w, M = 2, 2, 130, 40, 64, 4
    print(f"[case] logit decode B{B} H{H} T0 {T0} n{n} d{d}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.8
    inp = inputs(B, H, T0, d, M, seed=d + 5)
    dec = make_decode_inputs(n, B, H, d, d, seed=d + 6, with_gate_logits=True)
    x = to_dev(inp)
    pre = lz.hybrid_fwd(x["q"], x["k"], x["v"], x["gate_x"], x["meta_k"], x["meta_v"], w, scale=s,
                        mix=mix, return_state=True, return_ring=True)
    state, rk, rv = pre["hT"], pre["ring_k"], pre["ring_v"]
    pos = torch.full((B,), T0, dtype=torch.int64, device="cuda")
    outs = []
    for i in range(n):
        outs.append(lz.decode_step(dec["q"][i].cuda(), dec["k"][i].cuda(), dec["v"][i].cuda(),
                                   dec["gate_x"][i].cuda(), state, rk, rv, pos, x["meta_k"],
                                   x["meta_v"], scale=s, mix=mix))
    torch.cuda.synchronize()
    r, dq = f64(inp), f64(dec)
    full = {n_: np.concatenate([r[n_], np.moveaxis(dq[n_], 0, 2)], axis=2)
            for n_ in ("q", "k", "v", "gate_x")}
    ref = oracle.hybrid_forward(full["q"], full["k"], full["v"], oracle.log_sigmoid(full["gate_x"]),
                                r["meta_k"], r["meta_v"], w, s, mix=mix)
    assert_close("decode o", torch.stack(outs, dim=2), ref["o"][:, :, T0:], BF)
    assert_close("state", state, ref["hT"], BF)


@pytest.mark.parametrize("T,w,M,gate_mean", [(200, 64, 4, 2.0), (257, 16, 0, -3.0)])
def test_backward_gate_logits(T, w, M, gate_mean):
    B, H, d = 2, 2, 64
    print(f"[case] logit bwd B{B} H{H} T{T} w{w} M{M} gate{gate_mean}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.75
    inp = inputs(B, H, T, d, M, seed=T, gate_mean=gate_mean, with_grad_out=True, with_h0=True)
    x = to_dev(inp)
    args = (x["q"], x["k"], x["v"], x["gate_x"], x["meta_k"], x["meta_v"], w)
    f = lz.hybrid_fwd(*args, scale=s, mix=mix, h0=x["h0"], save_for_backward=True)
    g = lz.hybrid_bwd(*args, f["o_swa"], f["lse"], x["dO"], scale=s, mix=mix, h0=x["h0"],
                      return_dh0=True)
    torch.cuda.synchronize()
    r = f64(inp)
    ref = oracle.hybrid_backward(r["q"], r["k"], r["v"], oracle.log_sigmoid(r["gate_x"]),
                                 r["meta_k"], r["meta_v"], w, s, r["dO"], mix=mix, h0=r["h0"])
    assert g["dlog_alpha"].dtype == torch.float32
    assert_close("d gate_x", g["dlog_alpha"], oracle.log_sigmoid_backward(r["gate_x"],
                                                                          ref["dlog_alpha"]), BF)
    for n in ("dq", "dk", "dv", "dmeta_k", "dmeta_v", "dh0"):
        if n.startswith("dmeta") and M == 0:
            continue
        assert_close(n, g[n], ref[n], BF)


def test_full_size_prefill_gate_logits_sampled_heads():
    wl = WORKLOADS["prefill_bf16_b2_h32_t4096_d128"]
    print("[case] logit full-size prefill B2 H32 T4096 d128", flush=True)
    s = 1.0 / math.sqrt(wl.dk)
    inp = inputs(wl.B, wl.H, wl.T, wl.dk, wl.n_meta, seed=0)
    x = to_dev(inp)
    out = lz.hybrid_fwd(x["q"], x["k"], x["v"], x["gate_x"], x["meta_k"], x["meta_v"], wl.window,
                        scale=s, return_state=True, return_ring=True)
    torch.cuda.synchronize()
    for b, h in [(0, 5), (1, 31)]:
        sl = {n: (t[b:b + 1, h:h + 1] if n not in ("meta_k", "meta_v") else t[h:h + 1])
              for n, t in inp.items()}
        ref = ref_forward(sl, wl.window, s, 1.0)
        assert_close(f"o[b{b},h{h}]", out["o"][b:b + 1, h:h + 1], ref["o"], BF)
        assert_close(f"hT[b{b},h{h}]", out["hT"][b:b + 1, h:h + 1], ref["hT"], BF)
        assert_close(f"ring_k[b{b},h{h}]", out["ring_k"][b:b + 1, h:h + 1], ref["ring_k"], BF,
                     tol=0.0)
