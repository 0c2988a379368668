"""GPU parity with separate window-branch queries and keys (q_w, k_w) against
the fp64 oracle, through the C ABI.

The gated branch reads q, k and the window branch q_w, k_w.  Cases: the
single-pass forward (bf16, d = 128) and the two-kernel forward (saved for the
backward pass, d = 64 and 128, fp32), both over several chunks with ragged
tails and a two-segment sequence; the window cache (which must hold k_w); the
decode step reproducing a longer prefill; and the backward, whose dq, dk are the
gated branch's and dq_w, dk_w the window branch's.
"""
import math

import numpy as np
import pytest
import torch

import gated_linear_attention_chunked_amd as lz
import oracle
from tests._gpu_helpers import assert_close, f64, to_dev
from workloads import make_decode_inputs, make_inputs

pytestmark = pytest.mark.gpu
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def ref_forward(inp, w, s, mix):
    r = f64(inp)
    return oracle.hybrid_forward(r["q"], r["k"], r["v"], r["log_alpha"], r["meta_k"],
                                 r["meta_v"], w, s, mix=mix, h0=r.get("h0"), q_w=r["q_w"],
                                 k_w=r["k_w"])


@pytest.mark.parametrize("B,H,T,d,w,M,dtype", [
    (2, 2, 300, 128, 128, 4, "bf16"),   # single pass, ragged tail
    (1, 2, 2100, 128, 64, 3, "bf16"),   # single pass, two state segments
    (2, 2, 257, 64, 64, 4, "bf16"),     # single pass at d = 64, three-chunk ring
    (1, 2, 130, 64, 40, 2, "f32"),
])
def test_forward_separate_window_inputs(B, H, T, d, w, M, dtype):
    print(f"[case] window inputs fwd B{B} H{H} T{T} d{d} w{w} M{M} {dtype}", flush=True)
    dt = DT[dtype]
    s, mix = 1.0 / math.sqrt(d), 0.8
    inp = make_inputs(B, H, T, d, d, M, dtype=dtype, seed=T + w, with_h0=True,
                      with_window_qk=True)
    x = to_dev(inp)
    ref = ref_forward(inp, w, s, mix)
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], w)
    kw = dict(scale=s, mix=mix, h0=x["h0"], return_state=True, return_ring=True,
              q_w=x["q_w"], k_w=x["k_w"])
    inf = lz.hybrid_fwd(*args, **kw)               # inference call
    sav = lz.hybrid_fwd(*args, save_for_backward=True, **kw)
    torch.cuda.synchronize()
    for tag, out in (("inference", inf), ("saved", sav)):
        assert_close(f"{tag}.o", out["o"], ref["o"], dt)
        assert_close(f"{tag}.hT", out["hT"], ref["hT"], dt)
        assert_close(f"{tag}.ring_k", out["ring_k"], ref["ring_k"], dt, tol=0.0)
        assert_close(f"{tag}.ring_v", out["ring_v"], ref["ring_v"], dt, tol=0.0)
    assert_close("saved.o_swa", sav["o_swa"], ref["o_swa"], dt)
    assert_close("saved.lse", sav["lse"], ref["lse"], dt, tol=1e-4)  # fp32 output


@pytest.mark.parametrize("d", [64, 128])
def test_decode_separate_window_inputs(d):
    B, H, T0, n, w, M = 2, 2, 150, 70, 64, 3
    print(f"[case] window inputs decode B{B} H{H} T0 {T0} n{n} d{d} w{w} M{M}", flush=True)
    dt = torch.bfloat16
    s, mix = 1.0 / math.sqrt(d), 0.6
    inp = make_inputs(B, H, T0, d, d, M, seed=d, with_window_qk=True)
    dec = make_decode_inputs(n, B, H, d, d, seed=d + 1, with_window_qk=True)
    x = to_dev(inp)
    pre = lz.hybrid_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], w,
                        scale=s, mix=mix, return_state=True, return_ring=True, q_w=x["q_w"],
                        k_w=x["k_w"])
    state, rk, rv = pre["hT"], pre["ring_k"], pre["ring_v"]
    pos = torch.full((B,), T0, dtype=torch.int64, device="cuda")
    outs = []
    for i in range(n):
        t = {k_: dec[k_][i].cuda() for k_ in dec}
        outs.append(lz.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], state, rk, rv, pos,
                                   x["meta_k"], x["meta_v"], scale=s, mix=mix, q_w=t["q_w"],
                                   k_w=t["k_w"]))
    torch.cuda.synchronize()
    r, dq = f64(inp), f64(dec)
    full = {n_: np.concatenate([r[n_], np.moveaxis(dq[n_], 0, 2)], axis=2)
            for n_ in ("q", "k", "v", "log_alpha", "q_w", "k_w")}
    ref = oracle.hybrid_forward(full["q"], full["k"], full["v"], full["log_alpha"], r["meta_k"],
                                r["meta_v"], w, s, mix=mix, q_w=full["q_w"], k_w=full["k_w"])
    assert_close("decode o", torch.stack(outs, dim=2), ref["o"][:, :, T0:], dt)
    assert_close("state", state, ref["hT"], dt)
    assert_close("ring_k", rk, ref["ring_k"], dt, tol=0.0)
    assert_close("ring_v", rv, ref["ring_v"], dt, tol=0.0)


@pytest.mark.parametrize("T,w,M", [(200, 64, 4), (257, 16, 0)])
def test_backward_separate_window_inputs(T, w, M):
    B, H, d = 2, 2, 64
    print(f"[case] window inputs bwd B{B} H{H} T{T} w{w} M{M}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.7
    inp = make_inputs(B, H, T, d, d, M, seed=T, with_grad_out=True, with_h0=True,
                      with_window_qk=True)
    dhT = torch.randn(B, H, d, d, generator=torch.Generator().manual_seed(T)) * 0.1
    x = to_dev(inp)
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], w)
    f = lz.hybrid_fwd(*args, scale=s, mix=mix, h0=x["h0"], save_for_backward=True,
                      q_w=x["q_w"], k_w=x["k_w"])
    g = lz.hybrid_bwd(*args, f["o_swa"], f["lse"], x["dO"], scale=s, mix=mix, h0=x["h0"],
                      dhT=dhT.cuda(), return_dh0=True, return_dmix=True, q_w=x["q_w"],
                      k_w=x["k_w"])
    torch.cuda.synchronize()
    r = f64(inp)
    ref = oracle.hybrid_backward(r["q"], r["k"], r["v"], r["log_alpha"], r["meta_k"],
                                 r["meta_v"], w, s, r["dO"], mix=mix, h0=r["h0"],
                                 dhT=dhT.double().numpy(), q_w=r["q_w"], k_w=r["k_w"])
    for n in ("dq", "dk", "dq_w", "dk_w", "dv", "dlog_alpha", "dmeta_k", "dmeta_v", "dh0"):
        if n.startswith("dmeta") and M == 0:
            continue
        assert_close(n, g[n], ref[n], torch.bfloat16)
    # dmix = sum(dO * o_swa) with o_swa saved in bf16: error <= 2^-8 sum|dO||o_swa|
    bound = 2.0 ** -8 * float((np.abs(r["dO"]) * np.abs(ref_forward(inp, w, s, mix)["o_swa"])).sum())
    err = abs(float(g["dmix"].item()) - ref["dmix"])
    print(f"  dmix: error {err:.2e} (bound {bound:.2e})")
    assert err <= bound
