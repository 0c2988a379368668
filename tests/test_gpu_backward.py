"""GPU parity of the hybrid backward against the fp64 oracle's reverse mode.

Every gradient (dq, dk, dv, dlog_alpha, dmeta_k, dmeta_v, dh0) is compared per
tensor with the normwise maximum relative error.  Cases: several chunks with
ragged tails, windows of 1 / inside / beyond T, M = 0 and 16, an initial state,
an upstream gradient of the final state, a sequence trained as two chained
segments, a mix weight other than 1, extreme gates, determinism, and the
full-size training workload (B=8, H=16, T=2048, d=64) on sampled heads (all
batch rows of a head, so its meta gradients are complete).
"""
import math

import numpy as np
import pytest
import torch

import gated_linear_attention_chunked_amd as lz
import oracle
from tests._gpu_helpers import assert_close, f64, to_dev
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dmeta_k", "dmeta_v", "dh0")


def run_grads(inp, w, s, mix, h0=None, dhT=None):
    x = to_dev(inp)
    h0d = None if h0 is None else h0.cuda()
    dhTd = None if dhT is None else dhT.cuda()
    f = lz.hybrid_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], w,
                      scale=s, mix=mix, h0=h0d, save_for_backward=True, return_state=True)
    g = lz.hybrid_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], w,
                      f["o_swa"], f["lse"], x["dO"], scale=s, mix=mix, h0=h0d, dhT=dhTd,
                      return_dh0=True, return_dmix=True)
    torch.cuda.synchronize()
    g["hT"] = f["hT"]
    return g


def ref_grads(inp, w, s, mix, h0=None, dhT=None):
    r = f64(inp)
    return oracle.hybrid_backward(r["q"], r["k"], r["v"], r["log_alpha"], r["meta_k"],
                                  r["meta_v"], w, s, r["dO"], mix=mix,
                                  h0=None if h0 is None else h0.double().numpy(),
                                  dhT=None if dhT is None else dhT.double().numpy())


DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def check(B, H, T, w, M, seed=0, mix=1.0, gate_mean=2.0, with_h0=False, steep_chunks=False,
          with_dhT=False, d=64, dtype="bf16"):
    print(f"[case] bwd B{B} H{H} T{T} d{d} {dtype} w{w} M{M} mix{mix} gate{gate_mean} "
          f"h0{with_h0} steep{steep_chunks} dhT{with_dhT}", flush=True)
    inp = make_inputs(B, H, T, d, d, M, dtype=dtype, seed=seed, gate_mean=gate_mean,
                      with_grad_out=True, with_h0=with_h0)
    if steep_chunks:
        # every third 64-token chunk decays 8x faster (about -94 per chunk in
        # natural log): chunks on both sides of the single-reference bound
        la = inp["log_alpha"].clone()
        for c0 in range(64, T, 192):
            la[:, :, c0:c0 + 64] *= 8.0
        inp["log_alpha"] = la
    h0 = inp.pop("h0", None)
    dhT = (torch.randn(B, H, d, d, generator=torch.Generator().manual_seed(seed + 7)) * 0.1
           if with_dhT else None)
    s = 1.0 / math.sqrt(d)
    g = run_grads(inp, w, s, mix, h0, dhT)
    ref = ref_grads(inp, w, s, mix, h0, dhT)
    for n in NAMES:
        if n.startswith("dmeta") and M == 0:
            continue
        assert_close(n, g[n], ref[n], DT[dtype])
    check_dmix(g["dmix"], ref["dmix"], inp, w, s, dtype)


def check_dmix(got, ref, inp, w, s, dtype="bf16"):
    # dmix = sum(dO * o_swa): o_swa is saved in the input precision (relative
    # rounding <= 2^-8 in bf16; in fp32 its error is the forward's, held to
    # 1e-4) and the sum runs in fp32, so |error| <= u sum(|dO| |o_swa|); the
    # bound is on that scale because the sum itself may cancel
    r = f64(inp)
    o_swa, _ = oracle.window_meta_attention(r["q"], r["k"], r["v"], r["meta_k"], r["meta_v"], w, s)
    scale = float((np.abs(r["dO"]) * np.abs(o_swa)).sum())
    err = abs(float(got.item()) - ref)
    u = 2.0 ** -8 if dtype == "bf16" else 1e-4
    print(f"  dmix: {float(got.item()):.6e} vs {ref:.6e} (error {err:.2e}, bound scale {scale:.2e})")
    assert err <= u * scale


@pytest.mark.parametrize("T,w,M", [(64, 64, 4), (200, 64, 4), (257, 16, 16), (130, 1, 0),
                                   (100, 300, 2)])
def test_backward_shapes(T, w, M):
    check(2, 2, T, w, M, seed=T + w)


@pytest.mark.parametrize("T,w,M", [(64, 64, 4), (200, 128, 4), (257, 16, 16), (130, 1, 0),
                                   (300, 200, 2), (400, 65, 4)])
def test_backward_bf16_d128(T, w, M):
    # the Llama-like head size: generic GLA gradient kernels, tiled window backward
    check(2, 2, T, w, M, seed=T + w, d=128)


@pytest.mark.parametrize("T,w,M", [(64, 64, 4), (200, 64, 4), (257, 16, 16), (130, 1, 0),
                                   (100, 300, 2)])
def test_backward_fp32_d64(T, w, M):
    check(2, 2, T, w, M, seed=T + w, dtype="f32")


@pytest.mark.parametrize("T,w,M", [(64, 64, 4), (200, 128, 4), (257, 16, 16), (130, 1, 0),
                                   (300, 200, 2)])
def test_backward_fp32_d128(T, w, M):
    # fp32 at d = 128: the chunk-gradient kernel reads dO, v and dS^T from global
    # memory; the window dq kernel shares LDS between query and key tiles
    check(1, 2, T, w, M, seed=T + w, d=128, dtype="f32")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "f32"), (128, "f32")])
def test_backward_generic_gate_ranges_and_states(d, dtype):
    check(1, 2, 192, 64, 4, seed=4, gate_mean=-3.0, d=d, dtype=dtype)
    check(2, 1, 450, 64, 4, seed=5, steep_chunks=True, d=d, dtype=dtype)
    check(2, 2, 200, 64, 4, seed=11, with_h0=True, with_dhT=True, mix=0.6, d=d, dtype=dtype)


@pytest.mark.parametrize("T,d,dtype", [(4500, 64, "bf16"), (2200, 128, "bf16"), (2100, 64, "f32"),
                                       (2150, 128, "f32")])
def test_backward_several_blocks(T, d, dtype):
    # longer than one 2048-token block: the block-start states (parked in the
    # gate-gradient output) and the reverse carry between blocks, with an
    # initial state and a final-state gradient
    check(1, 2, T, 64, 4, seed=T, with_h0=True, with_dhT=True, d=d, dtype=dtype)


def test_backward_h0_and_mix():
    check(1, 3, 190, 40, 4, seed=3, mix=0.45, with_h0=True)


def test_backward_state_gradients():
    # a loss term through the final state (dhT) and the initial state's gradient
    check(2, 2, 200, 64, 4, seed=11, with_h0=True, with_dhT=True)
    check(1, 2, 130, 16, 0, seed=12, with_dhT=True, gate_mean=-3.0)
    check(1, 1, 64, 64, 4, seed=13, with_dhT=True)


def test_backward_segments_chain():
    # With w = 1 and no meta slots the window branch is token-local, so a
    # sequence trained as two segments (forward: hT of the first as h0 of the
    # second; backward: dh0 of the second as dhT of the first) has the whole
    # sequence's gradients.
    B, H, T, T1, d = 2, 2, 300, 130, 64
    print(f"[case] bwd segments B{B} H{H} T{T} split {T1}", flush=True)
    inp = make_inputs(B, H, T, d, d, 0, dtype="bf16", seed=21, with_grad_out=True)
    s = 1.0 / math.sqrt(d)
    x = to_dev(inp)
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    seg = lambda a, b: {n: (part(t, a, b) if n not in ("meta_k", "meta_v") else t)
                        for n, t in x.items()}
    x1, x2 = seg(0, T1), seg(T1, T)
    f1 = lz.hybrid_fwd(x1["q"], x1["k"], x1["v"], x1["log_alpha"], None, None, 1, scale=s,
                       save_for_backward=True, return_state=True)
    f2 = lz.hybrid_fwd(x2["q"], x2["k"], x2["v"], x2["log_alpha"], None, None, 1, scale=s,
                       h0=f1["hT"], save_for_backward=True)
    g2 = lz.hybrid_bwd(x2["q"], x2["k"], x2["v"], x2["log_alpha"], None, None, 1, f2["o_swa"],
                       f2["lse"], x2["dO"], scale=s, h0=f1["hT"], return_dh0=True)
    g1 = lz.hybrid_bwd(x1["q"], x1["k"], x1["v"], x1["log_alpha"], None, None, 1, f1["o_swa"],
                       f1["lse"], x1["dO"], scale=s, dhT=g2["dh0"], return_dh0=True)
    torch.cuda.synchronize()
    ref = ref_grads(inp, 1, s, 1.0)
    for n in ("dq", "dk", "dv", "dlog_alpha"):
        assert_close(n, torch.cat([g1[n], g2[n]], dim=2), ref[n], BF)
    assert_close("dh0", g1["dh0"], ref["dh0"], BF)


def test_backward_extreme_gates():
    check(1, 2, 192, 64, 4, seed=4, gate_mean=-3.0)


def test_backward_mixed_gate_ranges():
    check(2, 2, 450, 64, 4, seed=5, steep_chunks=True)
    check(1, 2, 320, 100, 4, seed=6, gate_mean=0.3, with_h0=True)


def test_backward_deterministic():
    inp = make_inputs(2, 2, 300, 64, 64, 4, dtype="bf16", seed=9, with_grad_out=True)
    a = run_grads(inp, 64, 0.125, 1.0)
    b = run_grads(inp, 64, 0.125, 1.0)
    for n in NAMES + ("hT", "dmix"):
        assert torch.equal(a[n], b[n]), n


def test_full_size_training_sampled_heads():
    wl = WORKLOADS["train_bf16_b8_h16_t2048_d64"]
    print("[case] train_bf16_b8_h16_t2048_d64 heads 0, 15", flush=True)
    inp = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.n_meta, dtype=wl.dtype, seed=0,
                      with_grad_out=True)
    g = run_grads(inp, wl.window, wl.scale, wl.mix)
    for h in (0, 15):
        sl = {n: (t[:, h:h + 1] if n not in ("meta_k", "meta_v") else t[h:h + 1])
              for n, t in inp.items()}
        ref = ref_grads(sl, wl.window, wl.scale, wl.mix)
        for n in NAMES:
            got = g[n][h:h + 1] if n.startswith("dmeta") else g[n][:, h:h + 1]
            assert_close(f"{n}[h{h}]", got, ref[n], BF)
