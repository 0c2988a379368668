"""GPU parity with gates that all but reset the state at every token.

A log2 gate below -15 per token (alpha < 3.1e-5) would push the 16-token
sub-block factors past the bf16/fp32 exponent range; the kernels hold the
gate at 2^-15 there.  Two references: the fp64 oracle fed the same floor (the
kernels' semantics: every output at the usual bars), and the exact oracle
(no floor), from which the floor moves the outputs by at most 2^-15 of the
older state's share (o, dq, dk, dv at the usual normwise bars).  The gate
gradient is alpha-small for such tokens and comes from products that cancel,
so it is held to an absolute bound on the scale of those products (|q| |dq|);
the initial-state gradient, which every token's floored gate scales down,
to one on |dh0| itself.  Cases: uniformly extreme gates (log alpha about -14,
-30, -90), half the channels extreme and half moderate, bf16 logits of -40,
at d = 64 and 128, bf16 and fp32; and packed (variable-length) batches with
gates far below the floor, each sequence against the oracle run on it alone.
"""
import math

import numpy as np
import pytest
import torch

import gated_linear_attention_chunked_amd as lz
import oracle
from tests._gpu_helpers import assert_close, f64, rel_err, to_dev
from workloads import make_decode_inputs, make_inputs, make_packed_inputs

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}
FLOOR = -15.0 * math.log(2.0)  # log alpha = -15 ln 2, alpha = 2^-15


@pytest.mark.parametrize("d,dtype,gate_mean,mixed,logits", [
    (64, "bf16", -30.0, False, False),
    (128, "bf16", -90.0, False, False),
    (64, "bf16", -14.0, True, False),     # half the channels moderate
    (128, "bf16", -40.0, False, True),    # bf16 logits
    (64, "f32", -30.0, True, False),
    (128, "f32", -14.0, False, False),
])
def test_extreme_gates(d, dtype, gate_mean, mixed, logits):
    B, H, T, w, M = 2, 2, 300, 64, 4
    print(f"[case] extreme gates d{d} {dtype} gate{gate_mean} mixed{mixed} logits{logits}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.8
    inp = make_inputs(B, H, T, d, d, M, dtype=dtype, seed=d + int(-gate_mean), gate_mean=gate_mean,
                      with_grad_out=True, with_h0=True, with_gate_logits=logits)
    if mixed:
        # channels d/2.. take moderate gates (log alpha about -0.13)
        la = inp["log_alpha"].clone()
        la[..., d // 2:] = torch.nn.functional.logsigmoid(
            torch.randn(B, H, T, d - d // 2, generator=torch.Generator().manual_seed(5)) + 2.0)
        inp["log_alpha"] = la
    if logits:
        inp.pop("log_alpha")
    gname = "gate_x" if logits else "log_alpha"
    x = to_dev(inp)
    args = (x["q"], x["k"], x["v"], x[gname], x["meta_k"], x["meta_v"], w)
    f = lz.hybrid_fwd(*args, scale=s, mix=mix, h0=x["h0"], save_for_backward=True,
                      return_state=True, return_ring=True)
    g = lz.hybrid_bwd(*args, f["o_swa"], f["lse"], x["dO"], scale=s, mix=mix, h0=x["h0"],
                      return_dh0=True)
    o_gla, hT_gla = lz.gla_fwd(x["q"], x["k"], x["v"], x[gname], h0=x["h0"], return_state=True)
    torch.cuda.synchronize()
    r = f64(inp)
    la_exact = oracle.log_sigmoid(r["gate_x"]) if logits else r["log_alpha"]
    la = np.maximum(la_exact, FLOOR)  # the kernels' floor on log alpha
    dt = DT[dtype]
    bar = 2e-2 if dtype == "bf16" else 1e-4
    ref = oracle.hybrid_forward(r["q"], r["k"], r["v"], la, r["meta_k"], r["meta_v"], w, s,
                                mix=mix, h0=r["h0"])
    exact = oracle.hybrid_forward(r["q"], r["k"], r["v"], la_exact, r["meta_k"], r["meta_v"], w,
                                  s, mix=mix, h0=r["h0"])
    for n in ("o", "hT", "o_swa"):
        assert torch.isfinite(f[n]).all(), n
        assert_close(n, f[n], ref[n], dt)
    e = rel_err(f["o"], exact["o"])
    print(f"  o against the exact oracle: {e:.2e}", flush=True)
    assert e <= bar
    # The GLA-only entry point and the backward's chunk gradients gate
    # 64-token chunks from a running log2 sum that reaches 15 x 64 = 960 at the
    # floor, which fp32 holds to 2^-14: each decay factor then carries up to
    # about 1e-4 relative error (against 1e-7 at ordinary gates), seen
    # elementwise where outputs cancel.  Their fp32 elementwise bar here is
    # 1e-2 (normwise bars unchanged).
    gbar = 1e-2 if dtype == "f32" else None
    assert_close("gla.o", o_gla, ref["o_gla"], dt, pbar=gbar)
    assert_close("gla.hT", hT_gla, ref["hT"], dt, pbar=gbar)
    gr = oracle.hybrid_backward(r["q"], r["k"], r["v"], la, r["meta_k"], r["meta_v"], w, s,
                                r["dO"], mix=mix, h0=r["h0"])
    gx = oracle.hybrid_backward(r["q"], r["k"], r["v"], la_exact, r["meta_k"], r["meta_v"], w, s,
                                r["dO"], mix=mix, h0=r["h0"])
    for n in ("dq", "dk", "dv", "dmeta_k", "dmeta_v"):
        assert torch.isfinite(g[n]).all(), n
        assert_close(n, g[n], gr[n], dt, pbar=gbar if n in ("dq", "dk", "dv") else None)
    for n in ("dq", "dk", "dv"):
        e = rel_err(g[n], gx[n])
        print(f"  {n} against the exact oracle: {e:.2e}", flush=True)
        assert e <= bar
    d0 = g["dh0"].cpu().double().numpy()
    assert np.isfinite(d0).all()
    e0 = np.abs(d0 - gr["dh0"]).max()
    print(f"  dh0: max |error| {e0:.2e} (max |ref| {np.abs(gr['dh0']).max():.2e})", flush=True)
    assert e0 <= bar * max(np.abs(gr["dh0"]).max(), 1e-30) or e0 < 1e-30
    dgate = oracle.log_sigmoid_backward(r["gate_x"], gr["dlog_alpha"]) if logits else gr["dlog_alpha"]
    got = g["dlog_alpha"].cpu().double().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - dgate).max()
    scale = np.abs(r["q"]).max() * np.abs(gr["dq"]).max()
    u = 2.0 ** -8 if dtype == "bf16" else 1e-4
    print(f"  d gate: max |error| {err:.2e}, bound {u * scale:.2e} (max |ref| {np.abs(dgate).max():.2e})",
          flush=True)
    assert err <= u * scale

    # decode continues from the prefill with the same gate floor
    n = 4
    dec = make_decode_inputs(n, B, H, d, d, dtype=dtype, seed=d + 3, gate_mean=gate_mean,
                             with_gate_logits=logits)
    dname = "gate_x" if logits else "log_alpha"
    state, rk, rv = f["hT"].clone(), f["ring_k"].clone(), f["ring_v"].clone()
    pos = torch.full((B,), T, dtype=torch.int64, device="cuda")
    st_ref, rk_ref, rv_ref = ref["hT"], ref["ring_k"], ref["ring_v"]
    pos_ref = np.full(B, T)
    for i in range(n):
        o = lz.decode_step(dec["q"][i].cuda(), dec["k"][i].cuda(), dec["v"][i].cuda(),
                           dec[dname][i].cuda(), state, rk, rv, pos, x["meta_k"], x["meta_v"],
                           scale=s, mix=mix)
        torch.cuda.synchronize()
        dla = np.maximum(oracle.log_sigmoid(f64(dec)["gate_x"][i]) if logits
                         else f64(dec)["log_alpha"][i], FLOOR)
        o_ref, st_ref, rk_ref, rv_ref, pos_ref = oracle.decode_step(
            f64(dec)["q"][i], f64(dec)["k"][i], f64(dec)["v"][i], dla, st_ref, rk_ref, rv_ref,
            pos_ref, r["meta_k"], r["meta_v"], w, s, mix=mix)
        assert torch.isfinite(o).all()
        assert_close(f"decode[{i}].o", o, o_ref, dt)
    assert_close("decode.state", state, st_ref, dt)


@pytest.mark.parametrize("d,w,logits", [
    (128, 128, False),   # single-pass kernel
    (64, 64, True),      # d = 64 packed batches: GLA output pass + window kernel
])
def test_extreme_gates_packed(d, w, logits):
    """Packed (variable-length) prefill with gates far below the floor: every
    sequence against the oracle run on it alone with the same floor."""
    lengths = [0, 1, 33, 300, 1100, 70]
    print(f"[case] extreme gates packed d{d} w{w} logits{logits}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.8
    inp = make_packed_inputs(lengths, 2, d, d, 4, seed=d + 17, gate_mean=-30.0, with_h0=True,
                             with_gate_logits=logits)
    x = to_dev(inp)
    out = lz.hybrid_fwd_varlen(x["q"], x["k"], x["v"], x["gate_x"] if logits else x["log_alpha"],
                               x["meta_k"], x["meta_v"], w, x["cu_seqlens"], max(lengths), scale=s,
                               mix=mix, h0=x["h0"], return_state=True, return_ring=True)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    for b in range(len(lengths)):
        sl = lambda t: f64({"t": t[:, cu[b]:cu[b + 1]]})["t"][None]
        la = oracle.log_sigmoid(sl(inp["gate_x"])) if logits else sl(inp["log_alpha"])
        ref = oracle.hybrid_forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), np.maximum(la, FLOOR),
                                    f64(inp)["meta_k"], f64(inp)["meta_v"], w, s, mix=mix,
                                    h0=f64(inp)["h0"][b:b + 1])
        if lengths[b]:
            assert torch.isfinite(out["o"][:, cu[b]:cu[b + 1]]).all()
            assert_close(f"o[seq {b}]", out["o"][:, cu[b]:cu[b + 1]][None], ref["o"], torch.bfloat16)
        assert torch.isfinite(out["hT"][b]).all()
        assert_close(f"hT[seq {b}]", out["hT"][b:b + 1], ref["hT"], torch.bfloat16)
