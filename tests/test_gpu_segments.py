"""Segment-wise runs of one sequence against the fp64 oracle on the whole
sequence, through the C ABI (lizard_hybrid_fwd_segment / _bwd_segment).

A sequence is cut into segments run one after another: the gated branch is
chained through its state (hT -> h0 forward, dh0 -> dhT backward) and the window
branch gets each segment's halo, the window keys and values of the min(w-1,
tokens before) tokens before it; the backward passes each segment's halo
gradient to the segment before as its tail gradient.  Every output and
gradient must equal the unsplit oracle's (meta and mix gradients summed over
segments).  Cases: three segments with windows crossing both cuts, a halo
shorter than w-1, d = 128, fp32, separate window queries and keys, gate logits,
and a 32768-token sequence in eight segments (sampled head).  A segmented
prefill then continues into decoding: lizard_window_cache_fill builds the
decode window cache from the last segment and its halo (bit for bit the
oracle's cache after the whole prefill) and decode steps follow the oracle.
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


def run_segments(inp, cuts, w, s, mix, sep=False, logits=False):
    """GPU forward and backward of inp cut at the given token positions."""
    x = to_dev(inp)
    T = x["q"].shape[2]
    bounds = [0] + list(cuts) + [T]
    gate = x["gate_x"] if logits else x["log_alpha"]
    kw_full = x["k_w"] if sep else x["k"]
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    segs, h = [], None
    for a, b in zip(bounds[:-1], bounds[1:]):
        L = min(w - 1, a)
        halo = dict(halo_k=part(kw_full, a - L, a), halo_v=part(x["v"], a - L, a)) if L else {}
        extra = dict(q_w=part(x["q_w"], a, b), k_w=part(x["k_w"], a, b)) if sep else {}
        f = lz.hybrid_fwd(part(x["q"], a, b), part(x["k"], a, b), part(x["v"], a, b),
                          part(gate, a, b), x["meta_k"], x["meta_v"], w, scale=s, mix=mix, h0=h,
                          save_for_backward=True, return_state=True, **extra, **halo)
        segs.append(dict(a=a, b=b, f=f, halo=halo, extra=extra, h0=h))
        h = f["hT"]
    grads, dhT, tail = [None] * len(segs), None, {}
    for i in range(len(segs) - 1, -1, -1):
        sg = segs[i]
        a, b = sg["a"], sg["b"]
        g = lz.hybrid_bwd(part(x["q"], a, b), part(x["k"], a, b), part(x["v"], a, b),
                          part(gate, a, b), x["meta_k"], x["meta_v"], w, sg["f"]["o_swa"],
                          sg["f"]["lse"], part(x["dO"], a, b), scale=s, mix=mix, h0=sg["h0"],
                          dhT=dhT, return_dh0=True, return_dmix=True, return_dhalo=True,
                          **sg["extra"], **sg["halo"], **tail)
        grads[i] = g
        dhT = g["dh0"]
        # the segment before must hold the whole halo of this one
        if "dhalo_k" in g:
            assert g["dhalo_k"].shape[2] <= segs[i - 1]["b"] - segs[i - 1]["a"]
        tail = dict(tail_dk=g["dhalo_k"], tail_dv=g["dhalo_v"]) if "dhalo_k" in g else {}
    torch.cuda.synchronize()
    out = {n: torch.cat([sg["f"][n] for sg in segs], dim=2) for n in ("o", "o_swa", "lse")}
    out["hT"] = segs[-1]["f"]["hT"]
    names = ["dq", "dk", "dv", "dlog_alpha"] + (["dq_w", "dk_w"] if sep else [])
    for n in names:
        out[n] = torch.cat([g[n] for g in grads], dim=2)
    for n in ("dmeta_k", "dmeta_v", "dmix"):
        out[n] = sum(g[n] for g in grads)
    out["dh0"] = grads[0]["dh0"]
    return out


def reference(inp, w, s, mix, sep=False, logits=False):
    r = f64(inp)
    la = oracle.log_sigmoid(r["gate_x"]) if logits else r["log_alpha"]
    extra = dict(q_w=r["q_w"], k_w=r["k_w"]) if sep else {}
    fwd = oracle.hybrid_forward(r["q"], r["k"], r["v"], la, r["meta_k"], r["meta_v"], w, s,
                                mix=mix, **extra)
    bwd = oracle.hybrid_backward(r["q"], r["k"], r["v"], la, r["meta_k"], r["meta_v"], w, s,
                                 r["dO"], mix=mix, **extra)
    if logits:
        bwd["dlog_alpha"] = oracle.log_sigmoid_backward(r["gate_x"], bwd["dlog_alpha"])
    return fwd, bwd


def check(B, H, T, cuts, d, w, M, dtype="bf16", mix=1.0, sep=False, logits=False, seed=0,
          heads=None):
    print(f"[case] segments B{B} H{H} T{T} cuts {cuts} d{d} w{w} M{M} {dtype} sep{sep} "
          f"logits{logits}", flush=True)
    inp = make_inputs(B, H, T, d, d, M, dtype=dtype, seed=seed, with_grad_out=True,
                      with_window_qk=sep, with_gate_logits=logits)
    s = 1.0 / math.sqrt(d)
    got = run_segments(inp, cuts, w, s, mix, sep, logits)
    dt = DT[dtype]
    dmix_ref, dmix_scale = 0.0, 0.0
    for h in (range(H) if heads is None else heads):
        sl = {n: (t[h:h + 1] if n in ("meta_k", "meta_v") else t[:, h:h + 1]) for n, t in inp.items()}
        fwd, bwd = reference(sl, w, s, mix, sep, logits)
        hs = lambda t: t[:, h:h + 1]
        for n in ("o", "o_swa", "hT"):
            assert_close(f"{n}[h{h}]", hs(got[n]), fwd[n], dt)
        assert_close(f"lse[h{h}]", hs(got["lse"]), fwd["lse"], dt, tol=1e-4)
        for n in ["dq", "dk", "dv", "dlog_alpha", "dh0"] + (["dq_w", "dk_w"] if sep else []):
            assert_close(f"{n}[h{h}]", hs(got[n]), bwd[n], dt)
        if M > 0:  # every batch row of head h is in the slice, so its sums are complete
            for n in ("dmeta_k", "dmeta_v"):
                assert_close(f"{n}[h{h}]", got[n][h:h + 1], bwd[n], dt)
        r = f64(sl)
        dmix_ref += bwd["dmix"]
        dmix_scale += float((np.abs(r["dO"]) * np.abs(fwd["o_swa"])).sum())
    if heads is None:
        # dmix = sum(dO * o_swa) over everything, summed over segments
        u = 2.0 ** -8 if dtype == "bf16" else 1e-4
        err = abs(float(got["dmix"].item()) - dmix_ref)
        print(f"  dmix error {err:.2e} (bound {u * dmix_scale:.2e})", flush=True)
        assert err <= u * dmix_scale


@pytest.mark.parametrize("T,cuts,w,M", [(600, (200, 400), 64, 4), (600, (130, 470), 100, 2),
                                        (300, (250,), 64, 0)])
def test_three_and_two_segments_bf16(T, cuts, w, M):
    # windows reach across every cut (halo of w - 1 tokens); a last segment
    # shorter than the window (50 tokens, w = 64)
    check(2, 2, T, cuts, 64, w, M, seed=T + w)


def test_short_first_segment():
    # the first cut at 40 < w - 1: the second segment's halo is the 40 tokens
    # before it (a halo shorter than w - 1)
    check(1, 2, 300, (40, 200), 64, 64, 4, seed=3)


def test_segments_d128_and_fp32():
    check(1, 2, 700, (300,), 128, 128, 4, seed=5)
    check(1, 2, 300, (100, 200), 64, 40, 2, dtype="f32", seed=6)
    check(1, 1, 400, (150, 260), 128, 100, 3, dtype="f32", seed=10)


def test_segments_window_inputs_and_gate_logits():
    check(2, 1, 500, (180, 330), 64, 64, 4, sep=True, mix=0.7, seed=7)
    check(1, 2, 400, (150,), 64, 100, 3, logits=True, seed=8)


def test_long_sequence_eight_segments():
    # 32768 tokens in eight segments of 4096 (each backward itself walks two
    # 2048-token blocks), one sampled head against the oracle on the whole
    # sequence
    T = 32768
    check(1, 2, T, tuple(range(4096, T, 4096)), 64, 64, 4, seed=9, heads=[1])


@pytest.mark.parametrize("T,w,cuts,dtype", [
    (600, 64, [300], "bf16"),   # last segment longer than the window
    (300, 128, [250], "bf16"),  # last segment shorter: the cache reaches into the halo
    (40, 64, [25], "f32"),      # sequence shorter than the window: zero slots
    (200, 64, [], "bf16"),      # one segment from position 0: the prefill's own cache
])
def test_window_cache_after_segments_continues_decoding(T, w, cuts, dtype):
    """A prefill run in segments, then lizard_window_cache_fill on the last one,
    then decode steps: the cache equals the oracle's after the whole prefill
    (bit for bit: a copy) and the decode outputs follow the unsplit oracle."""
    B, H, d, M = 2, 2, 64, 4
    print(f"[case] window cache after segments T{T} w{w} cuts{cuts} {dtype}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.8
    dt = DT[dtype]
    inp = make_inputs(B, H, T, d, d, M, dtype=dtype, seed=T + w, with_h0=True)
    x = to_dev(inp)
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    bounds = [0] + list(cuts) + [T]
    h = x["h0"]
    for a, b in zip(bounds[:-1], bounds[1:]):
        L = min(w - 1, a)
        halo = dict(halo_k=part(x["k"], a - L, a), halo_v=part(x["v"], a - L, a)) if L else {}
        f = lz.hybrid_fwd(part(x["q"], a, b), part(x["k"], a, b), part(x["v"], a, b),
                          part(x["log_alpha"], a, b), x["meta_k"], x["meta_v"], w, scale=s,
                          mix=mix, h0=h, return_state=True, return_ring=not L, **halo)
        h = f["hT"]
    rk, rv = lz.window_cache_fill(part(x["k"], a, T), part(x["v"], a, T), w, a, **halo)
    torch.cuda.synchronize()
    r = f64(inp)
    ref = oracle.hybrid_forward(r["q"], r["k"], r["v"], r["log_alpha"], r["meta_k"], r["meta_v"],
                                w, s, mix=mix, h0=r["h0"])
    assert_close("ring_k", rk, ref["ring_k"], dt, tol=0.0)
    assert_close("ring_v", rv, ref["ring_v"], dt, tol=0.0)
    if not cuts:  # the same cache as the prefill call itself returned
        assert torch.equal(rk, f["ring_k"]) and torch.equal(rv, f["ring_v"])
    assert_close("hT", h, ref["hT"], dt)
    # an empty last segment: all w cache tokens come from its halo
    L = min(w, T)
    rk0, rv0 = lz.window_cache_fill(part(x["k"], T, T), part(x["v"], T, T), w, T,
                                    halo_k=part(x["k"], T - L, T), halo_v=part(x["v"], T - L, T))
    torch.cuda.synchronize()
    assert torch.equal(rk0, rk) and torch.equal(rv0, rv)
    # decoding continues from the segmented prefill
    dec = make_decode_inputs(3, B, H, d, d, dtype=dtype, seed=T + 1)
    rd = f64(dec)
    state = h.clone()
    pos = torch.full((B,), T, dtype=torch.int64, device="cuda")
    st_ref, rk_ref, rv_ref, pos_ref = ref["hT"], ref["ring_k"], ref["ring_v"], np.full(B, T)
    for i in range(3):
        o = lz.decode_step(dec["q"][i].cuda(), dec["k"][i].cuda(), dec["v"][i].cuda(),
                           dec["log_alpha"][i].cuda(), state, rk, rv, pos, x["meta_k"],
                           x["meta_v"], scale=s, mix=mix)
        torch.cuda.synchronize()
        o_ref, st_ref, rk_ref, rv_ref, pos_ref = oracle.decode_step(
            rd["q"][i], rd["k"][i], rd["v"][i], rd["log_alpha"][i], st_ref, rk_ref, rv_ref,
            pos_ref, r["meta_k"], r["meta_v"], w, s, mix=mix)
        assert_close(f"decode[{i}].o", o, o_ref, dt)
    assert_close("decode.ring_k", rk, rk_ref, dt, tol=0.0)
    assert_close("decode.state", state, st_ref, dt)
