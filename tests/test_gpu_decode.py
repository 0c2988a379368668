"""GPU parity of the constant-memory decode step against the fp64 oracle.

Prefill (GPU hybrid forward with state and window-cache handoff) followed by
decode steps must reproduce the oracle's decode and the oracle's longer prefill;
per-sequence positions may differ, including positions below the window.
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
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def prefill_then_decode(B, H, T0, n, d, w, M, dtype, mix=1.0, heads=None, seed=0):
    print(f"[case] decode B{B} H{H} T0 {T0} n{n} d{d} w{w} M{M} {dtype}", flush=True)
    dt = DT[dtype]
    s = 1.0 / math.sqrt(d)
    inp = make_inputs(B, H, T0, d, d, M, dtype=dtype, seed=seed)
    dec = make_decode_inputs(n, B, H, d, d, dtype=dtype, seed=seed + 1)
    x = to_dev(inp)
    pre = lz.hybrid_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], w,
                        scale=s, mix=mix, return_state=True, return_ring=True)
    state, rk, rv = pre["hT"], pre["ring_k"], pre["ring_v"]
    pos = torch.full((B,), T0, dtype=torch.int64, device="cuda")
    outs = []
    for i in range(n):
        outs.append(lz.decode_step(dec["q"][i].cuda(), dec["k"][i].cuda(), dec["v"][i].cuda(),
                                   dec["log_alpha"][i].cuda(), state, rk, rv, pos, x["meta_k"],
                                   x["meta_v"], scale=s, mix=mix))
    torch.cuda.synchronize()
    assert torch.all(pos.cpu() == T0 + n)
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    for b, h in heads:
        sl = lambda t: t[b:b + 1, h:h + 1]
        r = f64({n_: sl(t) for n_, t in inp.items() if n_ not in ("meta_k", "meta_v")})
        mk = f64({"m": inp["meta_k"][h:h + 1]})["m"]
        mv = f64({"m": inp["meta_v"][h:h + 1]})["m"]
        dq = f64({n_: t[:, b:b + 1, h:h + 1] for n_, t in dec.items()})
        # the longer prefill over prompt + decoded tokens gives the same outputs
        full = {n_: np.concatenate([r[n_], np.moveaxis(dq[n_], 0, 2)], axis=2)
                for n_ in ("q", "k", "v", "log_alpha")}
        ref = oracle.hybrid_forward(full["q"], full["k"], full["v"], full["log_alpha"], mk, mv,
                                    w, s, mix=mix)
        got = torch.stack([o[b:b + 1, h:h + 1] for o in outs], dim=2)
        assert_close(f"decode o[b{b},h{h}]", got, ref["o"][:, :, T0:], dt)
        assert_close(f"state[b{b},h{h}]", sl(state), ref["hT"], dt)
        assert_close(f"ring_k[b{b},h{h}]", sl(rk), ref["ring_k"], dt, tol=0.0)
        assert_close(f"ring_v[b{b},h{h}]", sl(rv), ref["ring_v"], dt, tol=0.0)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_decode_matches_longer_prefill(dtype, d):
    prefill_then_decode(2, 2, 40, 20, d, 16, 4, dtype, mix=0.8)


def test_decode_from_short_history_and_no_meta():
    prefill_then_decode(1, 2, 3, 12, 64, 8, 0, "f32")
    prefill_then_decode(1, 2, 0, 5, 64, 8, 2, "bf16")


def test_decode_ragged_positions():
    # sequences at different positions in one call
    B, H, d, w, M = 3, 2, 64, 8, 2
    s = 1.0 / math.sqrt(d)
    rng = torch.Generator().manual_seed(7)
    state = torch.randn(B, H, d, d, generator=rng) * 0.1
    rk = (torch.randn(B, H, w, d, generator=rng) / 8).float()
    rv = (torch.randn(B, H, w, d, generator=rng) / 8).float()
    mk = torch.randn(H, M, d, generator=rng)
    mv = torch.randn(H, M, d, generator=rng)
    pos = torch.tensor([0, 5, 100], dtype=torch.int64)
    dec = make_decode_inputs(1, B, H, d, d, dtype="f32", seed=3)
    ref = oracle.decode_step(*(dec[n][0].double().numpy() for n in ("q", "k", "v", "log_alpha")),
                             state.double().numpy(), rk.double().numpy(), rv.double().numpy(),
                             pos.numpy(), mk.double().numpy(), mv.double().numpy(), w, s)
    g = [t.cuda() for t in (state, rk, rv, pos)]
    o = lz.decode_step(*(dec[n][0].cuda() for n in ("q", "k", "v", "log_alpha")), *g,
                       mk.cuda(), mv.cuda(), scale=s)
    torch.cuda.synchronize()
    assert_close("o", o, ref[0], torch.float32)
    assert_close("state", g[0], ref[1], torch.float32)
    assert_close("ring_k", g[1], ref[2], torch.float32, tol=0.0)
    assert torch.equal(g[3].cpu(), torch.tensor([1, 6, 101]))


def test_full_size_decode_workload_sampled_heads():
    # the decode workload as defined: B=64 H=32 d=128 w=128 M=4, a 2048-token
    # prefill, then all 1024 sequential steps; two sampled heads are compared
    # with the oracle's 3072-token prefill (every step's output, the final state
    # and the window cache), so state drift and ring wrap-around over the whole
    # run are covered
    wl = WORKLOADS["decode_bf16_b64_h32_d128"]
    prefill_then_decode(wl.B, wl.H, wl.T, wl.steps, wl.dk, wl.window, wl.n_meta, wl.dtype,
                        heads=[(0, 0), (63, 31)])


def test_decode_position_advance_many_heads():
    # the position counter advances once per call however many heads a sequence
    # has; a negative position decodes as 0 and still advances by one
    B, H, d, w, M = 3, 32, 64, 8, 2
    rng = torch.Generator().manual_seed(11)
    state = torch.randn(B, H, d, d, generator=rng) * 0.1
    rk = torch.randn(B, H, w, d, generator=rng) / 8
    rv = torch.randn(B, H, w, d, generator=rng) / 8
    mk, mv = torch.randn(H, M, d, generator=rng), torch.randn(H, M, d, generator=rng)
    dec = make_decode_inputs(1, B, H, d, d, dtype="f32", seed=5)
    x = [dec[n][0].cuda() for n in ("q", "k", "v", "log_alpha")]
    outs = []
    for p0 in ([-3, 7, 1000], [0, 7, 1000]):
        g = [t.clone().cuda() for t in (state, rk, rv)]
        pos = torch.tensor(p0, dtype=torch.int64, device="cuda")
        o = lz.decode_step(*x, *g, pos, mk.cuda(), mv.cuda())
        torch.cuda.synchronize()
        assert torch.equal(pos.cpu(), torch.tensor(p0) + 1)
        outs.append([o] + [t.clone() for t in g])
        lz.decode_step(*x, *g, pos, mk.cuda(), mv.cuda())
        torch.cuda.synchronize()
        assert torch.equal(pos.cpu(), torch.tensor(p0) + 2)
    for a, b in zip(*outs):  # one step from position -3 is one step from 0
        assert torch.equal(a, b)
