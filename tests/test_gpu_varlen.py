"""GPU parity of the packed-batch (variable-length) hybrid forward against the
fp64 oracle run on every sequence alone.

Each sequence's o rows, final state and window cache must match the oracle's
single-sequence forward (its own h0, no window reaching into a neighbour).
Cases: lengths 0, 1, chunk-aligned and ragged, several state segments, a bound
max_seqlen larger than every length, d = 64 and windows past 129 (the
two-kernel path, with the streaming and the tiled window kernels), fp32, an
initial state per sequence, gate logits and separate window inputs, decode continuing
every sequence from its own position, and the serving-mix workload (16
sequences of 64..8192 tokens, H=32, d=128) on sampled sequences and heads.
"""
import math

import numpy as np
import pytest
import torch

import gated_linear_attention_chunked_amd as lz
import oracle
from tests._gpu_helpers import assert_close, to_dev
from workloads import make_decode_inputs, make_packed_inputs, packed_lengths, to_f64_numpy

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
D = 128


def seq_ref(inp, b, w, s, mix, heads=None, sep=False, logits=False):
    """Oracle forward of sequence b alone (heads: a subset of heads, or all)."""
    cu = inp["cu_seqlens"].tolist()
    hs = list(range(inp["q"].shape[0])) if heads is None else heads
    sl = lambda t: to_f64_numpy(t[hs, cu[b]:cu[b + 1]])[None]
    la = oracle.log_sigmoid(sl(inp["gate_x"])) if logits else sl(inp["log_alpha"])
    h0 = to_f64_numpy(inp["h0"][b:b + 1, hs]) if "h0" in inp else None
    return oracle.hybrid_forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), la,
                                 to_f64_numpy(inp["meta_k"][hs]), to_f64_numpy(inp["meta_v"][hs]),
                                 w, s, mix=mix, h0=h0,
                                 q_w=sl(inp["q_w"]) if sep else None,
                                 k_w=sl(inp["k_w"]) if sep else None)


def run(inp, w, s, mix, max_seqlen, sep=False, logits=False):
    x = to_dev(inp)
    out = lz.hybrid_fwd_varlen(x["q"], x["k"], x["v"], x["gate_x"] if logits else x["log_alpha"],
                               x["meta_k"], x["meta_v"], w, x["cu_seqlens"], max_seqlen, scale=s,
                               mix=mix, h0=x.get("h0"), return_state=True, return_ring=True,
                               q_w=x.get("q_w") if sep else None, k_w=x.get("k_w") if sep else None)
    torch.cuda.synchronize()
    return out


def check_all(inp, out, w, s, mix, sep=False, logits=False, seqs=None, heads=None, dt=BF):
    cu = inp["cu_seqlens"].tolist()
    hs = list(range(inp["q"].shape[0])) if heads is None else heads
    for b in (range(len(cu) - 1) if seqs is None else seqs):
        ref = seq_ref(inp, b, w, s, mix, heads, sep, logits)
        L = cu[b + 1] - cu[b]
        if L:
            assert_close(f"o[seq {b}, len {L}]", out["o"][hs, cu[b]:cu[b + 1]][None], ref["o"], dt)
        assert_close(f"hT[seq {b}]", out["hT"][b:b + 1, hs], ref["hT"], dt)
        assert_close(f"ring_k[seq {b}]", out["ring_k"][b:b + 1, hs], ref["ring_k"], dt, tol=0.0)
        assert_close(f"ring_v[seq {b}]", out["ring_v"][b:b + 1, hs], ref["ring_v"], dt, tol=0.0)


@pytest.mark.parametrize("lengths,d,w,M,bound", [
    ([0, 1, 31, 32, 33, 300, 2100, 129], 128, 128, 4, 0),  # single-pass kernel
    ([700, 64, 0, 1500], 128, 64, 0, 4096),                 # max_seqlen above every length
    ([5000], 128, 129, 16, 0),                              # one long sequence
    ([0, 1, 65, 300, 1300, 64], 64, 64, 4, 0),              # d = 64: two-kernel path
    ([257, 0, 900, 3], 64, 200, 2, 1000),                   # tiled window (w > 129)
    ([129, 640, 0, 77], 128, 300, 4, 0),
])
def test_packed_forward_matches_each_sequence(lengths, d, w, M, bound):
    print(f"[case] varlen lengths {lengths} d{d} w{w} M{M} bound{bound}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.85
    inp = make_packed_inputs(lengths, 2, d, d, M, seed=sum(lengths) % 97, with_h0=True)
    out = run(inp, w, s, mix, max(max(lengths), bound, 1))
    check_all(inp, out, w, s, mix)


@pytest.mark.parametrize("lengths,d,w,M", [
    ([0, 1, 65, 300, 1300, 64], 64, 64, 4),   # streaming window kernel
    ([257, 0, 900, 3], 128, 128, 2),           # d = 128: tiled window kernel
    ([700, 64, 1500], 64, 200, 0),             # tiled window, several state segments
])
def test_packed_forward_fp32(lengths, d, w, M):
    print(f"[case] varlen fp32 lengths {lengths} d{d} w{w} M{M}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.75
    inp = make_packed_inputs(lengths, 2, d, d, M, dtype="f32", seed=len(lengths) + d,
                             with_h0=True)
    out = run(inp, w, s, mix, max(lengths))
    check_all(inp, out, w, s, mix, dt=torch.float32)


@pytest.mark.parametrize("d,w", [(128, 100), (64, 64), (64, 180)])
def test_packed_forward_gate_logits_and_window_inputs(d, w):
    lengths = [257, 0, 1100, 40]
    print(f"[case] varlen logits + window inputs {lengths} d{d} w{w}", flush=True)
    s, mix = 1.0 / math.sqrt(d), 0.7
    inp = make_packed_inputs(lengths, 2, d, d, 4, seed=3, gate_mean=-1.0, with_h0=True,
                             with_window_qk=True, with_gate_logits=True)
    out = run(inp, w, s, mix, max(lengths), sep=True, logits=True)
    check_all(inp, out, w, s, mix, sep=True, logits=True)


def test_decode_continues_each_packed_sequence():
    lengths, n, w, M, H = [90, 0, 333, 1], 20, 64, 4, 2
    print(f"[case] varlen prefill + decode {lengths} n{n}", flush=True)
    s, mix = 1.0 / math.sqrt(D), 0.9
    inp = make_packed_inputs(lengths, H, D, D, M, seed=11)
    dec = make_decode_inputs(n, len(lengths), H, D, D, seed=12)
    x = to_dev(inp)
    pre = run(inp, w, s, mix, max(lengths))
    state, rk, rv = pre["hT"], pre["ring_k"], pre["ring_v"]
    pos = torch.tensor(lengths, dtype=torch.int64, device="cuda")
    outs = []
    for i in range(n):
        outs.append(lz.decode_step(dec["q"][i].cuda(), dec["k"][i].cuda(), dec["v"][i].cuda(),
                                   dec["log_alpha"][i].cuda(), state, rk, rv, pos, x["meta_k"],
                                   x["meta_v"], scale=s, mix=mix))
    torch.cuda.synchronize()
    assert pos.cpu().tolist() == [L + n for L in lengths]
    cu = inp["cu_seqlens"].tolist()
    for b, L in enumerate(lengths):
        sl = lambda t: to_f64_numpy(t[:, cu[b]:cu[b + 1]])[None]
        dq = {n_: to_f64_numpy(t[:, b:b + 1]) for n_, t in dec.items()}  # [n, 1, H, d]
        full = {n_: np.concatenate([sl(inp[n_]), np.moveaxis(dq[n_], 0, 2)], axis=2)
                for n_ in ("q", "k", "v", "log_alpha")}
        ref = oracle.hybrid_forward(full["q"], full["k"], full["v"], full["log_alpha"],
                                    to_f64_numpy(inp["meta_k"]), to_f64_numpy(inp["meta_v"]), w, s,
                                    mix=mix)
        got = torch.stack([o[b:b + 1] for o in outs], dim=2)
        assert_close(f"decode o[seq {b}]", got, ref["o"][:, :, L:], BF)
        assert_close(f"state[seq {b}]", state[b:b + 1], ref["hT"], BF)


def test_serving_mix_workload_sampled():
    lengths = packed_lengths(16, 64, 8192, seed=0)
    print(f"[case] serving mix H32 d128 lengths {lengths}", flush=True)
    s = 1.0 / math.sqrt(D)
    inp = make_packed_inputs(lengths, 32, D, D, 4, seed=0)
    out = run(inp, 128, s, 1.0, max(lengths))
    longest = int(np.argmax(lengths))
    check_all(inp, out, 128, s, 1.0, seqs=[0, longest, 15], heads=[0, 17, 31])


def test_binding_rejects_bad_lengths_and_out_buffers():
    # a sequence longer than max_seqlen, and cu_seqlens that do not end at N, are
    # refused before anything is enqueued; without max_seqlen the bound is taken
    # from cu_seqlens
    inp = make_packed_inputs([100, 300], 2, 64, 64, 2, dtype="bf16", seed=1)
    x = to_dev(inp)
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], 64)
    with pytest.raises(ValueError, match="max_seqlen"):
        lz.hybrid_fwd_varlen(*args, x["cu_seqlens"], 200)
    bad = torch.tensor([0, 100, 399], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="cu_seqlens"):
        lz.hybrid_fwd_varlen(*args, bad, 300)
    a = lz.hybrid_fwd_varlen(*args, x["cu_seqlens"])
    b = lz.hybrid_fwd_varlen(*args, x["cu_seqlens"], 300)
    torch.cuda.synchronize()
    assert torch.equal(a["o"], b["o"])
    # decode_step's out buffer must match [B, H, dv] in the problem's dtype
    B, H, d, w = 2, 2, 64, 8
    st = torch.zeros(B, H, d, d, device="cuda")
    rk = torch.zeros(B, H, w, d, device="cuda", dtype=BF)
    rv = torch.zeros_like(rk)
    pos = torch.zeros(B, dtype=torch.int64, device="cuda")
    dec = make_decode_inputs(1, B, H, d, d, dtype="bf16", seed=2)
    t = [dec[n][0].cuda() for n in ("q", "k", "v", "log_alpha")]
    for out in (torch.empty(B, H, d // 2, device="cuda", dtype=BF),
                torch.empty(B, H, d, device="cuda", dtype=torch.float32)):
        with pytest.raises(ValueError, match="out"):
            lz.decode_step(*t, st, rk, rv, pos, None, None, out=out)
    torch.cuda.synchronize()
    assert torch.equal(pos.cpu(), torch.zeros(B, dtype=torch.int64))
