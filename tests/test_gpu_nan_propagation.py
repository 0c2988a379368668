"""NaN inputs reach the outputs (the library's stated error convention).

A NaN gate of one token and channel of one head must poison that head's gated
branch from its chunk on (the state's row for that channel becomes NaN, and
every later output reads the whole state) and its final state, in the prefill,
the backward and the decode step, while every other head stays finite.  The
per-token gate floor must not mask it: a floor taken with fmaxf would return
the floor for a NaN gate.
"""
import math

import pytest
import torch

import gated_linear_attention_chunked_amd as lz
from tests._gpu_helpers import to_dev
from workloads import make_decode_inputs, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,dtype,logits", [
    (128, "bf16", False),  # single-pass kernel, generic backward
    (64, "bf16", True),    # d = 64 kernels, gate logits
    (64, "f32", False),    # fp32 output pass
])
def test_nan_gate_stays_in_its_head(d, dtype, logits):
    B, H, T, w, M = 1, 3, 200, 64, 2
    print(f"[case] NaN gate d{d} {dtype} logits{logits}", flush=True)
    s = 1.0 / math.sqrt(d)
    inp = make_inputs(B, H, T, d, d, M, dtype=dtype, seed=d + 1, with_grad_out=True,
                      with_gate_logits=logits)
    gname = "gate_x" if logits else "log_alpha"
    if logits:
        inp.pop("log_alpha")
    inp[gname][0, 1, 100, 5] = float("nan")  # head 1, token 100, channel 5
    x = to_dev(inp)
    args = (x["q"], x["k"], x["v"], x[gname], x["meta_k"], x["meta_v"], w)
    f = lz.hybrid_fwd(*args, scale=s, save_for_backward=True, return_state=True,
                      return_ring=True)
    g = lz.hybrid_bwd(*args, f["o_swa"], f["lse"], x["dO"], scale=s, return_dh0=True)
    torch.cuda.synchronize()
    o = f["o"].float()
    others = [0, 2]
    assert torch.isfinite(o[0, others]).all() and torch.isfinite(f["hT"][0, others]).all()
    assert torch.isfinite(o[0, 1, :64]).all()      # chunks before the NaN token
    assert torch.isnan(o[0, 1, 128:]).all()        # every later output reads the NaN state row
    assert torch.isnan(f["hT"][0, 1]).any()
    assert torch.isfinite(f["o_swa"].float()).all()  # the window branch reads no gate
    for n in ("dq", "dk", "dv", "dlog_alpha"):
        assert torch.isfinite(g[n][0, others].float()).all(), n
    assert torch.isnan(g["dq"][0, 1].float()).any() and torch.isnan(g["dlog_alpha"][0, 1]).any()
    assert torch.isfinite(g["dmeta_k"]).all() and torch.isfinite(g["dmeta_v"]).all()

    # decode: head 1 continues from its NaN state; a NaN gate in head 2's step
    # poisons head 2 from then on; head 0 stays finite
    dec = make_decode_inputs(2, B, H, d, d, dtype=dtype, seed=d + 2, with_gate_logits=logits)
    dname = "gate_x" if logits else "log_alpha"
    dec[dname][0, 0, 2, 7] = float("nan")
    state, rk, rv = f["hT"].clone(), f["ring_k"].clone(), f["ring_v"].clone()
    pos = torch.full((B,), T, dtype=torch.int64, device="cuda")
    for i in range(2):
        od = lz.decode_step(dec["q"][i].cuda(), dec["k"][i].cuda(), dec["v"][i].cuda(),
                            dec[dname][i].cuda(), state, rk, rv, pos, x["meta_k"], x["meta_v"],
                            scale=s).float()
        torch.cuda.synchronize()
        assert torch.isfinite(od[0, 0]).all() and torch.isfinite(state[0, 0]).all()
        assert torch.isnan(od[0, 1]).all() and torch.isnan(od[0, 2]).all()
        assert torch.isnan(state[0, 2]).any()
