"""GPU parity of the hybrid forward and backward on a seeded sweep of mixed
configurations, each against the fp64 oracle.

Each case draws (from a fixed seed) the head size (64, 128), the element type
(bf16, fp32), the gate format (log alpha; bf16 logits with bf16), the window
(1 .. 300, across the single-pass and tiled kernels), the meta slots (0 .. 16),
a ragged length, separate window queries and keys, an initial state, a
final-state gradient, the mix weight and the gate range, so that the features
meet in combinations the targeted tests do not enumerate.
"""
import math

import numpy as np
import pytest
import torch

import gated_linear_attention_chunked_amd as lz
import oracle
from tests._gpu_helpers import assert_close, f64, to_dev
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def draw(i):
    r = np.random.default_rng(1000 + i)
    dtype = ["bf16", "f32"][r.integers(2)]
    return dict(
        B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), T=int(r.integers(1, 401)),
        d=int([64, 128][r.integers(2)]), dtype=dtype,
        logits=dtype == "bf16" and bool(r.integers(2)),
        w=int([1, 2, 17, 33, 64, 65, 100, 128, 129, 130, 200, 300][r.integers(12)]),
        M=int([0, 1, 4, 16][r.integers(4)]), sep=bool(r.integers(2)), h0=bool(r.integers(2)),
        dhT=bool(r.integers(2)), mix=float(np.round(r.uniform(-1.5, 1.5), 3)),
        gate_mean=float([2.0, 0.3, -3.0][r.integers(3)]), seed=int(r.integers(1 << 20)))


@pytest.mark.parametrize("i", range(24))
def test_random_configuration(i):
    c = draw(i)
    print(f"[case] random {i}: {c}", flush=True)
    B, H, T, d, M, w = c["B"], c["H"], c["T"], c["d"], c["M"], c["w"]
    dt = DT[c["dtype"]]
    inp = make_inputs(B, H, T, d, d, M, dtype=c["dtype"], seed=c["seed"],
                      gate_mean=c["gate_mean"], with_grad_out=True, with_h0=c["h0"],
                      with_window_qk=c["sep"], with_gate_logits=c["logits"])
    if c["logits"]:
        inp.pop("log_alpha")
    gname = "gate_x" if c["logits"] else "log_alpha"
    if c["dhT"]:
        inp["dhT"] = torch.randn(B, H, d, d, generator=torch.Generator().manual_seed(c["seed"])) * 0.1
    s, mix = 1.0 / math.sqrt(d), c["mix"]
    x = to_dev(inp)
    args = (x["q"], x["k"], x["v"], x[gname], x["meta_k"], x["meta_v"], w)
    sep = dict(q_w=x.get("q_w"), k_w=x.get("k_w"))
    f = lz.hybrid_fwd(*args, scale=s, mix=mix, h0=x.get("h0"), save_for_backward=True,
                      return_state=True, **sep)
    g = lz.hybrid_bwd(*args, f["o_swa"], f["lse"], x["dO"], scale=s, mix=mix, h0=x.get("h0"),
                      dhT=x.get("dhT"), return_dh0=True, return_dmix=True, **sep)
    torch.cuda.synchronize()

    r = f64(inp)
    la = oracle.log_sigmoid(r["gate_x"]) if c["logits"] else r["log_alpha"]
    ow = dict(q_w=r.get("q_w"), k_w=r.get("k_w"))
    ref = oracle.hybrid_forward(r["q"], r["k"], r["v"], la, r["meta_k"], r["meta_v"], w, s,
                                mix=mix, h0=r.get("h0"), **ow)
    for n in ("o", "hT", "o_swa"):
        assert_close(n, f[n], ref[n], dt)
    assert_close("lse", f["lse"], ref["lse"], dt, tol=1e-4)
    gr = oracle.hybrid_backward(r["q"], r["k"], r["v"], la, r["meta_k"], r["meta_v"], w, s,
                                r["dO"], mix=mix, h0=r.get("h0"), dhT=r.get("dhT"), **ow)
    dgate = (oracle.log_sigmoid_backward(r["gate_x"], gr["dlog_alpha"]) if c["logits"]
             else gr["dlog_alpha"])
    assert_close("d gate_x" if c["logits"] else "dlog_alpha", g["dlog_alpha"], dgate, dt)
    names = ["dq", "dk", "dv", "dh0"] + (["dq_w", "dk_w"] if c["sep"] else [])
    names += ["dmeta_k", "dmeta_v"] if M > 0 else []
    for n in names:
        assert_close(n, g[n], gr[n], dt)
    # dmix = sum(dO * o_swa) in fp32 from the saved o_swa: bounded by the
    # rounding of o_swa in the element type, on the scale sum |dO| |o_swa|
    o_swa = ref["o_swa"]
    scale = float((np.abs(r["dO"]) * np.abs(o_swa)).sum())
    u = 2.0 ** -8 if c["dtype"] == "bf16" else 1e-4
    err = abs(float(g["dmix"].item()) - gr["dmix"])
    print(f"  dmix: error {err:.2e}, bound scale {scale:.2e}", flush=True)
    assert err <= u * scale + 1e-6
