"""The allocation-free hybrid forward (lizard_hybrid_fwd_static) against the
workspace entry point lizard_hybrid_fwd, through the C ABI.

Both run the same kernels, the first with its scratch in the library's fixed
per-device array, so their outputs must agree bit for bit; each is also held to
the oracle's bar.  Two calls in a row, the second on a smaller problem, show
that nothing left in the shared array from the first call leaks into the second.
"""
import ctypes
import math

import pytest
import torch

import gated_linear_attention_chunked_amd as lz
import oracle
from gated_linear_attention_chunked_amd import _abi
from tests._gpu_helpers import assert_close, f64, to_dev
from workloads import make_inputs

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_pair(B, H, T, d, w, M, saved, seed):
    print(f"[case] no-alloc B{B} H{H} T{T} d{d} w{w} M{M} saved={saved}", flush=True)
    inp = make_inputs(B, H, T, d, d, M, dtype="bf16", seed=seed, with_h0=True)
    x = to_dev(inp)
    s = 1.0 / math.sqrt(d)
    desc = lz.make_desc(B, H, T, d, d, w, M, s, 0.7, BF)
    need = lz.workspace_bytes(desc, _abi.OP_HYBRID_FWD)
    assert 0 < need <= _abi.STATIC_SCRATCH_BYTES
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def outputs():
        o = {"o": torch.full((B, H, T, d), float("nan"), device="cuda", dtype=BF),
             "hT": torch.full((B, H, d, d), float("nan"), device="cuda"),
             "ring_k": torch.full((B, H, w, d), float("nan"), device="cuda", dtype=BF),
             "ring_v": torch.full((B, H, w, d), float("nan"), device="cuda", dtype=BF)}
        if saved:
            o["lse"] = torch.full((B, H, T), float("nan"), device="cuda")
            o["o_swa"] = torch.full((B, H, T, d), float("nan"), device="cuda", dtype=BF)
        return o

    common = lambda o: (ctypes.byref(desc), _p(x["q"]), _p(x["k"]), _p(x["v"]),
                        _p(x["log_alpha"]), _p(x["meta_k"]), _p(x["meta_v"]), _p(x["h0"]),
                        _p(o["o"]), _p(o.get("lse")), _p(o.get("o_swa")), _p(o["hT"]),
                        _p(o["ring_k"]), _p(o["ring_v"]), None, None)
    ref_out, st_out = outputs(), outputs()
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    assert lz.lib().lizard_hybrid_fwd(*common(ref_out), _p(ws), need, stream) == 0
    assert lz.lib().lizard_hybrid_fwd_static(*common(st_out), stream) == 0
    torch.cuda.synchronize()
    for n in ref_out:
        assert torch.equal(st_out[n], ref_out[n]), n
    r = f64(inp)
    ref = oracle.hybrid_forward(r["q"], r["k"], r["v"], r["log_alpha"], r["meta_k"], r["meta_v"],
                                w, s, mix=0.7, h0=r["h0"])
    for n in ("o", "hT"):
        assert_close(f"static.{n}", st_out[n], ref[n], BF)
    for n in ("ring_k", "ring_v"):
        assert_close(f"static.{n}", st_out[n], ref[n], BF, tol=0.0)
    if saved:
        assert_close("static.o_swa", st_out["o_swa"], ref["o_swa"], BF)
        assert_close("static.lse", st_out["lse"], ref["lse"], BF, tol=1e-4)


def test_static_scratch_matches_workspace_entry_point():
    # single-pass kernel (d = 128, inference outputs), then a smaller problem
    run_pair(1, 8, 1000, 128, 128, 4, False, seed=3)
    run_pair(1, 4, 300, 128, 128, 4, False, seed=4)
    # two-kernel path (d = 64, saved lse and o_swa), larger then smaller
    run_pair(2, 3, 700, 64, 64, 4, True, seed=5)
    run_pair(1, 2, 130, 64, 64, 4, True, seed=6)


def test_static_scratch_rejects_bad_arguments_before_launch():
    lib = lz.lib()
    d = lz.make_desc(1, 2, 128, 96, 96, 64, 4, None, 1.0, BF)  # dk = 96: not built
    fake = ctypes.c_void_p(0x1000)
    assert lib.lizard_hybrid_fwd_static(ctypes.byref(d), *([fake] * 15), None) == 4
    assert lib.lizard_hybrid_fwd_static(None, *([fake] * 15), None) == 1
