"""LIZARD_SYNC_DEBUG=1: every call waits for its own work and reports its
status; outputs must be those of the normal asynchronous mode.  The switch is
read once per process, so the check runs in one child process that calls the
forward, backward and decode entry points and compares them with the oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import math, sys
import numpy as np, torch
sys.path.insert(0, sys.argv[1])
import gated_linear_attention_chunked_amd as lz
import oracle
from workloads import make_inputs, make_decode_inputs, to_f64_numpy
print("[child] sync-debug forward/backward/decode B1 H2 T300 d64", flush=True)
inp = make_inputs(1, 2, 300, 64, 64, 4, dtype="bf16", seed=1, with_grad_out=True)
x = {n: t.cuda() for n, t in inp.items()}
s = 0.125
f = lz.hybrid_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], 64, scale=s,
                  save_for_backward=True, return_state=True, return_ring=True)
g = lz.hybrid_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], 64,
                  f["o_swa"], f["lse"], x["dO"], scale=s)
dec = make_decode_inputs(1, 1, 2, 64, 64, dtype="bf16", seed=2)
pos = torch.full((1,), 300, dtype=torch.int64, device="cuda")
o = lz.decode_step(*(dec[n][0].cuda() for n in ("q", "k", "v", "log_alpha")), f["hT"].clone(),
                   f["ring_k"].clone(), f["ring_v"].clone(), pos, x["meta_k"], x["meta_v"], scale=s)
torch.cuda.synchronize()
r = {n: to_f64_numpy(t) for n, t in inp.items()}
ref = oracle.hybrid_forward(r["q"], r["k"], r["v"], r["log_alpha"], r["meta_k"], r["meta_v"], 64, s)
gref = oracle.hybrid_backward(r["q"], r["k"], r["v"], r["log_alpha"], r["meta_k"], r["meta_v"],
                              64, s, r["dO"])
rel = lambda a, b: float(np.max(np.abs(to_f64_numpy(a) - b)) / np.max(np.abs(b)))
errs = {"o": rel(f["o"], ref["o"]), "hT": rel(f["hT"], ref["hT"])}
errs.update({n: rel(g[n], gref[n]) for n in ("dq", "dk", "dv", "dlog_alpha")})
print("[child] errors", errs, "pos", int(pos.item()), flush=True)
assert all(e < 2e-2 for e in errs.values()), errs
assert int(pos.item()) == 301 and torch.isfinite(o.float()).all()
print("[child] ok", flush=True)
'''


def test_sync_debug_mode_matches_oracle():
    env = dict(os.environ, LIZARD_SYNC_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0
    assert "[child] ok" in r.stdout
