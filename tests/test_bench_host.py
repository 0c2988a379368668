"""Host-side checks of bench.py: the algorithmic byte and FLOP counts that the
roofline figures divide by, the counter-traffic record lookup, and the refusal
of multi-GPU runs.  No GPU is touched.

Each count is checked against a second derivation: the byte counts against a
sum over the tensors a call reads and writes (element count x element size),
the FLOP count against a brute-force enumeration of the (query, key) pairs that
the causal chunks and the sliding window contain.
"""
import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def tensor_bytes(*specs):
    return sum(int(np.prod(shape)) * size for shape, size in specs)


@pytest.mark.parametrize("B,H,T,d,w,M", [(2, 32, 4096, 128, 128, 4), (1, 3, 100, 64, 7, 0),
                                         (1, 32, 32768, 128, 128, 4)])
@pytest.mark.parametrize("gate_bytes", [4, 2])
def test_hybrid_bytes_match_tensor_sizes(B, H, T, d, w, M, gate_bytes):
    expect = tensor_bytes(((B, H, T, d), 2), ((B, H, T, d), 2), ((B, H, T, d), 2),  # q, k, v
                          ((B, H, T, d), gate_bytes),                                 # gates
                          ((B, H, T, d), 2),                                          # o
                          ((B, H, d, d), 4),                                          # hT
                          ((B, H, w, d), 2), ((B, H, w, d), 2),                       # window cache
                          ((H, M, d), 2), ((H, M, d), 2))                             # meta k, v
    assert bench.hybrid_bytes(B, H, T, d, w, M, gate_bytes=gate_bytes) == expect


def test_headline_bytes_value():
    # the figure the prefill roofline divides by
    assert bench.hybrid_bytes(2, 32, 4096, 128, 128, 4) == 411_107_328


@pytest.mark.parametrize("B,H,d,w,M,pos", [(64, 32, 128, 128, 4, 2048), (2, 3, 64, 5, 2, 0),
                                           (2, 3, 64, 5, 2, 3), (1, 1, 64, 1, 0, 10)])
def test_decode_bytes_match_tensor_sizes(B, H, d, w, M, pos):
    n_old = min(pos + 1, w) - 1  # cache slots read besides the new token's
    expect = tensor_bytes(((B, H, d, d), 4), ((B, H, d, d), 4),       # state read and written
                          ((B, H, n_old, d), 2), ((B, H, n_old, d), 2),  # older K, V slots read
                          ((B, H, d), 2), ((B, H, d), 2),              # new K, V slots written
                          ((B, H, d), 2), ((B, H, d), 2), ((B, H, d), 2),  # q, k, v
                          ((B, H, d), 4),                              # log alpha
                          ((B, H, d), 2),                              # o
                          ((H, M, d), 2), ((H, M, d), 2))              # meta k, v
    assert bench.decode_bytes_per_step(B, H, d, w, M, pos) == expect


def test_train_bytes_match_tensor_sizes():
    B, H, T, d = 8, 16, 2048, 64
    x = (B, H, T, d)
    fwd = tensor_bytes((x, 2), (x, 2), (x, 2), (x, 4),          # q, k, v, log alpha read
                       (x, 2), (x, 2), ((B, H, T), 4))          # o, o_swa, lse written
    bwd = tensor_bytes((x, 2), (x, 2), (x, 2), (x, 4), (x, 2),  # q, k, v, log alpha, dO
                       (x, 2), ((B, H, T), 4),                  # o_swa, lse
                       (x, 2), (x, 2), (x, 2), (x, 4))          # dq, dk, dv, dlog alpha
    assert bench.train_bytes(B, H, T, d) == fwd + bwd == 639_631_360


@pytest.mark.parametrize("T,C,w,M,d", [(256, 64, 64, 4, 64), (200, 64, 7, 0, 32), (130, 64, 300, 2, 16)])
def test_flops_match_pair_enumeration(T, C, w, M, d):
    # the count takes the intra-chunk triangles of whole chunks only (the
    # configured workloads have T a multiple of the chunk)
    macs = 0
    for t in range(T):
        c0 = (t // C) * C
        if c0 + C <= T:
            macs += (t - c0 + 1) * d * 2      # intra-chunk scores and A V, causal
        macs += d * d * 2                     # q S and the state update
        keys = sum(1 for s in range(t + 1) if t - s < w) + M
        macs += keys * d * 2                  # window scores and P V, meta slots included
    assert bench.algorithmic_flops(1, 1, T, d, C, w, M) == 2 * macs
    assert bench.algorithmic_flops(3, 2, T, d, C, w, M) == 2 * 6 * macs


def test_headline_flops_value():
    assert bench.algorithmic_flops(2, 32, 4096, 128, 64, 128, 4) == pytest.approx(38.992347136e9)


def test_counter_traffic_record_lookup():
    path = os.path.join(ROOT, "profiles", "prefill_hybrid_b2_h32_t4096_d128.md")
    recs = [json.loads(l.split(":", 1)[1]) for l in open(path) if l.startswith("traffic-record:")]
    assert len(recs) == 1
    rec = recs[0]
    assert re.fullmatch(r"[0-9a-f]{16}", rec["source_digest"])
    assert bench.counter_traffic(rec["workload"], rec["source_digest"]) == rec["bytes_per_launch"]
    # a record whose digest does not match the kernel sources is not reported
    assert bench.counter_traffic(rec["workload"], "0" * 16) is None
    assert bench.counter_traffic("no_such_workload", rec["source_digest"]) is None


def test_source_digest_follows_the_sources():
    d1 = bench.source_digest("gla_fwd.hip", "hybrid_fwd.hip", "common.hpp")
    d2 = bench.source_digest("gla_fwd.hip", "hybrid_fwd.hip")
    assert re.fullmatch(r"[0-9a-f]{16}", d1) and d1 != d2


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout.strip() == ""
