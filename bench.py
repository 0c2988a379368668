#!/usr/bin/env python3
"""Benchmark of the hybrid attention hot path on one MI355X.

A step is one hybrid prefill forward (GLA branch + window/meta branch + combine
+ state and window-cache handoff) over one batch of the bf16 workload
B=2, H=32, T=4096, d=128, chunk 64, w=128, M=4, with inputs resident in HBM.
Prints one JSON line with prefill tokens/s (value), the fraction of bf16 MFMA
peak, the HBM roofline of the dominant kernel, the fp64 oracle timed on the host
as a CPU baseline, and secondary lines for the decode workload (B=64, H=32,
1024 steps after a 2048-token prefill) and the training workload (B=8, H=16,
T=2048, d=64, forward + backward).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_flops(B, H, T, d, C, w, M):
    """Causal-triangle and real-window work only (no padded tiles), FLOP = 2 MAC."""
    nc = T // C
    gla = nc * C * (C + 1) / 2 * (2 * d) + T * d * d * 2
    win = sum(min(t + 1, w) for t in range(T)) + M * T
    return 2.0 * B * H * (gla + win * 2 * d)


def hybrid_bytes(B, H, T, d, w, M, gate_bytes=4):
    """Hybrid forward: q, k, v (bf16) and the gates (fp32 log_alpha, or bf16
    logits with gate_bytes=2) read once, o written once, the final state (fp32)
    and the window cache (bf16 K and V) written once, the meta keys and values
    read once."""
    return (B * H * (T * (3 * d * 2 + d * gate_bytes + d * 2) + d * d * 4 + 2 * w * d * 2)
            + H * M * d * 2 * 2)


def decode_bytes_per_step(B, H, d, w, M, pos):
    """Per step and (b,h): fp32 state read+write, the min(pos+1,w)-1 older ring
    slots read (K and V), the new K,V written, q,k,v,log_alpha read, o written."""
    n_old = min(pos + 1, w) - 1
    per = 2 * d * d * 4 + n_old * d * 2 * 2 + 2 * d * 2 + 3 * d * 2 + d * 4 + d * 2
    return B * H * per + H * M * d * 2 * 2


def source_digest(*names):
    """Digest of the kernel sources and of the per-source build flags they add
    (a flag change alters the code as a source change does)."""
    from gated_linear_attention_chunked_amd.build import EXTRA_FLAGS
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_linear_attention_chunked_amd", "csrc", n), "rb") as f:
            h.update(f.read())
        if EXTRA_FLAGS.get(n):
            h.update(" ".join(EXTRA_FLAGS[n]).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload, digest):
    """HBM bytes per call measured with rocprofv3 FETCH_SIZE/WRITE_SIZE (scaled by
    a copy-kernel calibration), as recorded in profiles/*.md; None when no record
    matches the current kernel source."""
    if not os.path.isdir(PROFILES):
        return None
    for fn in sorted(os.listdir(PROFILES)):
        if not fn.endswith(".md"):
            continue
        with open(os.path.join(PROFILES, fn)) as f:
            for line in f:
                if line.startswith("traffic-record:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("workload") == workload and rec.get("source_digest") == digest:
                        return rec.get("bytes_per_launch")
    return None


# minimum warm-up time of the secondary lines (a quarter of --min-warmup-seconds)
_MIN_WARM = [0.25]


def event_time_ms(fn, steps, warmup):
    import torch
    warm_up(fn, warmup, _MIN_WARM[0])
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def _oracle_worker(task):
    """One host process: the oracle on the same head again and again until
    `seconds` have passed; returns (heads done, seconds)."""
    x, wl, seconds = task
    import oracle
    from threadpoolctl import threadpool_limits
    heads = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while True:
            oracle.hybrid_forward(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"],
                                  x["meta_v"], wl["window"], wl["scale"], mix=wl["mix"])
            heads += 1
            if time.perf_counter() - t0 >= seconds:
                break
    return heads, time.perf_counter() - t0


def host_cores():
    """Host cores for the CPU baseline: the process's affinity set, capped at the
    16-core share a one-GPU machine gives a job."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, seconds, cores):
    """The fp64 oracle as it stands, on `cores` host processes (BLAS limited to
    one thread each), each running whole heads of the same workload for about
    `seconds`; reported in layer tokens/s.  Runs before the GPU is touched, so
    the worker processes are plain forks of a process with no GPU context."""
    import multiprocessing as mp
    from workloads import make_inputs, to_f64_numpy
    inp = make_inputs(1, 1, wl["T"], wl["dk"], wl["dv"], wl["n_meta"], dtype=wl["dtype"], seed=0)
    x = {n: to_f64_numpy(t) for n, t in inp.items()}
    task = (x, dict(wl), seconds)
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        res = pool.map(_oracle_worker, [task] * cores)
    wall = time.perf_counter() - t0
    heads = sum(h for h, _ in res)
    # one head of T tokens is 1/H of a batch element's work: tokens/s of the
    # whole layer = head-tokens/s / H
    return {"value": heads * wl["T"] / wall / wl["H"], "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{heads} head(s) x T={wl['T']} of the same workload (one head of one "
                      f"sequence per pass, heads spread over {cores} processes, BLAS 1 thread "
                      f"each), fp64 numpy, {wall:.1f} s wall"}


def warm_up(fn, steps, min_seconds=1.0):
    """At least `steps` untimed calls, and more until `min_seconds` have passed
    (the GPU runs about 10% slower until its clocks settle); returns the number
    of calls made."""
    import torch
    n, t0 = 0, time.perf_counter()
    while n < steps or time.perf_counter() - t0 < min_seconds:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # the first ~50 steps after set-up run before the GPU has reached steady
    # clocks (about 10% slower); the defaults time the steady state
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the decode and training lines")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    ap.add_argument("--train-only", action="store_true",
                    help="only time the training step (forward + backward), for profiling")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time the decode steps, for profiling")
    ap.add_argument("--decode-b", type=int, default=None,
                    help="batch of the --decode-only run (default 64, 1024 steps; else 256 steps)")
    ap.add_argument("--min-warmup-seconds", type=float, default=1.0,
                    help="keep warming up past --warmup steps until this much time has passed")
    args = ap.parse_args()
    _MIN_WARM[0] = args.min_warmup_seconds / 4
    if args.copy_probe:
        import torch
        a = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on a single GPU; multi-GPU runs are not supported "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    from workloads import WORKLOADS, make_inputs
    name = "prefill_bf16_b2_h32_t4096_d128"
    wl = WORKLOADS[name]
    cpu = None
    if not (args.no_cpu_baseline or args.decode_only or args.train_only):
        # before anything touches the GPU: the workers are forks of this process
        cpu = cpu_baseline(wl, args.cpu_seconds, host_cores())

    import torch
    import gated_linear_attention_chunked_amd as lz
    from gated_linear_attention_chunked_amd import _abi

    if args.decode_only:
        steps = None if args.decode_b is None else 256
        print(json.dumps({"decode": bench_decode(lz, torch, torch.device("cuda:0"), B=args.decode_b,
                                                 steps=steps)}), flush=True)
        return
    if args.train_only:
        print(json.dumps({"train": bench_train(lz, torch, torch.device("cuda:0"), args)}),
              flush=True)
        return
    B, H, T, d, w, M, C = wl.B, wl.H, wl.T, wl.dk, wl.window, wl.n_meta, wl.chunk
    dev = torch.device("cuda:0")
    inp = make_inputs(B, H, T, d, d, M, dtype=wl.dtype, seed=0)
    x = {n: t.to(dev) for n, t in inp.items()}
    o = torch.empty_like(x["v"])
    hT = torch.empty(B, H, d, d, device=dev)
    rk = torch.empty(B, H, w, d, device=dev, dtype=torch.bfloat16)
    rv = torch.empty_like(rk)
    desc = lz.make_desc(B, H, T, d, d, w, M, wl.scale, wl.mix, torch.bfloat16)
    nws = lz.workspace_bytes(desc, _abi.OP_HYBRID_FWD)
    ws = torch.empty(max(nws, 1), device=dev, dtype=torch.uint8)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    lib = lz.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dref = ctypes.byref(desc)
    hyb_args = (dref, P(x["q"]), P(x["k"]), P(x["v"]), P(x["log_alpha"]), P(x["meta_k"]),
                P(x["meta_v"]), None, P(o), None, None, P(hT), P(rk), P(rv), None, None, P(ws), nws,
                stream)

    def step():
        st = lib.lizard_hybrid_fwd(*hyb_args)
        if st != 0:
            raise RuntimeError(f"lizard_hybrid_fwd: status {st}")

    # ---- timed region: exactly K steps between two synchronisations
    warmup_run = warm_up(step, args.warmup, args.min_warmup_seconds)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    value = B * T / (ms / 1e3)
    flops = algorithmic_flops(B, H, T, d, C, w, M)

    # ---- the same step's two launches (GLA state pass, then the single-pass
    # output kernel) are the roofline unit; the separate branch entry points are
    # timed for context
    gws_n = lz.workspace_bytes(desc, _abi.OP_GLA_FWD)
    gla_args = (dref, P(x["q"]), P(x["k"]), P(x["v"]), P(x["log_alpha"]), None, P(o), P(hT),
                P(ws), gws_n, stream)
    gla_ms = event_time_ms(lambda: lib.lizard_gla_fwd(*gla_args), args.steps, args.warmup)
    swa_ms = event_time_ms(lambda: lib.lizard_swa_fwd(dref, P(x["q"]), P(x["k"]), P(x["v"]),
                                                      P(x["meta_k"]), P(x["meta_v"]), P(o), None,
                                                      stream), args.steps, args.warmup)
    hbytes = hybrid_bytes(B, H, T, d, w, M)
    achieved = hbytes / (ms / 1e3) / 1e9
    traffic = counter_traffic(name, source_digest("gla_fwd.hip", "hybrid_fwd.hip", "hybrid_fwd.hpp", "common.hpp"))

    out = {
        "metric": "prefill tokens/s + % bf16 MFMA peak; decode tokens/s + % HBM BW",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": warmup_run, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "B": B, "H": H, "T": T, "dk": d, "dv": d, "chunk": C,
                   "window": w, "n_meta": M, "parallelism": "single GPU"},
        "mfma": {"algorithmic_tflop_per_step": flops / 1e12,
                 "achieved_tflops": flops / (ms / 1e3) / 1e12,
                 "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                 "frac": flops / (ms / 1e3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                 # the step is below the ridge: its ceiling is min(peak, HBM BW x FLOP/B)
                 "roofline_ceiling_frac": min(1.0, flops / hbytes * HBM_PEAK_GBS * 1e9
                                              / (BF16_MFMA_PEAK_TFLOPS * 1e12)),
                 "frac_of_ceiling": (flops / (ms / 1e3)) / min(BF16_MFMA_PEAK_TFLOPS * 1e12,
                                                                flops / hbytes * HBM_PEAK_GBS * 1e9)},
        "roofline": {"kernel": "lizard_hybrid_fwd (gla_state_pass + hybrid_fwd_fused)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "launch_ms": ms, "algorithmic_bytes": hbytes},
        "separate_entry_points_ms": {"lizard_gla_fwd": gla_ms, "lizard_swa_fwd": swa_ms},
    }

    if not args.no_extras:
        out["prefill_gate_logits"] = bench_prefill_gate_logits(lz, torch, dev, args)
        out["long_prefill"] = bench_long_prefill(lz, torch, dev, args, ms / (B * T))
        out["prefill_varlen"] = bench_prefill_varlen(lz, torch, dev, args)
        out["decode"] = bench_decode(lz, torch, dev)
        # twice the batch: a 512 MiB working set (state + window cache), twice the
        # 256 MB last-level cache, so bytes / time cannot be served from it
        out["decode_b128"] = bench_decode(lz, torch, dev, B=128, steps=256)
        try:
            out["train"] = bench_train(lz, torch, dev, args)
        except lz.LizardError as e:
            out["train"] = {"error": str(e)}
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def bench_prefill_gate_logits(lz, torch, dev, args):
    """The headline prefill workload with the gates given as bf16 logits x
    (alpha = sigmoid(x), the same N(2, 1) draw), log-sigmoid taken in the
    kernels: half the gate bytes of fp32 log_alpha."""
    from gated_linear_attention_chunked_amd import _abi
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS["prefill_bf16_b2_h32_t4096_d128"]
    B, H, T, d, w, M = wl.B, wl.H, wl.T, wl.dk, wl.window, wl.n_meta
    x = {n: t.to(dev) for n, t in make_inputs(B, H, T, d, d, M, dtype=wl.dtype, seed=0,
                                              with_gate_logits=True).items()}
    o = torch.empty_like(x["v"])
    hT = torch.empty(B, H, d, d, device=dev)
    rk = torch.empty(B, H, w, d, device=dev, dtype=torch.bfloat16)
    rv = torch.empty_like(rk)
    desc = lz.make_desc(B, H, T, d, d, w, M, wl.scale, wl.mix, torch.bfloat16,
                        gate=_abi.LIZARD_GATE_LOGIT)
    nws = lz.workspace_bytes(desc, _abi.OP_HYBRID_FWD)
    ws = torch.empty(max(nws, 1), device=dev, dtype=torch.uint8)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = (ctypes.byref(desc), P(x["q"]), P(x["k"]), P(x["v"]), P(x["gate_x"]), P(x["meta_k"]),
         P(x["meta_v"]), None, P(o), None, None, P(hT), P(rk), P(rv), None, None, P(ws), nws, stream)
    lib = lz.lib()

    def step():
        st = lib.lizard_hybrid_fwd(*a)
        if st != 0:
            raise RuntimeError(f"lizard_hybrid_fwd (logit gates): status {st}")

    ms = event_time_ms(step, args.steps, args.warmup)
    nbytes = hybrid_bytes(B, H, T, d, w, M, gate_bytes=2)
    return {"workload": "prefill_bf16_b2_h32_t4096_d128, bf16 gate logits", "ms_per_step": ms,
            "tokens_per_s": B * T / (ms / 1e3), "algorithmic_bytes": nbytes,
            "achieved_GBs": nbytes / (ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}


def bench_long_prefill(lz, torch, dev, args, ms_per_token_headline):
    """Hybrid prefill of B=1, H=32, T=32768, d=128 (same value families); the time
    per token against the headline workload's shows whether time is linear in T
    (same B*H*T/8 work per token, 8x longer sequences)."""
    from workloads import WORKLOADS, make_inputs
    wl = WORKLOADS["prefill_bf16_b1_h32_t32768_d128"]
    x = {n: t.to(dev) for n, t in make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.n_meta,
                                              dtype=wl.dtype, seed=0).items()}

    def step():
        lz.hybrid_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"],
                      wl.window)

    ms = event_time_ms(step, max(5, args.steps // 5), max(5, args.warmup // 2))
    per_tok = ms / (wl.B * wl.T)
    return {"workload": "prefill_bf16_b1_h32_t32768_d128", "ms_per_call": ms,
            "tokens_per_s": wl.B * wl.T / (ms / 1e3),
            "time_per_token_vs_headline": per_tok / ms_per_token_headline}


def bench_prefill_varlen(lz, torch, dev, args):
    """Serving prefill: a packed batch of 16 sequences of 64..8192 tokens (seeded
    lengths), H=32, d=128, w=128, M=4, through lizard_hybrid_fwd_varlen with the
    final states and window caches; inputs drawn on the device with a seeded
    generator (the headline's value families)."""
    from gated_linear_attention_chunked_amd import _abi
    from workloads import packed_lengths
    lengths = packed_lengths(16, 64, 8192, seed=0)
    H, d, w, M = 32, 128, 128, 4
    N, B = sum(lengths), len(lengths)
    g = torch.Generator(device=dev).manual_seed(0)

    def rnd(*shape, mean=0.0, scale=1.0, dt=torch.bfloat16):
        return (torch.randn(*shape, device=dev, generator=g) * scale + mean).to(dt)

    s = 1.0 / math.sqrt(d)
    q, k, v = (rnd(H, N, d, scale=s) for _ in range(3))
    la = torch.nn.functional.logsigmoid(rnd(H, N, d, mean=2.0, dt=torch.float32))
    mk, mv = rnd(H, M, d), rnd(H, M, d)
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths), 0).to(torch.int32)
    cu = cu.to(dev)
    o = torch.empty_like(v)
    hT = torch.empty(B, H, d, d, device=dev)
    rk = torch.empty(B, H, w, d, device=dev, dtype=torch.bfloat16)
    rv = torch.empty_like(rk)
    desc = lz.make_desc(B, H, max(lengths), d, d, w, M, s, 1.0, torch.bfloat16)
    nws = lz.workspace_bytes(desc, _abi.OP_HYBRID_FWD)
    ws = torch.empty(max(nws, 1), device=dev, dtype=torch.uint8)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = (ctypes.byref(desc), P(cu), N, P(q), P(k), P(v), P(la), P(mk), P(mv), None, P(o), P(hT),
         P(rk), P(rv), None, None, P(ws), nws, stream)
    lib = lz.lib()

    def step():
        st = lib.lizard_hybrid_fwd_varlen(*a)
        if st != 0:
            raise RuntimeError(f"lizard_hybrid_fwd_varlen: status {st}")

    ms = event_time_ms(step, max(10, args.steps // 5), max(5, args.warmup // 5))
    nbytes = H * N * (3 * d * 2 + d * 4 + d * 2) + B * H * (d * d * 4 + 2 * w * d * 2) + H * M * d * 4
    return {"workload": "packed serving prefill: 16 sequences of 64..8192 tokens (seed 0), "
                        "H32 d128 w128 M4", "tokens": N, "ms_per_call": ms,
            "tokens_per_s": N / (ms / 1e3), "algorithmic_GBs": nbytes / (ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}


def bench_decode(lz, torch, dev, B=None, steps=None):
    """Decode steps (B=64, H=32, d=128, w=128, M=4; 1024 steps by default) after
    a 2048-token hybrid prefill; inputs drawn on the device with a seeded
    generator (same recipe)."""
    from workloads import WORKLOADS
    wl = WORKLOADS["decode_bf16_b64_h32_d128"]
    H, T, d, w, M = wl.H, wl.T, wl.dk, wl.window, wl.n_meta
    B = wl.B if B is None else B
    steps = wl.steps if steps is None else steps
    g = torch.Generator(device=dev).manual_seed(0)

    def rnd(*shape, mean=0.0, scale=1.0, dt=torch.bfloat16):
        return (torch.randn(*shape, device=dev, generator=g) * scale + mean).to(dt)

    s = 1.0 / math.sqrt(d)
    q, k, v = (rnd(B, H, T, d, scale=s) for _ in range(3))
    la = torch.nn.functional.logsigmoid(rnd(B, H, T, d, mean=2.0, dt=torch.float32))
    mk, mv = rnd(H, M, d), rnd(H, M, d)
    pre = lz.hybrid_fwd(q, k, v, la, mk, mv, w, return_state=True, return_ring=True)
    del q, k, v, la
    dq, dk_, dv_ = (rnd(steps, B, H, d, scale=s) for _ in range(3))
    dla = torch.nn.functional.logsigmoid(rnd(steps, B, H, d, mean=2.0, dt=torch.float32))
    state, rk, rv = pre["hT"], pre["ring_k"], pre["ring_v"]
    pos = torch.full((B,), T, dtype=torch.int64, device=dev)
    o = torch.empty(B, H, d, device=dev, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        lz.decode_step(dq[i], dk_[i], dv_[i], dla[i], state, rk, rv, pos, mk, mv, out=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    nbytes = sum(decode_bytes_per_step(B, H, d, w, M, T + i) for i in range(steps))
    gbs = nbytes / (ms / 1e3) / 1e9
    ws_mib = B * H * (d * d * 4 + 2 * w * d * 2) / 2**20
    return {"workload": f"decode_bf16_b{B}_h{H}_d{d}", "B": B, "steps": steps,
            "working_set_MiB": ws_mib, "ms_total": ms,
            "us_per_step": ms * 1e3 / steps, "tokens_per_s": B * steps / (ms / 1e3),
            "algorithmic_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "note": "algorithmic bytes: each state, ring and token byte moved once per step; "
                    "a working set near the 256 MB last-level cache may be served partly "
                    "from it, one of twice that size cannot"}


def train_bytes(B, H, T, d):
    """Algorithmic HBM bytes of one training step (bf16 tensors, fp32 gates):
    forward reads q, k, v, log_alpha and writes o, o_swa, lse; backward reads
    q, k, v, log_alpha, dO, o_swa, lse and writes dq, dk, dv, dlog_alpha (meta
    tensors are negligible)."""
    fwd = 3 * d * 2 + d * 4 + d * 2 + d * 2 + 4
    bwd = 5 * d * 2 + d * 4 + 4 + 3 * d * 2 + d * 4
    return B * H * T * (fwd + bwd)


TRAIN_SOURCES = ("common.hpp", "gla_fwd.hip", "swa_fwd.hip", "gla_bwd.hip", "swa_bwd.hip",
                 "hybrid_bwd.hip", "hybrid_fwd.hip", "hybrid_fwd.hpp", "hybrid_fwd_d64.hip")


def bench_train(lz, torch, dev, args):
    """Forward (saving lse and o_swa) + backward of B=8, H=16, T=2048, d=64, w=64, M=4."""
    from workloads import WORKLOADS, make_inputs
    name = "train_bf16_b8_h16_t2048_d64"
    wl = WORKLOADS[name]
    B, H, T, d, w, M = wl.B, wl.H, wl.T, wl.dk, wl.window, wl.n_meta
    x = {n: t.to(dev) for n, t in make_inputs(B, H, T, d, d, M, dtype=wl.dtype, seed=0,
                                              with_grad_out=True).items()}

    def step():
        f = lz.hybrid_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], w,
                          save_for_backward=True)
        lz.hybrid_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["meta_k"], x["meta_v"], w,
                      f["o_swa"], f["lse"], x["dO"])

    ms = event_time_ms(step, max(3, args.steps // 2), max(2, args.warmup // 2))
    nbytes = train_bytes(B, H, T, d)
    achieved = nbytes / (ms / 1e3) / 1e9
    return {"workload": name, "ms_per_step": ms, "tokens_per_s": B * T / (ms / 1e3),
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "algorithmic_bytes": nbytes,
                         "traffic": counter_traffic(name, source_digest(*TRAIN_SOURCES))}}


if __name__ == "__main__":
    main()
