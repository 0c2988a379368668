"""Seeded synthetic inputs for the hybrid attention path.

This module only draws random numbers and names workload shapes.  It holds none
of the method's arithmetic, and both the HIP tests/benchmark and the fp64 oracle
take their inputs from here.

Value recipe (shared by every workload):
  q, k, v        ~ N(0, 1) / sqrt(d)
  gate logits x  ~ N(2, 1);  log_alpha = logsigmoid(x) in fp32   (alpha in (0,1))
  meta_k, meta_v ~ N(0, 1)
  dO             ~ N(0, 1)
Values are drawn in fp32 from a CPU torch.Generator seeded with `seed`, in the
fixed order q, k, v, x, meta_k, meta_v, dO, and then rounded once (round to
nearest even) to the workload's dtype; log_alpha always stays fp32.
"""
import math

import torch

__all__ = ["WORKLOADS", "Workload", "make_inputs", "make_decode_inputs", "to_f64_numpy"]


class Workload(dict):
    """Shape record: B, H, T, dk, dv, chunk, window, n_meta, dtype, scale, mix."""

    def __getattr__(self, name):
        try:
            return self[name]
        except KeyError as e:
            raise AttributeError(name) from e


def _wl(**kw):
    kw.setdefault("mix", 1.0)
    kw.setdefault("scale", 1.0 / math.sqrt(kw["dk"]))
    kw.setdefault("chunk", 64)
    return Workload(**kw)


WORKLOADS = {
    # tiny fp32 hybrid forward
    "tiny_fp32_b1_h2_t256_d64": _wl(B=1, H=2, T=256, dk=64, dv=64, window=64, n_meta=4,
                                    dtype="f32"),
    # bf16 prefill with a Llama-3-8B-like head shape
    "prefill_bf16_b2_h32_t4096_d128": _wl(B=2, H=32, T=4096, dk=128, dv=128, window=128,
                                          n_meta=4, dtype="bf16"),
    # long-context bf16 prefill
    "prefill_bf16_b1_h32_t32768_d128": _wl(B=1, H=32, T=32768, dk=128, dv=128, window=128,
                                           n_meta=4, dtype="bf16"),
    # constant-memory decode: 2048-token prefill, then 1024 single-token steps
    "decode_bf16_b64_h32_d128": _wl(B=64, H=32, T=2048, dk=128, dv=128, window=128, n_meta=4,
                                    dtype="bf16", steps=1024),
    # training forward + backward with a 340M-model-like head shape
    "train_bf16_b8_h16_t2048_d64": _wl(B=8, H=16, T=2048, dk=64, dv=64, window=64, n_meta=4,
                                       dtype="bf16"),
}


def _torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(B, H, T, dk, dv, n_meta, dtype="bf16", seed=0, gate_mean=2.0,
                with_grad_out=False, with_h0=False, with_window_qk=False, with_gate_logits=False,
                **_ignored):
    """Draw one prefill/training batch on the CPU.  Returns a dict of tensors:
    q, k [B,H,T,dk]; v [B,H,T,dv]; log_alpha [B,H,T,dk] fp32; meta_k [H,M,dk];
    meta_v [H,M,dv]; optionally dO [B,H,T,dv], h0 [B,H,dk,dv] fp32, the window
    branch's own q_w, k_w [B,H,T,dk] (drawn last, like q and k) and, with
    with_gate_logits, gate_x [B,H,T,dk] bf16: the same gate draw x as logits
    (log_alpha = logsigmoid(x) is computed from the fp32 draw, so the two
    differ by the bf16 rounding of x)."""
    g = torch.Generator().manual_seed(seed)
    dt = _torch_dtype(dtype)
    q = torch.randn(B, H, T, dk, generator=g) / math.sqrt(dk)
    k = torch.randn(B, H, T, dk, generator=g) / math.sqrt(dk)
    v = torch.randn(B, H, T, dv, generator=g) / math.sqrt(dv)
    x = torch.randn(B, H, T, dk, generator=g) + gate_mean
    log_alpha = torch.nn.functional.logsigmoid(x).float()
    meta_k = torch.randn(H, n_meta, dk, generator=g)
    meta_v = torch.randn(H, n_meta, dv, generator=g)
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), log_alpha=log_alpha,
               meta_k=meta_k.to(dt), meta_v=meta_v.to(dt))
    if with_gate_logits:
        out["gate_x"] = x.to(torch.bfloat16)
    if with_grad_out:
        out["dO"] = torch.randn(B, H, T, dv, generator=g).to(dt)
    if with_h0:
        out["h0"] = torch.randn(B, H, dk, dv, generator=g) * 0.1
    if with_window_qk:
        out["q_w"] = (torch.randn(B, H, T, dk, generator=g) / math.sqrt(dk)).to(dt)
        out["k_w"] = (torch.randn(B, H, T, dk, generator=g) / math.sqrt(dk)).to(dt)
    return out


def packed_lengths(n_seq, lo, hi, seed):
    """Sequence lengths of a packed (serving) batch: n_seq draws uniform in
    [lo, hi] from a seeded generator."""
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (n_seq,), generator=g).tolist()


def make_packed_inputs(lengths, H, dk, dv, n_meta, dtype="bf16", seed=0, gate_mean=2.0,
                       with_h0=False, with_window_qk=False, with_gate_logits=False):
    """A packed batch: q, k, log_alpha [H, N, dk], v [H, N, dv] (N = sum of the
    lengths), sequence b at tokens cu[b] .. cu[b+1]-1; cu_seqlens int32 [B+1];
    meta_k/meta_v [H, M, d]; optionally h0 [B, H, dk, dv] fp32, the window
    branch's q_w, k_w and bf16 gate logits gate_x.  Same value families as
    make_inputs."""
    g = torch.Generator().manual_seed(seed)
    dt = _torch_dtype(dtype)
    N, B = int(sum(lengths)), len(lengths)
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    q = torch.randn(H, N, dk, generator=g) / math.sqrt(dk)
    k = torch.randn(H, N, dk, generator=g) / math.sqrt(dk)
    v = torch.randn(H, N, dv, generator=g) / math.sqrt(dv)
    x = torch.randn(H, N, dk, generator=g) + gate_mean
    meta_k = torch.randn(H, n_meta, dk, generator=g)
    meta_v = torch.randn(H, n_meta, dv, generator=g)
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt),
               log_alpha=torch.nn.functional.logsigmoid(x).float(),
               meta_k=meta_k.to(dt), meta_v=meta_v.to(dt), cu_seqlens=cu)
    if with_h0:
        out["h0"] = torch.randn(B, H, dk, dv, generator=g) * 0.1
    if with_window_qk:
        out["q_w"] = (torch.randn(H, N, dk, generator=g) / math.sqrt(dk)).to(dt)
        out["k_w"] = (torch.randn(H, N, dk, generator=g) / math.sqrt(dk)).to(dt)
    if with_gate_logits:
        out["gate_x"] = x.to(torch.bfloat16)
    return out


def make_decode_inputs(steps, B, H, dk, dv, dtype="bf16", seed=1, gate_mean=2.0,
                       with_window_qk=False, with_gate_logits=False, **_ignored):
    """Per-step decode tokens: q, k [steps,B,H,dk]; v [steps,B,H,dv];
    log_alpha [steps,B,H,dk] fp32, drawn in the order q, k, v, x (then q_w, k_w
    [steps,B,H,dk] with with_window_qk)."""
    g = torch.Generator().manual_seed(seed)
    dt = _torch_dtype(dtype)
    q = torch.randn(steps, B, H, dk, generator=g) / math.sqrt(dk)
    k = torch.randn(steps, B, H, dk, generator=g) / math.sqrt(dk)
    v = torch.randn(steps, B, H, dv, generator=g) / math.sqrt(dv)
    x = torch.randn(steps, B, H, dk, generator=g) + gate_mean
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt),
               log_alpha=torch.nn.functional.logsigmoid(x).float())
    if with_gate_logits:
        out["gate_x"] = x.to(torch.bfloat16)
    if with_window_qk:
        out["q_w"] = (torch.randn(steps, B, H, dk, generator=g) / math.sqrt(dk)).to(dt)
        out["k_w"] = (torch.randn(steps, B, H, dk, generator=g) / math.sqrt(dk)).to(dt)
    return out


def to_f64_numpy(t):
    """Upcast a (possibly bf16) tensor exactly to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
