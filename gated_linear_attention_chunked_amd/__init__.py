"""MI355X (gfx950) hybrid attention: chunked gated linear attention plus a
sliding-window + meta-memory softmax branch, with backward and a constant-memory
decode step.

The functions below are a thin torch-facing binding over the C ABI in
include/lizard.h (same names without the `lizard_` prefix).  torch only
allocates device memory and supplies the current HIP stream; every step of the
computation runs in liblizard.so.  Shapes follow the ABI: q, k [B,H,T,dk];
v [B,H,T,dv]; log_alpha [B,H,T,dk] float32; meta_k [H,M,dk]; meta_v [H,M,dv];
states [B,H,dk,dv] float32.  Wherever log_alpha is taken it may instead be a
bfloat16 tensor of gate logits x (alpha = sigmoid(x), bf16 problems only); the
gradient returned as dlog_alpha is then the float32 gradient with respect to x.
"""
import ctypes
import math

import torch

from . import _abi
from ._abi import LizardError, lib  # noqa: F401

__all__ = ["gla_fwd", "swa_fwd", "hybrid_fwd", "hybrid_fwd_varlen", "hybrid_bwd", "decode_step",
           "window_cache_fill", "workspace_bytes", "make_desc", "LizardError", "lib"]

_DTYPES = {torch.float32: _abi.LIZARD_F32, torch.bfloat16: _abi.LIZARD_BF16}


def make_desc(B, H, T, dk, dv, window=1, n_meta=0, scale=None, mix=1.0, dtype=torch.bfloat16,
              chunk=64, gate=_abi.LIZARD_GATE_LOG_ALPHA):
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    return _abi.Desc(B, H, T, dk, dv, chunk, window, n_meta,
                     0.0 if scale is None else float(scale), float(mix), _DTYPES[dtype], gate)


def _gate(log_alpha, name, shape):
    """The gate input is float32 log alpha, or bfloat16 logits x with
    alpha = sigmoid(x).  Returns the desc gate code."""
    if log_alpha is not None and log_alpha.dtype == torch.bfloat16:
        _need(log_alpha, name, shape, torch.bfloat16)
        return _abi.LIZARD_GATE_LOGIT
    _need(log_alpha, name, shape, torch.float32)
    return _abi.LIZARD_GATE_LOG_ALPHA


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, shape, dtype):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, name, shape, dtype):
    return None if t is None else _need(t, name, shape, dtype)


def _meta_pair(meta_k, meta_v, H, dk, dv, dt):
    if meta_k is None:
        meta_k = torch.empty(H, 0, dk, device="cuda", dtype=dt)
        meta_v = torch.empty(H, 0, dv, device="cuda", dtype=dt)
    M = meta_k.shape[1]
    _need(meta_k, "meta_k", (H, M, dk), dt)
    _need(meta_v, "meta_v", (H, M, dv), dt)
    return meta_k, meta_v, M


def workspace_bytes(desc, op):
    return int(lib().lizard_workspace_bytes(ctypes.byref(desc), op))


def gla_fwd(q, k, v, log_alpha, h0=None, return_state=False):
    """GLA branch alone: o_t = q_t S_t.  Returns o, or (o, hT) with return_state."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q", (B, H, T, dk), dt)
    _need(k, "k", (B, H, T, dk), dt)
    _need(v, "v", (B, H, T, dv), dt)
    gate = _gate(log_alpha, "log_alpha", (B, H, T, dk))
    _opt(h0, "h0", (B, H, dk, dv), torch.float32)
    o = torch.empty_like(v)
    hT = torch.empty(B, H, dk, dv, device=q.device, dtype=torch.float32) if return_state else None
    d = make_desc(B, H, T, dk, dv, dtype=dt, gate=gate)
    nws = workspace_bytes(d, _abi.OP_GLA_FWD)
    ws = torch.empty(nws, device=q.device, dtype=torch.uint8) if nws else None
    _abi.check("lizard_gla_fwd", lib().lizard_gla_fwd(
        ctypes.byref(d), _p(q), _p(k), _p(v), _p(log_alpha), _p(h0), _p(o), _p(hT),
        _p(ws), nws, _stream()))
    return (o, hT) if return_state else o


def swa_fwd(q, k, v, meta_k, meta_v, window, scale=None, return_lse=False):
    """Window + meta branch alone.  Returns o_swa, or (o_swa, lse)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q", (B, H, T, dk), dt)
    _need(k, "k", (B, H, T, dk), dt)
    _need(v, "v", (B, H, T, dv), dt)
    meta_k, meta_v, M = _meta_pair(meta_k, meta_v, H, dk, dv, dt)
    o = torch.empty_like(v)
    lse = torch.empty(B, H, T, device=q.device, dtype=torch.float32) if return_lse else None
    d = make_desc(B, H, T, dk, dv, window, M, scale, 1.0, dt)
    _abi.check("lizard_swa_fwd", lib().lizard_swa_fwd(
        ctypes.byref(d), _p(q), _p(k), _p(v), _p(meta_k), _p(meta_v), _p(o), _p(lse), _stream()))
    return (o, lse) if return_lse else o


def _window_pair(q_w, k_w, shape, dt):
    if (q_w is None) != (k_w is None):
        raise ValueError("q_w and k_w: give both or neither")
    if q_w is not None:
        _need(q_w, "q_w", shape, dt)
        _need(k_w, "k_w", shape, dt)


def _halo_pair(halo_k, halo_v, B, H, dk, dv, dt, window):
    """The window halo of a segment: [B, H, L, d] keys and values of the L tokens
    before it (L <= window - 1).  Returns L (0 without a halo)."""
    if (halo_k is None) != (halo_v is None):
        raise ValueError("halo_k and halo_v: give both or neither")
    if halo_k is None:
        return 0
    L = halo_k.shape[2]
    if L > window - 1:
        raise ValueError(f"a halo of {L} tokens exceeds window - 1 = {window - 1}")
    _need(halo_k, "halo_k", (B, H, L, dk), dt)
    _need(halo_v, "halo_v", (B, H, L, dv), dt)
    return L


def hybrid_fwd(q, k, v, log_alpha, meta_k, meta_v, window, scale=None, mix=1.0, h0=None,
               save_for_backward=False, return_state=False, return_ring=False, q_w=None,
               k_w=None, halo_k=None, halo_v=None):
    """o = o_gla + mix * o_swa.  Returns a dict with "o" and, on request, "lse" and
    "o_swa" (save_for_backward), "hT" (return_state), "ring_k"/"ring_v" (return_ring).
    q_w, k_w (optional, both or neither): the window branch's own queries and keys.
    halo_k, halo_v (optional, [B, H, L, d], L <= window - 1): the window keys and
    values of the L tokens before this segment of a longer sequence (segment-wise
    runs; no window cache output then)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q", (B, H, T, dk), dt)
    _need(k, "k", (B, H, T, dk), dt)
    _window_pair(q_w, k_w, (B, H, T, dk), dt)
    _need(v, "v", (B, H, T, dv), dt)
    gate = _gate(log_alpha, "log_alpha", (B, H, T, dk))
    meta_k, meta_v, M = _meta_pair(meta_k, meta_v, H, dk, dv, dt)
    _opt(h0, "h0", (B, H, dk, dv), torch.float32)
    dev = q.device
    out = {"o": torch.empty_like(v)}
    if save_for_backward:
        out["lse"] = torch.empty(B, H, T, device=dev, dtype=torch.float32)
        out["o_swa"] = torch.empty_like(v)
    if return_state:
        out["hT"] = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    if return_ring:
        out["ring_k"] = torch.empty(B, H, window, dk, device=dev, dtype=dt)
        out["ring_v"] = torch.empty(B, H, window, dv, device=dev, dtype=dt)
    L = _halo_pair(halo_k, halo_v, B, H, dk, dv, dt, window)
    if L and return_ring:
        raise ValueError("a segment with a halo returns no window cache")
    d = make_desc(B, H, T, dk, dv, window, M, scale, mix, dt, gate=gate)
    nws = workspace_bytes(d, _abi.OP_HYBRID_FWD)
    ws = torch.empty(nws, device=dev, dtype=torch.uint8) if nws else None
    if halo_k is not None:
        _abi.check("lizard_hybrid_fwd_segment", lib().lizard_hybrid_fwd_segment(
            ctypes.byref(d), _p(q), _p(k), _p(v), _p(log_alpha), _p(meta_k), _p(meta_v),
            _p(h0), _p(out["o"]), _p(out.get("lse")), _p(out.get("o_swa")), _p(out.get("hT")),
            _p(q_w), _p(k_w), _p(halo_k), _p(halo_v), L, _p(ws), nws, _stream()))
        return out
    _abi.check("lizard_hybrid_fwd", lib().lizard_hybrid_fwd(
        ctypes.byref(d), _p(q), _p(k), _p(v), _p(log_alpha), _p(meta_k), _p(meta_v), _p(h0),
        _p(out["o"]), _p(out.get("lse")), _p(out.get("o_swa")), _p(out.get("hT")),
        _p(out.get("ring_k")), _p(out.get("ring_v")), _p(q_w), _p(k_w), _p(ws), nws, _stream()))
    return out


def hybrid_fwd_varlen(q, k, v, log_alpha, meta_k, meta_v, window, cu_seqlens, max_seqlen=None,
                      scale=None, mix=1.0, h0=None, return_state=False, return_ring=False,
                      q_w=None, k_w=None, check_lengths=True):
    """Hybrid forward over a packed batch: q, k, log_alpha (and q_w, k_w) [H, N, dk],
    v [H, N, dv]; sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 (int32
    device tensor [B+1]); max_seqlen bounds every length (None: taken from
    cu_seqlens).  With check_lengths (the default) cu_seqlens is read back to the
    host once and must start at 0, be non-decreasing, end at N and have no length
    above max_seqlen, else ValueError; a caller that guarantees this may pass
    check_lengths=False and a max_seqlen to avoid the read-back.  Returns a dict
    with "o" [H, N, dv] and, on request, the per-sequence "hT" [B,H,dk,dv] and
    "ring_k"/"ring_v" [B,H,w,d]."""
    H, N, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    B = cu_seqlens.shape[0] - 1
    _need(q, "q", (H, N, dk), dt)
    _need(k, "k", (H, N, dk), dt)
    _need(v, "v", (H, N, dv), dt)
    _need(cu_seqlens, "cu_seqlens", (B + 1,), torch.int32)
    if check_lengths or max_seqlen is None:
        cu = cu_seqlens.cpu().tolist()
        lens = [b - a for a, b in zip(cu[:-1], cu[1:])]
        longest = max(lens, default=0)
        if check_lengths:
            if cu[0] != 0 or cu[-1] != N or any(n < 0 for n in lens):
                raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at N")
            if max_seqlen is not None and longest > max_seqlen:
                raise ValueError(f"a sequence of {longest} tokens exceeds max_seqlen={max_seqlen}")
        if max_seqlen is None:
            max_seqlen = max(longest, 1)
    _window_pair(q_w, k_w, (H, N, dk), dt)
    gate = _gate(log_alpha, "log_alpha", (H, N, dk))
    meta_k, meta_v, M = _meta_pair(meta_k, meta_v, H, dk, dv, dt)
    _opt(h0, "h0", (B, H, dk, dv), torch.float32)
    dev = q.device
    out = {"o": torch.empty_like(v)}
    if return_state:
        out["hT"] = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    if return_ring:
        out["ring_k"] = torch.empty(B, H, window, dk, device=dev, dtype=dt)
        out["ring_v"] = torch.empty(B, H, window, dv, device=dev, dtype=dt)
    d = make_desc(B, H, int(max_seqlen), dk, dv, window, M, scale, mix, dt, gate=gate)
    nws = workspace_bytes(d, _abi.OP_HYBRID_FWD)
    ws = torch.empty(nws, device=dev, dtype=torch.uint8) if nws else None
    _abi.check("lizard_hybrid_fwd_varlen", lib().lizard_hybrid_fwd_varlen(
        ctypes.byref(d), _p(cu_seqlens), N, _p(q), _p(k), _p(v), _p(log_alpha), _p(meta_k),
        _p(meta_v), _p(h0), _p(out["o"]), _p(out.get("hT")), _p(out.get("ring_k")),
        _p(out.get("ring_v")), _p(q_w), _p(k_w), _p(ws), nws, _stream()))
    return out


def hybrid_bwd(q, k, v, log_alpha, meta_k, meta_v, window, o_swa, lse, dO, scale=None, mix=1.0,
               h0=None, dhT=None, return_dh0=False, return_dmix=False, q_w=None, k_w=None,
               halo_k=None, halo_v=None, return_dhalo=False, tail_dk=None, tail_dv=None):
    """Gradients of sum(dO * o) + sum(dhT * hT) (dhT: the gradient of the final
    state, optional).  Returns a dict dq, dk, dv, dlog_alpha, dmeta_k, dmeta_v and,
    with return_dh0, dh0 (the gradient of the initial state), with return_dmix,
    dmix (a one-element float32 tensor, the gradient of the mix weight).  With the
    window branch's own q_w, k_w, dq and dk are the gated branch's gradients and
    the dict also holds dq_w, dk_w.  Segment-wise runs: halo_k, halo_v as given to
    hybrid_fwd (with return_dhalo the dict holds their float32 gradients dhalo_k,
    dhalo_v), and tail_dk, tail_dv [B, H, L, d] float32, the next segment's dhalo,
    added to the gradients of this segment's last L window keys and values."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    _need(q, "q", (B, H, T, dk), dt)
    _need(k, "k", (B, H, T, dk), dt)
    _window_pair(q_w, k_w, (B, H, T, dk), dt)
    _need(v, "v", (B, H, T, dv), dt)
    gate = _gate(log_alpha, "log_alpha", (B, H, T, dk))
    meta_k, meta_v, M = _meta_pair(meta_k, meta_v, H, dk, dv, dt)
    _opt(h0, "h0", (B, H, dk, dv), torch.float32)
    _opt(dhT, "dhT", (B, H, dk, dv), torch.float32)
    _need(o_swa, "o_swa", (B, H, T, dv), dt)
    _need(lse, "lse", (B, H, T), torch.float32)
    _need(dO, "dO", (B, H, T, dv), dt)
    dev = q.device
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "dlog_alpha": torch.empty(log_alpha.shape, device=dev, dtype=torch.float32),
         "dmeta_k": torch.empty(H, M, dk, device=dev, dtype=torch.float32),
         "dmeta_v": torch.empty(H, M, dv, device=dev, dtype=torch.float32)}
    if return_dh0:
        g["dh0"] = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    if return_dmix:
        g["dmix"] = torch.empty(1, device=dev, dtype=torch.float32)
    if q_w is not None:
        g["dq_w"] = torch.empty_like(q_w)
        g["dk_w"] = torch.empty_like(k_w)
    L = _halo_pair(halo_k, halo_v, B, H, dk, dv, dt, window)
    if (tail_dk is None) != (tail_dv is None):
        raise ValueError("tail_dk and tail_dv: give both or neither")
    Lt = 0 if tail_dk is None else tail_dk.shape[2]
    if tail_dk is not None:
        _need(tail_dk, "tail_dk", (B, H, Lt, dk), torch.float32)
        _need(tail_dv, "tail_dv", (B, H, Lt, dv), torch.float32)
    if return_dhalo and L:
        g["dhalo_k"] = torch.empty(B, H, L, dk, device=dev, dtype=torch.float32)
        g["dhalo_v"] = torch.empty(B, H, L, dv, device=dev, dtype=torch.float32)
    d = make_desc(B, H, T, dk, dv, window, M, scale, mix, dt, gate=gate)
    nws = workspace_bytes(d, _abi.OP_HYBRID_BWD)
    ws = torch.empty(max(nws, 1), device=dev, dtype=torch.uint8)
    if L or Lt:
        _abi.check("lizard_hybrid_bwd_segment", lib().lizard_hybrid_bwd_segment(
            ctypes.byref(d), _p(q), _p(k), _p(v), _p(log_alpha), _p(meta_k), _p(meta_v),
            _p(h0), _p(o_swa), _p(lse), _p(dO), _p(g["dq"]), _p(g["dk"]), _p(g["dv"]),
            _p(g["dlog_alpha"]), _p(g["dmeta_k"]), _p(g["dmeta_v"]), _p(dhT), _p(g.get("dh0")),
            _p(g.get("dmix")), _p(q_w), _p(k_w), _p(g.get("dq_w")), _p(g.get("dk_w")),
            _p(halo_k), _p(halo_v), L, _p(g.get("dhalo_k")), _p(g.get("dhalo_v")),
            _p(tail_dk), _p(tail_dv), Lt, _p(ws), nws, _stream()))
        return g
    _abi.check("lizard_hybrid_bwd", lib().lizard_hybrid_bwd(
        ctypes.byref(d), _p(q), _p(k), _p(v), _p(log_alpha), _p(meta_k), _p(meta_v), _p(h0),
        _p(o_swa), _p(lse), _p(dO), _p(g["dq"]), _p(g["dk"]), _p(g["dv"]), _p(g["dlog_alpha"]),
        _p(g["dmeta_k"]), _p(g["dmeta_v"]), _p(dhT), _p(g.get("dh0")), _p(g.get("dmix")),
        _p(q_w), _p(k_w), _p(g.get("dq_w")), _p(g.get("dk_w")), _p(ws), nws, _stream()))
    return g


def decode_step(q, k, v, log_alpha, state, ring_k, ring_v, pos, meta_k, meta_v, scale=None,
                mix=1.0, out=None, q_w=None, k_w=None):
    """One generation step for B sequences.  Updates state, ring_k/ring_v and pos
    (int64 [B], device) in place and returns o [B,H,dv].  q_w, k_w (optional, both
    or neither): the window branch's own query and key."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = q.dtype
    window = ring_k.shape[2]
    _need(q, "q", (B, H, dk), dt)
    _need(k, "k", (B, H, dk), dt)
    _window_pair(q_w, k_w, (B, H, dk), dt)
    _need(v, "v", (B, H, dv), dt)
    gate = _gate(log_alpha, "log_alpha", (B, H, dk))
    _need(state, "state", (B, H, dk, dv), torch.float32)
    _need(ring_k, "ring_k", (B, H, window, dk), dt)
    _need(ring_v, "ring_v", (B, H, window, dv), dt)
    _need(pos, "pos", (B,), torch.int64)
    meta_k, meta_v, M = _meta_pair(meta_k, meta_v, H, dk, dv, dt)
    o = torch.empty(B, H, dv, device=q.device, dtype=dt) if out is None else _need(
        out, "out", (B, H, dv), dt)
    d = make_desc(B, H, 0, dk, dv, window, M, scale, mix, dt, gate=gate)
    _abi.check("lizard_decode_step", lib().lizard_decode_step(
        ctypes.byref(d), _p(q), _p(k), _p(v), _p(log_alpha), _p(state), _p(ring_k), _p(ring_v),
        _p(pos), _p(meta_k), _p(meta_v), _p(q_w), _p(k_w), _p(o), _stream()))
    return o


def window_cache_fill(k, v, window, pos0, halo_k=None, halo_v=None, ring_k=None,
                      ring_v=None):
    """Decode window cache after a prefill run in segments.  k, v [B, H, T, d]:
    the last segment's window keys (k_w when the window branch has its own) and
    values, at positions pos0 .. pos0+T-1; halo_k, halo_v [B, H, L, d]: the L
    tokens before it (L <= window; when T < window at least min(pos0, window - T)
    of them).  Returns (ring_k, ring_v) [B, H, window, d]: slot p mod window holds
    token p for the last min(window, pos0 + T) positions, zeros elsewhere."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    _need(k, "k", (B, H, T, dk), dt)
    _need(v, "v", (B, H, T, dv), dt)
    if (halo_k is None) != (halo_v is None):
        raise ValueError("halo_k and halo_v: give both or neither")
    L = 0
    if halo_k is not None:
        L = halo_k.shape[2]
        _need(halo_k, "halo_k", (B, H, L, dk), dt)
        _need(halo_v, "halo_v", (B, H, L, dv), dt)
    dev = k.device
    rk = torch.empty(B, H, window, dk, device=dev, dtype=dt) if ring_k is None else _need(
        ring_k, "ring_k", (B, H, window, dk), dt)
    rv = torch.empty(B, H, window, dv, device=dev, dtype=dt) if ring_v is None else _need(
        ring_v, "ring_v", (B, H, window, dv), dt)
    d = make_desc(B, H, T, dk, dv, window, 0, None, 1.0, dt)
    _abi.check("lizard_window_cache_fill", lib().lizard_window_cache_fill(
        ctypes.byref(d), _p(k), _p(v), _p(halo_k), _p(halo_v), L, int(pos0), _p(rk), _p(rv),
        _stream()))
    return rk, rv


def default_scale(dk):
    return 1.0 / math.sqrt(dk)
