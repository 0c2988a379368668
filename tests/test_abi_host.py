"""Host-side checks of the C ABI (no GPU needed).

The library validates every argument before it touches HIP, so these run on a
machine without a GPU: the shared library loads, exports every function that
include/lizard.h declares, and maps each kind of bad argument to its status.
"""
import ctypes
import os
import subprocess

import pytest

from gated_linear_attention_chunked_amd import _abi

pytestmark = pytest.mark.skipif(not os.path.exists(_abi.LIB_PATH),
                                reason="liblizard.so not built")

NULLP = None


def desc(**kw):
    base = dict(B=1, H=2, T=128, dk=64, dv=64, chunk=64, window=64, n_meta=4, scale=0.0, mix=1.0,
                dtype=_abi.LIZARD_BF16, gate=_abi.LIZARD_GATE_LOG_ALPHA)
    base.update(kw)
    return _abi.Desc(base["B"], base["H"], base["T"], base["dk"], base["dv"], base["chunk"],
                     base["window"], base["n_meta"], base["scale"], base["mix"], base["dtype"],
                     base["gate"])


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails validation first


def gla(d, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, la=FAKE, h0=None, o=FAKE, hT=None)
    p.update(ptrs)
    return _abi.lib().lizard_gla_fwd(ctypes.byref(d) if d is not None else None, p["q"], p["k"],
                                     p["v"], p["la"], p["h0"], p["o"], p["hT"], None, 0, None)


def test_exports_every_declared_symbol():
    declared = _abi.header_symbols()
    assert set(declared) >= {"lizard_gla_fwd", "lizard_swa_fwd", "lizard_hybrid_fwd",
                             "lizard_hybrid_bwd", "lizard_decode_step", "lizard_status_str",
                             "lizard_workspace_bytes", "lizard_version"}
    lib = _abi.lib()
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared) <= exported


def test_status_strings_and_version():
    lib = _abi.lib()
    for code in range(8):
        assert lib.lizard_status_str(code)
    assert lib.lizard_status_str(99) == b"unknown status"
    assert lib.lizard_version() == 10200


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 3), (dict(gate=2), 3), (dict(gate=-1), 3),
    (dict(gate=_abi.LIZARD_GATE_LOGIT, dtype=_abi.LIZARD_F32), 4),
    (dict(B=-1), 2), (dict(T=-5), 2), (dict(dk=0), 2), (dict(window=0), 2), (dict(n_meta=-1), 2),
    (dict(chunk=0), 2), (dict(scale=float("nan")), 2), (dict(mix=float("inf")), 2),
    (dict(chunk=32), 4), (dict(dk=96, dv=96), 4), (dict(dk=64, dv=128), 4),
    (dict(n_meta=17), 4),
    (dict(B=300, H=300), 4),
])
def test_bad_descriptor_is_rejected_before_launch(kw, status):
    assert gla(desc(**kw)) == status


def test_null_pointers():
    assert gla(None) == 1
    assert gla(desc(), q=None) == 1
    assert gla(desc(), la=None) == 1
    lib = _abi.lib()
    d = desc()
    # meta slots requested but no meta pointers
    assert lib.lizard_swa_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, None, None) == 1
    # one ring pointer without the other
    assert lib.lizard_hybrid_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                 None, None, None, FAKE, None, None, None, None, 0, None) == 1
    assert lib.lizard_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, None, None, FAKE, None) == 1


def test_window_inputs_come_in_pairs():
    # the window branch's own queries and keys: both or neither (and, in the
    # backward, with both their gradient outputs)
    lib = _abi.lib()
    d = desc()
    for qw, kw in ((FAKE, None), (None, FAKE)):
        assert lib.lizard_hybrid_fwd(ctypes.byref(d), *([FAKE] * 13), qw, kw, FAKE, 1 << 30,
                                     None) == 1
        assert lib.lizard_decode_step(ctypes.byref(d), *([FAKE] * 10), qw, kw, FAKE, None) == 1
    for four in ((FAKE, FAKE, FAKE, None), (FAKE, None, None, None), (None, None, FAKE, FAKE)):
        assert lib.lizard_hybrid_bwd(ctypes.byref(d), *([FAKE] * 19), *four, FAKE, 1 << 30,
                                     None) == 1


def test_packed_forward_arguments_are_checked():
    lib = _abi.lib()
    d = desc(dk=128, dv=128, T=4096)
    need = lib.lizard_workspace_bytes(ctypes.byref(d), 2)
    call = lambda dd, cu=FAKE, n=100, ws_bytes=need, qw=None, kw=None: lib.lizard_hybrid_fwd_varlen(
        ctypes.byref(dd), cu, n, *([FAKE] * 6), None, FAKE, None, None, None, qw, kw, FAKE,
        ws_bytes, None)
    assert call(d, n=-1) == 2
    assert call(d, cu=None) == 1
    assert call(d, qw=FAKE) == 1
    assert call(d, ws_bytes=need - 1) == 5
    assert call(desc(T=4096, dtype=_abi.LIZARD_F32, gate=_abi.LIZARD_GATE_LOGIT)) == 4  # logits: bf16
    assert call(desc(T=4096, dtype=_abi.LIZARD_F32), cu=None) == 1  # fp32 packed: checked like bf16
    assert call(desc(dk=128, dv=128, T=0)) == 4               # the longest length must be >= 1
    assert call(desc(dk=128, dv=128, T=4096, B=0)) == 0       # nothing to do


def test_window_cache_fill_arguments_are_checked():
    # cache from the last segment of a segmented prefill: the halo must hold the
    # positions before the segment that the last w of pos0 + T keep
    lib = _abi.lib()
    call = lambda d, halo_len, pos0, k=FAKE, hk=FAKE, rk=FAKE: lib.lizard_window_cache_fill(
        ctypes.byref(d), k, FAKE, hk, FAKE, halo_len, pos0, rk, FAKE, None)
    d = desc(T=50, window=64)                 # T < w: min(pos0, 14) halo tokens needed
    assert call(d, 13, 100) == 2
    assert call(d, 10, 10, hk=None) == 1      # enough halo, but no halo pointer
    assert call(d, 14, 100, rk=None) == 1
    assert call(d, 5, -1) == 2                # negative start
    assert call(d, 65, 100) == 2              # more than w halo tokens
    assert call(d, 6, 5) == 2                 # more halo than tokens before
    assert call(desc(T=0, window=64), 63, 100) == 2   # an empty segment needs all w
    assert call(desc(T=70, window=64, B=0), 0, 100, k=None, hk=None, rk=None) == 0
    assert call(desc(T=70, window=64), 0, 100, k=None) == 1


def test_empty_problems_enqueue_nothing():
    # B*H == 0: valid, nothing to do, no HIP call
    assert gla(desc(B=0), q=None, k=None, v=None, la=None, o=None) == 0
    lib = _abi.lib()
    d = desc(H=0)
    assert lib.lizard_swa_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None) == 0


def test_workspace_query():
    lib = _abi.lib()
    for op in (1, 4):
        assert lib.lizard_workspace_bytes(ctypes.byref(desc()), op) == 0
    # forward: per-segment states, bounded and independent of T for long sequences
    f1 = lib.lizard_workspace_bytes(ctypes.byref(desc(B=1, H=32, T=4096, dk=128, dv=128)), 0)
    f2 = lib.lizard_workspace_bytes(ctypes.byref(desc(B=1, H=32, T=32768, dk=128, dv=128)), 2)
    assert f1 == f2 == 32 * 7 * (128 * 128 + 128) * 4
    assert lib.lizard_workspace_bytes(ctypes.byref(desc(B=64, H=32, T=4096)), 0) == 0
    assert lib.lizard_workspace_bytes(None, 3) == 0
    assert lib.lizard_workspace_bytes(ctypes.byref(desc(dtype=9)), 3) == 0
    a = lib.lizard_workspace_bytes(ctypes.byref(desc(T=1024)), 3)
    b = lib.lizard_workspace_bytes(ctypes.byref(desc(T=4096)), 3)
    assert a >= 0 and b >= a


def test_forward_rejects_small_workspace():
    lib = _abi.lib()
    d = desc(T=4096)
    need = lib.lizard_workspace_bytes(ctypes.byref(d), 0)
    assert need > 0
    assert gla(d) == 5  # no workspace passed
    st = lib.lizard_hybrid_fwd(ctypes.byref(d), *([FAKE] * 15), FAKE, need - 1, None)
    assert st == 5


def test_backward_workspace_and_support():
    lib = _abi.lib()
    d = desc(T=256)
    need = lib.lizard_workspace_bytes(ctypes.byref(d), 3)
    assert need > 0
    st = lib.lizard_hybrid_bwd(ctypes.byref(d), *([FAKE] * 23), FAKE, need - 1, None)
    assert st == 5
    # the backward covers d = 64 and 128 in both precisions
    for kw in (dict(dk=128, dv=128), dict(dtype=_abi.LIZARD_F32),
               dict(dk=128, dv=128, dtype=_abi.LIZARD_F32)):
        assert lib.lizard_workspace_bytes(ctypes.byref(desc(**kw)), 3) > 0
    d2 = desc(dk=96, dv=96)
    assert lib.lizard_workspace_bytes(ctypes.byref(d2), 3) == 0
    assert lib.lizard_hybrid_bwd(ctypes.byref(d2), *([FAKE] * 23), FAKE, 1 << 30, None) == 4


@pytest.mark.parametrize("kw", [dict(), dict(dk=128, dv=128), dict(dtype=_abi.LIZARD_F32),
                                dict(dk=128, dv=128, dtype=_abi.LIZARD_F32),
                                dict(B=8, H=16, window=200, n_meta=16)])
def test_backward_workspace_does_not_grow_with_T(kw):
    # the GLA part holds a fixed number of chunk states per head and the window
    # part a fixed number of meta partials per head, whatever the sequence length
    lib = _abi.lib()
    sizes = {T: lib.lizard_workspace_bytes(ctypes.byref(desc(T=T, **kw)), 3)
             for T in (1, 64, 1024, 2048, 32768, 262144)}
    assert len(set(sizes.values())) == 1, sizes
    assert sizes[1] > 0


def test_static_scratch_entry_checks_arguments_first():
    # the allocation-free forward runs lizard_hybrid_fwd's checks before any HIP
    # call (here: no GPU at all), and declares the size of its fixed array
    lib = _abi.lib()
    with open(_abi.HEADER) as f:
        assert "#define LIZARD_STATIC_SCRATCH_BYTES ((size_t)17 << 20)" in f.read()
    assert _abi.STATIC_SCRATCH_BYTES == 17 << 20
    call = lambda dd, *p: lib.lizard_hybrid_fwd_static(dd, *p, None)
    assert call(None, *([FAKE] * 15)) == 1
    assert call(ctypes.byref(desc(dk=96, dv=96)), *([FAKE] * 15)) == 4
    assert call(ctypes.byref(desc(dtype=7)), *([FAKE] * 15)) == 3
    assert call(ctypes.byref(desc()), FAKE, None, *([FAKE] * 13)) == 1
    assert call(ctypes.byref(desc(B=0, n_meta=0)), *([None] * 15)) == 0
    # the largest forward workspace of any accepted shape fits the array
    worst = max(lib.lizard_workspace_bytes(ctypes.byref(desc(B=1, H=h, T=65536, dk=128, dv=128)), 2)
                for h in range(1, 300))
    assert 0 < worst <= _abi.STATIC_SCRATCH_BYTES


def test_segment_entry_points_check_halo_and_tail():
    lib = _abi.lib()
    d = desc(T=128, window=64)
    need_f = lib.lizard_workspace_bytes(ctypes.byref(d), 2)
    need_b = lib.lizard_workspace_bytes(ctypes.byref(d), 3)
    fwd = lambda hk, hv, n: lib.lizard_hybrid_fwd_segment(ctypes.byref(d), *([FAKE] * 11), None,
                                                          None, hk, hv, n, FAKE, need_f, None)
    assert fwd(FAKE, FAKE, 64) == 2   # a halo longer than w - 1
    assert fwd(FAKE, FAKE, -1) == 2
    assert fwd(None, FAKE, 10) == 1   # halo tokens without keys
    bwd = lambda hlen, dh, tl, tail: lib.lizard_hybrid_bwd_segment(
        ctypes.byref(d), *([FAKE] * 19), None, None, None, None, FAKE, FAKE, hlen, dh[0], dh[1],
        tail, tail, tl, FAKE, need_b, None)
    assert bwd(64, (None, None), 0, None) == 2
    assert bwd(10, (FAKE, None), 0, None) == 1      # one halo gradient without the other
    assert bwd(0, (None, None), 64, FAKE) == 2      # tail longer than w - 1
    assert bwd(0, (None, None), 10, None) == 1      # tail length without the gradients
    d2 = desc(T=8, window=64)
    assert lib.lizard_hybrid_bwd_segment(
        ctypes.byref(d2), *([FAKE] * 19), None, None, None, None, None, None, 0, None, None,
        FAKE, FAKE, 9, FAKE, 1 << 30, None) == 2    # tail longer than the segment
