"""ctypes view of the C ABI declared in include/lizard.h.

Argument marshalling only: every step of the computation runs in the HIP
library.  The library must have been built (see build.py); if it is missing the
first call raises instead of falling back to anything else.
"""
import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
# LIZARD_LIB may name another build of the same library (e.g. the host-sanitizer
# build of build_sanitize.py); by default the in-tree liblizard.so is loaded
LIB_PATH = os.environ.get("LIZARD_LIB") or os.path.join(HERE, "liblizard.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "lizard.h")

LIZARD_F32, LIZARD_BF16 = 0, 1
LIZARD_GATE_LOG_ALPHA, LIZARD_GATE_LOGIT = 0, 1
OP_GLA_FWD, OP_SWA_FWD, OP_HYBRID_FWD, OP_HYBRID_BWD, OP_DECODE = range(5)
STATIC_SCRATCH_BYTES = 17 << 20  # LIZARD_STATIC_SCRATCH_BYTES
STATUS = {0: "LIZARD_OK", 1: "LIZARD_E_NULL", 2: "LIZARD_E_SHAPE", 3: "LIZARD_E_DTYPE",
          4: "LIZARD_E_UNSUPPORTED", 5: "LIZARD_E_WORKSPACE", 6: "LIZARD_E_HIP",
          7: "LIZARD_E_SCRATCH"}


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("window", ctypes.c_int32), ("n_meta", ctypes.c_int32),
                ("scale", ctypes.c_float), ("mix", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("gate", ctypes.c_int32)]


class LizardError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


P = ctypes.c_void_p
_SIGS = {
    "lizard_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Desc), ctypes.c_int32]),
    "lizard_gla_fwd": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 7 + [P, ctypes.c_size_t, P]),
    "lizard_swa_fwd": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 7 + [P]),
    "lizard_hybrid_fwd": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 15 + [P, ctypes.c_size_t, P]),
    "lizard_hybrid_fwd_static": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 15 + [P]),
    "lizard_hybrid_fwd_varlen": (ctypes.c_int, [ctypes.POINTER(Desc), P, ctypes.c_int32]
                                 + [P] * 13 + [P, ctypes.c_size_t, P]),
    "lizard_hybrid_bwd": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 23 + [P, ctypes.c_size_t, P]),
    "lizard_hybrid_fwd_segment": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 15
                                  + [ctypes.c_int32, P, ctypes.c_size_t, P]),
    "lizard_hybrid_bwd_segment": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 25
                                  + [ctypes.c_int32] + [P] * 4 + [ctypes.c_int32]
                                  + [P, ctypes.c_size_t, P]),
    "lizard_decode_step": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 13 + [P]),
    "lizard_window_cache_fill": (ctypes.c_int, [ctypes.POINTER(Desc)] + [P] * 4
                                 + [ctypes.c_int32, ctypes.c_int64, P, P, P]),
    "lizard_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "lizard_version": (ctypes.c_int32, []),
}

_lib = None


def lib():
    """Load liblizard.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def header_symbols():
    """Names of the functions declared in include/lizard.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(lizard_[a-z_0-9]+)\s*\(", text)))


def check(fn, status):
    if status != 0:
        raise LizardError(fn, status, lib().lizard_status_str(status).decode())
