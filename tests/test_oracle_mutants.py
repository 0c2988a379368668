"""Planted-mistake check of the oracle's pins (CPU only).

Each case copies the oracle's source, plants one plausible slip in it (a
dropped term, a wrong index, an off-by-one window, a missing factor), loads the
copy as a separate module and runs every pin in tests/test_oracle_pins.py
against it.  A pin set that lets a slip through would fail here.
"""
import importlib.util
import inspect
import os
import types

import pytest

import oracle.lizard_oracle as real
import tests.test_oracle_pins as pins

SRC = inspect.getsource(real)

MUTANTS = {
    "decay_applied_after_outer_product": (
        "S = np.exp(la[:, :, t, :])[..., :, None] * S \\\n            + k[:, :, t, :, None] * v[:, :, t, None, :]",
        "S = np.exp(la[:, :, t, :])[..., :, None] * (S \\\n            + k[:, :, t, :, None] * v[:, :, t, None, :])"),
    "decay_on_value_columns": (
        "S = np.exp(la[:, :, t, :])[..., :, None] * S",
        "S = np.exp(la[:, :, t, :])[..., None, :] * S"),
    "readout_uses_previous_state": (
        "        o[:, :, t, :] = np.matmul(q[:, :, t, None, :], S)[:, :, 0, :]\n    return o, S",
        "        o[:, :, t, :] = np.matmul(q[:, :, t, None, :], S - k[:, :, t, :, None] * v[:, :, t, None, :])[:, :, 0, :]\n    return o, S"),
    "window_excludes_current_token": (
        "keys = np.concatenate([k[:, :, lo:t + 1, :], mkb], axis=2)\n        vals = np.concatenate([v[:, :, lo:t + 1, :], mvb], axis=2)\n        logits = scale * np.matmul(keys, q[:, :, t, :, None])[..., 0]\n        m =",
        "keys = np.concatenate([k[:, :, lo:t, :], mkb], axis=2)\n        vals = np.concatenate([v[:, :, lo:t, :], mvb], axis=2)\n        logits = scale * np.matmul(keys, q[:, :, t, :, None])[..., 0]\n        m ="),
    "window_one_token_too_wide": (
        "    for t in range(T):\n        lo = max(0, t - window + 1)\n        keys",
        "    for t in range(T):\n        lo = max(0, t - window)\n        keys"),
    "meta_values_dropped": (
        "vals = np.concatenate([v[:, :, lo:t + 1, :], mvb], axis=2)\n        logits = scale * np.matmul(keys, q[:, :, t, :, None])[..., 0]\n        m =",
        "vals = np.concatenate([v[:, :, lo:t + 1, :], 0 * mvb], axis=2)\n        logits = scale * np.matmul(keys, q[:, :, t, :, None])[..., 0]\n        m ="),
    "softmax_scale_missing": (
        "logits = scale * np.matmul(keys, q[:, :, t, :, None])[..., 0]\n        m =",
        "logits = np.matmul(keys, q[:, :, t, :, None])[..., 0]\n        m ="),
    "mix_ignored": ("o=o_gla + mix * o_swa", "o=o_gla + o_swa"),
    "ring_slot_off_by_one": ("rk[:, :, p % window, :] = k[:, :, p, :]",
                             "rk[:, :, (p + 1) % window, :] = k[:, :, p, :]"),
    "decode_slot_off_by_one": ("slot = int(pos[b] % window)", "slot = int((pos[b] + 1) % window)"),
    "decode_valid_count_short": ("n = int(min(pos[b] + 1, window))", "n = int(min(pos[b], window) or 1)"),
    "bwd_state_grad_not_decayed": ("G = alpha[:, :, t, :, None] * G", "G = G"),
    "bwd_dlog_alpha_missing_alpha": ("dla[:, :, t, :] = alpha[:, :, t, :] * (G * S_prev)",
                                     "dla[:, :, t, :] = (G * S_prev)"),
    "bwd_dq_uses_previous_state": ("dq[:, :, t, :] = np.matmul(S_t, dO", "dq[:, :, t, :] = np.matmul(S_prev, dO"),
    "bwd_dv_transposed_state": ("dv_[:, :, t, :] = np.matmul(k[:, :, t, None, :], G)[:, :, 0, :]",
                                "dv_[:, :, t, :] = np.matmul(k[:, :, t, None, :], np.swapaxes(G, -1, -2))[:, :, 0, :]"),
    "bwd_softmax_centering_dropped": ("dl = p * (dp - D)", "dl = p * dp"),
    "bwd_meta_key_grad_unscaled": ("dmk += scale * (dl", "dmk += (dl"),
    "log_sigmoid_sign_of_x": ("return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))",
                              "return np.minimum(-x, 0.0) - np.log1p(np.exp(-np.abs(x)))"),
    "log_sigmoid_tail_dropped": ("return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))",
                                 "return np.minimum(x, 0.0)"),
    "log_sigmoid_grad_wrong_side": ("np.exp(log_sigmoid(-_f64(x)))", "np.exp(log_sigmoid(_f64(x)))"),
}

PIN_TESTS = [(name, fn) for name, fn in inspect.getmembers(pins, inspect.isfunction)
             if name.startswith("test_")]


def _load_mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique/found: {old[:60]!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _run_pins_against(mod):
    failed = []
    saved = pins.oracle
    pins.oracle = mod
    try:
        for name, fn in PIN_TESTS:
            params = [{}]
            if "mix" in inspect.signature(fn).parameters:
                params = [{"mix": 1.0}, {"mix": 0.6}]
            for kw in params:
                try:
                    fn(**kw)
                except Exception:       # AssertionError, or the slip breaks a shape
                    failed.append(name)
                    break
    finally:
        pins.oracle = saved
    return failed


def test_unmutated_copy_passes_every_pin():
    mod = _load_mutant("__all__ = [", "__all__ = [")
    assert _run_pins_against(mod) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    failed = _run_pins_against(_load_mutant(old, new))
    assert failed, f"no pin catches the planted mistake {name}"
