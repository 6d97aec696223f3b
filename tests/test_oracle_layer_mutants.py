"""The prologue / epilogue pins must catch plausible mistakes in the oracle.

Each mutant is a copy of oracle/layer.py with one deliberate mistake (taps
reversed, a history off by one token, no reset at sequence boundaries, a
missing square root, a norm over the wrong axis, a sign flip, a mean taken
as a sum, a dropped weight or gate); it is loaded as a separate module and
every pin in test_oracle_layer_pins.py is run against it: at least one must
fail.  The real oracle is untouched.
"""
import importlib.util
import os
import tempfile

import pytest

from oracle import layer as ORACLE
import test_oracle_layer_pins as pins

SRC = open(ORACLE.__file__).read()

MUTANTS = {
    "conv taps reversed": ("w[:, CONV_WIDTH - 1 - j] * ext", "w[:, j] * ext"),
    "conv history off by one": ("new_hist[n] = ext[L:L + CONV_WIDTH - 1]",
                                "new_hist[n] = ext[L + 1:L + CONV_WIDTH]"),
    "no reset between sequences": ("bounds = _seq_bounds(T, cu_seqlens)",
                                   "bounds = _seq_bounds(T, None) * (1 if cu_seqlens is None else len(cu_seqlens) - 1)"),
    "history ignored": ("hist = np.zeros((CONV_WIDTH - 1, C)) if history is None else _f64(history[n])",
                        "hist = np.zeros((CONV_WIDTH - 1, C))"),
    "swish without the input factor": ("return y * sigmoid(y)", "return sigmoid(y)"),
    "l2 norm without sqrt": ("x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
                             "x / (np.sum(x * x, axis=-1, keepdims=True) + eps)"),
    "l2 norm over heads": ("x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
                           "x / np.sqrt(np.sum(x * x, axis=-2, keepdims=True) + eps)"),
    "decay sign": ("DECAY_LOWER * sigmoid(_f64(a) + _f64(bias)[None])",
                   "DECAY_LOWER * sigmoid(-(_f64(a) + _f64(bias)[None]))"),
    "decay bias dropped": ("DECAY_LOWER * sigmoid(_f64(a) + _f64(bias)[None])",
                           "DECAY_LOWER * sigmoid(_f64(a))"),
    "rms as a sum": ("np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)",
                     "np.sqrt(np.sum(o * o, axis=-1, keepdims=True) + eps)"),
    "rms weight dropped": ("return o / r * _f64(w)[None]", "return o / r"),
    "gate dropped": ("return head_rmsnorm(o, norm_w, eps) * sigmoid(g)",
                     "return head_rmsnorm(o, norm_w, eps)"),
    "v normalised too": ("q, k = l2_normalize(q, l2_eps), l2_normalize(k, l2_eps)",
                         "q, k, v = (l2_normalize(q, l2_eps), l2_normalize(k, l2_eps),\n"
                         "               l2_normalize(v, l2_eps))"),
    "k left unnormalised": ("q, k = l2_normalize(q, l2_eps), l2_normalize(k, l2_eps)",
                            "q = l2_normalize(q, l2_eps)"),
    "conv state in wrong slot": ("states[:, i] = nh.reshape(N, 3, H, D)",
                                 "states[:, 2 - i] = nh.reshape(N, 3, H, D)"),
}


def _load(src, name):
    d = tempfile.mkdtemp()
    path = os.path.join(d, name + ".py")
    with open(path, "w") as f:
        f.write(src)
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_real_oracle_passes_every_pin():
    for p in pins.PINS:
        p(ORACLE)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = _load(SRC.replace(old, new), "layer_mutant")
    caught = []
    for p in pins.PINS:
        try:
            p(mod)
        except Exception as e:  # an assertion or a shape error both expose it
            caught.append((p.__name__, type(e).__name__))
    assert caught, f"no pin caught the mutant {name!r}"
