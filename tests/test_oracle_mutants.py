"""The pins must catch plausible mistakes in the oracle.

Each mutant is a copy of the oracle's source with one deliberate mistake (a
dropped term, a wrong sign or index, a transposed operand, a wrong order of
the four steps).  It is compiled into a temporary library and every pin in
test_oracle_pins.py is run against it; at least one pin must fail.  The
mistakes are planted in copies on the CPU only; the real oracle is untouched.
"""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle import build as obuild
import test_oracle_pins as pins

BODY = os.path.join(os.path.dirname(obuild.LIB), "kda_oracle_body.h")

RETAIN = """        REAL a = EXPF(log_alpha[i]);
        REAL* row = S + (int64_t)i * Dv;
        for (j = j0; j < j1; ++j) row[j] *= a;"""


def _blocks(src):
    """Split the step function at its four commented steps."""
    i1 = src.index("    /* 1. retain")
    i2 = src.index("    /* 2. recall")
    i3 = src.index("    /* 3. correct")
    i4 = src.index("    /* 4. read")
    end = src.index("}\n", i4)
    return src[:i1], src[i1:i2], src[i2:i3], src[i3:i4], src[i4:end], src[end:]


def _swap_correct_read(src):
    pre, b1, b2, b3, b4, post = _blocks(src)
    return pre + b1 + b2 + b4 + b3 + post


def _retain_last(src):
    pre, b1, b2, b3, b4, post = _blocks(src)
    return pre + b2 + b3 + b1 + b4 + post


MUTANTS = {
    "scalar_decay": lambda s: s.replace(RETAIN, RETAIN.replace("log_alpha[i]", "log_alpha[0]")),
    "decay_sign": lambda s: s.replace(RETAIN, RETAIN.replace("EXPF(log_alpha[i])", "EXPF(-log_alpha[i])")),
    "decay_columns": lambda s: s.replace(
        RETAIN, """        REAL* row = S + (int64_t)i * Dv;
        for (j = j0; j < j1; ++j) row[j] *= EXPF(log_alpha[j % Dk]);"""),
    "no_beta": lambda s: s.replace("REAL c = beta * k[i];", "REAL c = k[i];"),
    "erase_sign": lambda s: s.replace("row[j] += c * (v[j] - p[j]);", "row[j] += c * (v[j] + p[j]);"),
    "no_erase": lambda s: s.replace("row[j] += c * (v[j] - p[j]);", "row[j] += c * v[j];"),
    "recall_with_q": lambda s: s.replace("REAL ki = k[i];", "REAL ki = q[i];"),
    "read_with_k": lambda s: s.replace("REAL qi = q[i];", "REAL qi = k[i];"),
    "read_before_update": _swap_correct_read,
    "decay_after_write": _retain_last,
    "ignore_h0": lambda s: s.replace("if (J->h0) {", "if (0) {"),
    "leak_across_docs": lambda s: s.replace(
        "for (t = J->cu[n]; t < J->cu[n + 1]; ++t) {",
        "for (t = (n > 0 ? J->cu[n] - 1 : 0); t < J->cu[n + 1]; ++t) {"),
    "state_transposed_read": lambda s: s.replace(
        "const REAL* row = S + (int64_t)i * Dv;\n        REAL qi = q[i];\n"
        "        for (j = j0; j < j1; ++j) o[j] += row[j] * qi;",
        "REAL qi = q[i];\n"
        "        for (j = j0; j < j1; ++j) o[j] += S[(int64_t)(j % Dk) * Dv + (i % Dv)] * qi;"),
}


def _pin_calls():
    calls = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        f = getattr(pins, name)
        if name == "test_golden_half_life":
            for case in pins.golden("half_life.json")["cases"]:
                calls.append((name, lambda f=f, c=case: f(c)))
        elif name == "test_brute_force_unrolled_products":
            for args in [(5, 3, 8), (3, 7, 6)]:
                calls.append((name, lambda f=f, a=args: f(*a)))
        else:
            calls.append((name, f))
    return calls


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="kda_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, mutant_dir, monkeypatch):
    with open(BODY) as f:
        src = f.read()
    bad = MUTANTS[mutant](src)
    assert bad != src, "mutation site not found: the oracle source changed"
    d = os.path.join(mutant_dir, mutant)
    os.makedirs(d, exist_ok=True)
    here = os.path.dirname(obuild.LIB)
    for fn in ("kda_oracle.c", "kda_oracle.h"):
        shutil.copy(os.path.join(here, fn), d)
    with open(os.path.join(d, "kda_oracle_body.h"), "w") as f:
        f.write(bad)
    so = os.path.join(d, "libmutant.so")
    obuild.build(out=so, sources=[os.path.join(d, "kda_oracle.c")])
    monkeypatch.setattr(oracle, "_LIB", oracle.load(so))
    caught = []
    for name, call in _pin_calls():
        try:
            call()
        except (AssertionError, ValueError):
            caught.append(name)
    assert caught, f"no pin catches the mutant {mutant}"
