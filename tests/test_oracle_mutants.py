"""Plant plausible mistakes in a COPY of the oracle (on the CPU) and require
that the pins catch every one.  This is evidence that the pins constrain each
step of the recurrence, not only the final numbers of one example."""
import functools
import os
import re
import subprocess

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")


def _move_block(src, start_marker, end_marker, before_marker):
    """Cut [start_marker, end_marker) and paste it right before before_marker."""
    i = src.index(start_marker)
    j = src.index(end_marker, i)
    block = src[i:j]
    rest = src[:i] + src[j:]
    k = rest.index(before_marker)
    return rest[:k] + block + rest[k:]


def _sub(pattern, repl, count=1):
    def f(src):
        out, n = re.subn(pattern, repl, src, count=count)
        assert n == count, pattern
        return out
    return f


MUTANTS = {
    "residual_sign": _sub(r"e\[j\] = \(double\)vt\[j\] - p\[j\];", "e[j] = p[j] - (double)vt[j];"),
    "no_scalar_decay": _sub(r"const double a = exp\(\(double\)g\[row\]\);", "const double a = 1.0;"),
    "decay_not_exponentiated": _sub(r"const double a = exp\(\(double\)g\[row\]\);",
                                    "const double a = 1.0 + (double)g[row];"),
    "per_channel_decay_on_value_axis": _sub(
        r"const double a = exp\(\(double\)gt\[i\]\);\n(\s*)double \*Si = S \+ i \* Dv;\n(\s*)for \(long j = 0; j < Dv; \+\+j\) Si\[j\] \*= a;",
        "(void)0;\n\\1double *Si = S + i * Dv;\n\\2for (long j = 0; j < Dv; ++j) Si[j] *= exp((double)gt[j % Dk]);"),
    "beta_not_in_write": _sub(r"const double bki = beta \* \(double\)kt\[i\];", "const double bki = (double)kt[i];"),
    "kaczmarz_uses_l1_norm": _sub(r"kk \+= \(double\)kt\[i\] \* \(double\)kt\[i\];", "kk += fabs((double)kt[i]);"),
    "kaczmarz_ignores_eps": _sub(r"/ \(kk \+ eps\);", "/ kk;"),
    "scale_ignored": _sub(r"ot\[j\] = scale \* p\[j\];", "ot[j] = p[j];"),
    "predict_with_query": _sub(r"const double ki = \(double\)kt\[i\];\n(\s*)const double \*Si = S \+ i \* Dv;",
                               "const double ki = (double)qt[i];\n\\1const double *Si = S + i * Dv;"),
    "forget_after_write": lambda s: _move_block(s, "/* steps 1-2: forget */", "if (delta_off) {",
                                                "/* step 7: read after write */"),
    "read_before_write": lambda s: _move_block(s, "/* step 7: read after write */",
                                               "\n    }\n\n    for (long x = 0; x < Dk * Dv; ++x) s_final",
                                               "if (delta_off) {"),
    "additive_write_in_delta_mode": _sub(r"for \(long j = 0; j < Dv; \+\+j\) e\[j\] = \(double\)vt\[j\] - p\[j\];",
                                         "for (long j = 0; j < Dv; ++j) e[j] = (double)vt[j];"),
    "state_not_carried": _sub(r"for \(long t = 0; t < T; \+\+t\) \{",
                              "for (long t = 0; t < T; ++t) { if (t) memset(S, 0, sizeof(double) * Dk * Dv);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path, golden):
    src = open(SRC).read()
    mutated = MUTANTS[name](src)
    assert mutated != src
    c = tmp_path / f"mut_{name}.c"
    so = tmp_path / f"libmut_{name}.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o", str(so),
                    str(c), "-lm"], check=True)
    fwd = functools.partial(oracle.oracle_fwd, lib=oracle.bind(str(so)), threads=1)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(fwd, golden) if pins.needs_golden(pin) else pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant {name}"


def test_unmutated_copy_passes_every_pin(tmp_path, golden):
    """Control for the harness above: the same build route without a mutation
    passes all pins."""
    c = tmp_path / "copy.c"
    so = tmp_path / "libcopy.so"
    c.write_text(open(SRC).read())
    subprocess.run(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o", str(so),
                    str(c), "-lm"], check=True)
    fwd = functools.partial(oracle.oracle_fwd, lib=oracle.bind(str(so)), threads=1)
    for pin in pins.ALL_PINS:
        pin(fwd, golden) if pins.needs_golden(pin) else pin(fwd)
