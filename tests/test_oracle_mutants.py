"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
each to fail at least one pin, so that the pins are known to constrain every
step of the recurrence: fade, erase, write, read, and the state carry."""

import re

import pytest

from oracle.kda_oracle import SOURCE, build_variant
from pins import ALL_PINS

FADE = re.compile(r"    /\* fade:.*?\n    }\n", re.S)
ERASE = re.compile(r"    /\* erase:.*?p\[j\] \+= S\[\(size_t\)i \* dv \+ j\] \* k\[i\];\n", re.S)
READ = re.compile(r"    /\* read from the updated state.*?\* q\[i\];\n", re.S)


def _sub(src, old, new):
    assert old in src, old
    return src.replace(old, new, 1)


def _move_fade_after_write(src):
    fade = FADE.search(src).group(0)
    src = src.replace(fade, "", 1)
    return _sub(src, "    /* read from the updated state", fade + "    /* read from the updated state")


def _erase_before_fade(src):
    fade = FADE.search(src).group(0)
    erase = ERASE.search(src).group(0)
    src = src.replace(fade, "", 1)
    return src.replace(erase, erase + fade, 1)


def _read_before_write(src):
    read = READ.search(src).group(0)
    src = src.replace(read, "", 1)
    return _sub(src, "    /* write: S += beta k (v - p)^T */", read + "    /* write: S += beta k (v - p)^T */")


MUTANTS = {
    "no_fade": lambda s: _sub(s, "const double alpha = exp(g[i]);", "const double alpha = 1.0;"),
    "fade_base2": lambda s: _sub(s, "const double alpha = exp(g[i]);", "const double alpha = exp2(g[i]);"),
    "fade_value_axis": lambda s: _sub(s, "S[(size_t)i * dv + j] *= alpha;",
                                      "S[(size_t)i * dv + j] *= exp(g[j < dk ? j : 0]);"),
    "fade_after_write": _move_fade_after_write,
    "erase_before_fade": _erase_before_fade,
    "erase_full_strength": lambda s: _sub(s, "beta * k[i] * (v[j] - p[j])", "k[i] * (beta * v[j] - p[j])"),
    "erase_sign": lambda s: _sub(s, "beta * k[i] * (v[j] - p[j])", "beta * k[i] * (v[j] + p[j])"),
    "no_erase": lambda s: _sub(s, "beta * k[i] * (v[j] - p[j])", "beta * k[i] * v[j]"),
    "erase_with_query": lambda s: _sub(s, "p[j] += S[(size_t)i * dv + j] * k[i];",
                                       "p[j] += S[(size_t)i * dv + j] * q[i];"),
    "read_with_key": lambda s: _sub(s, "o[j] += S[(size_t)i * dv + j] * q[i];",
                                    "o[j] += S[(size_t)i * dv + j] * k[i];"),
    "read_before_write": _read_before_write,
    "ignore_S0": lambda s: _sub(s, "        if (S0)\n            memcpy", "        if (0)\n            memcpy"),
    "beta_squared": lambda s: _sub(s, "beta * k[i] * (v[j] - p[j])", "beta * beta * k[i] * (v[j] - p[j])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with open(SOURCE) as f:
        src = f.read()
    mutated = MUTANTS[name](src)
    assert mutated != src
    orc = build_variant(mutated)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
