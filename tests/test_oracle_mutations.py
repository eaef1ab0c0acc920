"""The oracle's pins have teeth: plausible mistakes planted in a copy of the
oracle's C source (compiled on the CPU into a temporary directory) must each be
caught by at least one independent check (hand example, exact brute force,
closed forms, chunk-vs-step consistency).  The real oracle must pass them all.
"""
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact

from test_oracle_pins import HAND, _hand_arrays, _rational_case, _rand_inputs, _to_oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

DECAY = "for (int64_t c = 0; c < dk; ++c) row[c] *= a[c];"
WRITE = "for (int64_t c = 0; c < dk; ++c) row[c] += u * k[c];"
READ = "for (int64_t c = 0; c < dk; ++c) p += row[c] * k[c];"
OUT = "for (int64_t c = 0; c < dk; ++c) acc += row[c] * q[c];"

MUTATIONS = {
    "no_decay": [(DECAY, "")],
    "no_beta": [("double u = beta * (v[i] - p);", "double u = (v[i] - p);")],
    "sign": [("double u = beta * (v[i] - p);", "double u = beta * (v[i] + p);")],
    "read_with_q": [(READ, "for (int64_t c = 0; c < dk; ++c) p += row[c] * q[c];")],
    "erase_then_decay": [
        (DECAY, ""),
        ("double u = beta * (v[i] - p);",
         "double u = beta * (v[i] - p); double up = -beta * p;"),
        (WRITE, "for (int64_t c = 0; c < dk; ++c) row[c] = (row[c] + up * k[c]) * a[c]"
                " + beta * v[i] * k[c];"),
    ],
    "output_before_write": [
        (WRITE, "double acc0 = 0.0; for (int64_t c = 0; c < dk; ++c) acc0 += row[c] * q[c];"
                " " + WRITE),
        ("o[i] = acc;", "o[i] = acc0;"),
    ],
    "ignore_s0": [("if (J->S0)", "if (0)")],
    "scalar_gate_only": [("a[c] = exp(channel_gate ? log_alpha[c] : log_alpha[0]);",
                          "a[c] = exp(log_alpha[0]);")],
    "beta_ignores_head": [("J->beta[bth]", "J->beta[b * T + t]")],
    "decay_twice": [(DECAY, DECAY + " " + DECAY)],
}


def _checks(lib):
    """Return the list of failed check names for one oracle library."""
    failed = []
    q, k, v, la, be, S0 = _hand_arrays()
    o, st = oracle.chunk_fwd(q, k, v, la, be, S0, lib=lib)
    want_o = np.array([[float(x) for x in r] for r in HAND["o"]])
    want_s = np.array([[float(x) for x in r] for r in HAND["S_T"]])
    if not (np.allclose(o[0, :, 0, :], want_o, atol=1e-14, rtol=0)
            and np.allclose(st[0, 0], want_s, atol=1e-14, rtol=0)):
        failed.append("hand")
    for channel in (False, True):
        case = _rational_case(7, 6, 3, 2, channel)
        o_ex, s_ex = exact.run(*case)
        o, st = oracle.chunk_fwd(*_to_oracle(*case, channel), lib=lib)
        o_ex = np.array([[float(x) for x in r] for r in o_ex])
        s_ex = np.array([[float(x) for x in r] for r in s_ex])
        if not (np.allclose(o[0, :, 0, :], o_ex, atol=1e-12, rtol=0)
                and np.allclose(st[0, 0], s_ex, atol=1e-12, rtol=0)):
            failed.append("brute_%s" % channel)
    q, k, v, la, be, S0 = _rand_inputs(300, channel=True, T=6)
    o, st = oracle.chunk_fwd(q, k, v, la, be, S0, lib=lib)
    S = S0.copy()
    ok = True
    for t in range(q.shape[1]):
        ot, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], la[:, t], be[:, t], S, lib=lib)
        ok &= np.allclose(ot, o[:, t], atol=1e-13, rtol=0)
    ok &= np.allclose(S, st, atol=1e-13, rtol=0)
    if not ok:
        failed.append("chunk_vs_step")
    return failed


def _build_variant(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, (name, old)
        src = src.replace(old, new, 1)
    path = os.path.join(str(tmp_path), name + ".c")
    with open(path, "w") as fh:
        fh.write(src)
    return oracle.load(oracle.build(src=path, out=os.path.join(str(tmp_path), name + ".so")))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_unmutated_oracle_passes_all_checks(tmp_path):
    lib = _build_variant(tmp_path, "clean", [])
    assert _checks(lib) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    lib = _build_variant(tmp_path, name, MUTATIONS[name])
    assert _checks(lib), "mutation %s escaped every check" % name
