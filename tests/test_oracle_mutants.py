"""Planted mistakes in a copy of the C oracle must be caught by the pins.

Each mutant is a one-line edit of ``oracle/gdn_oracle.c`` of the kind a
careless implementation makes (dropped term, wrong sign, misplaced gate, eps in
the wrong place, un-normalised query, transposed state index).  The copy is
compiled into a temporary library; at least one pin must fail for it.  The real
oracle is never modified.
"""
import glob
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle.chunked import chunked_scan
from tests.test_oracle_pins import _closed_form_head, _load_golden, _rand_case, GOLDEN

MUTANTS = {
    "beta_dropped_on_write": ("at * erased + bt * vr * kh[c]", "at * erased + vr * kh[c]"),
    "erase_sign_flipped": ("S[r * Dk + c] - bt * x[r] * kh[c]", "S[r * Dk + c] + bt * x[r] * kh[c]"),
    "gate_dropped": ("at * erased + bt", "erased + bt"),
    "gate_on_write_too": ("at * erased + bt * vr * kh[c]", "at * (erased + bt * vr * kh[c])"),
    "eps_outside_sqrt": ("1.0 / sqrt(ss + eps)", "1.0 / (sqrt(ss) + eps)"),
    "query_not_normalised": ("normalise(J->q + tok * Dk, Dk, J->l2norm", "normalise(J->q + tok * Dk, Dk, 0"),
    "state_transposed_on_load": ("J->S0[((b * H + h) * Dv + (r0 + r)) * Dk + c]",
                                 "J->S0[((b * H + h) * Dk + c) * Dv + (r0 + r)]"),
    "scale_ignored": ("J->scale * s", "s"),
    "reverse_ignored": ("J->reverse ? (T - 1 - step) : step", "step"),
}


def _pins_pass(lib):
    """Run a compact battery of the pins against the oracle build ``lib``."""
    for path in sorted(glob.glob(os.path.join(GOLDEN, "hand_*.txt"))):
        g = _load_golden(path)
        o, S = oracle.scan(g["q"], g["k"], g["v"], g["a"], g["beta"], g["S0"], reverse=g["reverse"],
                           l2norm=g["l2norm"], eps=g["eps"], scale=g["scale"], threads=1, lib=lib)
        if not (np.allclose(o, g["o"], rtol=0, atol=1e-15) and np.allclose(S, g["S"], rtol=0, atol=1e-15)):
            return False
    rng = np.random.default_rng(11)
    q, k, v, a, beta, S0 = _rand_case(rng, 1, 7, 1, 5, 3)
    for rev in (False, True):
        o, S = oracle.scan(q, k, v, a, beta, S0, reverse=rev, scale=0.5, lib=lib)
        oe, Se = _closed_form_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], beta[0, :, 0], S0[0, 0],
                                   reverse=rev, l2norm=True, eps=1e-6, scale=0.5)
        if not (np.allclose(o[0, :, 0], oe, rtol=1e-12, atol=1e-13) and np.allclose(S[0, 0], Se, rtol=1e-12)):
            return False
    return True


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def test_unmutated_copy_passes(mutant_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")).read()
    lib = _compile(mutant_dir, "clean", src)
    assert _pins_pass(lib)


def _compile(d, name, src):
    c = os.path.join(str(d), name + ".c")
    so = os.path.join(str(d), name + ".so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-o", so, c, "-lpthread", "-lm"], check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant_dir, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    lib = _compile(mutant_dir, name, src.replace(old, new))
    assert not _pins_pass(lib), f"pins did not catch planted mistake {name}"
