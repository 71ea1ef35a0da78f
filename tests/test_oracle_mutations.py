"""Plant plausible mistakes in copies of the oracle's C source (CPU only) and
check that the pins catch every one of them.

Each mutant is the oracle source with one textual change, compiled to a
temporary library; the checks below are the same independent references the
pins use (numpy.convolve prep, dense unrolling, the scalar closed form,
the beta = 0 decay-only form).
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import kda_synth as syn
from kda_synth import Workload, to_f64
import k3_checks
from ref_math import bruteforce_core, gated_rmsnorm, head_channels, prep_numpy

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "kda_oracle.c")

MUTANTS = {
    "tap order": ("(double)w[3] * x[c]", "(double)w[2] * x[c]"),
    "history not shifted in": ("hist[2 * nc + c] = x[c];", "hist[2 * nc + c] = 0.0;"),
    "no SiLU": ("xt[c] = silu(acc);", "xt[c] = acc;"),
    "dk^-1/2 on k": ("const double rk = 1.0 / sqrt(sk + L2_EPS);",
                     "const double rk = 1.0 / sqrt(sk + L2_EPS) / sqrt((double)dk);"),
    "L2 eps": ("L2_EPS = 1e-6", "L2_EPS = 1e-4"),
    "decay sign": ("const double a = exp(gi);", "const double a = exp(-gi);"),
    "correction sign": ("(vh[j] - y[j])", "(vh[j] + y[j])"),
    "beta dropped": ("const double bk = beta * kh[i];", "const double bk = kh[i];"),
    "y from q": ("y[j] += S[(size_t)i * dv + j] * kh[i];", "y[j] += S[(size_t)i * dv + j] * qh[i];"),
    "RMS eps": ("RMS_EPS = 1e-5", "RMS_EPS = 1e-6"),
    "gate sign": ("sigmoid(load(in->gate", "sigmoid(-load(in->gate"),
    "sum instead of mean": ("ms /= (double)dv;", "ms /= 1.0;"),
    "k uses q conv weights": ("ch = (size_t)H * dk + (size_t)h * dk + (c - dk);",
                              "ch = (size_t)h * dk + (c - dk);"),
    "v channel offset": ("ch = (size_t)2 * H * dk + (size_t)h * dv + (c - 2 * dk);",
                         "ch = (size_t)2 * H * dk + (c - 2 * dk);"),
    # K3's gate parameterisation
    "K3 decay sign": ("-5.0 * sigmoid(exp(A) * z)", "-5.0 * sigmoid(-exp(A) * z)"),
    "K3 bound": ("-5.0 * sigmoid(exp(A) * z)", "-4.0 * sigmoid(exp(A) * z)"),
    "K3 A not exponentiated": ("-5.0 * sigmoid(exp(A) * z)", "-5.0 * sigmoid(A * z)"),
    "K3 A of head 0 for all": ("in->A[(size_t)h * dk + i]", "in->A[i]"),
    "K3 beta logit not mapped": ("if (in->decay_form == KDAO_DECAY_K3) beta = sigmoid(beta);", ""),
    "K3 decay not mapped": ("if (in->decay_form == KDAO_DECAY_K3) gi = ", "if (0) gi = "),
}


def _checks_fail(oracle_mod, lib) -> bool:
    """True if any independent reference disagrees with this oracle build."""
    B, T, H, dk, dv = 2, 13, 2, 8, 12
    w = Workload("m", B, T, H, dk, dv, 16, "f32", s0_sigma=0.3, conv_hist="normal", seed=21)
    inp = syn.prefill_inputs_np(w)
    r = oracle_mod.prefill(inp, want_prep=True, lib=lib)
    conv_in = to_f64(inp["conv_in"], "f32")
    for i, p in enumerate(r["heads"]):
        b, h = divmod(int(p), H)
        hist = conv_in[b][:, head_channels(H, dk, dv, h)]
        qn, kn, vn = prep_numpy(inp, "f32", b, h, hist)
        if not np.allclose(r["prep"][i], np.concatenate([qn, kn, vn], 1), rtol=1e-11, atol=1e-14):
            return True
        oc, ST = bruteforce_core(qn, kn, vn, inp["g"][b, :, h].astype(np.float64),
                                 inp["beta"][b, :, h].astype(np.float64),
                                 inp["S0"][b, h].astype(np.float64))
        if not np.allclose(r["S_T"][i], ST, rtol=1e-10, atol=1e-13):
            return True
        if not np.allclose(r["o"][i], gated_rmsnorm(oc, inp["gate"][b, :, h].astype(np.float64)),
                           rtol=1e-9, atol=1e-12):
            return True
        want_hist = np.concatenate([hist, np.concatenate(
            [inp["q"][b, :, h], inp["k"][b, :, h], inp["v"][b, :, h]], 1).astype(np.float64)])[-3:]
        if not np.array_equal(r["conv_out"][i], want_hist):
            return True
    return bool(k3_checks.failures(oracle_mod, lib))


def test_unmutated_oracle_passes_checks(oracle_mod):
    assert not _checks_fail(oracle_mod, None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(oracle_mod, tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not unique in the oracle source"
    mutated = tmp_path / "kda_oracle.c"
    mutated.write_text(src.replace(old, new))
    so = oracle_mod.build(force=True, src=str(mutated), out=str(tmp_path / "libmut.so"))
    lib = oracle_mod.load_library(so)
    assert _checks_fail(oracle_mod, lib), f"mutant {name!r} passed every check"
