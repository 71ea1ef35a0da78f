"""Pins of the fp64 oracle against mathematics that does not come from the oracle.

Each test names the mistake class it is meant to catch.  Shapes use dk != dv
wherever possible so a transposed operand cannot pass.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import kda_synth as syn
from kda_synth import Workload, to_f64
import k3_checks
from ref_math import (bruteforce_core, conv_numpy, gated_rmsnorm, head_channels, prep_numpy,
                      raw_head, silu)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small(B=1, T=24, H=2, dk=8, dv=12, dtype="f32", s0=0.3, hist="normal", seed=7):
    w = Workload("t", B, T, H, dk, dv, 16, dtype, s0_sigma=s0, conv_hist=hist, seed=seed)
    return w, syn.prefill_inputs_np(w)


# -- P7: the conv + SiLU + L2 stage --------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prep_matches_numpy_convolve(oracle_mod, dtype):
    """Catches: tap order, channel packing (q/k/v, head-major), history row order,
    q/k normalisation and the 1/sqrt(dk) factor landing on q."""
    w, inp = small(B=2, T=19, H=3, dk=8, dv=12, dtype=dtype)
    r = oracle_mod.prefill(inp, want_prep=True)
    conv_in = to_f64(inp["conv_in"], dtype)
    for i, p in enumerate(r["heads"]):
        b, h = divmod(int(p), w.H)
        hist = conv_in[b][:, head_channels(w.H, w.dk, w.dv, h)]
        qn, kn, vn = prep_numpy(inp, dtype, b, h, hist)
        got = r["prep"][i]
        np.testing.assert_allclose(got[:, 2 * w.dk:], vn, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(got[:, :w.dk], qn, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(got[:, w.dk:2 * w.dk], kn, rtol=1e-12, atol=1e-15)
        # |k^| <= 1 and |q^| <= 1/sqrt(dk): normalisation, not some other scaling
        assert np.all(np.linalg.norm(got[:, w.dk:2 * w.dk], axis=1) <= 1 + 1e-12)
        assert np.all(np.linalg.norm(got[:, :w.dk], axis=1) <= 1 / math.sqrt(w.dk) + 1e-12)


def test_conv_numpy_helper_is_causal_convolution():
    """The test helper itself: an impulse at token 0 must reproduce the taps in
    reverse time order (tap 3 on the current token, tap 0 three tokens later)."""
    x = np.zeros((6, 1))
    x[0, 0] = 1.0
    w = np.array([[0.1, 0.2, 0.3, 0.4]])
    out = conv_numpy(x, np.zeros((3, 1)), w)[:, 0]
    np.testing.assert_allclose(out, [0.4, 0.3, 0.2, 0.1, 0.0, 0.0])
    # history only: the oldest history row meets tap 0 at token 0
    h = np.array([[1.0], [0.0], [0.0]])
    out = conv_numpy(np.zeros((3, 1)), h, w)[:, 0]
    np.testing.assert_allclose(out, [0.1, 0.0, 0.0])


# -- P1: dense unrolling ----------------------------------------------------------------

@pytest.mark.parametrize("dtype,B,T,H,dk,dv", [("f32", 1, 64, 2, 16, 16), ("f32", 2, 21, 3, 8, 12),
                                               ("bf16", 1, 17, 2, 12, 8)])
def test_bruteforce_unrolling(oracle_mod, dtype, B, T, H, dk, dv):
    """Catches: update order (decay before the delta correction), read-out from the
    pre-update state, beta placement, sign of the correction, transposes, wrong
    (b,t,h) indexing of g/beta/gate."""
    w, inp = small(B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype)
    r = oracle_mod.prefill(inp)
    g = to_f64(inp["g"], dtype)
    beta = to_f64(inp["beta"], dtype)
    gate = to_f64(inp["gate"], dtype)
    conv_in = to_f64(inp["conv_in"], dtype)
    for i, p in enumerate(r["heads"]):
        b, h = divmod(int(p), H)
        hist = conv_in[b][:, head_channels(H, dk, dv, h)]
        qn, kn, vn = prep_numpy(inp, dtype, b, h, hist)
        S0 = inp["S0"][b, h].astype(np.float64)
        oc, ST = bruteforce_core(qn, kn, vn, g[b, :, h], beta[b, :, h], S0)
        np.testing.assert_allclose(r["S_T"][i], ST, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(r["o"][i], gated_rmsnorm(oc, gate[b, :, h]),
                                   rtol=1e-10, atol=1e-12)


def test_matrix_form_twin_agrees(oracle_mod):
    """The literal (I - b k k^T) Diag(a) S + b k v^T route and the C recurrence."""
    w, inp = small(B=2, T=40, H=2, dk=8, dv=12)
    a = oracle_mod.prefill(inp)
    b = oracle_mod.prefill_matrix_form(inp)
    np.testing.assert_allclose(a["o"], b["o"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(a["S_T"], b["S_T"], rtol=1e-11, atol=1e-13)
    np.testing.assert_array_equal(a["conv_out"], b["conv_out"])


# -- P2: dk = dv = 1 closed form ------------------------------------------------------

def test_scalar_closed_form(oracle_mod):
    """s_t = a_t s_{t-1} + b_t with a_t = (1 - beta k^2) e^g, b_t = beta k v; the
    product/sum closed form is evaluated with cumulative products, not a loop."""
    T = 30
    w, inp = small(B=1, T=T, H=1, dk=1, dv=1, s0=0.7)
    r = oracle_mod.prefill(inp)
    qn, kn, vn = prep_numpy(inp, "f32", 0, 0, to_f64(inp["conv_in"], "f32")[0])
    qn, kn, vn = qn[:, 0], kn[:, 0], vn[:, 0]
    g = inp["g"][0, :, 0, 0].astype(np.float64)
    beta = inp["beta"][0, :, 0].astype(np.float64)
    gate = inp["gate"][0, :, 0, 0].astype(np.float64)
    a = (1.0 - beta * kn * kn) * np.exp(g)
    bb = beta * kn * vn
    s0 = float(inp["S0"][0, 0, 0, 0])
    s = np.empty(T)
    for t in range(T):   # s_t = prod_{j<=t} a_j s0 + sum_{i<=t} prod_{i<j<=t} a_j b_i
        s[t] = np.prod(a[:t + 1]) * s0 + sum(np.prod(a[i + 1:t + 1]) * bb[i] for i in range(t + 1))
    oc = s * qn
    o = oc / np.sqrt(oc * oc + 1e-5) / (1.0 + np.exp(-gate))
    np.testing.assert_allclose(r["S_T"][0, 0, 0], s[-1], rtol=1e-12)
    np.testing.assert_allclose(r["o"][0, :, 0], o, rtol=1e-10, atol=1e-14)
    # k^2 = k~^2 / (k~^2 + 1e-6) exactly: a unit key is not exactly unit
    kt = silu(conv_numpy(raw_head(inp, "f32", 0, 0), to_f64(inp["conv_in"], "f32")[0],
                         inp["conv_w"].astype(np.float64))[:, 1])
    np.testing.assert_allclose(kn * kn, kt * kt / (kt * kt + 1e-6), rtol=1e-13)


# -- P3: beta = 0 ------------------------------------------------------------------------

def test_beta_zero_only_decays(oracle_mod):
    """With beta = 0 the state only decays: S_T = diag(exp sum g) S0 and
    o_core_t = S0^T (q_t * exp(sum_{j<=t} g_j)).  Catches exp(-g), a decay applied to
    the wrong axis of S (dk vs dv), and an off-by-one in the token index of g."""
    w, inp = small(B=1, T=20, H=2, dk=8, dv=12, s0=1.0)
    inp["beta"][:] = 0.0
    r = oracle_mod.prefill(inp)
    g = inp["g"].astype(np.float64)
    gate = inp["gate"].astype(np.float64)
    conv_in = to_f64(inp["conv_in"], "f32")
    for i, p in enumerate(r["heads"]):
        b, h = divmod(int(p), w.H)
        S0 = inp["S0"][b, h].astype(np.float64)
        G = np.cumsum(g[b, :, h], axis=0)                       # [T, dk]
        np.testing.assert_allclose(r["S_T"][i], np.exp(G[-1])[:, None] * S0, rtol=1e-12)
        qn, _, _ = prep_numpy(inp, "f32", b, h, conv_in[b][:, head_channels(w.H, w.dk, w.dv, h)])
        oc = (qn * np.exp(G)) @ S0
        np.testing.assert_allclose(r["o"][i], gated_rmsnorm(oc, gate[b, :, h]), rtol=1e-10)


# -- K3's gate parameterisation --------------------------------------------------------

def test_k3_decay_and_beta_properties(oracle_mod):
    """The KDA_DECAY_K3 form: the bound, its limits, z = 0, the symmetry, e^A scaling,
    A per head and beta = sigmoid(b) (tests/k3_checks.py says what each pins).
    Catches a flipped sign, a wrong bound, A used without exp, head 0's A for
    every head, and an unmapped beta or decay logit."""
    assert k3_checks.failures(oracle_mod) == []


def test_k3_matrix_form_twin_agrees(oracle_mod):
    """The NumPy matrix-form route maps the logits with its own code; the C
    recurrence agrees with it on K3-form inputs."""
    w = Workload("t", 1, 20, 2, 8, 12, 16, "f32", s0_sigma=0.3, conv_hist="normal", seed=9)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w)
    a = oracle_mod.prefill(inp)
    b = oracle_mod.prefill_matrix_form(inp)
    np.testing.assert_allclose(a["o"], b["o"], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(a["S_T"], b["S_T"], rtol=1e-10, atol=1e-13)


# -- P4 / P6: carry -----------------------------------------------------------------------

def test_split_invariance_every_point(oracle_mod):
    """prefill(0..T) == prefill(0..T1) ; prefill(T1..T) with S and the raw conv
    history carried, bit for bit, for every T1 (including T1 < 3, where the carried
    history still holds rows of conv_in)."""
    w = syn.WORKLOADS["tiny"]
    inp = syn.prefill_inputs_np(w)
    inp["conv_in"] = syn.prefill_inputs_np(Workload("h", 1, 1, 2, 16, 16, 16, "f32",
                                                    conv_hist="normal", seed=3))["conv_in"]
    full = oracle_mod.prefill(inp)
    for T1 in range(0, w.T + 1):
        a = {x: inp[x][:, :T1] for x in ("q", "k", "v", "g", "beta", "gate")}
        c = {x: inp[x][:, T1:] for x in ("q", "k", "v", "g", "beta", "gate")}
        a["conv_w"] = c["conv_w"] = inp["conv_w"]
        S, hist = oracle_mod.initial_carry(w.B, w.H, w.dk, w.dv, None, inp["S0"], inp["conv_in"])
        ra = oracle_mod.prefill(a, S=S, hist=hist)
        rc = oracle_mod.prefill(c, S=S, hist=hist)
        o = np.concatenate([ra["o"], rc["o"]], axis=1)
        assert np.array_equal(o, full["o"]), T1
        assert np.array_equal(rc["S_T"], full["S_T"]), T1
        assert np.array_equal(rc["conv_out"], full["conv_out"]), T1


def test_conv_out_is_last_three_raw_tokens(oracle_mod):
    """conv_out rows are the last three raw tokens (oldest first); for T < 3 the
    leading rows still come from conv_in."""
    w, inp = small(B=1, T=2, H=2, dk=8, dv=12)
    r = oracle_mod.prefill(inp)
    conv_in = to_f64(inp["conv_in"], "f32")
    for i, p in enumerate(r["heads"]):
        b, h = divmod(int(p), w.H)
        ch = head_channels(w.H, w.dk, w.dv, h)
        x = raw_head(inp, "f32", b, h)
        want = np.concatenate([conv_in[b][:, ch], x])[-3:]
        np.testing.assert_array_equal(r["conv_out"][i], want)


def test_decode_steps_equal_prefill(oracle_mod):
    """T single-token decode steps reproduce prefill(T) bit for bit."""
    w, inp = small(B=2, T=9, H=2, dk=8, dv=12, dtype="bf16")
    full = oracle_mod.prefill(inp)
    S, hist = oracle_mod.initial_carry(w.B, w.H, w.dk, w.dv, None, inp["S0"], inp["conv_in"])
    for t in range(w.T):
        step = {x: inp[x][:, t] for x in ("q", "k", "v", "g", "beta", "gate")}
        step["conv_w"] = inp["conv_w"]
        o = oracle_mod.decode_step(step, S, hist)
        assert np.array_equal(o, full["o"][:, t])
    assert np.array_equal(S, full["S_T"])
    assert np.array_equal(hist, full["conv_out"])


# -- P5: delta identity ----------------------------------------------------------------

def test_delta_identity_each_token(oracle_mod):
    """S_t^T k_t = (1 - beta |k|^2) (D_t S_{t-1})^T k_t + beta |k|^2 v_t for every t."""
    w, inp = small(B=1, T=12, H=1, dk=8, dv=12, s0=0.5)
    S, hist = oracle_mod.initial_carry(1, 1, 8, 12, None, inp["S0"], inp["conv_in"])
    qn, kn, vn = prep_numpy(inp, "f32", 0, 0, to_f64(inp["conv_in"], "f32")[0])
    g = inp["g"][0, :, 0].astype(np.float64)
    beta = inp["beta"][0, :, 0].astype(np.float64)
    for t in range(w.T):
        prev = S[0].copy()
        step = {x: inp[x][:, t] for x in ("q", "k", "v", "g", "beta", "gate")}
        step["conv_w"] = inp["conv_w"]
        oracle_mod.decode_step(step, S, hist)
        kk = kn[t] @ kn[t]
        lhs = S[0].T @ kn[t]
        rhs = (1 - beta[t] * kk) * ((np.exp(g[t])[:, None] * prev).T @ kn[t]) + beta[t] * kk * vn[t]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-14)


# -- epilogue special cases -------------------------------------------------------------

def test_epilogue_gate_and_rms(oracle_mod):
    """gate = 0 halves the normalised output; a large gate passes it unchanged;
    the normalised row has mean square m/(m+1e-5) where m is that of o_core."""
    w, inp = small(B=1, T=10, H=2, dk=8, dv=12)
    inp["gate"][:] = 0.0
    r0 = oracle_mod.prefill(inp)
    inp["gate"][:] = 80.0
    r1 = oracle_mod.prefill(inp)
    np.testing.assert_allclose(r0["o"] * 2.0, r1["o"], rtol=1e-14)
    ms = (r1["o"] ** 2).mean(-1)
    assert np.all(ms < 1.0) and np.all(ms > 0.5)
    # independent o_core from the dense unrolling gives the exact mean square
    conv_in = to_f64(inp["conv_in"], "f32")
    qn, kn, vn = prep_numpy(inp, "f32", 0, 0, conv_in[0][:, head_channels(2, 8, 12, 0)])
    oc, _ = bruteforce_core(qn, kn, vn, inp["g"][0, :, 0].astype(np.float64),
                            inp["beta"][0, :, 0].astype(np.float64),
                            inp["S0"][0, 0].astype(np.float64))
    m = (oc ** 2).mean(-1)
    np.testing.assert_allclose(ms[0], m / (m + 1e-5), rtol=1e-12)


def test_empty_sequence_keeps_carry(oracle_mod):
    w, inp = small(B=1, T=0, H=2, dk=8, dv=12)
    S, hist = oracle_mod.initial_carry(1, 2, 8, 12, None, inp["S0"], inp["conv_in"])
    S_in, h_in = S.copy(), hist.copy()
    r = oracle_mod.prefill(inp, S=S, hist=hist)
    assert r["o"].shape == (2, 0, 12)
    assert np.array_equal(r["S_T"], S_in) and np.array_equal(r["conv_out"], h_in)


def test_oracle_rejects_bad_pairs(oracle_mod):
    w, inp = small()
    with pytest.raises(ValueError):
        oracle_mod.prefill(inp, heads=[0, 99])


# -- P10: structural facts the pages print ------------------------------------------------

def test_page_facts():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    kda = facts["kda_shape"]
    w = syn.WORKLOADS["k3width"]
    assert (w.H, w.dk, w.dv) == (kda["heads"], kda["head_dim"], kda["head_dim"])
    st = facts["kda_state_serving"]
    per_rank = st["layers"] * kda["heads"] * kda["head_dim"] ** 2 * 4 / st["tp"]
    assert abs(per_rank / 2 ** 20 - st["approx_mb"]) < 0.5           # 51.75 MiB ~ "52 MB"
    t = facts["tile_rescaling"]
    bf16_max = (2 - 2 ** -7) * 2.0 ** 127
    assert math.exp(t["max_decay_per_token"] * t["tile_tokens"]) < bf16_max
    assert math.exp(t["max_decay_per_token"] * 2 * t["tile_tokens"]) > bf16_max
    assert facts["rms_norm_eps"]["value"] == 1e-5


# -- the input recipe ------------------------------------------------------------------------

def test_bf16_rounding_is_rne():
    """bf16_bits_from_f64 against exact ties and torch's fp32 -> bf16 conversion."""
    import torch
    one = 1.0
    ulp = 2.0 ** -7
    x = np.array([one + ulp / 2, one + 3 * ulp / 2, -(one + ulp / 2), one + ulp / 2 + 2 ** -40,
                  3.0e38 / 2, 1e-30, 0.0])
    got = syn.bf16_bits_to_f64(syn.bf16_bits_from_f64(x))
    np.testing.assert_array_equal(got[:4], [one, one + 2 * ulp, -one, one + ulp])
    rng = np.random.default_rng(0)
    y = rng.standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(syn.bf16_bits_from_f64(y.astype(np.float64)), ref)


def test_input_recipe_statistics():
    w = syn.WORKLOADS["tiny"]
    inp = syn.prefill_inputs_np(Workload("s", 1, 4096, 4, 16, 16, 16, "f32"))
    g = inp["g"].astype(np.float64)
    assert np.all(g < 0)
    assert abs(np.exp(g).mean() - 0.93) < 0.02
    b = inp["beta"].astype(np.float64)
    assert np.all((b > 0) & (b < 1)) and abs(b.mean() - 0.5) < 0.02
    assert abs(inp["q"].std() - 1) < 0.02 and abs(inp["conv_w"]).max() <= 0.5
    again = syn.prefill_inputs_np(Workload("s", 1, 4096, 4, 16, 16, 16, "f32"))
    assert np.array_equal(again["q"], inp["q"])
