"""Pins of the oracle's context-parallel algebra (segment fragments and their
prefix composition) against results that do not come from that algebra.

The long-context training row of "Gemma 4 31B vs Kimi K3" (component table)
says only that ranks exchange fixed-size state fragments.  The reading taken:
the update is affine in the
state, a segment maps its entering state S to M S + N, and composing the
segments' (M, N) in order gives each segment its entering state.  M is built
from the per-token product definition, not from the recurrence, so agreement
with the recurrence pins both.  Shapes use dk != dv so that a transposed
operand cannot pass.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from kda_synth import Workload


def case(B=2, T=48, H=2, dk=8, dv=12, dtype="f32", seed=11, k3=False, hist="normal", s0=0.3):
    w = Workload("cp", B, T, H, dk, dv, 16, dtype, s0_sigma=s0, conv_hist=hist, seed=seed)
    inp = syn.prefill_inputs_np(w)
    if k3:
        inp = syn.with_k3_logits(inp, w)
    return w, inp


@pytest.mark.parametrize("k3", [False, True])
def test_state_map_is_affine_with_the_product_transition(oracle_mod, k3):
    """S_T(S0) - S_T(0) = M S0 for random S0, with M the ordered product of the
    per-token maps and S_T from the C recurrence.  Catches: the product taken in
    the wrong order (M D instead of D M), the decay on the wrong side of the
    rank-1 term, a missing beta, a transposed k k^T."""
    w, inp = case(k3=k3)
    n = w.B * w.H
    M = oracle_mod.segment_transition(inp)
    assert M.shape == (n, w.dk, w.dk)
    S_zero, h0 = oracle_mod.initial_carry(w.B, w.H, w.dk, w.dv, None, None, inp["conv_in"])
    oracle_mod.prefill(inp, S=S_zero, hist=h0.copy(), want_o=False)
    rng = np.random.default_rng(3)
    for _ in range(2):
        S0 = rng.standard_normal((n, w.dk, w.dv))
        S = S0.copy()
        oracle_mod.prefill(inp, S=S, hist=h0.copy(), want_o=False)
        want = np.einsum("nij,njk->nik", M, S0)
        assert np.abs((S - S_zero) - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


def test_transition_without_delta_term_is_the_decay(oracle_mod):
    """beta = 0 removes the rank-1 terms: M = Diag(exp(sum_t g_t)) (closed form).
    Catches: exp of the per-token g instead of its sum, a decay applied twice."""
    w, inp = case(T=37, k3=False)
    inp["beta"] = np.zeros_like(inp["beta"])
    M = oracle_mod.segment_transition(inp)
    g, _ = oracle_mod.decay_and_beta(inp)
    for i in range(w.B * w.H):
        b, h = divmod(i, w.H)
        want = np.diag(np.exp(g[b, :, h].sum(axis=0)))
        assert np.abs(M[i] - want).max() <= 1e-13


def test_one_segment_is_the_affine_map(oracle_mod):
    """R = 1: M S0 + N is the prefill's final state from S0."""
    w, inp = case(B=1, T=40, H=3)
    M, N = oracle_mod.segment_fragments(inp)
    S0, _ = oracle_mod.initial_carry(w.B, w.H, w.dk, w.dv, None, inp["S0"], None)
    r = oracle_mod.prefill(inp)
    want = r["S_T"]
    got = np.einsum("nij,njk->nik", M, S0) + N
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


@pytest.mark.parametrize("segments,T,dtype,k3", [(2, 48, "f32", False), (3, 48, "bf16", False),
                                                 (4, 64, "bf16", True), (6, 48, "f32", True)])
def test_context_parallel_equals_sequential(oracle_mod, segments, T, dtype, k3):
    """Fragments from S = 0 per segment (each with the previous segment's last
    three raw tokens as its conv history), composed from S0, then every segment
    rerun from its entering state: o and S_T equal the sequential prefill's.
    Catches: a segment started without its conv halo, segments composed in the
    wrong order, M and N of different segments mixed, S0 dropped."""
    w, inp = case(B=2, T=T, dtype=dtype, k3=k3, seed=20 + segments)
    seq = oracle_mod.prefill(inp)
    cp = oracle_mod.prefill_context_parallel(inp, segments)
    for got, want in ((cp["o"], seq["o"]), (cp["S_T"], seq["S_T"])):
        assert np.abs(got - want).max() <= 1e-11 * np.abs(want).max()
    # the entering state of each segment is the sequential state at its boundary
    L = T // segments
    for r in range(1, segments):
        part = {x: inp[x][:, :r * L] for x in ("q", "k", "v", "g", "beta", "gate")}
        part.update(conv_w=inp["conv_w"], S0=inp["S0"], conv_in=inp["conv_in"], A=inp.get("A"))
        want = oracle_mod.prefill(part, want_o=False)["S_T"]
        assert np.abs(cp["S_start"][r] - want).max() <= 1e-11 * np.abs(want).max()


def test_segment_needs_its_conv_halo(oracle_mod):
    """The check above is sensitive to the halo: starting a segment with a zero
    conv history (the plausible mistake) changes o by far more than rounding."""
    w, inp = case(B=1, T=32)
    seq = oracle_mod.prefill(inp)
    seg = {x: inp[x][:, 16:] for x in ("q", "k", "v", "g", "beta", "gate")}
    seg.update(conv_w=inp["conv_w"], A=None)
    S_mid = oracle_mod.prefill({**{x: inp[x][:, :16] for x in ("q", "k", "v", "g", "beta", "gate")},
                                "conv_w": inp["conv_w"], "S0": inp["S0"], "conv_in": inp["conv_in"]},
                               want_o=False)["S_T"]
    no_halo = oracle_mod.prefill(seg, S=S_mid.copy(),
                                 hist=np.zeros((w.B * w.H, 3, 2 * w.dk + w.dv)))
    assert np.abs(no_halo["o"] - seq["o"][:, 16:]).max() > 1e-3
