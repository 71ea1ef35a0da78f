"""Pins of the fp64 gradient reference (oracle/backward.py).

The reference differentiates a second, torch-float64 writing of the forward
with autograd.  It is pinned to things that do not come from autograd: the
forward equals the C recurrence; central finite differences in float64 of the
loss <dO, o> + <dS_T, S_T> agree with every gradient along random directions;
v cannot reach the outputs when beta = 0; the state gradient through a segment
is the transpose of the segment's transition M (built from the per-token
product in oracle/__init__.py).
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from kda_synth import Workload

ob = pytest.importorskip("oracle.backward")

INPUTS = ("q", "k", "v", "g", "beta", "gate", "S0", "conv_in")


def case(B=2, T=20, H=2, dk=8, dv=12, dtype="f32", seed=5):
    w = Workload("bw", B, T, H, dk, dv, 16, dtype, s0_sigma=0.3, conv_hist="normal", seed=seed)
    return w, syn.prefill_inputs_np(w)


def as_f64(inp):
    return {x: (ob._f64(a) if x not in ("conv_w", "S0") else np.asarray(a, dtype=np.float64))
            for x, a in inp.items() if a is not None}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_torch_forward_equals_c_recurrence(oracle_mod, dtype):
    """The function autograd differentiates is the oracle's prefill (dk != dv)."""
    w, inp = case(dtype=dtype)
    f = ob.forward(inp)
    r = oracle_mod.prefill(inp)
    o = f["o"].transpose(0, 2, 1, 3).reshape(w.B * w.H, w.T, w.dv)
    assert np.abs(o - r["o"]).max() <= 1e-12 * np.abs(r["o"]).max()
    assert np.abs(f["S_T"].reshape(-1, w.dk, w.dv) - r["S_T"]).max() <= 1e-12 * np.abs(r["S_T"]).max()


@pytest.mark.parametrize("name", INPUTS)
def test_gradients_match_central_differences(name):
    """Directional derivative along a random direction, float64 central
    difference (step 1e-6) against the autograd gradient, for a loss on o, S_T
    and conv_out.  Catches a gradient path autograd would miss if the forward
    detached or reused a value."""
    w, inp = case(T=18, seed=9)
    x = as_f64(inp)
    rng = np.random.default_rng(100 + INPUTS.index(name))
    f = ob.forward(x)
    dO = rng.standard_normal(f["o"].shape)
    dS = rng.standard_normal(f["S_T"].shape)
    dC = rng.standard_normal(f["conv_out"].shape)
    grads = ob.backward(x, dO, dS, dC)
    d = rng.standard_normal(x[name].shape)
    eps = 1e-6
    hi, lo = dict(x), dict(x)
    hi[name] = x[name] + eps * d
    lo[name] = x[name] - eps * d
    fd = (ob.loss(hi, dO, dS, dC) - ob.loss(lo, dO, dS, dC)) / (2 * eps)
    an = float(np.sum(grads[name] * d))
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_v_has_no_gradient_without_the_delta_term():
    """beta = 0: v never reaches o or S_T, so dv = 0 exactly, while dbeta is not 0."""
    w, inp = case()
    inp["beta"] = np.zeros_like(inp["beta"])
    rng = np.random.default_rng(1)
    f = ob.forward(inp)
    grads = ob.backward(inp, rng.standard_normal(f["o"].shape), rng.standard_normal(f["S_T"].shape))
    assert np.all(grads["v"] == 0.0)
    assert np.abs(grads["beta"]).max() > 1e-3


def test_state_gradient_is_the_transposed_transition(oracle_mod):
    """With dO = 0 the loss is <dS_T, M S0 + N>, so dS0 = M^T dS_T per (b, h), M
    the oracle's per-token product transition."""
    w, inp = case(dk=8, dv=8, seed=13)
    M = oracle_mod.segment_transition(inp)
    rng = np.random.default_rng(2)
    f = ob.forward(inp)
    dS = rng.standard_normal(f["S_T"].shape)
    grads = ob.backward(inp, np.zeros(f["o"].shape), dS)
    want = np.einsum("nji,njk->nik", M, dS.reshape(-1, w.dk, w.dv))
    assert np.abs(grads["S0"].reshape(-1, w.dk, w.dv) - want).max() <= 1e-11 * np.abs(want).max()


def test_conv_out_is_the_c_recurrences(oracle_mod):
    """The torch forward's conv_out (the last three raw rows) equals the C
    recurrence's, in the packed channel order."""
    w, inp = case(T=2)
    f = ob.forward(inp)
    r = oracle_mod.prefill(inp)
    for i, p in enumerate(r["heads"]):
        b, h = divmod(int(p), w.H)
        ch = oracle_mod._head_channels(w.H, w.dk, w.dv, h)
        assert np.array_equal(f["conv_out"][b][:, ch], r["conv_out"][i])


def test_segment_chain_equals_whole_sequence(oracle_mod):
    """Backward of two segments, the later first: its gradients of S0 and of
    the conv history become the earlier segment's gradients of S_T and of
    conv_out.  The result equals the whole sequence's gradients (the
    composition a segment-wise backward over a long sequence relies on)."""
    w, inp = case(B=1, T=30, seed=17)
    x = as_f64(inp)
    rng = np.random.default_rng(5)
    f = ob.forward(x)
    dO = rng.standard_normal(f["o"].shape)
    dS = rng.standard_normal(f["S_T"].shape)
    whole = ob.backward(x, dO, dS)
    cut = 13
    first = {k: x[k][:, :cut] for k in ("q", "k", "v", "g", "beta", "gate")}
    first.update(conv_w=x["conv_w"], S0=x["S0"], conv_in=x["conv_in"])
    mid = ob.forward(first)
    second = {k: x[k][:, cut:] for k in ("q", "k", "v", "g", "beta", "gate")}
    second.update(conv_w=x["conv_w"], S0=mid["S_T"], conv_in=mid["conv_out"])
    g2 = ob.backward(second, dO[:, cut:], dS)
    g1 = ob.backward(first, dO[:, :cut], g2["S0"], g2["conv_in"])
    for k in ("q", "k", "v", "g", "beta", "gate"):
        got = np.concatenate([g1[k], g2[k]], axis=1)
        assert np.abs(got - whole[k]).max() <= 1e-11 * np.abs(whole[k]).max(), k
    for k in ("S0", "conv_in"):
        assert np.abs(g1[k] - whole[k]).max() <= 1e-11 * np.abs(whole[k]).max(), k
