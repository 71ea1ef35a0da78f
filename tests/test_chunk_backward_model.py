"""The chunkwise backward model (tests/chunk_backward_model.py) against torch
autograd of the token-serial recurrence core, in float64: ragged last chunks,
every chunk size the kernels use, dk != dv, strong decay (g near K3's bound of
-5 per token) and beta = 0."""
from __future__ import annotations

import numpy as np
import pytest

import chunk_backward_model as cbm

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _serial_core_grads(q, k, v, g, beta, S0, dO, dS_T):
    """The definition, token by token (S' = Diag(e^g) S, u = beta (v - S'^T k),
    S = S' + k u^T, o = S^T q), differentiated by torch autograd."""
    torch = pytest.importorskip("torch")
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for n, a in dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0).items()}
    S = t["S0"]
    outs = []
    for i in range(q.shape[0]):
        Sp = torch.exp(t["g"][i])[:, None] * S
        u = t["beta"][i] * (t["v"][i] - Sp.T @ t["k"][i])
        S = Sp + torch.outer(t["k"][i], u)
        outs.append(S.T @ t["q"][i])
    O = torch.stack(outs) if outs else torch.zeros((0, v.shape[1]), dtype=torch.float64)
    loss = (O * torch.tensor(dO)).sum() + (S * torch.tensor(dS_T)).sum()
    loss.backward()
    return O.detach().numpy(), S.detach().numpy(), {n: x.grad.numpy() if x.grad is not None else np.zeros_like(x.detach().numpy())
                                                     for n, x in t.items()}


def _case(T, dk, dv, seed, g_scale=1.0, beta_zero=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)       # k^ is unit-norm after the L2 step
    v = rng.standard_normal((T, dv))
    g = -g_scale * np.log1p(np.exp(rng.standard_normal((T, dk)) - 3.0))
    beta = np.zeros(T) if beta_zero else 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = 0.1 * rng.standard_normal((dk, dv))
    dO = rng.standard_normal((T, dv))
    dS_T = rng.standard_normal((dk, dv))
    return q, k, v, g, beta, S0, dO, dS_T


def _check(args, C, tol=1e-10):
    q, k, v, g, beta, S0, dO, dS_T = args
    O_ref, S_ref, ref = _serial_core_grads(*args)
    O, S_T, _ = cbm.forward(q, k, v, g, beta, S0, C)
    assert np.allclose(O, O_ref, rtol=0, atol=tol * max(1.0, np.abs(O_ref).max()))
    assert np.allclose(S_T, S_ref, rtol=0, atol=tol * max(1.0, np.abs(S_ref).max()))
    got = cbm.backward(q, k, v, g, beta, S0, dO, dS_T, C)
    for n in ("q", "k", "v", "g", "beta", "S0"):
        scale = max(1e-300, np.sqrt(np.mean(ref[n] ** 2)))
        err = np.abs(got[n] - ref[n]).max() / scale if ref[n].size else 0.0
        assert err <= tol, f"d{n}: max|err|/RMS {err:.3e}"


@pytest.mark.parametrize("T,C", [(1, 16), (17, 16), (64, 64), (100, 32), (130, 64), (77, 16)])
def test_matches_autograd(T, C):
    _check(_case(T, 16, 16, seed=T + C), C)


def test_dk_ne_dv():
    _check(_case(90, 16, 24, seed=5), 32)


def test_strong_decay():
    """g near K3's bound (-5 per token, e^-80 over a 16-token tile): every decay
    factor the chunk form uses stays <= 1, so the gradients keep full accuracy."""
    _check(_case(70, 16, 16, seed=9, g_scale=40.0), 64, tol=1e-9)


def test_beta_zero():
    """beta = 0: U = 0, the state only decays and dv vanishes."""
    args = _case(50, 8, 8, seed=3, beta_zero=True)
    _check(args, 16)
    got = cbm.backward(*args, C=16)
    assert np.abs(got["v"]).max() == 0.0


def test_planted_mistakes_are_caught():
    """A plausible slip in the derivation (dropping the chunk-level G_C term,
    through Diag(e^{G_C}) S_in, from dg) moves the gradient far beyond the
    tolerance, so the comparison above is sensitive to it."""
    args = _case(40, 8, 8, seed=11)
    q, k, v, g, beta, S0, dO, dS_T = args
    _, _, ref = _serial_core_grads(*args)
    good = cbm.backward(q, k, v, g, beta, S0, dO, dS_T, C=16)
    assert np.abs(good["g"] - ref["g"]).max() < 1e-9
    orig = cbm._chunk_backward

    def no_gc(*a):
        dq, dk, dv, dg, dbeta, dS = orig(*a)
        f = cbm._chunk_terms(*a[:6])
        dGC = np.exp(f["GC"]) * np.sum(a[7] * a[5], axis=1)
        return dq, dk, dv, dg - dGC[None, :], dbeta, dS

    cbm._chunk_backward = no_gc
    try:
        bad = cbm.backward(q, k, v, g, beta, S0, dO, dS_T, C=16)
    finally:
        cbm._chunk_backward = orig
    assert np.abs(bad["g"] - ref["g"]).max() > 1e-3


@pytest.mark.parametrize("T,C", [(130, 64), (77, 16)])
def test_phased_equals_chunk_by_chunk(T, C):
    """The three-phase order (operands of every chunk, the serial dS pass, the
    gradients of every chunk) gives the chunk-by-chunk reverse's gradients."""
    args = _case(T, 16, 16, seed=T)
    a = cbm.backward(*args, C=C)
    b = cbm.backward_phased(*args, C=C)
    for n in a:
        assert np.allclose(a[n], b[n], rtol=1e-12, atol=1e-12 * max(1.0, np.abs(a[n]).max())), n


@pytest.mark.parametrize("T,chunk,dtype", [(20, 8, "f32"), (37, 16, "bf16"), (2, 16, "f32"), (70, 32, "bf16")])
def test_whole_backward_chunkwise_equals_autograd(T, chunk, dtype):
    """The whole backward (conv, SiLU, norms, RMSNorm * sigmoid(gate) around the
    chunkwise core) against the fp64 autograd reference on the prefill inputs:
    ragged chunks, bf16 inputs, fewer tokens than the conv history."""
    ob = pytest.importorskip("oracle.backward")
    import backward_model as bm
    import kda_synth as syn
    from kda_synth import Workload
    w = Workload("cbm", 2, T, 2, 8, 8, 16, dtype, s0_sigma=0.3, conv_hist="normal", seed=7 + T)
    inp = syn.prefill_inputs_np(w)
    rng = np.random.default_rng(T + 1)
    f = ob.forward(inp)
    dO = rng.standard_normal(f["o"].shape)
    dS = rng.standard_normal(f["S_T"].shape)
    dC = rng.standard_normal(f["conv_out"].shape)
    ref = ob.backward(inp, dO, dS, dC)
    orig = bm.backward_pair
    calls = []

    def chunkwise(*a, **kw):
        calls.append(1)
        return cbm.backward_pair_chunkwise(*a, **kw)

    bm.backward_pair = chunkwise      # the same per-(b, h) layout handling
    try:
        got = bm.backward(inp, dO, dS, chunk=chunk, dconv_out=dC)
    finally:
        bm.backward_pair = orig
    assert len(calls) == 2 * 2        # every (b, h) went through the chunkwise model
    for x in ref:
        assert np.abs(got[x] - ref[x]).max() <= 1e-10 * max(1.0, np.abs(ref[x]).max()), x


def test_float32_chunks_of_32_within_the_backward_bound():
    """The chunk form in float32 (the precision a matrix-core kernel would use)
    at K3-like decay (mean about -0.6 per token, tails near -8): every gradient
    within 5e-5 x RMS of float64 for 32-token chunks, under the 1e-4 bound of
    the GPU backward.  Token by token float32 is about 5e-6; the error grows
    with the chunk length under strong decay (through the decay-weighted row
    and column sums and the reverse cumulative sum of dG), so longer chunks
    would need more care."""
    args = _case(128, 64, 64, seed=64, g_scale=8.0)
    ref = cbm.backward(*args, C=32)
    got = cbm.backward(*[np.asarray(x, dtype=np.float32) for x in args], C=32)
    assert got["g"].dtype == np.float32
    for n in ref:
        err = np.abs(got[n].astype(np.float64) - ref[n]).max() / np.sqrt(np.mean(ref[n] ** 2))
        assert err <= 5e-5, f"d{n}: {err:.2e}"
