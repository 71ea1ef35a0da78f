"""The chunkwise algebra the kernels implement, checked against the oracle (CPU).

* exact in fp64 for several chunk sizes, ragged tails and a non-zero state;
* the operand-precision budget on prefill-like data: bf16 matrix-core operands
  put the max error at several times 1e-2 x RMS, too close to (or past) the
  2e-2 x RMS bound, while fp16 operands (same matrix-core rate, three more
  mantissa bits) stay under 0.4 of it.  That fixes the kernels' scheme:
  fp16 operands, fp32 accumulation, fp32 state, fp32 output;
* strong decay ("wide" chunks, a tile decaying by more than e^8): the scheme
  the kernels take there (fp32 in-tile blocks, U as an fp16 pair) against the
  bf16 operands of an earlier design, at K3's -5 bound and on mixed inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from chunk_model import chunk_core, chunk_core_kernel
from kda_synth import Workload, to_f64
from ref_math import gated_rmsnorm, head_channels, prep_numpy


def _case(T, dk, dv, dtype="f32", s0=0.2, seed=11, H=1):
    w = Workload("c", 1, T, H, dk, dv, 64, dtype, s0_sigma=s0, conv_hist="normal", seed=seed)
    return w, syn.prefill_inputs_np(w)


@pytest.mark.parametrize("form", ["wy", "tx"])
@pytest.mark.parametrize("C", [1, 2, 16, 64])
@pytest.mark.parametrize("T", [1, 15, 17, 64, 100])
def test_chunk_algebra_exact(oracle_mod, C, T, form):
    w, inp = _case(T, 16, 24)
    r = oracle_mod.prefill(inp, want_prep=True)
    prep = r["prep"][0]
    qn, kn, vn = prep[:, :16], prep[:, 16:32], prep[:, 32:]
    g = inp["g"][0, :, 0].astype(np.float64)
    beta = inp["beta"][0, :, 0].astype(np.float64)
    oc, S = chunk_core(qn, kn, vn, g, beta, inp["S0"][0, 0].astype(np.float64), C=C, form=form)
    o = gated_rmsnorm(oc, inp["gate"][0, :, 0].astype(np.float64))
    np.testing.assert_allclose(S, r["S_T"][0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(o, r["o"][0], rtol=1e-9, atol=1e-11)


def test_tile_references_bound_factors():
    """With g >= -5 no decay factor inside a 16-token tile exceeds e^80 (bf16 and fp32
    finite), which is what lets the decay-weighted products run as bf16 products."""
    g = np.full((64, 4), -5.0)
    G = np.cumsum(g, axis=0)
    worst = 0.0
    for a0 in range(0, 64, 16):
        rho = G[a0 - 1] if a0 else np.zeros(4)
        worst = max(worst, float(np.max(rho - G[a0:a0 + 16])))
        assert np.all(G[a0:a0 + 16] - rho <= 0)
    assert worst == 80.0 and np.isfinite(np.float32(np.exp(worst)))


def _operand_error(oracle_mod, operands, T=512, d=128, form="wy"):
    """max |err| / RMS for o and S_T with the given operand type, C = 64."""
    w, inp = _case(T, d, d, dtype="bf16", s0=0.01, seed=5, H=2)
    r = oracle_mod.prefill(inp, want_prep=True)
    errs_o, errs_s, ro, rs = [], [], [], []
    for i in range(2):
        prep = r["prep"][i]
        qn, kn, vn = prep[:, :d], prep[:, d:2 * d], prep[:, 2 * d:]
        g = to_f64(inp["g"], "bf16")[0, :, i]
        beta = to_f64(inp["beta"], "bf16")[0, :, i]
        gate = to_f64(inp["gate"], "bf16")[0, :, i]
        oc, S = chunk_core(qn, kn, vn, g, beta, inp["S0"][0, i].astype(np.float64), C=64,
                           operands=operands, form=form)
        o = gated_rmsnorm(oc, gate)
        errs_o.append(np.abs(o - r["o"][i]).max())
        errs_s.append(np.abs(S - r["S_T"][i]).max())
        ro.append(r["o"][i])
        rs.append(r["S_T"][i])
    rms_o = np.sqrt(np.mean(np.square(ro)))
    rms_s = np.sqrt(np.mean(np.square(rs)))
    return max(errs_o) / rms_o, max(errs_s) / rms_s


@pytest.mark.parametrize("form", ["wy", "tx"])
def test_operand_precision_budget(oracle_mod, form):
    """fp16 operands (d = 128, C = 64, bf16 inputs, non-zero initial state) keep the
    max error under 0.4 of the 2e-2 x RMS bound for o and S_T, in both orders of
    the U product; bf16 operands would not (their error is above half the bound)."""
    eo, es = _operand_error(oracle_mod, "fp16", form=form)
    assert eo < 0.4 * 2e-2 and es < 0.4 * 2e-2, (eo, es)
    if form == "tx":
        return
    bo, bs = _operand_error(oracle_mod, "bf16")
    assert max(bo, bs) > 0.5 * 2e-2, (bo, bs)


def test_cancellation_needs_full_precision_u(oracle_mod):
    """On a head of the B2 T4096 H32 workload where the state predicts the new
    values well (U = U~ - W S cancels), passing U~ in fp16 puts the state's max
    error past the 2e-2 x RMS bound, while both orders the kernels use (fp32
    U~ - W S in one kernel; T diag(beta) (V - (K e^G) S) with the difference
    in fp32 accumulators in the other) stay well inside it."""
    w = syn.WORKLOADS["prefill"]
    inp = syn.prefill_inputs_np(w)
    b, h = divmod(55, w.H)
    r = oracle_mod.prefill(inp, heads=[55], want_prep=True)
    d = w.dk
    prep = r["prep"][0]
    args = (prep[:, :d], prep[:, d:2 * d], prep[:, 2 * d:], syn.to_f64(inp["g"], "bf16")[b, :, h],
            syn.to_f64(inp["beta"], "bf16")[b, :, h], np.zeros((d, d)))
    rms_s = np.sqrt(np.mean(oracle_mod.prefill(inp, want_o=False)["S_T"] ** 2))  # over the workload
    err = {}
    for name, kw in [("wy", {}), ("tx", {"form": "tx"}), ("ut16", {"ut_rounded": True})]:
        _, S = chunk_core(*args, C=64, operands="fp16", **kw)
        err[name] = np.abs(S - r["S_T"][0]).max() / rms_s
    assert err["ut16"] > 2e-2, err
    assert err["wy"] < 0.6 * 2e-2 and err["tx"] < 0.6 * 2e-2, err


def _wide_case_error(oracle_mod, w, inp, scheme):
    """max |err| / RMS for o and S_T of the kernels' rounding model, and the
    number of wide chunks, over every head of the case."""
    r = oracle_mod.prefill(inp, want_prep=True)
    g_all, beta_all = oracle_mod.decay_and_beta(inp)
    d = w.dk
    eo, es, ro, rs, nwide = 0.0, 0.0, [], [], 0
    for p in range(w.B * w.H):
        b, h = divmod(p, w.H)
        prep = r["prep"][p]
        S0 = inp["S0"][b, h].astype(np.float64)
        oc, S, nw = chunk_core_kernel(prep[:, :d], prep[:, d:2 * d], prep[:, 2 * d:], g_all[b, :, h],
                                      beta_all[b, :, h], S0, wide_scheme=scheme)
        o = gated_rmsnorm(oc, to_f64(inp["gate"], "bf16")[b, :, h])
        eo, es = max(eo, np.abs(o - r["o"][p]).max()), max(es, np.abs(S - r["S_T"][p]).max())
        ro.append(r["o"][p])
        rs.append(r["S_T"][p])
        nwide += nw
    return eo / np.sqrt(np.mean(np.square(ro))), es / np.sqrt(np.mean(np.square(rs))), nwide


def test_wide_chunks_precision_design(oracle_mod):
    """Strong decay, modelled with the kernels' rounding points.  At K3's bound
    (every channel at -5 per token, tiles spanning e^80) bf16 decay-weighted
    operands put the largest o error past the 2e-2 x RMS bound; fp32 diagonal
    blocks plus U as an fp16 pair keep o and S_T under 0.6 of it.  The same
    scheme holds a few fast channels among normal ones, and g = -2 per token,
    under half of it."""
    w = Workload("k3b", 1, 160, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=53)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w, z_mean=6.0)
    bo, bs, nb = _wide_case_error(oracle_mod, w, inp, "bf16")
    so, ss, ns = _wide_case_error(oracle_mod, w, inp, "split")
    assert nb == ns == 2 * 3, (nb, ns)  # every chunk of both heads is wide
    assert bo > 2e-2, bo
    assert so < 0.6 * 2e-2 and ss < 0.6 * 2e-2, (so, ss)

    w = Workload("k3m", 1, 256, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=57)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w, fast_channels=8)
    so, ss, ns = _wide_case_error(oracle_mod, w, inp, "split")
    assert ns == 2 * 4, ns
    assert so < 0.5 * 2e-2 and ss < 0.5 * 2e-2, (so, ss)

    w = Workload("sd", 1, 160, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=31)
    inp = syn.prefill_inputs_np(w)
    gbits = syn.bf16_bits_from_f64(np.full(inp["g"].shape, -2.0))
    gbits[:, 64:128] = syn.bf16_bits_from_f64(np.full(inp["g"][:, 64:128].shape, -0.05))
    inp["g"] = gbits
    so, ss, ns = _wide_case_error(oracle_mod, w, inp, "split")
    assert ns == 2 * 2, ns  # the middle chunk decays slowly
    assert so < 0.5 * 2e-2 and ss < 0.5 * 2e-2, (so, ss)
