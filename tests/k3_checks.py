"""Properties of K3's gate parameterisation that pin the oracle's KDA_DECAY_K3
form without restating its formula.

The pages ("Kimi K3.1 Pro vs gpt-oss-120b" and "Gemma 4 31B vs Kimi K3",
component tables, row "Gated DeltaNet / KDA") give the log-decay as the bounded
form g = -5 sigmoid(e^A z).  What follows from that alone:
  * e^A z -> +inf gives g -> -5 (the bound); e^A z -> -inf gives g -> 0;
  * z = 0 gives g = -5/2 whatever A is;
  * g(z) + g(-z) = -5 (sigmoid(x) + sigmoid(-x) = 1);
  * A enters only through e^A z: (z, A + ln 2) and (2z, A) decay alike;
  * A is per head: a head whose e^A is ~0 decays by -5/2 per token whatever z.
beta = sigmoid(b) gives beta = 1/2 at b = 0 and beta = 0 at b -> -inf.

Each check runs the oracle with beta = 0 (logit -1e4), where the state only
decays: S_T = diag(exp(sum_t g_t)) S0, so S_T / S0 exposes sum_t g_t.
"""
from __future__ import annotations

import math

import numpy as np

import kda_synth as syn
from kda_synth import Workload


def _base(T=9, H=2, dk=8, dv=12, seed=5):
    w = Workload("k3", 1, T, H, dk, dv, 16, "f32", s0_sigma=0.5, conv_hist="normal", seed=seed)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w)
    inp["beta"] = np.full(inp["beta"].shape, -1e4, np.float32)   # beta = 0
    return w, inp


def _ST(oracle_mod, inp, lib):
    return oracle_mod.prefill(inp, lib=lib)["S_T"]


def failures(oracle_mod, lib=None) -> list[str]:
    """Names of the properties this oracle build violates (empty: all hold)."""
    bad = []
    w, inp = _base()
    S0 = inp["S0"][0].astype(np.float64)                           # [H, dk, dv]
    T = w.T

    def with_(**kw):
        d = dict(inp)
        d.update(kw)
        return d

    z_shape = inp["g"].shape
    # the bound: g -> -5 for e^A z -> +inf (A = 0), g -> 0 for -inf
    zero_A = np.zeros((w.H, w.dk), np.float32)
    S = _ST(oracle_mod, with_(g=np.full(z_shape, 30.0, np.float32), A=zero_A), lib)
    if not np.allclose(S, S0 * math.exp(-5.0 * T), rtol=1e-9, atol=0):
        bad.append("bound -5")
    S = _ST(oracle_mod, with_(g=np.full(z_shape, -30.0, np.float32), A=zero_A), lib)
    if not np.allclose(S, S0, rtol=1e-9, atol=0):
        bad.append("limit 0")
    # z = 0: -5/2 per token for any A
    S = _ST(oracle_mod, with_(g=np.zeros(z_shape, np.float32)), lib)
    if not np.allclose(S, S0 * math.exp(-2.5 * T), rtol=1e-12, atol=0):
        bad.append("z = 0")
    # g(z) + g(-z) = -5
    z = inp["g"].astype(np.float32)
    Sp, Sm = _ST(oracle_mod, with_(g=z), lib), _ST(oracle_mod, with_(g=-z), lib)
    if not np.allclose(Sp * Sm, S0 * S0 * math.exp(-5.0 * T), rtol=1e-10, atol=0):
        bad.append("symmetry")
    # A only through e^A z
    A = inp["A"]
    S1 = _ST(oracle_mod, with_(g=(2.0 * z).astype(np.float32), A=A), lib)
    S2 = _ST(oracle_mod, with_(g=z, A=(A + np.float32(math.log(2.0))).astype(np.float32)), lib)
    if not np.allclose(S1, S2, rtol=1e-6, atol=0):
        bad.append("e^A scaling")
    # A per head: head 1 with e^A ~ 0 decays by -5/2 per token, head 0 does not
    A_h = A.copy()
    A_h[1, :] = -100.0
    S = _ST(oracle_mod, with_(g=z, A=A_h), lib)
    if not np.allclose(S[1], S0[1] * math.exp(-2.5 * T), rtol=1e-12, atol=0):
        bad.append("A of head 1")
    if np.allclose(S[0], S0[0] * math.exp(-2.5 * T), rtol=1e-3, atol=0):
        bad.append("A of head 0")
    # beta = sigmoid(b): b = 0 gives beta = 1/2; compare with the direct form
    # (g = 0 there; in the K3 form A = 0 and z = -60 give g ~ -4e-26)
    direct = with_(g=np.zeros(z_shape, np.float32), beta=np.full(inp["beta"].shape, 0.5, np.float32))
    direct.pop("A")
    k3 = with_(g=np.full(z_shape, -60.0, np.float32), A=zero_A,
               beta=np.zeros(inp["beta"].shape, np.float32))
    rd, rk = oracle_mod.prefill(direct, lib=lib), oracle_mod.prefill(k3, lib=lib)
    if not (np.allclose(rd["S_T"], rk["S_T"], rtol=1e-9, atol=1e-15)
            and np.allclose(rd["o"], rk["o"], rtol=1e-8, atol=1e-12)):
        bad.append("beta = sigmoid(b)")
    return bad
