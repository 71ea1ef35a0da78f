"""Independent reference computations used to pin the oracle (test helpers).

None of this imports the oracle's arithmetic: the convolution goes through
numpy.convolve, the recurrence through explicit products of dense transition
matrices, and the scalar case through closed-form products and sums.
"""
from __future__ import annotations

import numpy as np

from kda_synth import to_f64

L2_EPS = 1e-6
RMS_EPS = 1e-5


def head_channels(H, dk, dv, h):
    return np.concatenate([h * dk + np.arange(dk), H * dk + h * dk + np.arange(dk),
                           2 * H * dk + h * dv + np.arange(dv)])


def raw_head(inp, dtype, b, h):
    """Raw (pre-conv) q|k|v tokens of pair (b,h): [T, 2dk+dv] fp64."""
    q, k, v = (to_f64(inp[x], dtype) for x in ("q", "k", "v"))
    return np.concatenate([q[b, :, h], k[b, :, h], v[b, :, h]], axis=1)


def conv_numpy(x_raw, hist, w):
    """Causal depthwise conv (kernel 4) per channel with numpy.convolve.

    out[t] = sum_j w[j] x[t-3+j]; with a = hist ++ x, that is
    numpy.convolve(a, w[::-1])[t+3].
    """
    T, nc = x_raw.shape
    out = np.empty((T, nc))
    for c in range(nc):
        a = np.concatenate([hist[:, c], x_raw[:, c]])
        out[:, c] = np.convolve(a, w[c, ::-1], mode="full")[3:T + 3]
    return out


def silu(x):
    return x / (1.0 + np.exp(-x))


def prep_numpy(inp, dtype, b, h, hist=None):
    """q^, k^, v^ of one pair via numpy.convolve + SiLU + L2 normalisation."""
    q = inp["q"]
    B, T, H, dk = q.shape
    dv = inp["v"].shape[3]
    nc = 2 * dk + dv
    x_raw = raw_head(inp, dtype, b, h)
    if hist is None:
        hist = np.zeros((3, nc))
    w = np.asarray(inp["conv_w"], dtype=np.float64)[head_channels(H, dk, dv, h)]
    xt = silu(conv_numpy(x_raw, hist, w))
    qt, kt, vt = xt[:, :dk], xt[:, dk:2 * dk], xt[:, 2 * dk:]
    qn = qt / np.sqrt((qt ** 2).sum(1, keepdims=True) + L2_EPS) / np.sqrt(dk)
    kn = kt / np.sqrt((kt ** 2).sum(1, keepdims=True) + L2_EPS)
    return qn, kn, vt


def bruteforce_core(qn, kn, vn, g, beta, S0):
    """Dense unrolling of the recurrence.

    M_t = (I - beta_t k_t k_t^T) diag(exp g_t);  Phi_{t,i} = M_t ... M_{i+1}.
    o_core_t = (Phi_{t,0} S0)^T q_t + sum_{i<=t} beta_i (q_t^T Phi_{t,i} k_i) v_i
    S_T      = Phi_{T,0} S0 + sum_i Phi_{T,i} beta_i k_i v_i^T
    (indices 1-based in the formulas, 0-based below).  Returns (o_core [T,dv], S_T).
    """
    T, dk = qn.shape
    M = [(np.eye(dk) - beta[t] * np.outer(kn[t], kn[t])) @ np.diag(np.exp(g[t]))
         for t in range(T)]
    o = np.zeros((T, vn.shape[1]))
    for t in range(T):
        # Phi_{t,i} for i = t, t-1, ..., -1 (Phi_{t,t} = I; i = -1 is the initial state)
        phi = np.eye(dk)
        attn = np.zeros(t + 1)
        for i in range(t, -1, -1):
            attn[i] = beta[i] * qn[t] @ phi @ kn[i]
            phi = phi @ M[i]
        o[t] = (phi @ S0).T @ qn[t] + attn @ vn[:t + 1]
    phi = np.eye(dk)
    S_T = np.zeros_like(S0)
    for i in range(T - 1, -1, -1):
        S_T += phi @ (beta[i] * np.outer(kn[i], vn[i]))
        phi = phi @ M[i]
    S_T += phi @ S0
    return o, S_T


def gated_rmsnorm(o_core, gate):
    """o_core / sqrt(mean(o_core^2) + eps) * sigmoid(gate), row-wise."""
    r = np.sqrt((o_core ** 2).mean(-1, keepdims=True) + RMS_EPS)
    return o_core / r / (1.0 + np.exp(-gate))
