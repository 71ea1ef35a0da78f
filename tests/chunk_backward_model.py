"""CPU model (float64 NumPy) of a chunkwise backward of the KDA recurrence core,
per (b, h): the gradients reach every chunk through one reverse recurrence of
the state gradient over chunks, and each chunk's gradients are matrix products
over the chunk, the shape a matrix-core kernel takes (the chunkwise form of
the forward run in reverse, instead of a token-by-token walk).  It uses no
autograd; tests/test_chunk_backward_model.py compares it with torch autograd of
the token-serial core.

Core of the recurrence ("Kimi K3, previewed", section "Kimi Delta Attention -
the workhorse": fine-grained per-channel decay with the delta rule), per token
t with q^, k^, v^ given (after the conv, SiLU and norms):
  S' = Diag(e^{g_t}) S_{t-1},  u_t = beta_t (v^_t - S'^T k^_t),
  S_t = S' + k^_t u_t^T,       o_t = S_t^T q^_t.
Chunk of C tokens entering with S_in, G the chunk-local inclusive cumulative
sum of g (per channel), G_C its last row:
  F = K e^G,  Qg = Q e^G,  H = K e^{G_C - G}            (all factors <= 1)
  A_ij = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}   (j < i),  T = (I + A)^-1
  P_ij = sum_c q_ic k_jc e^{G_ic - G_jc}          (j <= i)
  W = diag(beta) (V - F S_in),  U = T W
  O = Qg S_in + P U,  S_out = Diag(e^{G_C}) S_in + H^T U.
Reverse of one chunk, given dO and dS_out:
  dU = P^T dO + H dS_out,  dW = T^T dU,  dT = dU W^T,  dA = -T^T dT T^T (j < i),
  dP = dO U^T (j <= i),  dV = diag(beta) dW,  dbeta = rowsum(dW * (V - F S_in)) + ...,
  dF = -diag(beta) dW S_in^T,  dQg = dO S_in^T,  dH = U dS_out^T,
  dS_in = Qg^T dO + Diag(e^{G_C}) dS_out + F^T (-diag(beta) dW),
then through A, P, F, Qg, H and Diag(e^{G_C}) to q, k, beta and G, and from G to
g by the reverse cumulative sum (G_C depends on every g of the chunk).
"""
from __future__ import annotations

import numpy as np


def _chunk_terms(q, k, v, g, beta, S_in):
    """Forward quantities of one chunk (rows = tokens)."""
    C = q.shape[0]
    G = np.cumsum(g, axis=0)
    GC = G[-1]
    # [i, j, c] e^{G_i - G_j}; only j <= i is used (exponent <= 0), the rest is
    # clamped so that it cannot overflow in float32
    E = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))
    low = np.tril(np.ones((C, C)), -1)                  # j < i
    lowd = np.tril(np.ones((C, C)))                     # j <= i
    Ap = np.einsum("ic,jc,ijc->ij", k, k, E) * low      # A' (without beta)
    A = beta[:, None] * Ap
    P = np.einsum("ic,jc,ijc->ij", q, k, E) * lowd
    T = np.linalg.inv(np.eye(C) + A)
    F = k * np.exp(G)
    Qg = q * np.exp(G)
    H = k * np.exp(GC[None, :] - G)
    R = v - F @ S_in                                    # V - F S_in
    W = beta[:, None] * R
    U = T @ W
    O = Qg @ S_in + P @ U
    S_out = np.exp(GC)[:, None] * S_in + H.T @ U
    return dict(G=G, GC=GC, E=E, low=low, lowd=lowd, Ap=Ap, A=A, P=P, T=T, F=F, Qg=Qg, H=H, R=R, W=W, U=U,
                O=O, S_out=S_out)


def forward(q, k, v, g, beta, S0, C=64):
    """Chunkwise forward of the core over T tokens: O [T, dv], S_T, and the
    state entering every chunk."""
    Tn = q.shape[0]
    S = S0.copy()
    O = np.zeros((Tn, v.shape[1]))
    states = []
    for c0 in range(0, Tn, C):
        sl = slice(c0, min(Tn, c0 + C))
        states.append(S.copy())
        f = _chunk_terms(q[sl], k[sl], v[sl], g[sl], beta[sl], S)
        O[sl] = f["O"]
        S = f["S_out"]
    return O, S, states


def _chunk_backward(q, k, v, g, beta, S_in, dO, dS_out):
    """Gradients of one chunk's (O, S_out) map; returns dq, dk, dv, dg, dbeta, dS_in."""
    f = _chunk_terms(q, k, v, g, beta, S_in)
    T, P, U, W, R, E, H, F, Qg = f["T"], f["P"], f["U"], f["W"], f["R"], f["E"], f["H"], f["F"], f["Qg"]
    G, GC = f["G"], f["GC"]
    # through U = T W, O = Qg S_in + P U, S_out = Diag(e^{G_C}) S_in + H^T U
    dU = P.T @ dO + H @ dS_out
    dW = T.T @ dU
    dT = dU @ W.T
    dA = -(T.T @ dT @ T.T) * f["low"]
    dP = (dO @ U.T) * f["lowd"]
    dR = beta[:, None] * dW
    dbeta = np.sum(dW * R, axis=1) + np.sum(dA * f["Ap"], axis=1)
    dv = dR.copy()
    dF = -dR @ S_in.T
    dQg = dO @ S_in.T
    dH = U @ dS_out.T
    dS_in = Qg.T @ dO + np.exp(GC)[:, None] * dS_out - F.T @ dR
    dGC = np.exp(GC) * np.sum(dS_out * S_in, axis=1)
    # through A_ij = beta_i sum_c k_ic k_jc E_ijc and P_ij = sum_c q_ic k_jc E_ijc
    dAb = dA * beta[:, None]                               # d/dA'
    dq = np.einsum("ij,jc,ijc->ic", dP, k, E)
    dk = (np.einsum("ij,jc,ijc->ic", dAb, k, E) + np.einsum("ij,ic,ijc->jc", dAb, k, E)
          + np.einsum("ij,ic,ijc->jc", dP, q, E))
    # G enters E with + at row i and - at column j
    tA = np.einsum("ij,ic,jc,ijc->ijc", dAb, k, k, E)
    tP = np.einsum("ij,ic,jc,ijc->ijc", dP, q, k, E)
    dG = tA.sum(axis=1) - tA.sum(axis=0) + tP.sum(axis=1) - tP.sum(axis=0)
    # through F = K e^G, Qg = Q e^G, H = K e^{G_C - G}
    eG = np.exp(G)
    dk += dF * eG + dH * np.exp(GC[None, :] - G)
    dq += dQg * eG
    dG += dF * F + dQg * Qg - dH * H
    dGC += np.sum(dH * H, axis=0)
    # G = cumsum(g) within the chunk; G_C = G[-1] depends on every g
    dg = np.cumsum(dG[::-1], axis=0)[::-1] + dGC[None, :]
    return dq, dk, dv, dg, dbeta, dS_in


def backward(q, k, v, g, beta, S0, dO, dS_T, C=64):
    """Gradients of <dO, O> + <dS_T, S_T> with respect to q, k, v, g, beta, S0,
    chunk by chunk from the last (one state per chunk kept by the forward)."""
    Tn = q.shape[0]
    _, _, states = forward(q, k, v, g, beta, S0, C)
    dq, dk, dv, dg = (np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(g))
    dbeta = np.zeros_like(beta)
    dS = dS_T.copy()
    starts = list(range(0, Tn, C))
    for n in range(len(starts) - 1, -1, -1):
        sl = slice(starts[n], min(Tn, starts[n] + C))
        dq[sl], dk[sl], dv[sl], dg[sl], dbeta[sl], dS = _chunk_backward(
            q[sl], k[sl], v[sl], g[sl], beta[sl], states[n], dO[sl], dS)
    return dict(q=dq, k=dk, v=dv, g=dg, beta=dbeta, S0=dS)


def backward_phased(q, k, v, g, beta, S0, dO, dS_T, C=64):
    """The same gradients in the three phases a kernel set would run:
      1. every chunk at once, from its entering state: the operands Qg, F, H,
         T diag(beta), P and e^{G_C};
      2. one serial pass over the chunks, last first, carrying only dS:
         dS_in = Diag(e^{G_C}) dS_out + Qg^T dO - F^T Z,
         Z = diag(beta) T^T (P^T dO + H dS_out)
         (the transpose of the forward's chunk transition, plus the output term);
      3. every chunk at once again, from its dS_out: the gradients of q, k, v, g
         and beta (the chunk reverse above, whose dS_in is not used).
    Phase 2 is the only sequential part; its work per chunk is the forward
    recurrence's (a d x C by C x d product chain)."""
    Tn = q.shape[0]
    _, _, states = forward(q, k, v, g, beta, S0, C)
    starts = list(range(0, Tn, C))
    sls = [slice(c0, min(Tn, c0 + C)) for c0 in starts]
    ops = [_chunk_terms(q[sl], k[sl], v[sl], g[sl], beta[sl], states[n]) for n, sl in enumerate(sls)]
    dS_out = [None] * len(sls)
    dS = dS_T.copy()
    for n in range(len(sls) - 1, -1, -1):
        f, sl = ops[n], sls[n]
        dS_out[n] = dS
        Z = beta[sl][:, None] * (f["T"].T @ (f["P"].T @ dO[sl] + f["H"] @ dS))
        dS = np.exp(f["GC"])[:, None] * dS + f["Qg"].T @ dO[sl] - f["F"].T @ Z
    out = dict(q=np.zeros_like(q), k=np.zeros_like(k), v=np.zeros_like(v), g=np.zeros_like(g),
               beta=np.zeros_like(beta), S0=dS)
    for n, sl in enumerate(sls):
        dq, dk, dv, dg, db, _ = _chunk_backward(q[sl], k[sl], v[sl], g[sl], beta[sl], states[n], dO[sl], dS_out[n])
        out["q"][sl], out["k"][sl], out["v"][sl], out["g"][sl], out["beta"][sl] = dq, dk, dv, dg, db
    return out


L2_EPS = 1e-6
RMS_EPS = 1e-5


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def backward_pair_chunkwise(raw, hist, w, g, beta, gate, S0, dO, dS_T, chunk=64, dC=None):
    """The whole backward of one (b, h), with the arguments and results of the
    token-by-token model (tests/backward_model.py, backward_pair), organised as
    a chunkwise kernel set would be: per-token work (conv, SiLU, norms, the
    RMSNorm * sigmoid(gate) backward, the norm / SiLU / conv-transpose backward)
    on all tokens at once, and the recurrence core's gradients by the three
    phases of backward_phased."""
    T, nc = raw.shape
    d = nc // 3
    full = np.concatenate([hist, raw], axis=0)              # row t + 3 = token t
    a = w[:, 0] * full[0:T] + w[:, 1] * full[1:T + 1] + w[:, 2] * full[2:T + 2] + w[:, 3] * full[3:T + 3]
    x = a * _sig(a)
    qt, kt, vn = x[:, :d], x[:, d:2 * d], x[:, 2 * d:]
    nq = np.sum(qt * qt, axis=1) + L2_EPS
    nk = np.sum(kt * kt, axis=1) + L2_EPS
    rq, rk = nq ** -0.5 / np.sqrt(d), nk ** -0.5
    qn, kn = qt * rq[:, None], kt * rk[:, None]
    z, _, _ = forward(qn, kn, vn, g, beta, S0, chunk)
    # RMSNorm * sigmoid(gate), per token
    r = np.sqrt(np.mean(z * z, axis=1) + RMS_EPS)
    n = z / r[:, None]
    s = _sig(gate)
    dgate = dO * n * s * (1 - s)
    dn = dO * s
    dz = (dn - n * np.mean(dn * n, axis=1, keepdims=True)) / r[:, None]
    core = backward_phased(qn, kn, vn, g, beta, S0, dz, dS_T, chunk)
    dqn, dkn, dvn = core["q"], core["k"], core["v"]
    # L2 norms, SiLU, conv transpose
    dqt = rq[:, None] * (dqn - qt * (np.sum(qt * dqn, axis=1) / nq)[:, None])
    dkt = rk[:, None] * (dkn - kt * (np.sum(kt * dkn, axis=1) / nk)[:, None])
    dx = np.concatenate([dqt, dkt, dvn], axis=1)
    sa = _sig(a)
    da = dx * sa * (1 + a * (1 - sa))
    pad = np.concatenate([da, np.zeros((3, nc))], axis=0)  # da of tokens t .. t + 3
    draw = w[:, 3] * pad[0:T] + w[:, 2] * pad[1:T + 1] + w[:, 1] * pad[2:T + 2] + w[:, 0] * pad[3:T + 3]
    dhist = np.zeros((3, nc))
    for hr in range(3):                                     # history row hr is token hr - 3
        for t in range(0, min(hr + 1, T)):
            dhist[hr] += w[:, hr - t] * da[t]
    if dC is not None:                                      # conv_out's rows: the last three raw rows
        for kk in range(3):
            t = T - 3 + kk
            if t >= 0:
                draw[t] += dC[kk]
            else:
                dhist[t + 3] += dC[kk]
    return draw, dhist, core["g"], core["beta"], dgate, core["S0"]
