"""CPU model (float64 NumPy) of the GPU backward's algorithm, per (b, h): the
forward token loop with the state stored at every chunk start, then the chunks
in reverse, each recomputed from its stored state (keeping the state entering
every token and the per-token vectors) and walked back token by token with the
state gradient dS carried.  It uses no autograd; tests compare it with the
autograd reference (oracle/backward.py), so the step-by-step derivation the
kernel follows is checked on the CPU.

Per token t (forward): a = conv(raw), x~ = SiLU(a), q^ = q~ rq, k^ = k~ rk,
v^ = v~, S' = Diag(alpha) S_{t-1}, y = S'^T k^, u = beta (v^ - y),
S_t = S' + k^ u^T, z = S_t^T q^, n = z / r, o = n sigmoid(gate).
Reverse, with dS = dL/dS_t from the later tokens and do = dL/do_t:
  dgate = do n s (1 - s)                      (s = sigmoid(gate))
  dz    = (do s - n mean(do s n)) / r
  dq^   = S_t dz;      dS += q^ dz^T
  du    = dS^T k^;     dk^ = dS u
  dbeta = du . (v^ - y);  dv^ = beta du;  dy = -beta du
  dS'   = dS + k^ dy^T;   dk^ += S' dy
  dg    = rowsum(dS' * S');  dS_{t-1} = Diag(alpha) dS'
  dq~   = rq (dq^ - q~ (q~ . dq^) / nq),  nq = |q~|^2 + 1e-6  (same for k)
  da    = dx~ sigmoid(a) (1 + a (1 - sigmoid(a)))
  dx_s  = sum_{j=0..3} w_j da_{s+3-j}         (conv transpose; a 3-token ring of da)
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6
RMS_EPS = 1e-5


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def backward_pair(raw, hist, w, g, beta, gate, S0, dO, dS_T, chunk=64, dC=None):
    """One (b, h): raw [T, 3d] raw q|k|v, hist [3, 3d], w [3d, 4], g [T, d],
    beta [T], gate [T, d], S0 [d, d], dO [T, d], dS_T [d, d], dC [3, 3d] the
    gradient of the last three raw rows (all float64).
    Returns (draw [T, 3d], dhist [3, 3d], dg, dbeta, dgate, dS0)."""
    T, nc = raw.shape
    d = nc // 3
    full = np.concatenate([hist, raw], axis=0)  # row t + 3 = token t

    def token_vectors(t):
        a = w[:, 0] * full[t] + w[:, 1] * full[t + 1] + w[:, 2] * full[t + 2] + w[:, 3] * full[t + 3]
        x = a * _sig(a)
        qt, kt, vt = x[:d], x[d:2 * d], x[2 * d:]
        nq, nk = qt @ qt + L2_EPS, kt @ kt + L2_EPS
        rq, rk = nq ** -0.5 / np.sqrt(d), nk ** -0.5
        return dict(a=a, x=x, qt=qt, kt=kt, nq=nq, nk=nk, rq=rq, rk=rk, qn=qt * rq, kn=kt * rk, vn=vt)

    # forward: states at chunk starts
    nchunks = (T + chunk - 1) // chunk
    ckpt = np.zeros((nchunks, d, d))
    S = S0.copy()
    for t in range(T):
        if t % chunk == 0:
            ckpt[t // chunk] = S
        tv = token_vectors(t)
        Sp = np.exp(g[t])[:, None] * S
        y = Sp.T @ tv["kn"]
        u = beta[t] * (tv["vn"] - y)
        S = Sp + np.outer(tv["kn"], u)

    dS = dS_T.copy()
    draw = np.zeros((T, nc))
    dhist = np.zeros((3, nc))
    dg = np.zeros((T, d))
    dbeta = np.zeros(T)
    dgate = np.zeros((T, d))
    ring = np.zeros((3, nc))  # da of tokens t+1, t+2, t+3
    for c in range(nchunks - 1, -1, -1):
        t0, t1 = c * chunk, min(T, (c + 1) * chunk)
        # recompute the chunk: the state entering each token and its vectors
        S = ckpt[c].copy()
        entering, vecs = [], []
        for t in range(t0, t1):
            tv = token_vectors(t)
            alpha = np.exp(g[t])
            Sp = alpha[:, None] * S
            tv["y"] = Sp.T @ tv["kn"]
            tv["u"] = beta[t] * (tv["vn"] - tv["y"])
            entering.append(S)
            S = Sp + np.outer(tv["kn"], tv["u"])
            tv["z"] = S.T @ tv["qn"]
            vecs.append(tv)
        for t in range(t1 - 1, t0 - 1, -1):
            tv, Sprev = vecs[t - t0], entering[t - t0]
            alpha = np.exp(g[t])
            Sp = alpha[:, None] * Sprev
            St = Sp + np.outer(tv["kn"], tv["u"])
            r = np.sqrt(np.mean(tv["z"] ** 2) + RMS_EPS)
            n = tv["z"] / r
            s = _sig(gate[t])
            dgate[t] = dO[t] * n * s * (1 - s)
            dn = dO[t] * s
            dz = (dn - n * np.mean(dn * n)) / r
            dqn = St @ dz
            dS = dS + np.outer(tv["qn"], dz)
            du = dS.T @ tv["kn"]
            dkn = dS @ tv["u"]
            dbeta[t] = du @ (tv["vn"] - tv["y"])
            dvn = beta[t] * du
            dy = -beta[t] * du
            dSp = dS + np.outer(tv["kn"], dy)
            dkn = dkn + Sp @ dy
            dg[t] = np.sum(dSp * Sp, axis=1)
            dS = alpha[:, None] * dSp
            dqt = tv["rq"] * (dqn - tv["qt"] * (tv["qt"] @ dqn) / tv["nq"])
            dkt = tv["rk"] * (dkn - tv["kt"] * (tv["kt"] @ dkn) / tv["nk"])
            dx = np.concatenate([dqt, dkt, dvn])
            sa = _sig(tv["a"])
            da = dx * sa * (1 + tv["a"] * (1 - sa))
            draw[t] = w[:, 3] * da + w[:, 2] * ring[0] + w[:, 1] * ring[1] + w[:, 0] * ring[2]
            if dC is not None and t >= T - 3:
                draw[t] += dC[t - (T - 3)]
            ring = np.stack([da, ring[0], ring[1]])
    # history rows 0..2 are tokens -3..-1: dx_s = sum over t = 0 .. s + 3 of w_{s-t+3} da_t
    for s in (-1, -2, -3):
        dhist[s + 3] = sum(w[:, s - t + 3] * ring[t] for t in range(0, s + 4))
    if dC is not None:  # rows of conv_out that are history rows (T < 3)
        for kk in range(3):
            if T - 3 + kk < 0:
                dhist[T + kk] += dC[kk]
    return draw, dhist, dg, dbeta, dgate, dS


def backward(inp: dict, dO, dS_T, chunk=64, dconv_out=None) -> dict:
    """All (b, h) pairs; gradients in the layouts of the inputs (float64)."""
    def f64(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.astype(np.float64)

    q, k, v, g, beta, gate = (f64(inp[x]) for x in ("q", "k", "v", "g", "beta", "gate"))
    conv_w = np.asarray(inp["conv_w"], dtype=np.float64)
    B, T, H, d = q.shape
    cch = 3 * H * d
    S0 = np.zeros((B, H, d, d)) if inp.get("S0") is None else np.asarray(inp["S0"], dtype=np.float64)
    ci = np.zeros((B, 3, cch)) if inp.get("conv_in") is None else f64(inp["conv_in"])
    out = {x: np.zeros_like(a) for x, a in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                                             ("gate", gate), ("S0", S0), ("conv_in", ci))}
    dO = np.asarray(dO, dtype=np.float64)
    dS_T = np.zeros((B, H, d, d)) if dS_T is None else np.asarray(dS_T, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            ch = np.concatenate([h * d + np.arange(d), H * d + h * d + np.arange(d), 2 * H * d + h * d + np.arange(d)])
            raw = np.concatenate([q[b, :, h], k[b, :, h], v[b, :, h]], axis=1)
            dC = None if dconv_out is None else np.asarray(dconv_out, dtype=np.float64)[b][:, ch]
            draw, dhist, dg, dbeta, dgate, dS0 = backward_pair(raw, ci[b][:, ch], conv_w[ch], g[b, :, h],
                                                               beta[b, :, h], gate[b, :, h], S0[b, h],
                                                               dO[b, :, h], dS_T[b, h], chunk, dC)
            out["q"][b, :, h], out["k"][b, :, h], out["v"][b, :, h] = draw[:, :d], draw[:, d:2 * d], draw[:, 2 * d:]
            out["conv_in"][b][:, ch] = dhist
            out["g"][b, :, h], out["beta"][b, :, h], out["gate"][b, :, h] = dg, dbeta, dgate
            out["S0"][b, h] = dS0
    return out
