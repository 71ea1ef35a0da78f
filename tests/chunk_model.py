"""NumPy model of the chunkwise form of the KDA recurrence (test helper).

This is the algebra the GPU kernels implement, written out plainly so it can be
checked against the token-by-token oracle, and so the effect of rounding the
matrix-core operands to bf16 can be measured on the CPU before any GPU code.

Per chunk of C tokens entering with state S (dk x dv), with G the inclusive
cumulative sum of g inside the chunk (G_{-1} = 0):
  A_rj = beta_r sum_c k_rc k_jc e^{G_rc - G_jc}     (j < r)
  T    = (I + A)^-1
  W    = T diag(beta) (K * e^G) ;  U~ = T diag(beta) V
  U    = U~ - W S  ( = T diag(beta) (V - (K * e^G) S) )
  P_rj = sum_c q_rc k_jc e^{G_rc - G_jc}            (j <= r)
  O    = (Q * e^G) S + P U
  S'   = diag(e^{G_C}) S + (K * e^{G_C - G})^T U
The decay-weighted products use 16-token tiles: row tile a takes the reference
rho_a = G at the token before the tile (0 for the first tile), so the row factor
e^{G_r - rho_a} <= 1 and the column factor e^{rho_a - G_j} is <= 1 for earlier
tiles and bounded by e^{16 max|g|} inside the tile.
"""
from __future__ import annotations

import numpy as np

TILE = 16


def _bf16(x):
    """Round to bf16 (nearest even) and back, elementwise, through float32."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _fp16(x):
    """Round to IEEE half (nearest even) and back."""
    return np.asarray(x, dtype=np.float16).astype(np.float64)


def _id(x):
    return np.asarray(x, dtype=np.float64)


def _f32(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float64)


def _fp16_fin(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float16).astype(np.float64)


WIDE_SPAN = 8.0  # a chunk is "wide" when some tile decays by more than e^8 in some channel


def chunk_core_kernel(qn, kn, vn, g, beta, S0, wide_scheme="split", C=64, span=WIDE_SPAN):
    """The two-kernel path's rounding points, chunk by chunk (C = 64, 16-token tiles).

    fp16 operands everywhere, fp32 accumulation and state, as the kernels do:
    row factors e^{G - rho_a} <= 1; off-diagonal column factors referenced to
    the end of the column tile (<= 1); the diagonal column factor
    e^{rho_a - G} (up to e^{span} of the tile).  A chunk is wide when some
    tile's span exceeds e^8.  wide_scheme decides what a wide chunk does:
      "bf16":  every decay-weighted A / P operand in bf16 (an earlier design);
      "split": diagonal blocks of A and P from fp32 operands (q's row as its
               fp16 normalised value times the fp32 factor: the factor may
               underflow fp16 while the column factor makes up for it), and U
               passed to the P U and (K e^{G_C-G})^T U products as fp16 hi + lo.
    Returns (o_core [T, dv], S_T, number of wide chunks).
    """
    T, dk = qn.shape
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, vn.shape[1]))
    nwide = 0
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        n = c1 - c0
        Q, K, V, b = _f32(qn[c0:c1]), _f32(kn[c0:c1]), _f32(vn[c0:c1]), _f32(beta[c0:c1])
        G = _f32(np.cumsum(g[c0:c1], axis=0))
        tiles = list(range(0, n, TILE))
        refs = [G[a0 - 1] if a0 > 0 else np.zeros(dk) for a0 in tiles]
        wide = any(np.any(refs[i] - G[min(n, a0 + TILE) - 1] > span) for i, a0 in enumerate(tiles))
        nwide += wide
        op = _bf16 if (wide and wide_scheme == "bf16") else _fp16_fin
        A = np.zeros((n, n))
        P = np.zeros((n, n))
        for ai, a0 in enumerate(tiles):
            a1 = min(n, a0 + TILE)
            rho = refs[ai]
            rowf = np.exp(G[a0:a1] - rho)
            Kr, Qr = K[a0:a1] * rowf, Q[a0:a1] * rowf
            Kc = K[a0:a1] * np.exp(rho - G[a0:a1])
            with np.errstate(over="ignore", invalid="ignore"):
                if wide and wide_scheme == "split":
                    # q's fp32 row: its fp16 normalised value times the fp32 factor
                    Ad, Pd = _f32(Kr) @ _f32(Kc).T, _f32(_fp16(Q[a0:a1]) * rowf) @ _f32(Kc).T
                else:
                    Ad, Pd = op(Kr) @ op(Kc).T, op(Qr) @ op(Kc).T
            A[a0:a1, a0:a1] = np.where(np.isfinite(Ad), Ad, 0.0)   # upper part is discarded below
            P[a0:a1, a0:a1] = np.where(np.isfinite(Pd), Pd, 0.0)
            for bi in range(ai):
                b0 = tiles[bi]
                rb1 = G[b0 + TILE - 1]                              # end of column tile b
                cc = op(K[b0:b0 + TILE] * np.exp(rb1 - G[b0:b0 + TILE]))
                if bi < ai - 1:
                    cc = op(cc * np.exp(rho - rb1))
                A[a0:a1, b0:b0 + TILE] = op(Kr) @ cc.T
                P[a0:a1, b0:b0 + TILE] = op(Qr) @ cc.T
        A = np.tril(A, -1) * b[:, None]
        P = np.tril(P, 0)
        Tm = np.linalg.inv(np.eye(n) + A)
        Tb = _fp16(Tm * b[None, :])
        X = _fp16(V) - _fp16(K * np.exp(G)) @ _fp16(S)
        U = Tb @ _fp16(X)
        Ub = _fp16(U)
        if wide and wide_scheme == "split":
            Ub = Ub + _fp16(U - Ub)
        o[c0:c1] = _fp16(_fp16(Q * np.exp(G)) @ _fp16(S) + _fp16(P) @ Ub)
        S = np.exp(G[-1])[:, None] * S + _fp16(K * np.exp(G[-1] - G)).T @ Ub
    return o, S, nwide


def chunk_core(qn, kn, vn, g, beta, S0, C=64, operands=None, tile=TILE, form="wy", ut_rounded=False):
    """Chunkwise o_core [T,dv] and final state for one (b,h).

    qn, kn [T,dk] (q already scaled by dk^-1/2), vn [T,dv], g [T,dk], beta [T].
    operands = None (exact fp64), "bf16" or "fp16": every matrix-core operand is
    rounded to that type while accumulation, decay factors and the state stay in
    higher precision, as in the GPU kernels.
    form = "wy": U = U~ - W S with W, U~ formed inside the chunk (single-kernel
    path); "tx": U = (T diag(beta)) (V - (K e^G) S), the same product taken in
    the other order (two-kernel path), with its operand rounding points.
    ut_rounded: also round U~ to the operand type before U = U~ - W S (a
    hand-over the kernels do not use: see test_chunk_algebra).
    """
    rnd = {None: _id, "bf16": _bf16, "fp16": _fp16}[operands]
    f32 = _id if operands is None else (lambda x: np.asarray(x, dtype=np.float32).astype(np.float64))
    T, dk = qn.shape
    dv = vn.shape[1]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        n = c1 - c0
        Q, K, V = f32(qn[c0:c1]), f32(kn[c0:c1]), f32(vn[c0:c1])
        b = f32(beta[c0:c1])
        G = f32(np.cumsum(g[c0:c1], axis=0))
        A = np.zeros((n, n))
        P = np.zeros((n, n))
        for a0 in range(0, n, tile):
            a1 = min(n, a0 + tile)
            rho = G[a0 - 1] if a0 > 0 else np.zeros(dk)
            rowf = np.exp(G[a0:a1] - rho)                        # <= 1
            colf = np.exp(rho - G[:a1])                          # <= 1 before a0
            Kr, Qr, Kc = rnd(K[a0:a1] * rowf), rnd(Q[a0:a1] * rowf), rnd(K[:a1] * colf)
            A[a0:a1, :a1] = Kr @ Kc.T
            P[a0:a1, :a1] = Qr @ Kc.T
        A = np.tril(A, -1) * b[:, None]
        P = np.tril(P, 0)
        Tm = np.linalg.inv(np.eye(n) + A)
        Tb = rnd(Tm * b[None, :])
        if form == "tx":
            X = rnd(V) - rnd(K * np.exp(G)) @ rnd(S)
            U = Tb @ rnd(X)
        else:
            W = Tb @ rnd(K * np.exp(G))
            Ut = Tb @ rnd(V)
            U = (rnd(Ut) if ut_rounded else Ut) - rnd(W) @ rnd(S)
        Ub = rnd(U)
        o[c0:c1] = rnd(Q * np.exp(G)) @ rnd(S) + rnd(P) @ Ub
        S = np.exp(G[-1])[:, None] * S + rnd(K * np.exp(G[-1] - G)).T @ Ub
    return o, S
