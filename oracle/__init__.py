"""fp64 CPU oracle for Kimi Delta Attention (KDA) -- TEST INFRASTRUCTURE.

Only the test-suite, the smoke check (`__graft_entry__.smoke`) and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library and never imports it.

Two independent routes to the same definition (see kda_oracle.h for the steps,
and the pages: "Kimi K3, previewed", section "Kimi Delta Attention - the
workhorse"; the component tables of "Kimi K3.1 Pro vs gpt-oss-120b" and
"Gemma 4 31B vs Kimi K3", rows "Gated DeltaNet / KDA" and "Output gate + sink";
rms_norm_eps from the "Kimi K3" model card config):

* `prefill` -- the C recurrence (kda_oracle.c): S <- diag(a) S, then the
  delta-rule correction S += beta k (v - S^T k)^T, read-out S^T q.
* `prefill_matrix_form` -- NumPy, the state update written literally as the
  matrix product S_t = (I - beta k k^T) Diag(alpha_t) S_{t-1} + beta k v^T with
  an explicit dk x dk transition.  Slow; for small shapes.

Context parallelism ("Gemma 4 31B vs Kimi K3", component table, long-context
training row): a segment maps its entering state S to M S + N.
`segment_transition` builds M as the ordered product of the per-token maps,
`segment_fragments` returns (M, N), `compose_segments` the entering states, and
`prefill_context_parallel` the whole prefill computed segment by segment.

Inputs are numpy arrays: float32, or uint16 holding bf16 bits.  All
arithmetic is fp64 on the exact input values.

K3's gate parameterisation ("Kimi K3.1 Pro vs gpt-oss-120b" and "Gemma 4 31B
vs Kimi K3", component tables, row "Gated DeltaNet / KDA"): when `inp` holds
"A" (fp32 [H, dk]), g and beta are logits z and b, and the recurrence uses the
bounded log-decay g = -5 sigmoid(e^A z) and beta = sigmoid(b) (`k3_log_decay`,
`k3_beta`).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

L2_EPS = 1e-6
RMS_EPS = 1e-5


def build(force: bool = True, src: str = _SRC, out: str = _SO) -> str:
    """Compile the C oracle with gcc (no fast-math) into oracle/liboracle.so."""
    if force or not os.path.exists(out):
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-I", _HERE, "-o", out + ".tmp", src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return out


class _Inputs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("in_dtype", ctypes.c_int),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("conv_w", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("decay_form", ctypes.c_int), ("A", ctypes.c_void_p)]


_lib_handle = None


def load_library(path: str):
    """ctypes handle of a compiled oracle library (the default one, or a test build)."""
    lib = ctypes.CDLL(path)
    lib.kdao_prefill.restype = ctypes.c_int
    lib.kdao_prefill.argtypes = [ctypes.POINTER(_Inputs), ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int]
    lib.kdao_max_threads.restype = ctypes.c_int
    return lib


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        _lib_handle = load_library(_SO)
    return _lib_handle


def max_threads() -> int:
    return int(_lib().kdao_max_threads())


def k3_log_decay(z, A):
    """K3's bounded log-decay -5 sigmoid(e^A z) (fp64), z [..., dk], A broadcast over it."""
    return -5.0 / (1.0 + np.exp(-np.exp(A) * z))


def k3_beta(b):
    """beta = sigmoid(b) of a beta logit (fp64)."""
    return 1.0 / (1.0 + np.exp(-b))


def decay_and_beta(inp: dict):
    """fp64 log-decay g [B,T,H,dk] and beta [B,T,H] that `prefill` uses for these inputs."""
    g, beta = _f64(inp["g"]), _f64(inp["beta"])
    if inp.get("A") is None:
        return g, beta
    A = np.asarray(inp["A"], dtype=np.float32).astype(np.float64)
    return k3_log_decay(g, A[None, None]), k3_beta(beta)


def _dtype_of(a) -> str:
    if a.dtype == np.uint16:
        return "bf16"
    if a.dtype == np.float32:
        return "f32"
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _f64(a) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _pairs(B, H, heads):
    if heads is None:
        return np.arange(B * H, dtype=np.int32)
    bh = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    if bh.size and (bh.min() < 0 or bh.max() >= B * H):
        raise ValueError(f"(b,h) pair index out of range [0, {B * H})")
    return bh


def _head_channels(H, dk, dv, h):
    """conv channel indices of head h in the packed order q | k | v (head-major)."""
    return np.concatenate([h * dk + np.arange(dk), H * dk + h * dk + np.arange(dk),
                           2 * H * dk + h * dv + np.arange(dv)])


def initial_carry(B, H, dk, dv, heads=None, S0=None, conv_in=None):
    """fp64 per-pair initial state [n,dk,dv] and raw conv history [n,3,2dk+dv]."""
    bh = _pairs(B, H, heads)
    n = len(bh)
    S = np.zeros((n, dk, dv))
    hist = np.zeros((n, 3, 2 * dk + dv))
    S0a = None if S0 is None else np.asarray(S0)
    ci = None
    if conv_in is not None:
        ci = _f64(conv_in) if conv_in.dtype in (np.uint16, np.float32) else conv_in
    for i, p in enumerate(bh):
        b, h = divmod(int(p), H)
        if S0a is not None:
            S[i] = S0a[b, h]
        if ci is not None:
            hist[i] = ci[b][:, _head_channels(H, dk, dv, h)]
    return S, hist


def prefill(inp: dict, heads=None, S=None, hist=None, want_o=True, want_prep=False,
            nthreads: int = 0, lib=None) -> dict:
    """Run the C recurrence over the (b,h) pairs `heads` (default: all).

    `inp` holds q k v g gate beta conv_w (numpy; shapes [B,T,H,.]) and optionally
    S0 / conv_in.  `S` / `hist` (fp64, per pair) override S0 / conv_in and are
    updated in place, so consecutive calls carry the state.
    Returns dict(o [n,T,dv], S_T [n,dk,dv], conv_out [n,3,2dk+dv], prep [n,T,2dk+dv]).
    """
    q, k, v, g, beta, gate = (np.ascontiguousarray(inp[x]) for x in
                              ("q", "k", "v", "g", "beta", "gate"))
    conv_w = np.ascontiguousarray(inp["conv_w"], dtype=np.float32)
    dt = _dtype_of(q)
    for a in (k, v, g, beta, gate):
        if _dtype_of(a) != dt:
            raise TypeError("all activation inputs must share one dtype")
    B, T, H, dk = q.shape
    dv = v.shape[3]
    bh = _pairs(B, H, heads)
    if S is None or hist is None:
        S0, h0 = initial_carry(B, H, dk, dv, bh, inp.get("S0"), inp.get("conv_in"))
        S = S0 if S is None else S
        hist = h0 if hist is None else hist
    assert S.dtype == np.float64 and S.flags.c_contiguous and S.shape == (len(bh), dk, dv)
    assert hist.dtype == np.float64 and hist.flags.c_contiguous
    o = np.zeros((len(bh), T, dv)) if want_o else None
    prep = np.zeros((len(bh), T, 2 * dk + dv)) if want_prep else None
    A = inp.get("A")
    if A is not None:
        A = np.ascontiguousarray(A, dtype=np.float32)
        if A.shape != (H, dk):
            raise ValueError(f"A must be [H, dk] = [{H}, {dk}], got {A.shape}")
    st = _Inputs(B, T, H, dk, dv, 1 if dt == "bf16" else 0, q.ctypes.data, k.ctypes.data,
                 v.ctypes.data, conv_w.ctypes.data, g.ctypes.data, beta.ctypes.data,
                 gate.ctypes.data, 0 if A is None else 1, None if A is None else A.ctypes.data)
    rc = (lib or _lib()).kdao_prefill(ctypes.byref(st), _ptr(bh), len(bh), _ptr(S), _ptr(hist),
                             _ptr(o) if o is not None else None,
                             _ptr(prep) if prep is not None else None, int(nthreads))
    if rc != 0:
        raise ValueError("kdao_prefill rejected its arguments")
    return {"o": o, "S_T": S, "conv_out": hist, "prep": prep, "heads": bh}


def decode_step(step_inp: dict, S: np.ndarray, hist: np.ndarray, heads=None,
                nthreads: int = 0) -> np.ndarray:
    """One decode step: inputs [N,H,.] (one token per sequence).  S and hist
    (fp64, per listed pair) are updated in place; returns o [n, dv]."""
    one = {x: step_inp[x][:, None] for x in ("q", "k", "v", "g", "beta", "gate")}
    one["conv_w"] = step_inp["conv_w"]
    one["A"] = step_inp.get("A")
    r = prefill(one, heads=heads, S=S, hist=hist, nthreads=nthreads)
    return r["o"][:, 0, :]


# ----------------------------------------------------------------------------
# NumPy twin in the literal matrix form (second arithmetic route, small shapes)
# ----------------------------------------------------------------------------

def _silu(x):
    return x / (1.0 + np.exp(-x))


def prep_matrix_form(x_raw, hist, w):
    """conv (kernel 4, causal, history rows oldest-first) + SiLU for one head.

    x_raw [T, nc] raw tokens, hist [3, nc], w [nc, 4] (tap 3 = current token).
    Written as a sum over taps of shifted copies of the padded sequence.
    """
    T = x_raw.shape[0]
    padded = np.concatenate([hist, x_raw], axis=0)          # [T+3, nc]
    acc = np.zeros_like(x_raw)
    for j in range(4):
        acc = acc + w[:, j][None, :] * padded[j:j + T]
    return _silu(acc)


def prefill_matrix_form(inp: dict, heads=None, S=None, hist=None) -> dict:
    """Same outputs as `prefill`, with the state update as an explicit matrix product."""
    q, k, v = _f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"])
    gate = _f64(inp["gate"])
    g, beta = _f64(inp["g"]), _f64(inp["beta"])
    if inp.get("A") is not None:  # K3's logits, mapped here with NumPy's own exp
        A = np.asarray(inp["A"], dtype=np.float32).astype(np.float64)
        g = -5.0 * (1.0 / (1.0 + np.exp(-(np.exp(A)[None, None] * g))))
        beta = 1.0 / (1.0 + np.exp(-beta))
    conv_w = np.asarray(inp["conv_w"], dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    bh = _pairs(B, H, heads)
    if S is None or hist is None:
        S0, h0 = initial_carry(B, H, dk, dv, bh, inp.get("S0"), inp.get("conv_in"))
        S = S0 if S is None else S
        hist = h0 if hist is None else hist
    o = np.zeros((len(bh), T, dv))
    S_T = np.zeros_like(S)
    hist_out = np.zeros_like(hist)
    eye = np.eye(dk)
    for i, p in enumerate(bh):
        b, h = divmod(int(p), H)
        ch = _head_channels(H, dk, dv, h)
        x_raw = np.concatenate([q[b, :, h], k[b, :, h], v[b, :, h]], axis=1)  # [T, nc]
        xt = prep_matrix_form(x_raw, hist[i], conv_w[ch])
        qt, kt, vt = xt[:, :dk], xt[:, dk:2 * dk], xt[:, 2 * dk:]
        qn = qt / np.sqrt((qt * qt).sum(1, keepdims=True) + L2_EPS) / np.sqrt(dk)
        kn = kt / np.sqrt((kt * kt).sum(1, keepdims=True) + L2_EPS)
        St = S[i].copy()
        for t in range(T):
            kk = kn[t][:, None]
            M = (eye - beta[b, t, h] * (kk @ kk.T)) @ np.diag(np.exp(g[b, t, h]))
            St = M @ St + beta[b, t, h] * (kk @ vt[t][None, :])
            oc = St.T @ qn[t]
            rms = np.sqrt(np.mean(oc * oc) + RMS_EPS)
            o[i, t] = oc / rms / (1.0 + np.exp(-gate[b, t, h]))
        S_T[i] = St
        full = np.concatenate([hist[i], x_raw], axis=0)
        hist_out[i] = full[-3:]
    return {"o": o, "S_T": S_T, "conv_out": hist_out, "heads": bh}


# ----------------------------------------------------------------------------
# Context parallelism ("Gemma 4 31B vs Kimi K3", component table, long-context
# training row: ranks exchange only fixed-size state fragments).  Plainest
# reading: the state update is affine in the state, so a segment acts on the
# state entering it as
# S_out = M S_in + N; each rank forms (M, N) for its segment, the fragments are
# gathered, and a prefix composition gives every segment its entering state.
# ----------------------------------------------------------------------------

def segment_transition(inp: dict, heads=None, hist=None) -> np.ndarray:
    """M [n, dk, dk] per (b, h) pair: the product, over the tokens in order, of the
    per-token maps (I - beta k^ k^T) Diag(e^g) -- the linear part of the update,
    so that S_T = M S_0 + N for every initial state S_0.

    k^ (conv + SiLU + L2 norm from the raw history `hist`, default from
    inp["conv_in"] or zeros) comes from the C oracle's prep output; g and beta
    as the recurrence takes them.  Each token is applied as the rank-1 form
    D M - beta k^ (k^T D M) of the same product."""
    q = inp["q"]
    B, T, H, dk = q.shape
    dv = inp["v"].shape[3]
    bh = _pairs(B, H, heads)
    S0, h0 = initial_carry(B, H, dk, dv, bh, None, inp.get("conv_in"))
    r = prefill(inp, heads=bh, S=S0, hist=h0 if hist is None else hist.copy(), want_o=False,
                want_prep=True)
    g, beta = decay_and_beta(inp)
    M = np.zeros((len(bh), dk, dk))
    for i, p in enumerate(bh):
        b, h = divmod(int(p), H)
        Mi = np.eye(dk)
        kn = r["prep"][i][:, dk:2 * dk]
        for t in range(T):
            DM = np.exp(g[b, t, h])[:, None] * Mi
            Mi = DM - beta[b, t, h] * np.outer(kn[t], kn[t] @ DM)
        M[i] = Mi
    return M


def segment_fragments(inp: dict, heads=None, hist=None) -> tuple:
    """(M, N) of each listed pair for one segment: N is the state after the
    segment from S = 0 (the C recurrence), M its `segment_transition`."""
    q = inp["q"]
    B, T, H, dk = q.shape
    dv = inp["v"].shape[3]
    bh = _pairs(B, H, heads)
    S, h0 = initial_carry(B, H, dk, dv, bh, None, inp.get("conv_in"))
    h0 = h0 if hist is None else hist.copy()
    M = segment_transition(inp, heads=bh, hist=h0)
    prefill(inp, heads=bh, S=S, hist=h0.copy(), want_o=False)
    return M, S


def compose_segments(M: np.ndarray, N: np.ndarray, S0: np.ndarray) -> tuple:
    """Prefix composition: M, N [R, n, dk, .] per segment, S0 [n, dk, dv] entering
    segment 0.  Returns (S_start [R, n, dk, dv], S_end [n, dk, dv]) with
    S_start[0] = S0 and S_start[r + 1] = M[r] S_start[r] + N[r] (fp64)."""
    R = M.shape[0]
    S_start = np.zeros((R,) + S0.shape)
    S = np.array(S0, dtype=np.float64)
    for r in range(R):
        S_start[r] = S
        S = np.einsum("nij,njk->nik", M[r], S) + N[r]
    return S_start, S


def _segment_inputs(inp: dict, t0: int, t1: int) -> tuple:
    """Inputs of tokens [t0, t1) and the raw conv history [B, 3, Cch] entering them
    (the caller's conv_in before token 0, zeros before that)."""
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[3]
    seg = {x: inp[x][:, t0:t1] for x in ("q", "k", "v", "g", "beta", "gate")}
    seg["conv_w"] = inp["conv_w"]
    seg["A"] = inp.get("A")
    raw = np.concatenate([_f64(inp["q"]).reshape(B, T, H * dk), _f64(inp["k"]).reshape(B, T, H * dk),
                          _f64(inp["v"]).reshape(B, T, H * dv)], axis=2)
    ci = np.zeros((B, 3, raw.shape[2]))
    if inp.get("conv_in") is not None:
        ci = _f64(inp["conv_in"])
    full = np.concatenate([ci, raw], axis=1)  # row t + 3 holds token t
    return seg, full[:, t0:t0 + 3]


def prefill_context_parallel(inp: dict, segments: int) -> dict:
    """`prefill` of the whole sequence computed the context-parallel way: the T
    tokens cut into `segments` equal segments, each segment's (M, N) formed from
    S = 0 with its own 3-token raw history, the entering states by
    `compose_segments` from S0, then every segment run from its entering state.
    Returns o [B*H, T, dv] and S_T [B*H, dk, dv] like `prefill`."""
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[3]
    if T % segments:
        raise ValueError("T must be a multiple of the segment count")
    L = T // segments
    n = B * H
    Ms, Ns, hists = np.zeros((segments, n, dk, dk)), np.zeros((segments, n, dk, dv)), []
    for r in range(segments):
        seg, ci = _segment_inputs(inp, r * L, (r + 1) * L)
        _, h = initial_carry(B, H, dk, dv, None, None, ci)
        hists.append(h)
        Ms[r], Ns[r] = segment_fragments(seg, hist=h)
    S0, _ = initial_carry(B, H, dk, dv, None, inp.get("S0"), None)
    S_start, S_end = compose_segments(Ms, Ns, S0)
    o = np.zeros((n, T, dv))
    for r in range(segments):
        seg, _ = _segment_inputs(inp, r * L, (r + 1) * L)
        res = prefill(seg, S=S_start[r].copy(), hist=hists[r].copy())
        o[:, r * L:(r + 1) * L] = res["o"]
    return {"o": o, "S_T": S_end, "S_start": S_start, "M": Ms, "N": Ns}
