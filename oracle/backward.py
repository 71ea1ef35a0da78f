"""fp64 gradients of the KDA prefill -- TEST INFRASTRUCTURE (imported only by the
tests; shares no code with the GPU library).

The forward is written once more, token by token, in plain PyTorch CPU ops in
float64, and differentiated by torch.autograd: the reference for the backward
pass that training at the pages' long context needs (1M-token context in
"Gemma 4 31B vs Kimi K3", component table, long-context training row).  The definition is the
one `oracle.prefill` computes ("Kimi K3, previewed", section "Kimi Delta
Attention - the workhorse"; the component tables of "Kimi K3.1 Pro vs
gpt-oss-120b" and "Gemma 4 31B vs Kimi K3", rows "Gated DeltaNet / KDA" and
"Output gate + sink"):

  x~ = SiLU(causal depthwise conv, kernel 4, of the raw q, k, v channels)
  q^ = q~ (|q~|^2 + 1e-6)^-1/2 dk^-1/2,  k^ = k~ (|k~|^2 + 1e-6)^-1/2,  v^ = v~
  S_t = (I - beta k^ k^T) Diag(e^g) S_{t-1} + beta k^ v^T,  o = RMSNorm(S_t^T q^) sigmoid(gate)

`prefill_torch` must equal `oracle.prefill` (pinned), so autograd differentiates
the same function.  Gradients are taken with respect to the exact input values
(bf16 inputs are their bf16 values), for a loss <dO, o> + <dS_T, S_T> +
<dconv_out, conv_out>: the last two terms carry a later segment's gradient
into this one when a long sequence is processed in segments.
Direct decay form only (g is the log-decay, beta in [0, 1]).
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6
RMS_EPS = 1e-5


def _torch():
    import torch
    return torch


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _head_channels(H, dk, dv, h):
    return np.concatenate([h * dk + np.arange(dk), H * dk + h * dk + np.arange(dk),
                           2 * H * dk + h * dv + np.arange(dv)])


def prefill_torch(q, k, v, conv_w, g, beta, gate, S0, conv_in, want_conv_out=False):
    """The prefill in float64 torch ops on [B,T,H,.] tensors; conv_w [Cch,4],
    S0 [B,H,dk,dv], conv_in [B,3,Cch].  Returns (o [B,T,H,dv], S_T [B,H,dk,dv]),
    and conv_out [B,3,Cch] (the last three raw rows) when want_conv_out."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[3]
    nc = 2 * dk + dv
    # raw channels per (b, h): [B, H, T, nc] with the 3-token history in front
    raw = torch.cat([q, k, v], dim=3)                             # [B,T,H,nc] (per head: q | k | v)
    hist = torch.stack([conv_in[:, :, torch.as_tensor(_head_channels(H, dk, dv, h))] for h in range(H)], dim=2)
    w = torch.stack([conv_w[torch.as_tensor(_head_channels(H, dk, dv, h))] for h in range(H)], dim=0)  # [H,nc,4]
    full = torch.cat([hist, raw], dim=1)                          # [B,T+3,H,nc]
    acc = sum(w[None, None, :, :, j] * full[:, j:j + T] for j in range(4))
    x = acc * torch.sigmoid(acc)                                  # SiLU
    qt, kt, vt = x[..., :dk], x[..., dk:2 * dk], x[..., 2 * dk:]
    qn = qt / torch.sqrt((qt * qt).sum(-1, keepdim=True) + L2_EPS) / np.sqrt(dk)
    kn = kt / torch.sqrt((kt * kt).sum(-1, keepdim=True) + L2_EPS)
    S = S0
    outs = []
    for t in range(T):
        S = torch.exp(g[:, t])[..., None] * S                      # Diag(e^g) S
        y = torch.einsum("bhij,bhi->bhj", S, kn[:, t])
        u = beta[:, t][..., None] * (vt[:, t] - y)
        S = S + kn[:, t][..., None] * u[..., None, :]
        z = torch.einsum("bhij,bhi->bhj", S, qn[:, t])
        rms = torch.sqrt((z * z).mean(-1, keepdim=True) + RMS_EPS)
        outs.append(z / rms * torch.sigmoid(gate[:, t]))
    if not want_conv_out:
        return torch.stack(outs, dim=1), S
    # last three raw rows of history + tokens, back in the packed channel order
    last = full[:, T:T + 3]                                       # [B,3,H,nc]
    cch = H * nc
    conv_out = torch.zeros((B, 3, cch), dtype=last.dtype)
    for h in range(H):
        conv_out = conv_out.index_add(2, torch.as_tensor(_head_channels(H, dk, dv, h)), last[:, :, h])
    return torch.stack(outs, dim=1), S, conv_out


def _leaves(inp, B, H, dk, dv):
    torch = _torch()
    cch = H * (2 * dk + dv)
    vals = {x: torch.tensor(_f64(inp[x]), dtype=torch.float64, requires_grad=True)
            for x in ("q", "k", "v", "g", "beta", "gate")}
    vals["conv_w"] = torch.tensor(np.asarray(inp["conv_w"], dtype=np.float64))
    S0 = inp.get("S0")
    vals["S0"] = torch.tensor(np.zeros((B, H, dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64),
                              requires_grad=True)
    ci = inp.get("conv_in")
    vals["conv_in"] = torch.tensor(np.zeros((B, 3, cch)) if ci is None else _f64(ci), requires_grad=True)
    return vals


def forward(inp: dict) -> dict:
    """o [B,T,H,dv] and S_T of `prefill_torch` on numpy inputs (for the pin against
    the C recurrence)."""
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[3]
    if inp.get("A") is not None:
        raise ValueError("the backward reference covers the direct decay form only")
    vals = _leaves(inp, B, H, dk, dv)
    o, S_T, conv_out = prefill_torch(vals["q"], vals["k"], vals["v"], vals["conv_w"], vals["g"], vals["beta"],
                                     vals["gate"], vals["S0"], vals["conv_in"], want_conv_out=True)
    return {"o": o.detach().numpy(), "S_T": S_T.detach().numpy(), "conv_out": conv_out.detach().numpy()}


def backward(inp: dict, dO, dS_T=None, dconv_out=None) -> dict:
    """Gradients of <dO, o> + <dS_T, S_T> + <dconv_out, conv_out> with respect to
    q, k, v, g, beta, gate, S0 and conv_in (all float64, shapes of the inputs);
    conv_out is the last three raw rows [B, 3, Cch]."""
    torch = _torch()
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[3]
    if inp.get("A") is not None:
        raise ValueError("the backward reference covers the direct decay form only")
    vals = _leaves(inp, B, H, dk, dv)
    o, S_T, conv_out = prefill_torch(vals["q"], vals["k"], vals["v"], vals["conv_w"], vals["g"], vals["beta"],
                                     vals["gate"], vals["S0"], vals["conv_in"], want_conv_out=True)
    outs, gouts = [o], [torch.tensor(np.asarray(dO, dtype=np.float64))]
    if dS_T is not None:
        outs.append(S_T)
        gouts.append(torch.tensor(np.asarray(dS_T, dtype=np.float64)))
    if dconv_out is not None:
        outs.append(conv_out)
        gouts.append(torch.tensor(np.asarray(dconv_out, dtype=np.float64)))
    names = ["q", "k", "v", "g", "beta", "gate", "S0", "conv_in"]
    grads = torch.autograd.grad(outs, [vals[x] for x in names], gouts, allow_unused=True)
    return {x: (np.zeros(vals[x].shape) if gr is None else gr.numpy()) for x, gr in zip(names, grads)}


def loss(inp: dict, dO, dS_T=None, dconv_out=None) -> float:
    """<dO, o> + <dS_T, S_T> + <dconv_out, conv_out> at these inputs (float64),
    for finite differences."""
    r = forward(inp)
    val = float(np.sum(np.asarray(dO, dtype=np.float64) * r["o"]))
    if dS_T is not None:
        val += float(np.sum(np.asarray(dS_T, dtype=np.float64) * r["S_T"]))
    if dconv_out is not None:
        val += float(np.sum(np.asarray(dconv_out, dtype=np.float64) * r["conv_out"]))
    return val
