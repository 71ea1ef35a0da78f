"""Seeded synthetic inputs for the KDA prefill and decode workloads.

Shared by the tests, the benchmark and the smoke check.  This module holds no
KDA arithmetic: only random draws, the workloads' input distributions and
round-to-nearest-even conversion to bf16.

Workloads (Kimi-K3-like shapes: 96 heads, 128-dim q/k/v and a 128 x 128 state
per head, as the "Kimi K3.1 Pro vs gpt-oss-120b" and "Gemma 4 31B vs Kimi K3"
component tables give for KDA):

  tiny      B1 T64 H2 d16, fp32 inputs, chunk 16
  prefill   B2 T4096 H32 d128, bf16 inputs, chunk 64
  k3width   B1 T65536 H96 d128, bf16 inputs, chunk 64, S0 ~ N(0, 0.01^2)
  long1m    B1 T1048576 H96 d128, bf16 inputs, 16 segments of 65536, S0 = 0
  decode    N256 H96 d128, one token per step, 1000 steps, S ~ N(0, 0.05^2)

Value recipe (all workloads): q, k, v ~ N(0,1); conv_w ~ U(-1/2, 1/2) per
(channel, tap); g = -softplus(z), z ~ N(-3, 1) per channel; beta = sigmoid(N(0,1))
per (token, head); gate ~ N(0,1).  The second parameter of N(., .) is the
standard deviation.

K3-logit inputs (`with_k3_logits`, for the KDA_DECAY_K3 form): the same
tensors, except that g holds decay logits z ~ N(z_mean, 1) per channel, beta
holds beta logits ~ N(0, 1) per (token, head) (so beta has the distribution
above), and A ~ N(0, 0.1) fp32 per (head, key channel).  The default
z_mean = -4.7 gives the log-decay -5 sigmoid(e^A z) the same mean as the
recipe above (-0.075 per token; 0.7% of values below -0.5 against 0.5%).
With z_mean = 6 nearly every log-decay sits at K3's bound of -5 per token.
`fast_channels` = n redraws the logits of n seeded key channels per head from
N(6, 1) (the rest as above): a few fast-forgetting channels put every chunk of
every head past fp16's in-tile decay range.  Draws are fp64 (numpy backend) or fp32 (torch backend,
used for the large workloads on the device), then rounded once to the
workload's dtype.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 0x4B444100


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str                 # "f32" or "bf16"
    s0_sigma: float = 0.0      # initial state N(0, s0_sigma^2); 0 -> zeros
    segments: int = 1          # prefill processed as this many equal segments
    steps: int = 0             # decode steps (decode workload only)
    conv_hist: str = "zero"    # initial raw conv history: "zero" or "normal"
    seed: int = SEED_BASE

    @property
    def cch(self) -> int:
        return self.H * (2 * self.dk + self.dv)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 2, 16, 16, 16, "f32", seed=SEED_BASE + 0),
    "prefill": Workload("prefill", 2, 4096, 32, 128, 128, 64, "bf16", seed=SEED_BASE + 1),
    "k3width": Workload("k3width", 1, 65536, 96, 128, 128, 64, "bf16", s0_sigma=0.01,
                        seed=SEED_BASE + 2),
    "long1m": Workload("long1m", 1, 1048576, 96, 128, 128, 64, "bf16", segments=16,
                       seed=SEED_BASE + 3),
    "decode": Workload("decode", 256, 1, 96, 128, 128, 1, "bf16", s0_sigma=0.05, steps=1000,
                       conv_hist="normal", seed=SEED_BASE + 4),
}


# ----------------------------------------------------------------------------
# bf16 helpers (bits held in uint16 arrays)
# ----------------------------------------------------------------------------

def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (round to nearest, ties to even); return the bits.

    bf16 keeps 8 significant bits.  With x = m * 2**e (0.5 <= |m| < 1), m * 256 is
    exact in fp64, np.rint rounds it half-to-even, and the rounded value is exact
    in fp32, whose upper 16 bits are then the bf16 encoding.  Values must lie in
    the normal bf16 range (or be zero).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(m * 256.0), e - 8)
    f = r.astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bf16 bits."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of an input array stored as f32 or as bf16 bits."""
    return bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f64(x64) if dtype == "bf16" else x64.astype(np.float32)


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


# ----------------------------------------------------------------------------
# numpy backend (host, fp64 draws): small workloads and oracle-only cases
# ----------------------------------------------------------------------------

def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def prefill_inputs_np(w: Workload, T: int | None = None, seed: int | None = None) -> dict:
    """Prefill inputs as numpy arrays (f32, or uint16 bf16 bits for bf16 workloads).

    Keys: q k v g gate [B,T,H,d]; beta [B,T,H]; conv_w [Cch,4] f32;
    S0 [B,H,dk,dv] f32 or None; conv_in [B,3,Cch] (dtype of the inputs) or None.
    """
    T = w.T if T is None else T
    seed = w.seed if seed is None else seed
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    rq, rk, rv, rw, rz, rb, rg, rs, rh = _streams(seed, 9)
    d = w.dtype
    out = {
        "q": _round(rq.standard_normal((B, T, H, dk)), d),
        "k": _round(rk.standard_normal((B, T, H, dk)), d),
        "v": _round(rv.standard_normal((B, T, H, dv)), d),
        "conv_w": rw.uniform(-0.5, 0.5, (w.cch, 4)).astype(np.float32),
        "g": _round(-_softplus(rz.normal(-3.0, 1.0, (B, T, H, dk))), d),
        "beta": _round(1.0 / (1.0 + np.exp(-rb.standard_normal((B, T, H)))), d),
        "gate": _round(rg.standard_normal((B, T, H, dv)), d),
        "S0": None,
        "conv_in": None,
    }
    if w.s0_sigma > 0:
        out["S0"] = (rs.standard_normal((B, H, dk, dv)) * w.s0_sigma).astype(np.float32)
    if w.conv_hist == "normal":
        out["conv_in"] = _round(rh.standard_normal((B, 3, w.cch)), d)
    return out


def _fast_channel_sets(seed: int, H: int, dk: int, n: int) -> np.ndarray:
    """n distinct key channels per head [H, n], seeded (shared by both backends)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed + 0x2000))
    return np.stack([rng.choice(dk, n, replace=False) for _ in range(H)])


def with_k3_logits(inp: dict, w: Workload, seed: int | None = None, z_mean: float = -4.7,
                   fast_channels: int = 0) -> dict:
    """Copy of prefill or decode inputs whose g and beta are K3's logits, plus A [H, dk]."""
    seed0 = w.seed if seed is None else seed
    seed = seed0 + 0x1000
    rz, rb, ra, rf = _streams(seed, 4)
    out = dict(inp)
    z = rz.normal(z_mean, 1.0, inp["g"].shape)
    if fast_channels:
        chans = _fast_channel_sets(seed0, w.H, w.dk, fast_channels)
        for h in range(w.H):
            z[..., h, chans[h]] = rf.normal(6.0, 1.0, z[..., h, chans[h]].shape)
    out["g"] = _round(z, w.dtype)
    out["beta"] = _round(rb.standard_normal(inp["beta"].shape), w.dtype)
    out["A"] = (ra.standard_normal((w.H, w.dk)) * 0.1).astype(np.float32)
    return out


def decode_inputs_np(w: Workload, steps: int, seed: int | None = None) -> dict:
    """Decode inputs for `steps` consecutive steps (numpy backend).

    Keys: q k v g gate [steps,N,H,d]; beta [steps,N,H]; conv_w [Cch,4];
    S [N,H,dk,dv] f32 initial state; conv_state [N,3,Cch] initial raw history.
    """
    seed = w.seed if seed is None else seed
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    rq, rk, rv, rw, rz, rb, rg, rs, rh = _streams(seed, 9)
    d = w.dtype
    return {
        "q": _round(rq.standard_normal((steps, N, H, dk)), d),
        "k": _round(rk.standard_normal((steps, N, H, dk)), d),
        "v": _round(rv.standard_normal((steps, N, H, dv)), d),
        "conv_w": rw.uniform(-0.5, 0.5, (w.cch, 4)).astype(np.float32),
        "g": _round(-_softplus(rz.normal(-3.0, 1.0, (steps, N, H, dk))), d),
        "beta": _round(1.0 / (1.0 + np.exp(-rb.standard_normal((steps, N, H)))), d),
        "gate": _round(rg.standard_normal((steps, N, H, dv)), d),
        "S": (rs.standard_normal((N, H, dk, dv)) * w.s0_sigma).astype(np.float32),
        "conv_state": _round(rh.standard_normal((N, 3, w.cch)), d),
    }


# ----------------------------------------------------------------------------
# torch backend (device-side fp32 draws): the large workloads
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _gen(device, seed):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _tdtype(d: str):
    torch = _torch()
    return torch.bfloat16 if d == "bf16" else torch.float32


def _normal_fill(out, gen, mean=0.0, std=1.0, rows=1 << 22):
    """Fill `out` (any dtype) with N(mean, std^2) drawn in fp32, slab by slab."""
    torch = _torch()
    flat = out.view(-1)
    n = flat.numel()
    step = rows
    for s in range(0, n, step):
        e = min(n, s + step)
        tmp = torch.empty(e - s, dtype=torch.float32, device=out.device)
        tmp.normal_(mean, std, generator=gen)
        flat[s:e].copy_(tmp)
    return out


def _transform_fill(out, gen, kind, rows=1 << 22):
    """g = -softplus(N(-3,1)) or beta = sigmoid(N(0,1)), drawn in fp32 and rounded once."""
    torch = _torch()
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, rows):
        e = min(n, s + rows)
        tmp = torch.empty(e - s, dtype=torch.float32, device=out.device)
        if kind == "g":
            tmp.normal_(-3.0, 1.0, generator=gen)
            tmp = -torch.nn.functional.softplus(tmp)
        else:
            tmp.normal_(0.0, 1.0, generator=gen)
            tmp = torch.sigmoid(tmp)
        flat[s:e].copy_(tmp)
    return out


def prefill_inputs_torch(w: Workload, device, T: int | None = None, seed: int | None = None,
                         slab: int = 1 << 24) -> dict:
    """Prefill inputs as torch tensors on `device` (draws made on that device)."""
    torch = _torch()
    T = w.T if T is None else T
    seed = w.seed if seed is None else seed
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    dt = _tdtype(w.dtype)
    out = {}
    for i, (name, shape) in enumerate([("q", (B, T, H, dk)), ("k", (B, T, H, dk)),
                                       ("v", (B, T, H, dv)), ("gate", (B, T, H, dv))]):
        out[name] = _normal_fill(torch.empty(shape, dtype=dt, device=device),
                                 _gen(device, seed * 16 + i), rows=slab)
    out["g"] = _transform_fill(torch.empty((B, T, H, dk), dtype=dt, device=device),
                               _gen(device, seed * 16 + 4), "g", rows=slab)
    out["beta"] = _transform_fill(torch.empty((B, T, H), dtype=dt, device=device),
                                  _gen(device, seed * 16 + 5), "beta", rows=slab)
    cw = torch.empty((w.cch, 4), dtype=torch.float32, device=device)
    cw.uniform_(-0.5, 0.5, generator=_gen(device, seed * 16 + 6))
    out["conv_w"] = cw
    out["S0"] = None
    if w.s0_sigma > 0:
        out["S0"] = _normal_fill(torch.empty((B, H, dk, dv), dtype=torch.float32, device=device),
                                 _gen(device, seed * 16 + 7), std=w.s0_sigma)
    out["conv_in"] = None
    if w.conv_hist == "normal":
        out["conv_in"] = _normal_fill(torch.empty((B, 3, w.cch), dtype=dt, device=device),
                                      _gen(device, seed * 16 + 8))
    return out


def with_k3_logits_torch(inp: dict, w: Workload, device, seed: int | None = None,
                         z_mean: float = -4.7, fast_channels: int = 0) -> dict:
    """Device-side twin of `with_k3_logits`: g and beta replaced by K3's logits, plus A."""
    torch = _torch()
    seed = w.seed if seed is None else seed
    out = dict(inp)
    out["g"] = _normal_fill(torch.empty_like(inp["g"]), _gen(device, seed * 16 + 9), mean=z_mean)
    if fast_channels:
        chans = _fast_channel_sets(seed, w.H, w.dk, fast_channels)
        gen = _gen(device, seed * 16 + 12)
        for h in range(w.H):
            idx = torch.as_tensor(chans[h], device=device)
            sel = out["g"][..., h, :].index_select(-1, idx)
            out["g"][..., h, :].index_copy_(-1, idx, _normal_fill(torch.empty_like(sel), gen, mean=6.0))
    out["beta"] = _normal_fill(torch.empty_like(inp["beta"]), _gen(device, seed * 16 + 10))
    out["A"] = _normal_fill(torch.empty((w.H, w.dk), dtype=torch.float32, device=device),
                            _gen(device, seed * 16 + 11), std=0.1)
    return out


def decode_inputs_torch(w: Workload, device, steps: int, seed: int | None = None) -> dict:
    """Decode inputs for `steps` steps as torch tensors on `device`."""
    torch = _torch()
    seed = w.seed if seed is None else seed
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    dt = _tdtype(w.dtype)
    out = {}
    for i, (name, shape) in enumerate([("q", (steps, N, H, dk)), ("k", (steps, N, H, dk)),
                                       ("v", (steps, N, H, dv)), ("gate", (steps, N, H, dv))]):
        out[name] = _normal_fill(torch.empty(shape, dtype=dt, device=device),
                                 _gen(device, seed * 16 + i))
    out["g"] = _transform_fill(torch.empty((steps, N, H, dk), dtype=dt, device=device),
                               _gen(device, seed * 16 + 4), "g")
    out["beta"] = _transform_fill(torch.empty((steps, N, H), dtype=dt, device=device),
                                  _gen(device, seed * 16 + 5), "beta")
    cw = torch.empty((w.cch, 4), dtype=torch.float32, device=device)
    cw.uniform_(-0.5, 0.5, generator=_gen(device, seed * 16 + 6))
    out["conv_w"] = cw
    out["S"] = _normal_fill(torch.empty((N, H, dk, dv), dtype=torch.float32, device=device),
                            _gen(device, seed * 16 + 7), std=w.s0_sigma)
    out["conv_state"] = _normal_fill(torch.empty((N, 3, w.cch), dtype=dt, device=device),
                                     _gen(device, seed * 16 + 8))
    return out


def torch_to_np(t):
    """Host numpy copy of an input tensor: f32 stays f32, bf16 becomes uint16 bits."""
    torch = _torch()
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def np_to_torch(a, dtype: str, device):
    """Device tensor from a numpy input array (f32, or uint16 bits for bf16)."""
    torch = _torch()
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)
