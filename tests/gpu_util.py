"""Helpers for the GPU parity tests (inputs, tolerance checks)."""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn

TOL_BF16 = 2e-2   # max |gpu - oracle| <= TOL x RMS(oracle), bf16 inputs
TOL_F32 = 1e-4    # same, fp32 inputs


def tol_for(dtype: str) -> float:
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_28_amd as kda
    kda.lib()  # raises if the library is missing: no silent fallback
    return torch, kda


def err_ratio(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.abs(got - ref).max()) / rms if rms > 0 else float(np.abs(got).max())


def assert_rms_close(got, ref, tol, what):
    r = err_ratio(got, ref)
    print(f"  {what}: max|err|/RMS = {r:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite values"
    assert r <= tol, f"{what}: max|err|/RMS {r:.3e} > {tol:.0e}"


def to_dev(inp: dict, dtype: str, device="cuda") -> dict:
    out = {}
    for kk, a in inp.items():
        if a is None:
            out[kk] = None
        elif kk in ("conv_w", "S0", "S", "A"):
            out[kk] = syn.np_to_torch(np.ascontiguousarray(a, dtype=np.float32), "f32", device)
        else:
            out[kk] = syn.np_to_torch(np.ascontiguousarray(a), dtype, device)
    return out


def gather_heads(t, heads, H):
    """[B,T,H,d] device tensor -> numpy [n, T, d] for the listed (b*H+h) pairs."""
    arr = t.float().cpu().numpy()
    return np.stack([arr[p // H, :, p % H] for p in heads])
