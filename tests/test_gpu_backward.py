"""kda_prefill_backward on the GPU against the fp64 autograd reference
(oracle/backward.py, itself pinned by finite differences).

The kernel computes in fp32 throughout, so the bound is the fp32 one of the
forward (1e-4 x RMS of each reference gradient), for f32 and bf16 inputs alike
(bf16 inputs are exact values; only the arithmetic rounds).
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from kda_synth import Workload
from gpu_util import assert_rms_close, need_gpu, to_dev

pytestmark = pytest.mark.gpu

TOL_GRAD = 1e-4
NAMES = ("q", "k", "v", "g", "beta", "gate", "S0", "conv_in")


def _run(kda, torch, inp, dtype, dO, dS):
    dev = to_dev(inp, dtype)
    go = torch.from_numpy(dO.astype(np.float32)).cuda()
    gs = None if dS is None else torch.from_numpy(dS.astype(np.float32)).cuda()
    out = kda.prefill_backward(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"], dev["gate"],
                               go, S0=dev.get("S0"), conv_in=dev.get("conv_in"), grad_S_T=gs)
    torch.cuda.synchronize()
    return {x: out[x].cpu().numpy() for x in NAMES}


CASES = [
    # B, T, H, d, dtype
    (1, 200, 2, 128, "bf16"),   # 7 stretches of 32 (ragged last)
    (2, 150, 2, 32, "f32"),
    (2, 70, 3, 16, "bf16"),
    (1, 64, 2, 64, "f32"),      # a whole number of stretches
    (2, 2, 2, 16, "f32"),       # fewer tokens than the conv history
    (1, 1100, 1, 32, "f32"),    # 35 stretches: two slabs of recompute (32 + 3), dS and the ring carried
    (1, 1100, 2, 128, "bf16"),  # the K3-width shape's kernels: 512 threads, two pipelined slabs
]


@pytest.mark.parametrize("B,T,H,d,dtype", CASES)
def test_backward_matches_autograd(B, T, H, d, dtype):
    torch, kda = need_gpu()
    ob = pytest.importorskip("oracle.backward")
    w = Workload("bwd", B, T, H, d, d, 64, dtype, s0_sigma=0.05, conv_hist="normal", seed=120 + T + d)
    inp = syn.prefill_inputs_np(w)
    rng = np.random.default_rng(T + d)
    dO = rng.standard_normal((B, T, H, d))
    dS = rng.standard_normal((B, H, d, d))
    print(f"  case B{B} T{T} H{H} d{d} {dtype}", flush=True)
    got = _run(kda, torch, inp, dtype, dO, dS)
    ref = ob.backward(inp, dO, dS)
    for x in NAMES:
        assert_rms_close(got[x], ref[x], TOL_GRAD, f"d{x}")


def test_backward_without_state_loss():
    """grad_S_T = NULL: the loss is <dO, o> only (S0 = NULL, conv_in = NULL too)."""
    torch, kda = need_gpu()
    ob = pytest.importorskip("oracle.backward")
    w = Workload("bwd0", 1, 90, 2, 32, 32, 64, "bf16", s0_sigma=0.0, conv_hist="zero", seed=131)
    inp = syn.prefill_inputs_np(w)
    inp["S0"] = None
    inp["conv_in"] = None
    dO = np.random.default_rng(7).standard_normal((1, 90, 2, 32))
    got = _run(kda, torch, inp, "bf16", dO, None)
    ref = ob.backward(inp, dO, None)
    for x in NAMES:
        assert_rms_close(got[x], ref[x], TOL_GRAD, f"d{x} (no state loss)")


def test_backward_empty_sequence():
    """T = 0: the state gradient passes through, the history gradient is zero."""
    torch, kda = need_gpu()
    B, H, d = 2, 2, 32
    dev = {x: torch.zeros((B, 0, H, d), dtype=torch.bfloat16, device="cuda") for x in ("q", "k", "v", "g", "gate")}
    beta = torch.zeros((B, 0, H), dtype=torch.bfloat16, device="cuda")
    conv_w = torch.zeros((3 * H * d, 4), dtype=torch.float32, device="cuda")
    go = torch.zeros((B, 0, H, d), dtype=torch.float32, device="cuda")
    gs = torch.randn((B, H, d, d), device="cuda")
    out = kda.prefill_backward(dev["q"], dev["k"], dev["v"], conv_w, dev["g"], beta, dev["gate"], go, grad_S_T=gs)
    torch.cuda.synchronize()
    assert torch.equal(out["S0"], gs)
    assert torch.count_nonzero(out["conv_in"]).item() == 0


def _carry_to_input(a, dtype):
    """Raw rows carried from the reference forward (exact input values) in the
    input encoding: uint16 bits for bf16, float32 otherwise."""
    a = np.asarray(a, dtype=np.float64)
    if dtype == "bf16":
        bits = a.astype(np.float32).view(np.uint32)
        assert np.all(bits & 0xFFFF == 0), "carried rows are not bf16 values"
        return (bits >> 16).astype(np.uint16)
    return a.astype(np.float32)


@pytest.mark.parametrize("B,T,H,d,dtype", [(1, 100, 2, 32, "bf16"), (2, 2, 2, 16, "f32"), (1, 3, 2, 16, "bf16")])
def test_backward_with_conv_out_loss(B, T, H, d, dtype):
    """A loss on conv_out (the last three raw rows) as well as on o and S_T;
    T = 2 also sends one row of that gradient into the history."""
    torch, kda = need_gpu()
    ob = pytest.importorskip("oracle.backward")
    w = Workload("bwdc", B, T, H, d, d, 64, dtype, s0_sigma=0.05, conv_hist="normal", seed=140 + T)
    inp = syn.prefill_inputs_np(w)
    rng = np.random.default_rng(40 + T)
    dO = rng.standard_normal((B, T, H, d))
    dS = rng.standard_normal((B, H, d, d))
    dC = rng.standard_normal((B, 3, 3 * H * d))
    print(f"  case B{B} T{T} H{H} d{d} {dtype} with grad_conv_out", flush=True)
    dev = to_dev(inp, dtype)
    out = kda.prefill_backward(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"], dev["gate"],
                               torch.from_numpy(dO.astype(np.float32)).cuda(), S0=dev["S0"],
                               conv_in=dev["conv_in"], grad_S_T=torch.from_numpy(dS.astype(np.float32)).cuda(),
                               grad_conv_out=torch.from_numpy(dC.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    ref = ob.backward(inp, dO, dS, dC)
    for x in NAMES:
        assert_rms_close(out[x].cpu().numpy(), ref[x], TOL_GRAD, f"d{x}")


def test_segment_chain_equals_whole_sequence():
    """A sequence differentiated as three carried segments, the last first: each
    segment's grad_S0 and grad_conv_in are the grad_S_T and grad_conv_out of
    the one before it.  The concatenated gradients match the reference's
    whole-sequence gradients (the carries S0 and conv_in of each segment come
    from the reference forward of the segments before it)."""
    torch, kda = need_gpu()
    ob = pytest.importorskip("oracle.backward")
    B, T, H, d, dtype = 1, 300, 2, 64, "bf16"
    w = Workload("bwds", B, T, H, d, d, 64, dtype, s0_sigma=0.05, conv_hist="normal", seed=151)
    inp = syn.prefill_inputs_np(w)
    rng = np.random.default_rng(52)
    dO = rng.standard_normal((B, T, H, d))
    dS = rng.standard_normal((B, H, d, d))
    whole = ob.backward(inp, dO, dS)
    cuts = [0, 70, 129, T]  # segments of 70, 59 and 171 tokens
    seq = ("q", "k", "v", "g", "beta", "gate")
    segs, S0, ci = [], inp["S0"], inp["conv_in"]
    for a, b in zip(cuts[:-1], cuts[1:]):
        seg = {x: inp[x][:, a:b] for x in seq}
        seg.update(conv_w=inp["conv_w"], S0=S0, conv_in=ci)
        segs.append(seg)
        f = ob.forward(seg)
        S0, ci = f["S_T"], _carry_to_input(f["conv_out"], dtype)
    gS = torch.from_numpy(dS.astype(np.float32)).cuda()
    gC = None
    got = [None] * len(segs)
    for i in range(len(segs) - 1, -1, -1):
        a, b = cuts[i], cuts[i + 1]
        print(f"  segment {i}: tokens {a}..{b}", flush=True)
        dev = to_dev(segs[i], dtype)
        out = kda.prefill_backward(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"], dev["gate"],
                                   torch.from_numpy(dO[:, a:b].astype(np.float32)).cuda(), S0=dev["S0"],
                                   conv_in=dev["conv_in"], grad_S_T=gS, grad_conv_out=gC)
        torch.cuda.synchronize()
        got[i] = {x: out[x].cpu().numpy() for x in NAMES}
        gS, gC = out["S0"], out["conv_in"]
    for x in seq:
        assert_rms_close(np.concatenate([g[x] for g in got], axis=1), whole[x], TOL_GRAD, f"d{x} (3 segments)")
    for x in ("S0", "conv_in"):
        assert_rms_close(got[0][x], whole[x], TOL_GRAD, f"d{x} (3 segments)")


def test_unpipelined_fallback_equals_pipelined():
    """232 heads leave too few compute units to split (the slabs then run one
    after the other on the caller's stream); heads are independent, so batch 0
    of that call equals, bit for bit, a 29-head call on batch 0's inputs, which
    takes the pipelined path (two slabs: 1100 tokens)."""
    torch, kda = need_gpu()
    B, T, H, d = 8, 1100, 29, 16
    # the library pipelines a call when its reverse width (heads rounded up to
    # 8) leaves at least 32 compute units: 232 + 32 > CUs >= 32 + 32 makes the
    # 232-head call run unpipelined and the 29-head call pipelined
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    assert 64 <= ncu < 264, f"{ncu} compute units: this test's two calls would take the same path"
    w = Workload("bwdp", B, T, H, d, d, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=171)
    inp = syn.prefill_inputs_np(w)
    rng = np.random.default_rng(71)
    dO = rng.standard_normal((B, T, H, d)).astype(np.float32)
    dS = rng.standard_normal((B, H, d, d)).astype(np.float32)
    dC = rng.standard_normal((B, 3, 3 * H * d)).astype(np.float32)

    def run(sl):
        part = {x: (a if x == "conv_w" else a[sl]) for x, a in inp.items() if a is not None}
        dev = to_dev(part, "bf16")
        out = kda.prefill_backward(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"], dev["gate"],
                                   torch.from_numpy(np.ascontiguousarray(dO[sl])).cuda(), S0=dev["S0"],
                                   conv_in=dev["conv_in"], grad_S_T=torch.from_numpy(np.ascontiguousarray(dS[sl])).cuda(),
                                   grad_conv_out=torch.from_numpy(np.ascontiguousarray(dC[sl])).cuda())
        torch.cuda.synchronize()
        return {x: out[x].cpu().numpy() for x in NAMES}

    print(f"  B{B} T{T} H{H} d{d}: all heads, then batch 0 alone", flush=True)
    whole = run(slice(0, B))
    first = run(slice(0, 1))
    for x in NAMES:
        assert np.array_equal(whole[x][:1], first[x]), x
