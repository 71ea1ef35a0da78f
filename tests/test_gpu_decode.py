"""Decode step on the GPU (kda_decode_step) against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from gpu_util import assert_rms_close, gather_heads, need_gpu, to_dev, tol_for
from kda_synth import Workload

pytestmark = pytest.mark.gpu


def _run_steps(oracle_mod, w: Workload, steps: int, heads=None, device_gen=False, k3=False):
    torch, kda = need_gpu()
    bh = np.arange(w.B * w.H) if heads is None else np.asarray(heads)
    if device_gen:
        # large shapes: draw on the device, copy the per-step inputs and the
        # sampled pairs' state to the host for the oracle
        dev = syn.decode_inputs_torch(w, "cuda", steps)
        inp = {x: syn.torch_to_np(dev[x]) for x in ("q", "k", "v", "g", "beta", "gate", "conv_w",
                                                      "conv_state")}
        S_host = dev["S"].view(w.B * w.H, w.dk, w.dv)[torch.as_tensor(bh, device="cuda").long()]
        S_o = np.ascontiguousarray(S_host.cpu().numpy().astype(np.float64))
        _, h_o = oracle_mod.initial_carry(w.B, w.H, w.dk, w.dv, heads, None, inp["conv_state"])
    else:
        inp = syn.decode_inputs_np(w, steps)
        if k3:  # g and beta as K3's logits, with A
            inp = syn.with_k3_logits(inp, w)
        dev = to_dev(inp, w.dtype)
        S_o, h_o = oracle_mod.initial_carry(w.B, w.H, w.dk, w.dv, heads, inp["S"], inp["conv_state"])
    S = dev["S"].clone()
    conv = dev["conv_state"].clone()
    tol = tol_for(w.dtype)
    for s in range(steps):
        step = {x: inp[x][s] for x in ("q", "k", "v", "g", "beta", "gate")}
        step["conv_w"] = inp["conv_w"]
        step["A"] = inp.get("A")
        o_ref = oracle_mod.decode_step(step, S_o, h_o, heads=heads)
        o = kda.decode_step(dev["q"][s], dev["k"][s], dev["v"][s], dev["conv_w"], dev["g"][s],
                            dev["beta"][s], dev["gate"][s], S, conv, A=dev.get("A"))
        torch.cuda.synchronize()
        o_np = o.cpu().numpy().reshape(w.B * w.H, w.dv)[bh]
        assert_rms_close(o_np, o_ref, tol, f"decode o step {s}")
    S_np = S.cpu().numpy().reshape(w.B * w.H, w.dk, w.dv)[bh]
    assert_rms_close(S_np, S_o, tol, "decode final S")
    # the history shift is data movement: bit-exact
    conv_np = syn.torch_to_np(conv)
    want = syn.bf16_bits_from_f64(h_o) if w.dtype == "bf16" else h_o.astype(np.float32)
    for i, p in enumerate(bh):
        n, h = divmod(int(p), w.H)
        ch = oracle_mod._head_channels(w.H, w.dk, w.dv, h)
        assert np.array_equal(conv_np[n][:, ch], want[i]), "conv history shift"


@pytest.mark.parametrize("d,dtype", [(16, "f32"), (64, "bf16"), (128, "bf16"), (128, "f32")])
def test_decode_small(oracle_mod, d, dtype):
    w = Workload("dec", 3, 1, 2, d, d, 1, dtype, s0_sigma=0.05, conv_hist="normal", seed=17 + d)
    _run_steps(oracle_mod, w, steps=6)


@pytest.mark.parametrize("d,dtype", [(16, "f32"), (128, "bf16")])
def test_decode_k3_logits(oracle_mod, d, dtype):
    """g and beta given as K3's logits (KDA_DECAY_K3, A per head and channel)."""
    w = Workload("dk3", 3, 1, 2, d, d, 1, dtype, s0_sigma=0.05, conv_hist="normal", seed=29 + d)
    _run_steps(oracle_mod, w, steps=6, k3=True)


def test_decode_k3_batch_sampled(oracle_mod):
    """The serving shape (256 sequences x 96 heads, d = 128), three steps, 24 sampled pairs."""
    w = syn.WORKLOADS["decode"]
    rng = np.random.default_rng(3)
    heads = np.sort(rng.choice(w.B * w.H, 24, replace=False)).astype(np.int32)
    _run_steps(oracle_mod, w, steps=3, heads=heads, device_gen=True)


def test_decode_equals_prefill_gpu(oracle_mod):
    """T decode steps on the GPU reproduce a GPU prefill of the same T tokens."""
    torch, kda = need_gpu()
    w = Workload("dp", 2, 37, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=99)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    o_p, S_p, c_p = kda.prefill(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"],
                                dev["gate"], S0=dev["S0"], conv_in=dev["conv_in"], chunk=64)
    S = dev["S0"].clone()
    conv = dev["conv_in"].clone()
    outs = []
    for t in range(w.T):
        sl = lambda x: dev[x][:, t].contiguous()
        outs.append(kda.decode_step(sl("q"), sl("k"), sl("v"), dev["conv_w"], sl("g"), sl("beta"),
                                    sl("gate"), S, conv))
    o_d = torch.stack(outs, 1)
    torch.cuda.synchronize()
    assert_rms_close(o_d.cpu().numpy(), o_p.cpu().numpy(), 1e-2, "decode vs prefill o")
    assert_rms_close(S.cpu().numpy(), S_p.cpu().numpy(), 1e-2, "decode vs prefill S")
    assert torch.equal(conv, c_p)


# -- M tokens per call (kda_decode_multi) ---------------------------------------------------

def _multi_case(N, M, H, d, dtype, seed, k3=False):
    """Inputs of M tokens for N sequences ([N, M, H, .], a prefill of T = M tokens),
    with an initial state and raw conv history."""
    w = Workload("dm", N, M, H, d, d, 1, dtype, s0_sigma=0.05, conv_hist="normal", seed=seed)
    inp = syn.prefill_inputs_np(w)
    if k3:
        inp = syn.with_k3_logits(inp, w)
    return w, inp


def _decode_multi(kda, dev, S, conv, accept=None):
    return kda.decode_multi(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"],
                            dev["gate"], S, conv, accept=accept, A=dev.get("A"))


def _expect_carry(oracle_mod, w, inp, n, a):
    """State and raw history of sequence n after its first a tokens (the oracle)."""
    one = {x: inp[x][n:n + 1, :a] for x in ("q", "k", "v", "g", "beta", "gate")}
    one["conv_w"] = inp["conv_w"]
    one["S0"] = inp["S0"][n:n + 1]
    one["conv_in"] = inp["conv_in"][n:n + 1]
    one["A"] = inp.get("A")
    S, hist = oracle_mod.initial_carry(1, w.H, w.dk, w.dv, None, one["S0"], one["conv_in"])
    if a > 0:
        oracle_mod.prefill(one, S=S, hist=hist)
    return S, hist


@pytest.mark.parametrize("d,dtype,M", [(16, "f32", 3), (128, "bf16", 1), (128, "bf16", 2), (128, "bf16", 5),
                                       (128, "bf16", 16), (64, "bf16", 8), (128, "f32", 4),
                                       (128, "f32", 12), (16, "f32", 10), (32, "bf16", 9),
                                       (64, "bf16", 13)])
def test_decode_multi_matches_oracle(oracle_mod, d, dtype, M):
    """All M tokens committed: o for every token, the state and the raw history after
    the last one, equal to the oracle's prefill of the M tokens.  M > 8 runs the
    lane-sum layout of the token loop, smaller M the row-group layout (one loop
    up to 2 tokens, split at the accept point from 3)."""
    torch, kda = need_gpu()
    w, inp = _multi_case(3, M, 2, d, dtype, seed=71 + d + M)
    dev = to_dev(inp, dtype)
    S, conv = dev["S0"].clone(), dev["conv_in"].clone()
    o = _decode_multi(kda, dev, S, conv)
    torch.cuda.synchronize()
    r = oracle_mod.prefill(inp)
    tol = tol_for(dtype)
    assert_rms_close(gather_heads(o, r["heads"], w.H), r["o"], tol, f"multi M={M} o")
    assert_rms_close(S.cpu().numpy().reshape(w.B * w.H, d, d), r["S_T"], tol, f"multi M={M} S")
    conv_np = syn.torch_to_np(conv)
    want = syn.bf16_bits_from_f64(r["conv_out"]) if dtype == "bf16" else r["conv_out"].astype(np.float32)
    for i, p in enumerate(r["heads"]):
        n, h = divmod(int(p), w.H)
        assert np.array_equal(conv_np[n][:, oracle_mod._head_channels(w.H, d, d, h)], want[i])


@pytest.mark.parametrize("k3,M", [(False, 2), (False, 3), (False, 6), (True, 6), (False, 12), (True, 15)])
def test_decode_multi_accept_counts(oracle_mod, k3, M):
    """Per-sequence accept counts 0, 1, 2, 4, M - 1 and M, and one above M (taken
    as M): o still covers all M tokens; S and the raw history are those after each
    sequence's accepted prefix (unchanged at 0)."""
    torch, kda = need_gpu()
    w, inp = _multi_case(7, M, 2, 128, "bf16", seed=83 + M, k3=k3)
    dev = to_dev(inp, "bf16")
    acc = [0, 1, 2, 4, M - 1, M, M + 3]
    S, conv = dev["S0"].clone(), dev["conv_in"].clone()
    o = _decode_multi(kda, dev, S, conv, accept=torch.tensor(acc, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    r = oracle_mod.prefill(inp)
    tol = tol_for("bf16")
    assert_rms_close(gather_heads(o, r["heads"], w.H), r["o"], tol, "accept o")
    S_np = S.cpu().numpy()
    conv_np = syn.torch_to_np(conv)
    for n, a in enumerate(acc):
        S_ref, h_ref = _expect_carry(oracle_mod, w, inp, n, min(a, M))
        assert_rms_close(S_np[n], S_ref, tol, f"accept {a}: S")
        for h in range(w.H):
            ch = oracle_mod._head_channels(w.H, 128, 128, h)
            assert np.array_equal(conv_np[n][:, ch], syn.bf16_bits_from_f64(h_ref[h])), f"accept {a}: history"


@pytest.mark.parametrize("M", [4, 11])
def test_decode_multi_equals_single_steps(oracle_mod, M):
    """M tokens in one call and M single-token steps give the same outputs and state
    (the single steps read and write the state M times)."""
    torch, kda = need_gpu()
    w, inp = _multi_case(4, M, 3, 128, "bf16", seed=85 + M)
    dev = to_dev(inp, "bf16")
    S1, c1 = dev["S0"].clone(), dev["conv_in"].clone()
    o1 = _decode_multi(kda, dev, S1, c1)
    S2, c2 = dev["S0"].clone(), dev["conv_in"].clone()
    o2 = torch.stack([kda.decode_step(dev["q"][:, t].contiguous(), dev["k"][:, t].contiguous(),
                                      dev["v"][:, t].contiguous(), dev["conv_w"], dev["g"][:, t].contiguous(),
                                      dev["beta"][:, t].contiguous(), dev["gate"][:, t].contiguous(), S2, c2)
                      for t in range(M)], dim=1)
    torch.cuda.synchronize()
    rms = o2.float().pow(2).mean().sqrt().item()
    assert (o1 - o2).abs().max().item() <= 1e-4 * rms
    assert (S1 - S2).abs().max().item() <= 1e-4 * S2.pow(2).mean().sqrt().item()
    assert torch.equal(c1, c2)


@pytest.mark.parametrize("M", [7, 14])
def test_decode_multi_bf16_output(oracle_mod, M):
    """bf16 output is the fp32 output rounded once (same kernel arithmetic)."""
    torch, kda = need_gpu()
    w, inp = _multi_case(2, M, 3, 128, "bf16", seed=90 + M)
    dev = to_dev(inp, "bf16")
    S1, c1 = dev["S0"].clone(), dev["conv_in"].clone()
    o32 = _decode_multi(kda, dev, S1, c1)
    S2, c2 = dev["S0"].clone(), dev["conv_in"].clone()
    o16 = kda.decode_multi(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"], dev["gate"],
                           S2, c2, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(S1, S2) and torch.equal(c1, c2)


def test_decode_multi_fp32_k3_accept(oracle_mod):
    """fp32 inputs (bound 1e-4 x RMS) with K3's logits and accept counts 3, 0, 16."""
    torch, kda = need_gpu()
    M = 16
    w, inp = _multi_case(3, M, 2, 32, "f32", seed=101, k3=True)
    dev = to_dev(inp, "f32")
    acc = [3, 0, M]
    S, conv = dev["S0"].clone(), dev["conv_in"].clone()
    o = _decode_multi(kda, dev, S, conv, accept=torch.tensor(acc, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    r = oracle_mod.prefill(inp)
    tol = tol_for("f32")
    assert_rms_close(gather_heads(o, r["heads"], w.H), r["o"], tol, "fp32 K3 o")
    S_np, conv_np = S.cpu().numpy(), conv.cpu().numpy()
    for n, a in enumerate(acc):
        S_ref, h_ref = _expect_carry(oracle_mod, w, inp, n, a)
        assert_rms_close(S_np[n], S_ref, tol, f"fp32 K3 accept {a}: S")
        for h in range(w.H):
            ch = oracle_mod._head_channels(w.H, 32, 32, h)
            assert np.array_equal(conv_np[n][:, ch], h_ref[h].astype(np.float32)), f"accept {a}: history"
