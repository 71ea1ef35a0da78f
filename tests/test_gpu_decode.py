"""Decode step on the GPU (kda_decode_step) against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from gpu_util import assert_rms_close, need_gpu, to_dev, tol_for
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
