"""Context-parallel prefill on the GPU (kda_cp_compose, kda_prefill_cp) against
the oracle.

kda_prefill_cp computes the prefill from R segments per sequence, each run from
S = 0 and from S = I (its fragments), composed, and run again from its entering
state.  Its results are compared with the oracle's plain sequential prefill, so
the whole chain (segment histories, fragments, composition, rerun, the last
segment's state, conv_out) is checked against the definition; the composition
kernel alone is compared with the oracle's composition.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from kda_synth import Workload
from gpu_util import TOL_BF16, TOL_F32, assert_rms_close, gather_heads, need_gpu, to_dev, tol_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [16, 128])
def test_cp_compose_matches_oracle(oracle_mod, d):
    """S_start and S_T of kda_cp_compose against the oracle's fp64 composition, on
    random contractive maps (fp32 arithmetic: bound 1e-5 x RMS)."""
    torch, kda = need_gpu()
    B, R, H = 2, 5, 3
    rng = np.random.default_rng(40 + d)
    M = (rng.standard_normal((B * R, H, d, d)) * 0.9 / np.sqrt(d)).astype(np.float32)
    N = rng.standard_normal((B * R, H, d, d)).astype(np.float32)
    S0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    P = (M.astype(np.float64) + N).astype(np.float32)
    dev = {x: torch.from_numpy(a).cuda() for x, a in (("N", N), ("P", P), ("S0", S0))}
    S_start, S_T = kda.cp_compose(dev["N"], dev["P"], S0=dev["S0"], B=B)
    torch.cuda.synchronize()
    # oracle layout: [R, n = b*H + h, d, d]
    Mo = (P.astype(np.float64) - N).reshape(B, R, H, d, d).transpose(1, 0, 2, 3, 4).reshape(R, B * H, d, d)
    No = N.astype(np.float64).reshape(B, R, H, d, d).transpose(1, 0, 2, 3, 4).reshape(R, B * H, d, d)
    want_start, want_end = oracle_mod.compose_segments(Mo, No, S0.astype(np.float64).reshape(B * H, d, d))
    got_start = S_start.cpu().numpy().reshape(B, R, H, d, d).transpose(1, 0, 2, 3, 4).reshape(R, B * H, d, d)
    assert_rms_close(got_start, want_start, 1e-5, f"compose d={d} S_start")
    assert_rms_close(S_T.cpu().numpy().reshape(B * H, d, d), want_end, 1e-5, f"compose d={d} S_T")


CASES = [
    # B, T, H, d, dtype, chunk, segments, K3 logits
    (2, 1024, 3, 128, "bf16", 64, 4, False),    # two-kernel path, 4 chunks per segment
    (1, 16384, 2, 128, "bf16", 64, 2, True),    # pipelined segments of 128 chunks, K3's logits
    (1, 600, 3, 64, "bf16", 32, 5, False),      # segments of 120 tokens: ragged chunk tails
    (2, 96, 2, 16, "f32", 16, 3, False),        # single-kernel path, fp32
    (3, 48, 2, 32, "f32", 16, 16, True),        # 3 tokens per segment: halos reach the previous segment's start
]


@pytest.mark.parametrize("B,T,H,d,dtype,chunk,R,k3", CASES)
def test_prefill_cp_matches_oracle(oracle_mod, B, T, H, d, dtype, chunk, R, k3):
    """o, S_T and conv_out of the context-parallel prefill against the oracle's
    sequential prefill (S0 and conv_in given)."""
    torch, kda = need_gpu()
    w = Workload("cp", B, T, H, d, d, chunk, dtype, s0_sigma=0.05, conv_hist="normal", seed=60 + R + d)
    inp = syn.prefill_inputs_np(w)
    if k3:
        inp = syn.with_k3_logits(inp, w)
    dev = to_dev(inp, dtype)
    print(f"  case B{B} T{T} H{H} d{d} {dtype} chunk {chunk} segments {R} k3={k3}", flush=True)
    o, S_T, conv_out = kda.prefill_cp(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"],
                                      dev["gate"], R, S0=dev["S0"], conv_in=dev["conv_in"], chunk=chunk,
                                      A=dev.get("A"))
    torch.cuda.synchronize()
    r = oracle_mod.prefill(inp)
    tol = tol_for(dtype)
    assert_rms_close(gather_heads(o, r["heads"], H), r["o"], tol, f"cp R={R} o")
    assert_rms_close(S_T.cpu().numpy().reshape(B * H, d, d), r["S_T"], tol, f"cp R={R} S_T")
    conv_np = syn.torch_to_np(conv_out)
    want = syn.bf16_bits_from_f64(r["conv_out"]) if dtype == "bf16" else r["conv_out"].astype(np.float32)
    for i, p in enumerate(r["heads"]):
        b, h = divmod(int(p), H)
        assert np.array_equal(conv_np[b][:, oracle_mod._head_channels(H, d, d, h)], want[i])


def test_prefill_cp_carry_in_place(oracle_mod):
    """Two consecutive context-parallel calls carrying S and the conv history in
    place (S_T = S0, conv_out = conv_in) equal one prefill of the whole sequence."""
    torch, kda = need_gpu()
    B, T, H, d = 1, 2048, 4, 128
    w = Workload("cpc", B, T, H, d, d, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=77)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    S, conv = dev["S0"].clone(), dev["conv_in"].clone()
    o = torch.empty((B, T, H, d), dtype=torch.float32, device="cuda")
    half = T // 2
    for t0 in (0, half):
        sl = {x: dev[x][:, t0:t0 + half].contiguous() for x in ("q", "k", "v", "g", "beta", "gate")}
        kda.prefill_cp(sl["q"], sl["k"], sl["v"], dev["conv_w"], sl["g"], sl["beta"], sl["gate"], 8,
                       S0=S, conv_in=conv, o=o[:, t0:t0 + half], S_T=S, conv_out=conv)
    torch.cuda.synchronize()
    r = oracle_mod.prefill(inp)
    assert_rms_close(gather_heads(o, r["heads"], H), r["o"], TOL_BF16, "cp carry o")
    assert_rms_close(S.cpu().numpy().reshape(B * H, d, d), r["S_T"], TOL_BF16, "cp carry S_T")
    conv_np = syn.torch_to_np(conv)
    want = syn.bf16_bits_from_f64(r["conv_out"])
    for h in range(H):
        assert np.array_equal(conv_np[0][:, oracle_mod._head_channels(H, d, d, h)], want[h])


@pytest.mark.timeout(600)
def test_prefill_cp_k3width_sixteen_segments(oracle_mod):
    """The K3-width shape, B1 T65536 H96 d128, in 16 segments of 4096 tokens (the
    per-rank share of 16 ranks): sampled heads over all 65536 tokens against the
    oracle's sequential prefill."""
    torch, kda = need_gpu()
    w = syn.WORKLOADS["k3width"]
    dev = syn.prefill_inputs_torch(w, "cuda")
    o, S_T, _ = kda.prefill_cp(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"],
                               dev["gate"], 16, S0=dev["S0"], chunk=w.chunk)
    torch.cuda.synchronize()
    heads = [0, 37, 95]
    host = {x: syn.torch_to_np(dev[x][:, :, heads].contiguous()) for x in ("q", "k", "v", "g", "beta", "gate")}
    chans = np.concatenate([h * w.dk + np.arange(w.dk) for h in heads]
                           + [w.H * w.dk + h * w.dk + np.arange(w.dk) for h in heads]
                           + [2 * w.H * w.dk + h * w.dv + np.arange(w.dv) for h in heads])
    host["conv_w"] = syn.torch_to_np(dev["conv_w"])[chans]
    host["S0"] = dev["S0"][:, heads].cpu().numpy()
    r = oracle_mod.prefill(host)
    o_got = o[0][:, heads].float().cpu().numpy().transpose(1, 0, 2)
    assert_rms_close(o_got, r["o"], TOL_BF16, "k3width 16 segments o")
    assert_rms_close(S_T[0, heads].cpu().numpy(), r["S_T"], TOL_BF16, "k3width 16 segments S_T")


RANK_CASES = [
    # B, T, H, d, dtype, chunk, K3 logits
    (1, 4096 + 17, 2, 128, "bf16", 64, False),   # two-kernel path: kept chunk blocks, ragged last chunk
    (2, 700, 3, 128, "bf16", 64, True),          # two-kernel path, K3's logits
    (2, 96, 2, 32, "f32", 16, False),            # other sizes: plain prefills
]


@pytest.mark.parametrize("B,T,H,d,dtype,chunk,k3", RANK_CASES)
def test_cp_rank_share_matches_oracle(oracle_mod, B, T, H, d, dtype, chunk, k3):
    """One rank's share in two calls: kda_cp_fragments gives the segment's
    final states from S = 0 and from S = I (against the oracle run from those
    states), kda_cp_finish reruns it from an entering state with the kept
    workspace (o, S_T, conv_out against the oracle's prefill from that state).
    conv_in stands for the three raw tokens before the rank's segment."""
    torch, kda = need_gpu()
    w = Workload("rk", B, T, H, d, d, chunk, dtype, s0_sigma=0.05, conv_hist="normal", seed=90 + d + T)
    inp = syn.prefill_inputs_np(w)
    if k3:
        inp = syn.with_k3_logits(inp, w)
    dev = to_dev(inp, dtype)
    print(f"  rank share B{B} T{T} H{H} d{d} {dtype} chunk {chunk} k3={k3}", flush=True)
    args = [dev[x] for x in ("q", "k", "v", "conv_w", "g", "beta", "gate")]
    ws, N, P = kda.cp_fragments(*args, conv_in=dev["conv_in"], chunk=chunk, A=dev.get("A"))
    o, S_T, conv_out = kda.cp_finish(ws, *args, dev["S0"], conv_in=dev["conv_in"], chunk=chunk, A=dev.get("A"))
    torch.cuda.synchronize()
    tol = tol_for(dtype)
    zero = dict(inp, S0=np.zeros((B, H, d, d), dtype=np.float32))
    eye = dict(inp, S0=np.broadcast_to(np.eye(d, dtype=np.float32), (B, H, d, d)).copy())
    rN = oracle_mod.prefill(zero, want_o=False)
    rP = oracle_mod.prefill(eye, want_o=False)
    assert_rms_close(N.cpu().numpy().reshape(B * H, d, d), rN["S_T"], tol, "fragment N (from S = 0)")
    assert_rms_close(P.cpu().numpy().reshape(B * H, d, d), rP["S_T"], tol, "fragment P (from S = I)")
    r = oracle_mod.prefill(inp)
    assert_rms_close(gather_heads(o, r["heads"], H), r["o"], tol, "finish o")
    assert_rms_close(S_T.cpu().numpy().reshape(B * H, d, d), r["S_T"], tol, "finish S_T")
    conv_np = syn.torch_to_np(conv_out)
    want = syn.bf16_bits_from_f64(r["conv_out"]) if dtype == "bf16" else r["conv_out"].astype(np.float32)
    for i, p in enumerate(r["heads"]):
        b, h = divmod(int(p), H)
        assert np.array_equal(conv_np[b][:, oracle_mod._head_channels(H, d, d, h)], want[i])


def test_cp_rank_share_finish_twice(oracle_mod):
    """The kept workspace serves several finishing calls (here from two
    entering states): each equals the oracle's prefill from its state."""
    torch, kda = need_gpu()
    w = Workload("rk2", 1, 1000, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=97)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    args = [dev[x] for x in ("q", "k", "v", "conv_w", "g", "beta", "gate")]
    ws, N, P = kda.cp_fragments(*args, conv_in=dev["conv_in"])
    for s, S_in in enumerate((dev["S0"], torch.zeros_like(dev["S0"]))):
        o, S_T, _ = kda.cp_finish(ws, *args, S_in, conv_in=dev["conv_in"], want_conv=False)
        torch.cuda.synchronize()
        r = oracle_mod.prefill(dict(inp, S0=S_in.cpu().numpy()))
        assert_rms_close(gather_heads(o, r["heads"], 2), r["o"], TOL_BF16, f"finish {s} o")
        assert_rms_close(S_T.cpu().numpy().reshape(2, 128, 128), r["S_T"], TOL_BF16, f"finish {s} S_T")
