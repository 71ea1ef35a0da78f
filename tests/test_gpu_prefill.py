"""Prefill on the GPU (kda_prefill, kda_prep) against the fp64 oracle.

Sizes with a two-kernel path (bf16 inputs, chunk 64, dk = dv = 128) run both
paths: "split" passes the workspace kda_prefill_workspace_bytes asks for,
"fused" passes none (the single-kernel path)."""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from gpu_util import assert_rms_close, gather_heads, need_gpu, to_dev, tol_for
from kda_synth import Workload

pytestmark = pytest.mark.gpu

PATHS = {"split": "auto", "fused": None}
path = pytest.mark.parametrize("path", list(PATHS))


def _gpu_prefill(kda, dev, chunk, **kw):
    return kda.prefill(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"],
                       dev["gate"], S0=dev.get("S0"), conv_in=dev.get("conv_in"), chunk=chunk,
                       A=dev.get("A"), **kw)


def _check_vs_oracle(oracle_mod, w: Workload, inp, o, S_T, conv_out, heads=None, what="", tol=None):
    torch, _ = need_gpu()
    torch.cuda.synchronize()
    r = oracle_mod.prefill(inp, heads=heads)
    bh = r["heads"]
    tol = tol_for(w.dtype) if tol is None else tol
    assert_rms_close(gather_heads(o, bh, w.H), r["o"], tol, f"{what} o")
    S_np = S_T.cpu().numpy().reshape(w.B * w.H, w.dk, w.dv)[bh]
    assert_rms_close(S_np, r["S_T"], tol, f"{what} S_T")
    conv_np = syn.torch_to_np(conv_out)
    want = syn.bf16_bits_from_f64(r["conv_out"]) if w.dtype == "bf16" else r["conv_out"].astype(np.float32)
    for i, p in enumerate(bh):
        b, h = divmod(int(p), w.H)
        ch = oracle_mod._head_channels(w.H, w.dk, w.dv, h)
        assert np.array_equal(conv_np[b][:, ch], want[i]), f"{what} conv_out"
    return r


# -- stage 1 on its own -------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,chunk,T", [("f32", 16, 16, 64), ("bf16", 128, 64, 130),
                                             ("bf16", 64, 32, 45)])
def test_prep_stage(oracle_mod, dtype, d, chunk, T):
    torch, kda = need_gpu()
    w = Workload("p", 2, T, 3, d, d, chunk, dtype, conv_hist="normal", seed=5 + d)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, dtype)
    qn, kn, vn, G = kda.prep(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"],
                             conv_in=dev["conv_in"], chunk=chunk)
    torch.cuda.synchronize()
    r = oracle_mod.prefill(inp, want_prep=True)
    prep = r["prep"]
    tol = 1e-5  # fp32 arithmetic (1-ulp hardware exp, rcp, rsqrt) on exact inputs
    assert_rms_close(gather_heads(qn, r["heads"], w.H), prep[:, :, :d], tol, "q^")
    assert_rms_close(gather_heads(kn, r["heads"], w.H), prep[:, :, d:2 * d], tol, "k^")
    assert_rms_close(gather_heads(vn, r["heads"], w.H), prep[:, :, 2 * d:], tol, "v^")
    # G: inclusive cumsum of g restarting at every chunk boundary
    g = syn.to_f64(inp["g"], dtype)
    Gr = np.zeros_like(g)
    for c0 in range(0, T, chunk):
        Gr[:, c0:c0 + chunk] = np.cumsum(g[:, c0:c0 + chunk], axis=1)
    np.testing.assert_allclose(G.cpu().numpy(), Gr, rtol=1e-5, atol=1e-5)


# -- the fused prefill ----------------------------------------------------------------------

def test_tiny_fp32(oracle_mod):
    """Tiny workload: B1 T64 H2 d16, fp32, chunk 16, tolerance 1e-4 x RMS."""
    torch, kda = need_gpu()
    w = syn.WORKLOADS["tiny"]
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, w.dtype)
    o, S_T, c = _gpu_prefill(kda, dev, w.chunk)
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what="tiny")


@path
@pytest.mark.parametrize("T", [1, 3, 15, 17, 63, 64, 65, 130])
def test_ragged_lengths_bf16_d128(oracle_mod, T, path):
    torch, kda = need_gpu()
    w = Workload("r", 1, T, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=40 + T)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, w.dtype)
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} T={T}")


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 32, 64), ("bf16", 64, 32), ("bf16", 128, 16),
                                           ("bf16", 128, 32), ("f32", 64, 64), ("f32", 128, 32),
                                           ("f32", 32, 16)])
def test_dims_chunks_dtypes(oracle_mod, dtype, d, chunk):
    torch, kda = need_gpu()
    w = Workload("dc", 2, 150, 2, d, d, chunk, dtype, s0_sigma=0.05, conv_hist="normal", seed=d + chunk)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, dtype)
    o, S_T, c = _gpu_prefill(kda, dev, chunk)
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{dtype} d={d} C={chunk}")


@path
def test_split_in_place_carry(oracle_mod, path):
    """Two calls with S and the conv history carried in place (S_T aliases S0,
    conv_out aliases conv_in) match the oracle over the whole sequence."""
    torch, kda = need_gpu()
    w = Workload("s", 2, 200, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=8)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    S = dev["S0"].clone()
    conv = dev["conv_in"].clone()
    outs = []
    for t0, t1 in [(0, 77), (77, 200)]:
        part = {x: dev[x][:, t0:t1].contiguous() for x in ("q", "k", "v", "g", "beta", "gate")}
        part["conv_w"] = dev["conv_w"]
        o, _, _ = kda.prefill(part["q"], part["k"], part["v"], part["conv_w"], part["g"],
                              part["beta"], part["gate"], S0=S, conv_in=conv, chunk=64, S_T=S,
                              conv_out=conv, workspace=PATHS[path])
        outs.append(o)
    o = torch.cat(outs, 1)
    _check_vs_oracle(oracle_mod, w, inp, o, S, conv, what=f"{path} carried")


@pytest.mark.parametrize("per_slab", [1, 3])
def test_slabs_of_a_small_workspace(oracle_mod, per_slab):
    """A workspace smaller than the preferred size runs the chunks in several
    launches with the state carried in the workspace: 5 chunks (T = 300) with
    room for 1 or 3 chunks per launch."""
    torch, kda = need_gpu()
    w = Workload("sl", 2, 300, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=9)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    per_chunk = w.B * w.H * 64 * 1024
    nbytes = per_slab * per_chunk + w.B * w.H * w.dk * w.dv * 4
    assert nbytes >= kda.workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, minimum=True)
    assert nbytes < kda.workspace_bytes(w.B, w.T, w.H, w.dk, w.dv)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=ws)
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{per_slab} chunk(s) per launch")


@pytest.mark.parametrize("per_buf", [None, 10])
def test_pipelined_slabs(oracle_mod, per_buf):
    """70 chunks (T = 4480) exceed one slab of 64 chunks: the preferred
    workspace runs two slabs of 35 on streams restricted to disjoint compute
    units, each in a region of its own, and one recurrence launch that waits on
    a flag per slab; a workspace with room for three buffers of 10 chunks runs
    7 slabs, a recurrence launch each (the state carried between them), so
    every buffer is reused."""
    torch, kda = need_gpu()
    before = kda.wait_timeouts()
    w = Workload("pp", 1, 70 * 64, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=17)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    per_chunk = w.B * w.H * 64 * 1024
    carry = w.B * w.H * w.dk * w.dv * 4
    assert kda.workspace_bytes(w.B, w.T, w.H, w.dk, w.dv) == 2 * 35 * per_chunk + carry
    ws = "auto" if per_buf is None else torch.empty(3 * per_buf * per_chunk + carry, dtype=torch.uint8,
                                                     device="cuda")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=ws)
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"pipelined slabs, buffers of {per_buf or 35} chunks")
    assert kda.wait_timeouts() == before


def test_pipelined_half_first_slab(oracle_mod):
    """131 chunks (T = 8393, ragged): slabs of 32, 50 and 49 chunks (the first
    one half-size), three regions of 64 chunks at the preferred workspace, one
    recurrence launch that finds each slab's first chunk from the slab plan."""
    torch, kda = need_gpu()
    before = kda.wait_timeouts()
    w = Workload("pf", 1, 131 * 64 - 55, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=29)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    per_chunk = w.B * w.H * 64 * 1024
    assert kda.workspace_bytes(w.B, w.T, w.H, w.dk, w.dv) == 3 * 64 * per_chunk + w.B * w.H * w.dk * w.dv * 4
    o, S_T, c = _gpu_prefill(kda, dev, 64)
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what="half-size first slab")
    assert kda.wait_timeouts() == before


@pytest.mark.parametrize("wait_us,withhold", [(200, 0), (200, 1), (200, 2), (1, -1)])
def test_pipelined_stop_and_resume(oracle_mod, wait_us, withhold):
    """The one-launch recurrence's stop-and-resume path, forced from the host
    (kda_debug_pipeline).  With slab `withhold`'s flag never set, every
    workgroup's bounded wait for it expires (after 200 us): the workgroup stops
    before that slab, leaves its state in S_T, and the call's second launch
    finishes from there.  With a 1 us bound and every flag set, the waits
    expire wherever the intra-chunk kernel is not yet ahead.  131 chunks
    (slabs of 32, 50 and 49, ragged), S and the conv history carried in place
    (S_T aliases S0, conv_out aliases conv_in), against the oracle."""
    torch, kda = need_gpu()
    w = Workload("sr", 1, 131 * 64 - 55, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=31)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    S = dev["S0"].clone()
    conv = dev["conv_in"].clone()
    before = kda.wait_timeouts()
    kda.debug_pipeline(wait_us, withhold)
    try:
        o, _, _ = kda.prefill(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"], dev["gate"],
                              S0=S, conv_in=conv, chunk=64, S_T=S, conv_out=conv)
        torch.cuda.synchronize()
    finally:
        kda.debug_pipeline()
    stops = kda.wait_timeouts() - before
    if withhold >= 0:  # every workgroup waited for that slab in vain, once
        assert stops == w.B * w.H, stops
    _check_vs_oracle(oracle_mod, w, inp, o, S, conv, what=f"bound {wait_us} us, slab {withhold} withheld")


@pytest.mark.parametrize("B,H,T", [(2, 3, 70 * 64 + 17), (1, 130, 66 * 64 + 5)])
def test_slab_plans_at_other_shapes(oracle_mod, B, H, T):
    """Ragged last chunk, at the preferred workspace.  B*H = 6 pipelines two
    slabs on 8 compute units (6 rounded up to a multiple of 8); B*H = 130 is
    more than half the compute units, so its 67 chunks run in one slab on
    the caller's stream.  Checked on a few pairs."""
    torch, kda = need_gpu()
    w = Workload("ps", B, T, H, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=23)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    nch = -(-T // 64)
    per_chunk = B * H * 64 * 1024
    carry = B * H * 128 * 128 * 4
    if 2 * B * H <= 256:
        want = 2 * (-(-nch // 2)) * per_chunk + carry
    else:
        want = nch * per_chunk
    assert kda.workspace_bytes(B, T, H, 128, 128) == want
    o, S_T, c = _gpu_prefill(kda, dev, 64)
    pairs = sorted({0, B * H // 2, B * H - 1})
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, heads=pairs, what=f"B{B} H{H} T{T}")


@pytest.mark.skip(reason="a capture that forked onto the library's CU-masked streams crashed (host "
                         "segfault in the runtime's end of capture); the library now runs the slabs on the "
                         "capturing stream alone, and capture stays off the GPU until that crash is understood")
def test_prefill_in_captured_graph():
    """kda_prefill captured in a HIP graph (torch.cuda.graph) at the preferred
    workspace, 70 chunks (two pipelined slabs when not capturing).  Under
    capture the slabs run one after the other on the capturing stream.  Three
    replays, with eager work and a synchronisation between them, each equal
    the eager call (one recurrence launch) bit for bit."""
    torch, kda = need_gpu()
    w = Workload("gr", 1, 70 * 64, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=51)
    dev = to_dev(syn.prefill_inputs_np(w), "bf16")
    args = (dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"], dev["gate"])
    ws = torch.empty(kda.workspace_bytes(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device="cuda")
    # the eager call also creates the library's streams before the capture
    o_ref, S_ref, c_ref = kda.prefill(*args, S0=dev["S0"], conv_in=dev["conv_in"], workspace=ws)
    torch.cuda.synchronize()
    o, S, conv = torch.empty_like(o_ref), torch.empty_like(S_ref), torch.empty_like(c_ref)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        kda.prefill(*args, S0=dev["S0"], conv_in=dev["conv_in"], o=o, S_T=S, conv_out=conv, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        o.zero_()
        S.zero_()
        conv.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: o"
        assert torch.equal(S, S_ref), f"replay {rep}: S_T"
        assert torch.equal(conv, c_ref), f"replay {rep}: conv_out"


def test_paths_agree(oracle_mod):
    """Both paths on the same inputs agree to well within the tolerance."""
    torch, kda = need_gpu()
    w = Workload("pa", 2, 256, 3, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=21)
    dev = to_dev(syn.prefill_inputs_np(w), "bf16")
    a = _gpu_prefill(kda, dev, 64, workspace="auto")
    b = _gpu_prefill(kda, dev, 64, workspace=None)
    torch.cuda.synchronize()
    for x, y, what in zip(a, b, ("o", "S_T", "conv_out")):
        x, y = x.float().cpu().numpy(), y.float().cpu().numpy()
        assert_rms_close(x, y, 2e-2, f"split vs fused {what}")


@pytest.mark.parametrize("d", [64, 128])
def test_empty_sequence_copies_carry(d):
    torch, kda = need_gpu()
    w = Workload("e", 2, 0, 2, d, d, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=2)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64)
    torch.cuda.synchronize()
    assert o.shape[1] == 0
    assert torch.equal(S_T, dev["S0"]) and torch.equal(c, dev["conv_in"])


@path
def test_no_initial_state_is_zero_state(oracle_mod, path):
    torch, kda = need_gpu()
    w = Workload("z", 1, 100, 3, 128, 128, 64, "bf16", seed=12)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} S0=None")


@path
def test_strong_decay_wide_chunks(oracle_mod, path):
    """g = -2 per token: a 16-token tile decays by e^32, beyond fp16's range, so
    those chunks are "wide": the in-tile (diagonal) blocks of A and P run on
    fp32 operands and U enters the state and output products as an fp16 pair.
    The middle chunk decays slowly (-0.05 per token) and takes the plain path;
    the bound is the workloads' 2e-2 x RMS."""
    torch, kda = need_gpu()
    w = Workload("sd", 1, 160, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=31)
    inp = syn.prefill_inputs_np(w)
    gbits = syn.bf16_bits_from_f64(np.full(inp["g"].shape, -2.0))
    gbits[:, 64:128] = syn.bf16_bits_from_f64(np.full(inp["g"][:, 64:128].shape, -0.05))
    inp["g"] = gbits
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} strong decay")


@path
def test_beta_zero_state_only_decays(oracle_mod, path):
    """beta = 0: no token writes the state, which only decays from S0 (the
    outputs read the decayed S0).  Also checks S_T = Diag(e^{sum g}) S0 row by
    row, which holds exactly in this case."""
    torch, kda = need_gpu()
    w = Workload("b0", 1, 130, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=41)
    inp = syn.prefill_inputs_np(w)
    inp["beta"] = syn.bf16_bits_from_f64(np.zeros(inp["beta"].shape))
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} beta=0")
    g = syn.bf16_bits_to_f64(inp["g"]).reshape(w.B, w.T, w.H, w.dk).sum(axis=1)  # [B, H, dk]
    want = inp["S0"].astype(np.float64).reshape(w.B, w.H, w.dk, w.dv) * np.exp(g)[..., None]
    got = S_T.cpu().numpy().astype(np.float64).reshape(w.B, w.H, w.dk, w.dv)
    assert_rms_close(got, want, 1e-5, f"{path} beta=0 S_T = decayed S0")


@path
def test_no_decay(oracle_mod, path):
    """g = 0: nothing is forgotten, every decay factor is exactly 1."""
    torch, kda = need_gpu()
    w = Workload("g0", 1, 130, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=43)
    inp = syn.prefill_inputs_np(w)
    inp["g"] = syn.bf16_bits_from_f64(np.zeros(inp["g"].shape))
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} g=0")


# -- K3's gate parameterisation (KDA_DECAY_K3) ----------------------------------------------

@path
@pytest.mark.parametrize("T", [17, 130])
def test_k3_logits(oracle_mod, path, T):
    """g and beta given as K3's logits: g = -5 sigmoid(e^A z), beta = sigmoid(b),
    computed in the kernels where they load g and beta."""
    torch, kda = need_gpu()
    w = Workload("k3", 2, T, 3, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=47)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w)
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} K3 logits")


@path
def test_k3_logits_at_the_bound(oracle_mod, path):
    """Decay logits around +6: nearly every channel decays by K3's bound of -5 per
    token, so a 16-token tile spans e^-80 (inside fp32's range, as the pages
    say for bf16) and every chunk is wide.  The state forgets nearly everything
    each token, so o and S_T are dominated by the last tokens' U, whose single
    fp16 rounding alone would reach the bound; the wide path splits it.  Held
    to the workloads' 2e-2 x RMS on the largest error, and the RMS error is
    printed."""
    torch, kda = need_gpu()
    w = Workload("k3b", 1, 160, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=53)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w, z_mean=6.0)
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S_T).all()
    r = _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} K3 bound")
    for got, want, what in ((gather_heads(o, r["heads"], w.H), r["o"], "o"),
                            (S_T.cpu().numpy().reshape(w.B * w.H, w.dk, w.dv), r["S_T"], "S_T")):
        err = np.asarray(got, dtype=np.float64) - want
        rms_err = float(np.sqrt(np.mean(err * err)) / np.sqrt(np.mean(want * want)))
        print(f"  {path} K3 bound {what}: RMS(err)/RMS = {rms_err:.3e}", flush=True)


@path
def test_k3_logits_mixed_fast_channels(oracle_mod, path):
    """K3's logits with 8 of 128 key channels per head drawn at z ~ N(6, 1):
    those channels forget at the -5 bound, so every chunk is wide while the
    other channels decay as in the workloads."""
    torch, kda = need_gpu()
    w = Workload("k3m", 2, 300, 3, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=57)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w, fast_channels=8)
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} K3 fast channels")


@pytest.mark.parametrize("dtype,d,chunk", [("f32", 16, 16), ("bf16", 64, 32)])
def test_k3_logits_other_sizes(oracle_mod, dtype, d, chunk):
    """The single-kernel path's other instantiations with K3's logits."""
    torch, kda = need_gpu()
    w = Workload("k3s", 1, 45, 2, d, d, chunk, dtype, s0_sigma=0.1, conv_hist="normal", seed=59 + d)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w)
    dev = to_dev(inp, dtype)
    o, S_T, c = _gpu_prefill(kda, dev, chunk)
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"K3 logits {dtype} d{d} C{chunk}")


def test_k3_prep_cumsum(oracle_mod):
    """kda_prep with K3's logits: G is the chunk-local cumulative sum of the
    bounded log-decay the oracle derives from the same logits."""
    torch, kda = need_gpu()
    w = Workload("k3p", 1, 100, 2, 128, 128, 64, "bf16", conv_hist="normal", seed=61)
    inp = syn.with_k3_logits(syn.prefill_inputs_np(w), w)
    dev = to_dev(inp, "bf16")
    _, _, _, G = kda.prep(dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"],
                          conv_in=dev["conv_in"], chunk=64, A=dev["A"])
    torch.cuda.synchronize()
    g, _ = oracle_mod.decay_and_beta(inp)
    want = np.concatenate([np.cumsum(g[:, c0:c0 + 64], axis=1) for c0 in range(0, w.T, 64)], axis=1)
    assert_rms_close(G.cpu().numpy(), want, 1e-5, "K3 G")


@path
def test_bf16_output(oracle_mod, path):
    torch, kda = need_gpu()
    w = Workload("bo", 1, 96, 2, 128, 128, 64, "bf16", s0_sigma=0.05, seed=13)
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    o32, _, _ = _gpu_prefill(kda, dev, 64, workspace=PATHS[path])
    o16, _, _ = _gpu_prefill(kda, dev, 64, out_dtype=torch.bfloat16, workspace=PATHS[path])
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))


@path
def test_deterministic(oracle_mod, path):
    torch, kda = need_gpu()
    w = Workload("det", 2, 300, 3, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=4)
    dev = to_dev(syn.prefill_inputs_np(w), "bf16")
    runs = [_gpu_prefill(kda, dev, 64, workspace=PATHS[path]) for _ in range(3)]
    torch.cuda.synchronize()
    for o, S, c in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(S, runs[0][1]) and torch.equal(c, runs[0][2])


@path
def test_prefill_workload_b2_t4096_h32(oracle_mod, path):
    """B2 T4096 H32 d128 bf16 chunk 64: every head against the oracle."""
    torch, kda = need_gpu()
    w = syn.WORKLOADS["prefill"]
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, w.chunk, workspace=PATHS[path])
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what=f"{path} B2 T4096 H32")


def _scale_bf16_bits(bits, factor_log2):
    """bf16 bit patterns times 2^factor_log2 (exact: only the exponent moves)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return syn.bf16_bits_from_f64(f * 2.0 ** factor_log2)


def test_values_beyond_fp16_range(oracle_mod):
    """v, S0 and the conv history times 2^15 (|v| up to about 1e5, the state
    about 1e4): V, S and the recurrence's products would leave fp16's range
    (65504).  The two-kernel path scales each math wave's columns by a power
    of two (the state and outputs come back unscaled), so the result stays
    within the workloads' 2e-2 x RMS of the oracle."""
    torch, kda = need_gpu()
    w = Workload("big", 1, 300, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=41)
    inp = syn.prefill_inputs_np(w)
    inp["v"] = _scale_bf16_bits(inp["v"], 15)
    inp["conv_in"] = _scale_bf16_bits(inp["conv_in"], 15)
    inp["S0"] = (inp["S0"] * 2.0 ** 15).astype(np.float32)
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace="auto")
    assert torch.isfinite(o).all() and torch.isfinite(S_T).all()
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what="values x 2^15")


def test_value_spike_mid_sequence(oracle_mod):
    """Ordinary values except two chunks of v times 2^16 in the middle of a
    pipelined 70-chunk sequence: the scale grows at the spike (the state is
    rescaled in place) and stays for the rest of the launch."""
    torch, kda = need_gpu()
    w = Workload("spk", 1, 70 * 64, 2, 128, 128, 64, "bf16", s0_sigma=0.05, conv_hist="normal", seed=43)
    inp = syn.prefill_inputs_np(w)
    inp["v"][:, 40 * 64:42 * 64] = _scale_bf16_bits(inp["v"][:, 40 * 64:42 * 64], 16)
    dev = to_dev(inp, "bf16")
    o, S_T, c = _gpu_prefill(kda, dev, 64, workspace="auto")
    assert torch.isfinite(o).all() and torch.isfinite(S_T).all()
    _check_vs_oracle(oracle_mod, w, inp, o, S_T, c, what="spike x 2^16")
