"""KDA benchmark on one MI355X.

Headline: prefill tokens/s on the K3-width workload (B1 T65536 H96 d128, bf16
inputs, fp32 state and output, chunk 64), one step = one kda_prefill over the
whole input.  Beside it: the batched decode step (256 sequences x 96 heads,
1000 consecutive steps) as HBM GB/s, the roofline of each kernel from
HIP-event timing of its launches, and the fp64 CPU oracle timed on a bounded
sample of the same prefill workload.

Prints one JSON line.  Options:
  --gpus N        only 1 is supported (the path runs on one GPU)
  --steps K       timed prefill steps (default 20)
  --warmup W      untimed prefill steps first (default 3)
  --workload      k3width (default) | prefill | long1m (16 x 65536 segments, carry in place)
  --decode-steps  decode steps timed back to back (default 1000; 0 skips decode)
  --no-cpu        skip the oracle leg
  --calibrate     also run a plain 1 GiB read + 1 GiB write kernel (for HBM counter scaling)
  --verify-tokens M tokens per sequence per kda_decode_multi call on the decode shape
                  (default 4; 0 skips): tokens/s and HBM GB/s
  --decay-form    direct (default: g and beta given) | k3 (g and beta given as K3's
                  logits, g = -5 sigmoid(e^A z) and beta = sigmoid(b) computed in the kernels)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFS = 2500.0  # dense bf16/fp16 matrix-core peak, TFLOP/s
METRIC = "KDA prefill tokens/s at H=96,d=128 (% MFMA peak); decode-step HBM GB/s"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_bytes_per_launch(B, T, H, dk, dv, in_bytes=2, out_bytes=4):
    """Compulsory HBM bytes of one prefill: q k v g gate in, beta in, o out, plus
    S0 read and S_T write and the conv history in/out per (b, h)."""
    per_token_head = in_bytes * (2 * dk + dv + dk + dv) + in_bytes + out_bytes * dv
    per_head = 4 * dk * dv * 2 + in_bytes * 3 * (2 * dk + dv) * 2
    return B * T * H * per_token_head + B * H * per_head


def prefill_flops(B, T, H, dk, dv, C=64):
    """Algorithmic FLOPs of the chunkwise form (exact triangular counts)."""
    n_full, tail = divmod(T, C)
    def chunk(c):
        tri_strict = c * (c - 1) // 2
        tri_incl = c * (c + 1) // 2
        mac = (tri_strict * dk          # A
               + tri_incl * dk          # P
               + tri_incl * dk          # W = T diag(beta) K
               + tri_incl * dv          # U~ = T diag(beta) V
               + c * dk * dv * 3        # W S, Q S, K^T U
               + tri_incl * dv)         # P U
        return 2 * mac
    return B * H * (n_full * chunk(C) + (chunk(tail) if tail else 0))


def decode_multi_bytes_per_call(N, M, H, dk, dv, in_bytes=2, out_bytes=4):
    """kda_decode_multi: the state once, M tokens of activations and outputs."""
    per = (4 * dk * dv * 2
           + M * (in_bytes * (2 * dk + dv + dk + dv) + in_bytes + out_bytes * dv)
           + 2 * 3 * (2 * dk + dv) * in_bytes)
    return N * H * per + H * (2 * dk + dv) * 4 * 4


def decode_bytes_per_step(N, H, dk, dv, in_bytes=2, out_bytes=4):
    per = (4 * dk * dv * 2                       # state read + write
           + in_bytes * (2 * dk + dv + dk + dv)  # q k v g gate
           + in_bytes                            # beta
           + out_bytes * dv                      # o
           + 2 * 3 * (2 * dk + dv) * in_bytes)   # conv history read + write
    conv_w = H * (2 * dk + dv) * 4 * 4
    return N * H * per + conv_w


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_key, src):
    """HBM traffic measured with rocprofv3 counters, if taken on this kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not d or d.get("source_sha256_16") != source_hash(src):
        return None
    return d.get("bytes_per_launch")


def timed_launches(torch, fn, n):
    """Run fn n times, one event pair per launch on the current stream; returns ms list."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(w, dev_inp, seconds_target=15.0):
    """The oracle on a bounded sample: the first n heads over the first Ts tokens."""
    import numpy as np
    import kda_synth as syn
    import oracle
    nthr = oracle.max_threads()
    nheads = min(w.H, 6 * max(1, nthr))
    Ts = min(w.T, 65536)
    dk, dv, H = w.dk, w.dv, w.H
    sl = {x: dev_inp[x][:, :Ts, :nheads].contiguous() for x in ("q", "k", "v", "g", "gate")}
    sl["beta"] = dev_inp["beta"][:, :Ts, :nheads].contiguous()
    cw = dev_inp["conv_w"]
    chans = list(range(0, nheads * dk)) + list(range(H * dk, H * dk + nheads * dk)) + \
        list(range(2 * H * dk, 2 * H * dk + nheads * dv))
    sl["conv_w"] = cw[chans].contiguous()
    host = {x: syn.torch_to_np(t) for x, t in sl.items()}
    if dev_inp.get("S0") is not None:
        host["S0"] = syn.torch_to_np(dev_inp["S0"][:, :nheads].contiguous())
    if dev_inp.get("A") is not None:
        host["A"] = syn.torch_to_np(dev_inp["A"][:nheads].contiguous())
    t0 = time.perf_counter()
    oracle.prefill(host)
    el = time.perf_counter() - t0
    head_tokens = w.B * Ts * nheads
    tok_s = head_tokens / el / H  # whole-token (all H heads) rate
    return {"value": tok_s, "unit": "tokens/s", "cores": nthr, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"fp64 C oracle, first {nheads} of {H} heads x first {Ts} tokens "
                      f"({head_tokens} head-tokens, {el:.1f} s); tokens/s = head-tokens/s / {H}"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_peaks(torch):
    """This GPU's own peaks (libkda_peaks.so): a fetch-modify-write of 1.61 GB of
    fp32 with the decode step's access pattern (the decode state's size), swept
    over workgroups per compute unit; the same blocks read and written in place
    or copied to a second buffer by workgroups of 256, 512 or 1024 threads; and
    loops of fp16 16x16x32 matrix-core instructions on register operands, swept
    over grid size and independent chains.  The best of each sweep is reported;
    every point is listed."""
    import ctypes
    path = os.path.join(ROOT, "gated_delta_rule_28_amd", "libkda_peaks.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run `python -m gated_delta_rule_28_amd.build`")
    L = ctypes.CDLL(path)
    L.kda_peak_fmw.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    L.kda_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 256 * 96 * 128 * 128 * 4
    buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    fmw = {}
    for lds in (0, 24 << 10, 32 << 10, 40 << 10, 54 << 10, 80 << 10):
        def run():
            assert L.kda_peak_fmw(ctypes.c_void_p(buf.data_ptr()), nbytes, lds, stream) == 0
        for _ in range(3):
            run()
        ms = sorted(timed_launches(torch, run, 15))[7]
        fmw[f"lds{lds >> 10}k"] = 2 * nbytes / (ms * 1e-3) / 1e9
    L.kda_peak_rw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    dst = torch.zeros_like(buf)
    rw = {}
    for mode in ("inplace", "copy"):
        for threads in (256, 512, 1024):
            d = buf if mode == "inplace" else dst
            def run():
                assert L.kda_peak_rw(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(d.data_ptr()), nbytes, threads,
                                     stream) == 0
            for _ in range(3):
                run()
            ms = sorted(timed_launches(torch, run, 15))[7]
            rw[f"{mode}_t{threads}"] = 2 * nbytes / (ms * 1e-3) / 1e9
    del dst
    L.kda_peak_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    buf.zero_()
    one_way = {}
    for direction, name in ((0, "read"), (1, "write")):
        def run():
            assert L.kda_peak_stream(ctypes.c_void_p(buf.data_ptr()), nbytes, direction, stream) == 0
        for _ in range(3):
            run()
        ms = sorted(timed_launches(torch, run, 15))[7]
        one_way[name] = nbytes / (ms * 1e-3) / 1e9
    del buf
    # a mix of X bytes read and X written at the two directions' own rates
    mix = 2.0 / (1.0 / one_way["read"] + 1.0 / one_way["write"])
    iters = 20000
    out = torch.empty(4096 * 256, dtype=torch.float32, device="cuda")
    mfma = {}
    for blocks in (1024, 2048, 4096):
        for chains in (4, 8):
            it = iters * 4 // chains
            def run():
                assert L.kda_peak_mfma(ctypes.c_void_p(out.data_ptr()), blocks, it, chains, stream) == 0
            run()
            ms = sorted(timed_launches(torch, run, 3))[1]
            mfma[f"b{blocks}c{chains}"] = blocks * 4 * chains * it * 16 * 16 * 32 * 2 / (ms * 1e-3) / 1e12
    return {"hbm_fetch_modify_write_gbs": max(fmw.values()), "hbm_fmw_sweep_gbs": fmw,
            "hbm_read_gbs": one_way["read"], "hbm_write_gbs": one_way["write"],
            "hbm_read_write_mix_gbs": mix,
            "hbm_read_write_gbs": max(rw.values()), "hbm_read_write_sweep_gbs": rw,
            "hbm_peak_gbs": max(max(fmw.values()), mix, max(rw.values())),
            "mfma_f16_tflops": max(mfma.values()), "mfma_sweep_tflops": mfma,
            "how": "median launch time with HIP events: kda_peak_fmw over 1.61 GB (decode access pattern; "
                   "dynamic LDS caps workgroups per CU); kda_peak_stream read-only and write-only over the same "
                   "blocks, combined as 2 / (1/read + 1/write) for an equal mix; kda_peak_rw over the same blocks "
                   "in place and as a copy to a second buffer, 256/512/1024-thread workgroups; kda_peak_mfma "
                   "(workgroups x chains); hbm_peak_gbs is the largest of the fetch-modify-write, the mix and the "
                   "read+write sweep"}


FP32_VALU_PEAK_TFS = 157.3


def backward_flops_per_head_token(d):
    """Algorithmic FLOP of the prefill gradient per (head, token), state side:
    one forward step (decay d^2, y 2d^2, rank-1 update 2d^2, read-out 2d^2 = 7d^2)
    and the reverse step (decay of the state and of its gradient 2d^2, S_t 2d^2,
    S_t dz 2d^2, q^ dz^T 2d^2, dS^T k^ 2d^2, dS u + S' dy 4d^2, k^ dy^T 2d^2,
    rowsum(dS' S') 2d^2 = 18d^2); the O(d) vector work is not counted."""
    return 25 * d * d


def time_backward_segments(torch, kda, w, inp, steps):
    """kda_prefill_backward of a workload run as carried segments (long1m: 16 x
    65536 tokens), segment by segment from the last: each call's grad_S0 and
    grad_conv_in are the earlier segment's grad_S_T and grad_conv_out.  Each
    segment's entering state and conv rows come from a segment-wise forward
    before the timed region; one random segment-sized grad_o serves every
    segment (the whole sequence's would not fit beside the inputs)."""
    dev = inp["q"].device
    R = w.segments
    L = w.T // R
    need = 6 * w.B * L * w.H * w.dk * 4 + kda.backward_workspace_bytes(w.B, L, w.H, w.dk, w.dv)
    free, _ = torch.cuda.mem_get_info(dev)
    if need > 0.9 * free:
        log(f"[bench] segment-wise backward skipped: needs {need / 2**30:.0f} GiB, {free / 2**30:.0f} GiB free")
        return {"skipped": f"needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} GiB free"}
    seq = ("q", "k", "v", "g", "beta", "gate")
    part = [{x: inp[x][:, r * L:(r + 1) * L] for x in seq} for r in range(R)]
    # the carries entering each segment
    S = inp["S0"].clone() if inp.get("S0") is not None else torch.zeros((w.B, w.H, w.dk, w.dv), device=dev)
    conv = torch.zeros((w.B, 3, w.cch), dtype=inp["q"].dtype, device=dev)
    S_in, conv_in = [], []
    for r in range(R):
        S_in.append(S.clone())
        conv_in.append(conv.clone())
        pr = part[r]
        kda.prefill(pr["q"], pr["k"], pr["v"], inp["conv_w"], pr["g"], pr["beta"], pr["gate"], S0=S,
                    conv_in=conv, chunk=w.chunk, S_T=S, conv_out=conv)
    torch.cuda.synchronize()
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    go = torch.randn((w.B, L, w.H, w.dv), generator=gen, device=dev)
    gs_T = torch.randn((w.B, w.H, w.dk, w.dv), generator=gen, device=dev)
    ws = torch.empty(kda.backward_workspace_bytes(w.B, L, w.H, w.dk, w.dv), dtype=torch.uint8, device=dev)

    def call():
        gS, gC = gs_T, None
        for r in range(R - 1, -1, -1):
            pr = part[r]
            g = kda.prefill_backward(pr["q"], pr["k"], pr["v"], inp["conv_w"], pr["g"], pr["beta"], pr["gate"], go,
                                     S0=S_in[r], conv_in=conv_in[r], grad_S_T=gS, grad_conv_out=gC, workspace=ws)
            gS, gC = g["S0"], g["conv_in"]
            del g  # this segment's 16 GB of input gradients go back before the next call allocates its own

    call()
    torch.cuda.synchronize()
    per = timed_launches(torch, call, steps)
    ms = sum(per) / len(per)
    flops = backward_flops_per_head_token(w.dk) * w.B * w.T * w.H
    tfs = flops / (ms * 1e-3) / 1e12
    log(f"[bench] backward, {R} segments of {L}: {ms:.1f} ms/call, {w.B * w.T / (ms * 1e-3) / 1e6:.3f} M tokens/s, "
        f"{tfs:.2f} TFLOP/s")
    return {"metric": "prefill backward tokens/s", "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s",
            "ms_per_call": ms, "calls_timed": steps,
            "config": f"kda_prefill_backward of B{w.B} T{w.T} H{w.H} dk=dv={w.dk} as {R} carried segments of "
                      f"{L} tokens (last first, state and conv gradients chained), bf16 inputs, fp32 gradients",
            "roofline": {"bound": "alu", "achieved": tfs, "peak": FP32_VALU_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": tfs / FP32_VALU_PEAK_TFS, "traffic": None,
                         "algorithmic_flops_per_launch": flops,
                         "launches": f"{R} calls, each " + backward_launches(L, w.dk)},
            "workspace_bytes": ws.numel()}


def time_backward(torch, kda, w, inp, steps):
    """kda_prefill_backward over the whole workload (all T tokens of each
    sequence), random fp32 output and final-state gradients."""
    if w.segments > 1:
        return time_backward_segments(torch, kda, w, inp, steps)
    dev = inp["q"].device
    # fp32 gradients of q, k, v, g, gate, grad_o, and the workspace
    need = 6 * w.B * w.T * w.H * w.dk * 4 + kda.backward_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv)
    free, _ = torch.cuda.mem_get_info(dev)
    if need > 0.9 * free:
        log(f"[bench] backward skipped: needs {need / 2**30:.0f} GiB, {free / 2**30:.0f} GiB free "
            "(a sequence this long takes segment-wise backward calls)")
        return {"skipped": f"needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} GiB free"}
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    go = torch.randn((w.B, w.T, w.H, w.dv), generator=gen, device=dev)
    gs = torch.randn((w.B, w.H, w.dk, w.dv), generator=gen, device=dev)
    ws = torch.empty(kda.backward_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8, device=dev)
    args = [inp[x] for x in ("q", "k", "v", "conv_w", "g", "beta", "gate")]
    holder = {}

    def call():
        holder["g"] = kda.prefill_backward(*args, go, S0=inp["S0"], grad_S_T=gs, workspace=ws)

    call()
    torch.cuda.synchronize()
    per = timed_launches(torch, call, steps)
    ms = sum(per) / len(per)
    flops = backward_flops_per_head_token(w.dk) * w.B * w.T * w.H
    tfs = flops / (ms * 1e-3) / 1e12
    log(f"[bench] backward: {ms:.1f} ms/call, {w.B * w.T / (ms * 1e-3) / 1e6:.3f} M tokens/s, {tfs:.2f} TFLOP/s")
    return {"metric": "prefill backward tokens/s", "value": w.B * w.T / (ms * 1e-3), "unit": "tokens/s",
            "ms_per_call": ms, "calls_timed": steps,
            "config": f"kda_prefill_backward B{w.B} T{w.T} H{w.H} dk=dv={w.dk}, bf16 inputs, fp32 gradients",
            "roofline": {"bound": "alu", "achieved": tfs, "peak": FP32_VALU_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": tfs / FP32_VALU_PEAK_TFS, "traffic": None,
                         "algorithmic_flops_per_launch": flops, "launches": backward_launches(w.T, w.dk)},
            "workspace_bytes": ws.numel()}


def backward_launches(T, d):
    """What one kda_prefill_backward call of T tokens launches (32-token stretches, 32 per slab)."""
    stretches = -(-T // 32)
    slabs = max(1, -(-stretches // 32))
    return (f"prefill_kernel<32, {d}, {d}, ., false, true> (the chunkwise forward with fp32 operands, storing the "
            f"state every 32 tokens) once, then {slabs} x (backward_kernel mode 2: recompute of a slab of 1,024 "
            "tokens, on the compute units the reverse leaves free, overlapping mode 3: the reverse walk of the "
            "previous slab)")


def time_context_parallel(torch, kda, w, inp, R, A, steps):
    """kda_prefill_cp of the whole workload (all T tokens of each sequence, whatever
    segmentation the workload's own timing uses) in R segments on this GPU (three prefill
    passes over all segments and the composition), and one rank's share of it at
    the rank's shape: kda_cp_fragments of its segment (the intra-chunk work once,
    the recurrence from S = 0 and from S = I side by side), the composition of
    the R gathered fragments and kda_cp_finish from the entering state (the
    exchange itself needs R GPUs and is not timed)."""
    if w.T % R or w.T // R < 3:
        raise SystemExit(f"--cp-segments {R} does not split workload {w.name}")
    dev = inp["q"].device
    L = w.T // R
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device=dev)
    S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    conv = torch.empty((w.B, 3, w.cch), dtype=torch.bfloat16, device=dev)
    nbytes = kda.cp_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, R, w.chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    args = [inp[x] for x in ("q", "k", "v", "conv_w", "g", "beta", "gate")]

    def call():
        kda.prefill_cp(*args, R, S0=inp["S0"], chunk=w.chunk, o=o, S_T=S, conv_out=conv, workspace=ws, A=A)

    call()
    torch.cuda.synchronize()
    per = timed_launches(torch, call, steps)
    ms = sum(per) / len(per)
    del ws, o
    log(f"[bench] context-parallel prefill, {R} segments on one GPU: {ms:.3f} ms/call")

    # one rank's share (segment 0's inputs; every segment has the same shape)
    seg = [t if t is inp["conv_w"] else t[:, :L].contiguous() for t in args]
    BH = w.B * w.H
    N1 = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    P1 = torch.empty_like(N1)
    NR = torch.randn((w.B * R, w.H, w.dk, w.dv), device=dev) * 0.01
    PR = NR + torch.randn_like(NR) * 0.01
    Sst = torch.empty_like(NR)
    o_r = torch.empty((w.B, L, w.H, w.dv), dtype=torch.float32, device=dev)
    ws_r = torch.empty(max(kda.cp_rank_workspace_bytes(w.B, L, w.H, w.dk, w.dv, w.chunk), 16), dtype=torch.uint8,
                       device=dev)

    def rank():
        kda.cp_fragments(*seg, chunk=w.chunk, N=N1, P=P1, workspace=ws_r, o=o_r, A=A)
        kda.cp_compose(NR, PR, S0=inp["S0"], B=w.B, S_start=Sst, want_state=False)
        kda.cp_finish(ws_r, *seg, Sst[:w.B], chunk=w.chunk, o=o_r, S_T=N1, want_conv=False, A=A)

    rank()
    torch.cuda.synchronize()
    rper = timed_launches(torch, rank, steps)
    rms = sum(rper) / len(rper)
    log(f"[bench] one rank's share ({L} tokens, {R} fragments composed): {rms:.3f} ms")
    nbytes_alg = prefill_bytes_per_launch(w.B, w.T, w.H, w.dk, w.dv)
    gbs = nbytes_alg / (ms * 1e-3) / 1e9
    return {"segments": R, "ms_per_call": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3), "calls_timed": steps,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                         "algorithmic_bytes_per_launch": nbytes_alg,
                         "note": "the prefill's algorithmic bytes; on one GPU the call runs all three passes "
                                 "of every segment"},
            "config": f"kda_prefill_cp of the {w.name} workload in {R} segments of {L} tokens on one GPU: "
                      "three prefill passes over all segments and the composition",
            "rank_share_ms": rms,
            "rank_share": f"kda_cp_fragments of one segment of B{w.B} T{L} H{w.H} (N from S = 0, P from S = I), "
                          f"kda_cp_compose of {R} fragments, kda_cp_finish; the all-gather of the fragments "
                          f"({2 * BH * w.dk * w.dv * 4} bytes per rank) needs {R} GPUs and is not timed",
            "workspace_bytes": nbytes}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="k3width", choices=["k3width", "prefill", "long1m"])
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate", action="store_true")
    ap.add_argument("--decay-form", default="direct", choices=["direct", "k3"])
    ap.add_argument("--verify-tokens", type=int, default=4)
    ap.add_argument("--backward-steps", type=int, default=0,
                    help="also time kda_prefill_backward over the workload (this many calls)")
    ap.add_argument("--cp-segments", type=int, default=0,
                    help="also time the context-parallel prefill (kda_prefill_cp) with this many segments")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU path only; run it with --gpus 1 "
              "(multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_28_amd as kda
    import kda_synth as syn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    kda.lib()
    dev = "cuda"
    w = syn.WORKLOADS[args.workload]
    seg = w.T // w.segments
    log(f"[bench] workload {w.name}: B{w.B} T{w.T} H{w.H} d{w.dk} C{w.chunk} ({w.segments} segment(s))")

    t0 = time.perf_counter()
    inp = syn.prefill_inputs_torch(w, dev)
    if args.decay_form == "k3":
        inp = syn.with_k3_logits_torch(inp, w, dev)
    A = inp.get("A")
    torch.cuda.synchronize()
    log(f"[bench] inputs generated on device in {time.perf_counter() - t0:.1f} s")
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device=dev)
    S = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    conv = torch.zeros((w.B, 3, w.cch), dtype=torch.bfloat16, device=dev)
    S0 = inp["S0"]

    def step():
        if w.segments == 1:
            kda.prefill(inp["q"], inp["k"], inp["v"], inp["conv_w"], inp["g"], inp["beta"], inp["gate"],
                        S0=S0, conv_in=None, chunk=w.chunk, o=o, S_T=S, conv_out=conv, A=A)
            return
        S.zero_()
        conv.zero_()
        for s in range(w.segments):
            t0_, t1_ = s * seg, (s + 1) * seg
            kda.prefill(inp["q"][:, t0_:t1_], inp["k"][:, t0_:t1_], inp["v"][:, t0_:t1_], inp["conv_w"],
                        inp["g"][:, t0_:t1_], inp["beta"][:, t0_:t1_], inp["gate"][:, t0_:t1_],
                        S0=S, conv_in=conv, chunk=w.chunk, o=o[:, t0_:t1_], S_T=S, conv_out=conv, A=A)

    if w.segments > 1:
        # segment views must be contiguous for the ABI: [B=1, seg, H, d] slices are
        assert w.B == 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    per = timed_launches(torch, step, args.steps)
    torch.cuda.synchronize()
    ms = sum(per) / len(per)
    timeouts = kda.wait_timeouts()
    if timeouts:  # a slab arrived late: the resume launch did part of the work
        log(f"[bench] {timeouts} per-slab waits expired (kernels serialised?): the timing includes resume launches")
    tokens = w.B * w.T
    value = tokens / (ms * 1e-3)
    launch_ms = ms / w.segments
    nbytes = prefill_bytes_per_launch(w.B, seg, w.H, w.dk, w.dv)
    flops = prefill_flops(w.B, seg, w.H, w.dk, w.dv, w.chunk)
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    # one kda_prefill call = every slab of the two kernels of the workspace path
    src = os.path.join(ROOT, "gated_delta_rule_28_amd", "csrc", "kda_prefill_split.hip")
    traffic = load_traffic("prefill_call", src)
    log(f"[bench] prefill {ms:.3f} ms/step, {value / 1e6:.2f} M tokens/s, {achieved:.0f} GB/s algorithmic")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": ("synthetic (seeded device draws; q,k,v,gate ~ N(0,1), g = -softplus(N(-3,1)), beta = sigmoid(N(0,1)))"
                 if A is None else
                 "synthetic (seeded device draws; q,k,v,gate ~ N(0,1); g, beta as K3 logits: z ~ N(-4.7,1), "
                 "b ~ N(0,1), A ~ N(0,0.1))"),
        "config": {"workload": f"{w.name}: KDA prefill B{w.B} T{w.T} H{w.H} dk=dv={w.dk} chunk {w.chunk}"
                               + (f", {w.segments} segments of {seg} with state carried" if w.segments > 1 else ""),
                   "inputs": "bf16", "state": "f32", "output": "f32", "decay_form": args.decay_form,
                   "matrix_core_operands": "f16 with f32 accumulation"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "kda_prefill (intra_chunk_kernel + inter_chunk_kernel, bf16 in, f32 out)",
                     "algorithmic_bytes_per_launch": nbytes, "launch_ms": launch_ms,
                     "workspace_bytes": kda.workspace_bytes(w.B, seg, w.H, w.dk, w.dv, w.chunk)},
        "mfma": {"algorithmic_flops_per_launch": flops,
                 "tflops": flops / (launch_ms * 1e-3) / 1e12,
                 "frac_of_bf16_f16_peak": flops / (launch_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFS},
    }
    del o

    if args.backward_steps > 0:
        out["backward"] = time_backward(torch, kda, w, inp, args.backward_steps)

    if args.cp_segments > 0:
        out["context_parallel"] = time_context_parallel(torch, kda, w, inp, args.cp_segments, A,
                                                        min(args.steps, 5))

    if args.decode_steps > 0:
        wd = syn.WORKLOADS["decode"]
        nsteps = args.decode_steps
        t0 = time.perf_counter()
        d = syn.decode_inputs_torch(wd, dev, nsteps)
        od = torch.empty((wd.B, wd.H, wd.dv), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        log(f"[bench] decode inputs ({nsteps} steps) generated in {time.perf_counter() - t0:.1f} s")

        def dstep(s):
            kda.decode_step(d["q"][s], d["k"][s], d["v"][s], d["conv_w"], d["g"][s], d["beta"][s],
                            d["gate"][s], d["S"], d["conv_state"], o=od)

        for s in range(min(20, nsteps)):
            dstep(s)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(nsteps):
            dstep(s)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / nsteps
        dbytes = decode_bytes_per_step(wd.B, wd.H, wd.dk, wd.dv)
        gbs = dbytes / (dms * 1e-3) / 1e9
        dsrc = os.path.join(ROOT, "gated_delta_rule_28_amd", "csrc", "kda_decode.hip")
        out["decode"] = {"metric": "decode-step HBM GB/s", "value": gbs, "unit": "GB/s",
                         "ms_per_step": dms, "steps_timed": nsteps,
                         "config": f"decode N{wd.B} H{wd.H} dk=dv={wd.dk}, bf16 inputs, f32 state",
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": gbs / HBM_PEAK_GBS,
                                      "traffic": load_traffic("decode_kernel", dsrc),
                                      "algorithmic_bytes_per_launch": dbytes}}
        log(f"[bench] decode {dms * 1e3:.1f} us/step, {gbs:.0f} GB/s")
        del d

    if args.decode_steps > 0 and args.verify_tokens > 0:
        wd = syn.WORKLOADS["decode"]
        M = args.verify_tokens
        ncalls = max(1, args.decode_steps // M)
        t0 = time.perf_counter()
        # ncalls sets of M tokens for N sequences: [ncalls * N, M, H, .]
        wm = syn.Workload("verify", ncalls * wd.B, M, wd.H, wd.dk, wd.dv, 1, "bf16", seed=wd.seed + 16)
        dm = syn.prefill_inputs_torch(wm, dev)
        st = syn.decode_inputs_torch(wd, dev, 1)
        om = torch.empty((wd.B, M, wd.H, wd.dv), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        log(f"[bench] multi-token decode inputs ({ncalls} calls x {M} tokens) generated in "
            f"{time.perf_counter() - t0:.1f} s")

        def mstep(c):
            r = slice(c * wd.B, (c + 1) * wd.B)
            kda.decode_multi(dm["q"][r], dm["k"][r], dm["v"][r], dm["conv_w"], dm["g"][r], dm["beta"][r],
                             dm["gate"][r], st["S"], st["conv_state"], o=om)

        for c in range(min(5, ncalls)):
            mstep(c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for c in range(ncalls):
            mstep(c)
        e1.record()
        torch.cuda.synchronize()
        mms = e0.elapsed_time(e1) / ncalls
        mbytes = decode_multi_bytes_per_call(wd.B, M, wd.H, wd.dk, wd.dv)
        mgbs = mbytes / (mms * 1e-3) / 1e9
        out["decode_multi"] = {"metric": "multi-token decode tokens/s", "value": wd.B * M / (mms * 1e-3),
                               "unit": "tokens/s", "tokens_per_call": M, "ms_per_call": mms,
                               "calls_timed": ncalls,
                               "config": f"kda_decode_multi N{wd.B} M{M} H{wd.H} dk=dv={wd.dk}, bf16 inputs, "
                                         "f32 state, all tokens committed",
                               "roofline": {"bound": "hbm", "achieved": mgbs, "peak": HBM_PEAK_GBS,
                                            "unit": "GB/s", "frac": mgbs / HBM_PEAK_GBS,
                                            "traffic": load_traffic("decode_multi_kernel", os.path.join(
                                                ROOT, "gated_delta_rule_28_amd", "csrc", "kda_decode.hip")),
                                            "algorithmic_bytes_per_launch": mbytes}}
        log(f"[bench] multi-token decode M={M}: {mms * 1e3:.1f} us/call, "
            f"{wd.B * M / (mms * 1e-3) / 1e6:.2f} M tokens/s, {mgbs:.0f} GB/s")
        del dm, st

    if args.calibrate:
        # an elementwise kernel that reads 1 GiB and writes 1 GiB: the known-size
        # reference for scaling the HBM byte counters
        n = 1 << 28
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = 2 * 4 * n

    peaks = measured_peaks(torch)
    out["measured_peaks"] = peaks
    mh, mm = peaks["hbm_peak_gbs"], peaks["mfma_f16_tflops"]
    out["roofline"]["measured_peak"] = mh
    out["roofline"]["frac_of_measured"] = out["roofline"]["achieved"] / mh
    out["mfma"]["frac_of_measured_f16_peak"] = out["mfma"]["tflops"] / mm
    if "decode" in out:
        out["decode"]["roofline"]["measured_peak"] = mh
        out["decode"]["roofline"]["frac_of_measured"] = out["decode"]["roofline"]["achieved"] / mh
    if "decode_multi" in out:
        out["decode_multi"]["roofline"]["measured_peak"] = mh
        out["decode_multi"]["roofline"]["frac_of_measured"] = out["decode_multi"]["roofline"]["achieved"] / mh
    log(f"[bench] measured peaks: fetch-modify-write {peaks['hbm_fetch_modify_write_gbs']:.0f} GB/s, read "
        f"{peaks['hbm_read_gbs']:.0f}, write {peaks['hbm_write_gbs']:.0f}, read+write mix {peaks['hbm_read_write_mix_gbs']:.0f}"
        f", read+write sweep {peaks['hbm_read_write_gbs']:.0f}"
        f" GB/s; fp16 matrix cores {mm:.0f} TFLOP/s")

    if not args.no_cpu:
        log("[bench] timing the oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(w, inp)
        log(f"[bench] oracle {out['cpu_baseline']['value']:.1f} tokens/s on {out['cpu_baseline']['cores']} threads")

    kda.release()  # the pipeline's streams, before the runtime's teardown
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
