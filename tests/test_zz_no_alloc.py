"""kda_prefill_noalloc (the allocation-free prefill) against kda_prefill.

Two calls in a row through the C ABI, the second on a smaller input, each
compared with kda_prefill on the same inputs (its preferred workspace): the
workloads' bound, 2e-2 x RMS, on o and S_T, and conv_out exactly.  The first
call needs more than one slab of the 128 MiB scratch; the second fits one.
"""
from __future__ import annotations

import numpy as np
import pytest

import kda_synth as syn
from gpu_util import assert_rms_close, need_gpu, to_dev
from kda_synth import Workload

pytestmark = pytest.mark.gpu


def _compare(kda, torch, w, seed_note):
    inp = syn.prefill_inputs_np(w)
    dev = to_dev(inp, "bf16")
    args = (dev["q"], dev["k"], dev["v"], dev["conv_w"], dev["g"], dev["beta"], dev["gate"])
    ref = kda.prefill(*args, S0=dev["S0"], conv_in=dev["conv_in"], chunk=64, workspace="auto")
    # outputs allocated up front: the no-allocation call itself allocates nothing
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    S_T = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    conv = torch.empty((w.B, 3, w.cch), dtype=torch.bfloat16, device="cuda")
    print(f"  {seed_note}: B{w.B} T{w.T} H{w.H} d{w.dk}", flush=True)
    got = kda.prefill(*args, S0=dev["S0"], conv_in=dev["conv_in"], chunk=64, o=o, S_T=S_T, conv_out=conv,
                      workspace="noalloc")
    torch.cuda.synchronize()
    for x, y, what in zip(got[:2], ref[:2], ("o", "S_T")):
        x, y = x.float().cpu().numpy(), y.float().cpu().numpy()
        assert_rms_close(x, y, 2e-2, f"no-alloc vs kda_prefill {what}")
        print(f"  {what} bit-identical: {np.array_equal(x, y)}", flush=True)
    assert torch.equal(got[2], ref[2]), "conv_out"


def test_noalloc_matches_prefill_twice():
    torch, kda = need_gpu()
    # 128 chunks x 32 heads x 64 KiB = 256 MiB of chunk blocks: several slabs of the scratch
    _compare(kda, torch, Workload("na1", 1, 8192, 32, 128, 128, 64, "bf16", s0_sigma=0.05,
                                  conv_hist="normal", seed=301), "first call")
    # smaller: one slab
    _compare(kda, torch, Workload("na2", 2, 300, 3, 128, 128, 64, "bf16", s0_sigma=0.05,
                                  conv_hist="normal", seed=302), "second call")
