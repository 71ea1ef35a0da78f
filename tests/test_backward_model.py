"""The CPU model of the GPU backward's algorithm (tests/backward_model.py)
against the fp64 autograd reference: the step-by-step reverse derivation the
kernel follows, checked on the CPU (ragged stretches, bf16 inputs, fewer tokens
than the conv history)."""
from __future__ import annotations

import numpy as np
import pytest

import backward_model as bm
import kda_synth as syn
from kda_synth import Workload

ob = pytest.importorskip("oracle.backward")


@pytest.mark.parametrize("T,chunk,dtype", [(20, 8, "f32"), (37, 16, "bf16"), (2, 16, "f32"), (64, 64, "bf16")])
def test_reverse_model_equals_autograd(T, chunk, dtype):
    w = Workload("bm", 2, T, 2, 8, 8, 16, dtype, s0_sigma=0.3, conv_hist="normal", seed=3 + T)
    inp = syn.prefill_inputs_np(w)
    rng = np.random.default_rng(T)
    f = ob.forward(inp)
    dO = rng.standard_normal(f["o"].shape)
    dS = rng.standard_normal(f["S_T"].shape)
    dC = rng.standard_normal(f["conv_out"].shape)
    ref = ob.backward(inp, dO, dS, dC)
    got = bm.backward(inp, dO, dS, chunk=chunk, dconv_out=dC)
    for x in ref:
        assert np.abs(got[x] - ref[x]).max() <= 1e-12 * max(1.0, np.abs(ref[x]).max()), x
