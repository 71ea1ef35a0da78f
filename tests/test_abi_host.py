"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

* libkda.so loads and exports every function include/kda.h declares;
* the ctypes structures of the binding match the C layout (offsets computed
  by gcc from the header itself);
* argument validation returns the documented codes before any HIP call.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def kda():
    import gated_delta_rule_28_amd as kda
    if not os.path.exists(kda.library_path):
        pytest.skip("libkda.so not built")
    kda.lib()
    return kda


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kda_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    for must in ("kda_prefill", "kda_decode_step", "kda_decode_multi", "kda_prefill_workspace_bytes", "kda_prep",
                 "kda_status_string", "kda_last_error", "kda_abi_version", "kda_cp_compose", "kda_prefill_cp",
                 "kda_prefill_cp_workspace_bytes", "kda_prefill_backward", "kda_prefill_backward_workspace_bytes",
                 "kda_release", "kda_cp_fragments", "kda_cp_finish", "kda_cp_rank_workspace_bytes",
                 "kda_wait_timeouts", "kda_debug_pipeline"):
        assert must in names


def test_every_declared_symbol_is_exported(kda):
    L = kda.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", kda.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (kda_\w+)", out))
    assert set(declared_functions()) <= exported


def _c_offsets(struct, fields):
    """offsetof/sizeof of a kda.h struct, computed by gcc from the header."""
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"kda.h\"\nint main(void){\n"
    src += f'printf("%zu\\n", sizeof({struct}));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof({struct}, {f}));\n'
    src += "return 0;}\n"
    d = os.path.join(ROOT, "_build_abi_check")
    os.makedirs(d, exist_ok=True)
    c = os.path.join(d, f"{struct}.c")
    exe = os.path.join(d, struct)
    open(c, "w").write(src)
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
    vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    return vals[0], vals[1:]


@pytest.mark.parametrize("name", ["PrefillArgs", "DecodeArgs", "PrepArgs", "DecodeMultiArgs", "CpComposeArgs",
                                  "PrefillCpArgs", "PrefillBackwardArgs"])
def test_ctypes_layout_matches_header(name):
    import gated_delta_rule_28_amd as kda
    cls = getattr(kda, name)
    struct = {"PrefillArgs": "kda_prefill_args", "DecodeArgs": "kda_decode_args",
              "PrepArgs": "kda_prep_args", "DecodeMultiArgs": "kda_decode_multi_args",
              "CpComposeArgs": "kda_cp_compose_args", "PrefillCpArgs": "kda_prefill_cp_args",
              "PrefillBackwardArgs": "kda_prefill_backward_args"}[name]
    fields = [f for f, _ in cls._fields_]
    size, offs = _c_offsets(struct, fields)
    assert ctypes.sizeof(cls) == size
    assert [getattr(cls, f).offset for f in fields] == offs


def _prefill_args(kda, **over):
    # fake, 16-byte aligned addresses: validation must reject before touching them
    base = dict(B=1, T=8, H=2, dk=16, dv=16, chunk=16, in_dtype=kda.KDA_BF16, out_dtype=kda.KDA_F32,
                q=0x1000, k=0x2000, v=0x3000, conv_w=0x4000, g=0x5000, beta=0x6000, gate=0x7000,
                S0=None, conv_in=None, o=0x8000, S_T=None, conv_out=None, workspace=None,
                workspace_bytes=0)
    base.update(over)
    return kda.PrefillArgs(**base)


CASES = [
    (dict(q=None), -1), (dict(o=None), -1), (dict(gate=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(T=-1), -2),
    (dict(in_dtype=7), -3), (dict(out_dtype=-1), -3),
    (dict(k=0x2008), -4), (dict(o=0x8004), -4), (dict(S0=0x9002), -4), (dict(beta=0x6001), -4),
    (dict(dk=48, dv=48), -5), (dict(dk=16, dv=32), -5), (dict(dk=256, dv=256), -5),
    (dict(chunk=48), -5), (dict(chunk=128), -5),
    # decay form: unknown value, K3's logits without A, A misaligned
    (dict(decay_form=2), -5), (dict(decay_form=-1), -5), (dict(decay_form=1), -1),
    (dict(decay_form=1, A=0xb008), -4),
]


@pytest.mark.parametrize("over,code", CASES)
def test_prefill_validation_codes(kda, over, code):
    a = _prefill_args(kda, **over)
    L = kda.lib()
    assert L.kda_prefill(ctypes.byref(a), None) == code
    assert L.kda_last_error().decode() != ""
    assert L.kda_status_string(code).decode() not in ("", "unknown status code")


def test_prefill_null_args_and_empty(kda):
    L = kda.lib()
    assert L.kda_prefill(None, None) == -1
    assert L.kda_wait_timeouts(None) == -1
    assert L.kda_debug_pipeline(0, -2) == -2
    assert L.kda_debug_pipeline(0, -1) == 0
    # T = 0 with nothing to carry: nothing to do, succeeds without a launch
    a = _prefill_args(kda, T=0, q=None, k=None, v=None, o=None)
    assert L.kda_prefill(ctypes.byref(a), None) == 0
    assert L.kda_prefill_workspace_bytes(ctypes.byref(a)) == 0


def test_prefill_workspace_sizes_and_check(kda):
    """Workspace sizes (no device needed) and the too-small check, which runs
    before anything is launched."""
    L = kda.lib()
    # sizes with a two-kernel path: bf16 inputs, chunk 64, dk = dv = 128
    a = _prefill_args(kda, B=2, T=300, H=3, dk=128, dv=128, chunk=64)
    per_chunk = 2 * 3 * 64 * 1024
    carry = 2 * 3 * 128 * 128 * 4
    assert L.kda_prefill_workspace_bytes(ctypes.byref(a)) == 5 * per_chunk   # all 5 chunks, one launch
    assert L.kda_prefill_workspace_min_bytes(ctypes.byref(a)) == per_chunk + carry
    one = _prefill_args(kda, B=2, T=64, H=3, dk=128, dv=128, chunk=64)
    assert L.kda_prefill_workspace_min_bytes(ctypes.byref(one)) == per_chunk
    # no two-kernel path: fp32 inputs, other chunk or head dims
    for over in (dict(in_dtype=kda.KDA_F32), dict(chunk=32), dict(dk=64, dv=64)):
        b = _prefill_args(kda, **{**dict(B=2, T=300, H=3, dk=128, dv=128, chunk=64), **over})
        assert L.kda_prefill_workspace_bytes(ctypes.byref(b)) == 0
        assert L.kda_prefill_workspace_min_bytes(ctypes.byref(b)) == 0
    # invalid arguments: 0
    assert L.kda_prefill_workspace_bytes(ctypes.byref(_prefill_args(kda, B=0))) == 0
    # a workspace below the minimum is rejected; misaligned too
    small = _prefill_args(kda, B=2, T=300, H=3, dk=128, dv=128, chunk=64, workspace=0x100000,
                          workspace_bytes=per_chunk + carry - 1)
    assert L.kda_prefill(ctypes.byref(small), None) == -6
    mis = _prefill_args(kda, B=2, T=300, H=3, dk=128, dv=128, chunk=64, workspace=0x100008,
                        workspace_bytes=10 * per_chunk)
    assert L.kda_prefill(ctypes.byref(mis), None) == -4
    # longer sequences run in pipelined slabs of up to 64 chunks (32, then 16 of
    # 62 at 65,536 tokens), each slab in a region of its own while all fit
    # 16 GiB, else in three buffers used in turn (1,048,576 tokens), plus a
    # state carry
    big = _prefill_args(kda, B=1, T=1 << 16, H=96, dk=128, dv=128, chunk=64)
    assert L.kda_prefill_workspace_bytes(ctypes.byref(big)) == 17 * 64 * 96 * 64 * 1024 + 96 * 128 * 128 * 4
    big = _prefill_args(kda, B=1, T=1 << 20, H=96, dk=128, dv=128, chunk=64)
    assert L.kda_prefill_workspace_bytes(ctypes.byref(big)) == 3 * 64 * 96 * 64 * 1024 + 96 * 128 * 128 * 4
    # 65 chunks: two balanced slabs of 33, one buffer each
    b65 = _prefill_args(kda, B=1, T=65 * 64, H=2, dk=128, dv=128, chunk=64)
    assert L.kda_prefill_workspace_bytes(ctypes.byref(b65)) == 2 * 33 * 2 * 64 * 1024 + 2 * 128 * 128 * 4


def test_decode_validation_codes(kda):
    L = kda.lib()
    base = dict(N=2, H=2, dk=16, dv=16, in_dtype=kda.KDA_BF16, out_dtype=kda.KDA_F32, q=0x1000,
                k=0x2000, v=0x3000, conv_w=0x4000, g=0x5000, beta=0x6000, gate=0x7000, S=0x8000,
                conv_state=0x9000, o=0xa000)
    for over, code in [(dict(S=None), -1), (dict(conv_state=None), -1), (dict(N=0), -2),
                       (dict(in_dtype=3), -3), (dict(S=0x8008), -4), (dict(dk=24, dv=24), -5),
                       (dict(decay_form=5), -5), (dict(decay_form=1), -1),
                       (dict(decay_form=1, A=0xb004), -4)]:
        a = kda.DecodeArgs(**{**base, **over})
        assert L.kda_decode_step(ctypes.byref(a), None) == code, over
    assert L.kda_decode_step(None, None) == -1


def test_decode_multi_validation_codes(kda):
    L = kda.lib()
    base = dict(N=2, M=4, H=2, dk=16, dv=16, in_dtype=kda.KDA_BF16, out_dtype=kda.KDA_F32, q=0x1000,
                k=0x2000, v=0x3000, conv_w=0x4000, g=0x5000, beta=0x6000, gate=0x7000, S=0x8000,
                conv_state=0x9000, o=0xa000, accept=None)
    for over, code in [(dict(S=None), -1), (dict(o=None), -1), (dict(N=0), -2), (dict(M=0), -2),
                       (dict(M=17), -2), (dict(in_dtype=3), -3), (dict(S=0x8008), -4),
                       (dict(accept=0xb002), -4), (dict(dk=24, dv=24), -5),
                       (dict(decay_form=4), -5), (dict(decay_form=1), -1)]:
        a = kda.DecodeMultiArgs(**{**base, **over})
        assert L.kda_decode_multi(ctypes.byref(a), None) == code, over
    assert L.kda_decode_multi(None, None) == -1


def test_prep_validation_codes(kda):
    L = kda.lib()
    base = dict(B=1, T=8, H=2, dk=16, dv=16, chunk=16, in_dtype=kda.KDA_F32, q=0x1000, k=0x2000,
                v=0x3000, conv_w=0x4000, g=0x5000, conv_in=None, q_out=0x6000, k_out=0x7000,
                v_out=0x8000, G_out=0x9000)
    for over, code in [(dict(G_out=None), -1), (dict(T=-2), -2), (dict(in_dtype=9), -3),
                       (dict(q_out=0x6004), -4), (dict(chunk=8), -5), (dict(decay_form=3), -5),
                       (dict(decay_form=1), -1)]:
        a = kda.PrepArgs(**{**base, **over})
        assert L.kda_prep(ctypes.byref(a), None) == code, over


def test_cp_compose_validation_codes(kda):
    L = kda.lib()
    base = dict(B=2, R=3, H=2, d=32, N=0x1000, P=0x2000, S0=None, S_start=0x3000, S_T=None)
    for over, code in [(dict(N=None), -1), (dict(P=None), -1), (dict(S_start=None), -1), (dict(B=0), -2),
                       (dict(R=0), -2), (dict(H=-1), -2), (dict(d=48), -5), (dict(d=256), -5),
                       (dict(S0=0x4008), -4), (dict(S_T=0x5004), -4), (dict(P=0x2002), -4)]:
        a = kda.CpComposeArgs(**{**base, **over})
        assert L.kda_cp_compose(ctypes.byref(a), None) == code, over
    assert L.kda_cp_compose(None, None) == -1


def _cp_args(kda, segments=4, ws=0x100000, ws_bytes=1 << 40, **over):
    return kda.PrefillCpArgs(_prefill_args(kda, **{**dict(B=2, T=256, H=3, dk=128, dv=128, chunk=64), **over}),
                             segments, ws, ws_bytes)


def test_prefill_cp_validation_and_workspace(kda):
    """Context-parallel prefill: segment count, split, workspace; nothing launched."""
    L = kda.lib()
    for a, code in [(_cp_args(kda, segments=0), -2), (_cp_args(kda, segments=3), -2),
                    (_cp_args(kda, segments=128), -2),   # 2 tokens per segment
                    (_cp_args(kda, ws=None), -1), (_cp_args(kda, ws=0x100008), -4),
                    (_cp_args(kda, ws_bytes=1000), -6), (_cp_args(kda, q=None), -1),
                    (_cp_args(kda, dk=64, dv=128), -5), (_cp_args(kda, chunk=8), -5),
                    (_cp_args(kda, decay_form=1), -1)]:
        assert L.kda_prefill_cp(ctypes.byref(a), None) == code
    assert L.kda_prefill_cp(None, None) == -1
    # workspace: histories + three state batches + the segment prefills' workspace
    a = _cp_args(kda, segments=4)
    seg = _prefill_args(kda, B=8, T=64, H=3, dk=128, dv=128, chunk=64)
    cch = 3 * 3 * 128
    r256 = lambda x: (x + 255) // 256 * 256
    want = (r256(8 * 3 * cch * 2) + 3 * r256(8 * 3 * 128 * 128 * 4)
            + L.kda_prefill_workspace_bytes(ctypes.byref(seg)))
    assert L.kda_prefill_cp_workspace_bytes(ctypes.byref(a)) == want
    assert L.kda_prefill_cp_workspace_bytes(ctypes.byref(_cp_args(kda, segments=3))) == 0
    assert L.kda_prefill_cp_workspace_bytes(None) == 0


def test_prefill_backward_validation_and_workspace(kda):
    L = kda.lib()
    base = dict(B=2, T=100, H=3, dk=32, dv=32, in_dtype=kda.KDA_BF16, q=0x1000, k=0x2000, v=0x3000,
                conv_w=0x4000, g=0x5000, beta=0x6000, gate=0x7000, S0=None, conv_in=None, grad_o=0x8000,
                grad_S_T=None, grad_conv_out=None, grad_q=0x9000, grad_k=0xa000, grad_v=0xb000, grad_g=0xc000, grad_beta=0xd000,
                grad_gate=0xe000, grad_S0=None, grad_conv_in=None, workspace=0x100000, workspace_bytes=1 << 40,
                decay_form=0, A=None)
    for over, code in [(dict(grad_o=None), -1), (dict(grad_k=None), -1), (dict(workspace=None), -1),
                       (dict(B=0), -2), (dict(in_dtype=5), -3), (dict(grad_q=0x9008), -4),
                       (dict(workspace=0x100004), -4), (dict(grad_beta=0xd002), -4),
                       (dict(grad_conv_out=0xf008), -4), (dict(dk=32, dv=64), -5),
                       (dict(decay_form=1, A=0xf000), -5), (dict(workspace_bytes=100), -6)]:
        a = kda.PrefillBackwardArgs(**{**base, **over})
        assert L.kda_prefill_backward(ctypes.byref(a), None) == code, over
    assert L.kda_prefill_backward(None, None) == -1
    # n d^2 + d^2 + 9 d + 2 min(n, 32) 32 (d^2 + 13 d + 8) floats per (b, h), n = ceil(T/32)
    a = kda.PrefillBackwardArgs(**base)
    want = 2 * 3 * (4 * 32 * 32 + 32 * 32 + 9 * 32 + 2 * 4 * 32 * (32 * 32 + 13 * 32 + 8)) * 4
    assert L.kda_prefill_backward_workspace_bytes(ctypes.byref(a)) == want
    assert L.kda_prefill_backward_workspace_bytes(None) == 0


def test_status_strings(kda):
    L = kda.lib()
    assert L.kda_status_string(0).decode() == "ok"
    assert L.kda_status_string(12345).decode() == "unknown status code"
    assert L.kda_abi_version() == 8


def test_release_with_nothing_kept(kda):
    """kda_release with no streams created makes no HIP call (safe without a GPU)
    and can be repeated."""
    L = kda.lib()
    assert L.kda_release() == 0 and L.kda_release() == 0


def test_noalloc_rejects_heads_beyond_its_scratch(kda):
    """kda_prefill_noalloc validates on the host: B*H whose minimum workspace
    (64 KiB + 64 KiB per head) exceeds the 128 MiB scratch is refused with
    KDA_E_WORKSPACE before any HIP call (so this runs without a GPU)."""
    L = kda.lib()
    fake = 1 << 20  # a 16-byte aligned stand-in address; nothing is launched
    a = kda.PrefillArgs(1, 128, 1025, 128, 128, 64, kda.KDA_BF16, kda.KDA_F32, fake, fake, fake, fake, fake,
                        fake, fake, None, None, fake, fake, fake, None, 0, kda.KDA_DECAY_DIRECT, None)
    assert L.kda_prefill_noalloc(ctypes.byref(a), None) == -6
    assert b"scratch" in L.kda_last_error()
    assert kda.NOALLOC_SCRATCH_BYTES == 128 << 20


def test_peaks_library_exports_its_header():
    """libkda_peaks.so (the measured-peak microbenchmarks the benchmark reports
    beside the vendor peaks) exports every function include/kda_peaks.h declares."""
    path = os.path.join(os.path.dirname(HEADER), "..", "gated_delta_rule_28_amd", "libkda_peaks.so")
    if not os.path.exists(path):
        pytest.skip("libkda_peaks.so not built")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(os.path.dirname(HEADER), "kda_peaks.h")).read(), flags=re.S)
    names = set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kda_\w+)\s*\(", text, flags=re.M))
    assert names == {"kda_peak_fmw", "kda_peak_stream", "kda_peak_rw", "kda_peak_mfma"}
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    assert names <= set(re.findall(r" T (kda_\w+)", out))
    L = ctypes.CDLL(path)
    L.kda_peak_fmw.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    L.kda_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    # argument checks run before any HIP call
    assert L.kda_peak_fmw(None, 65536, 0, None) == -1
    assert L.kda_peak_fmw(1 << 20, 1000, 0, None) == -2
    assert L.kda_peak_fmw((1 << 20) + 4, 65536, 0, None) == -3
    L.kda_peak_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    assert L.kda_peak_stream(1 << 20, 65536, 2, None) == -2
    L.kda_peak_rw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    assert L.kda_peak_rw(None, 1 << 20, 65536, 256, None) == -1
    assert L.kda_peak_rw(1 << 20, 1 << 24, 65536, 128, None) == -2            # workgroup size
    assert L.kda_peak_rw(1 << 20, (1 << 20) + 65536, 131072, 256, None) == -2  # partial overlap
    assert L.kda_peak_rw((1 << 20) + 4, 1 << 24, 65536, 256, None) == -3
    assert L.kda_peak_mfma(None, 1, 1, 4, None) == -1
    assert L.kda_peak_mfma(1 << 20, 1, 1, 5, None) == -2


def test_cp_rank_workspace_and_validation(kda):
    """kda_cp_rank_workspace_bytes: every 64-token chunk block (64 KiB per head)
    on the two-kernel path, one identity state per head otherwise; the two
    rank-share calls reject a missing fragment pointer or a short workspace
    before any HIP call."""
    L = kda.lib()
    a = kda.PrefillArgs(2, 130, 3, 128, 128, 64, kda.KDA_BF16, kda.KDA_F32)
    assert L.kda_cp_rank_workspace_bytes(ctypes.byref(a)) == 2 * 3 * 3 * 64 * 1024
    f = kda.PrefillArgs(2, 130, 3, 32, 32, 32, kda.KDA_F32, kda.KDA_F32)
    assert L.kda_cp_rank_workspace_bytes(ctypes.byref(f)) == (2 * 3 * 32 * 32 * 4 + 255) // 256 * 256
    bad = kda.PrefillArgs(2, 130, 3, 128, 64, 64, kda.KDA_BF16, kda.KDA_F32)
    assert L.kda_cp_rank_workspace_bytes(ctypes.byref(bad)) == 0
    fake = 1 << 20
    r = kda.PrefillArgs(1, 128, 2, 128, 128, 64, kda.KDA_BF16, kda.KDA_F32, fake, fake, fake, fake, fake,
                        fake, fake, None, None, fake, None, None, fake, 16, kda.KDA_DECAY_DIRECT, None)
    assert L.kda_cp_fragments(ctypes.byref(r), None, fake, None) == -1
    assert L.kda_cp_fragments(ctypes.byref(r), fake, fake, None) == -6
    assert L.kda_cp_finish(ctypes.byref(r), None) == -6
    r.workspace = None
    assert L.kda_cp_finish(ctypes.byref(r), None) == -1
