"""MI355X (gfx950) Kimi Delta Attention: Python binding of libkda.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/kda.h.  Torch supplies device
memory and the current stream.  If the library is missing the import still
works, but every call raises (there is no fallback implementation).

    o, S_T, conv_out = prefill(q, k, v, conv_w, g, beta, gate, S0=None, conv_in=None, chunk=64)
    nbytes = workspace_bytes(B, T, H, dk, dv, chunk, in_dtype)  # what prefill allocates
    o = decode_step(q, k, v, conv_w, g, beta, gate, S, conv_state)   # S, conv_state in place
    o = decode_multi(q, k, v, conv_w, g, beta, gate, S, conv_state, accept=None)  # [N, M, H, .]
    qn, kn, vn, G = prep(q, k, v, conv_w, g, conv_in=None, chunk=64)
    o, S_T, conv_out = prefill_cp(q, k, v, conv_w, g, beta, gate, segments=R, ...)  # context-parallel
    S_start, S_T = cp_compose(N, P, S0=None, B=1)   # the composition step alone
    ws, N, P = cp_fragments(q, k, v, conv_w, g, beta, gate, conv_in=None)   # one rank's share, part 1
    o, S_T, conv_out = cp_finish(ws, q, k, v, conv_w, g, beta, gate, S_start, conv_in=None)  # part 2
    grads = prefill_backward(q, k, v, conv_w, g, beta, gate, grad_o, S0=None, conv_in=None, grad_S_T=None)
    release()   # destroy the streams the library keeps between calls (kda_release)

Every call also takes A=None: given an fp32 [H, dk] tensor, g and beta are K3's
logits (g = -5 sigmoid(e^A z), beta = sigmoid(b), KDA_DECAY_K3) instead of the
log-decay and beta themselves.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["prefill", "decode_step", "decode_multi", "prep", "workspace_bytes", "library_path", "lib", "KDAError",
           "KDA_F32", "KDA_BF16", "KDA_DECAY_DIRECT", "KDA_DECAY_K3", "PrefillArgs", "DecodeArgs",
           "PrepArgs", "DecodeMultiArgs", "MAX_DECODE_TOKENS", "prefill_cp", "cp_compose",
           "cp_workspace_bytes", "CpComposeArgs", "PrefillCpArgs", "prefill_backward", "PrefillBackwardArgs",
           "backward_workspace_bytes", "release", "cp_fragments", "cp_finish", "cp_rank_workspace_bytes"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkda.so")

KDA_F32 = 0
KDA_BF16 = 1
KDA_DECAY_DIRECT = 0
KDA_DECAY_K3 = 1
ABI_VERSION = 8
MAX_DECODE_TOKENS = 16
NOALLOC_SCRATCH_BYTES = 128 << 20  # KDA_NOALLOC_SCRATCH_BYTES


class KDAError(RuntimeError):
    def __init__(self, fn, code, detail):
        super().__init__(f"{fn} failed with {code}: {detail}")
        self.code = code


_P = ctypes.c_void_p


class PrefillArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("chunk", ctypes.c_int),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("q", _P), ("k", _P), ("v", _P), ("conv_w", _P), ("g", _P), ("beta", _P),
                ("gate", _P), ("S0", _P), ("conv_in", _P), ("o", _P), ("S_T", _P),
                ("conv_out", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
                ("decay_form", ctypes.c_int), ("A", _P)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int),
                ("dv", ctypes.c_int), ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("q", _P), ("k", _P), ("v", _P), ("conv_w", _P), ("g", _P), ("beta", _P),
                ("gate", _P), ("S", _P), ("conv_state", _P), ("o", _P),
                ("decay_form", ctypes.c_int), ("A", _P)]


class DecodeMultiArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int), ("M", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int),
                ("dv", ctypes.c_int), ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
                ("q", _P), ("k", _P), ("v", _P), ("conv_w", _P), ("g", _P), ("beta", _P),
                ("gate", _P), ("S", _P), ("conv_state", _P), ("o", _P), ("accept", _P),
                ("decay_form", ctypes.c_int), ("A", _P)]


class PrepArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("chunk", ctypes.c_int),
                ("in_dtype", ctypes.c_int), ("q", _P), ("k", _P), ("v", _P), ("conv_w", _P),
                ("g", _P), ("conv_in", _P), ("q_out", _P), ("k_out", _P), ("v_out", _P),
                ("G_out", _P), ("decay_form", ctypes.c_int), ("A", _P)]


class CpComposeArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("R", ctypes.c_int), ("H", ctypes.c_int), ("d", ctypes.c_int),
                ("N", _P), ("P", _P), ("S0", _P), ("S_start", _P), ("S_T", _P)]


class PrefillCpArgs(ctypes.Structure):
    _fields_ = [("prefill", PrefillArgs), ("segments", ctypes.c_int), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t)]


class PrefillBackwardArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int),
                ("dv", ctypes.c_int), ("in_dtype", ctypes.c_int), ("q", _P), ("k", _P), ("v", _P),
                ("conv_w", _P), ("g", _P), ("beta", _P), ("gate", _P), ("S0", _P), ("conv_in", _P),
                ("grad_o", _P), ("grad_S_T", _P), ("grad_conv_out", _P), ("grad_q", _P), ("grad_k", _P),
                ("grad_v", _P),
                ("grad_g", _P), ("grad_beta", _P), ("grad_gate", _P), ("grad_S0", _P), ("grad_conv_in", _P),
                ("workspace", _P), ("workspace_bytes", ctypes.c_size_t), ("decay_form", ctypes.c_int),
                ("A", _P)]


_lib = None


def lib():
    """The loaded libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: run `python -m gated_delta_rule_28_amd.build`")
        L = ctypes.CDLL(library_path)
        L.kda_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _P]
        L.kda_prefill.restype = ctypes.c_int
        L.kda_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
        L.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.kda_prefill_workspace_min_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
        L.kda_prefill_workspace_min_bytes.restype = ctypes.c_size_t
        L.kda_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _P]
        L.kda_decode_step.restype = ctypes.c_int
        L.kda_decode_multi.argtypes = [ctypes.POINTER(DecodeMultiArgs), _P]
        L.kda_decode_multi.restype = ctypes.c_int
        L.kda_prep.argtypes = [ctypes.POINTER(PrepArgs), _P]
        L.kda_prep.restype = ctypes.c_int
        L.kda_cp_compose.argtypes = [ctypes.POINTER(CpComposeArgs), _P]
        L.kda_cp_compose.restype = ctypes.c_int
        L.kda_prefill_cp.argtypes = [ctypes.POINTER(PrefillCpArgs), _P]
        L.kda_prefill_cp.restype = ctypes.c_int
        L.kda_prefill_cp_workspace_bytes.argtypes = [ctypes.POINTER(PrefillCpArgs)]
        L.kda_prefill_cp_workspace_bytes.restype = ctypes.c_size_t
        L.kda_cp_fragments.argtypes = [ctypes.POINTER(PrefillArgs), _P, _P, _P]
        L.kda_cp_fragments.restype = ctypes.c_int
        L.kda_cp_finish.argtypes = [ctypes.POINTER(PrefillArgs), _P]
        L.kda_cp_finish.restype = ctypes.c_int
        L.kda_cp_rank_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
        L.kda_cp_rank_workspace_bytes.restype = ctypes.c_size_t
        L.kda_prefill_backward.argtypes = [ctypes.POINTER(PrefillBackwardArgs), _P]
        L.kda_prefill_backward.restype = ctypes.c_int
        L.kda_prefill_backward_workspace_bytes.argtypes = [ctypes.POINTER(PrefillBackwardArgs)]
        L.kda_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_last_error.restype = ctypes.c_char_p
        L.kda_abi_version.restype = ctypes.c_int
        L.kda_release.restype = ctypes.c_int
        L.kda_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint)]
        L.kda_wait_timeouts.restype = ctypes.c_int
        L.kda_debug_pipeline.argtypes = [ctypes.c_uint, ctypes.c_int]
        L.kda_debug_pipeline.restype = ctypes.c_int
        L.kda_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), _P]
        L.kda_prefill_noalloc.restype = ctypes.c_int
        if L.kda_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libkda ABI {L.kda_abi_version()} != binding ABI {ABI_VERSION}")
        _lib = L
    return _lib


def _check(fn, rc):
    if rc != 0:
        L = lib()
        raise KDAError(fn, rc, f"{L.kda_status_string(rc).decode()} ({L.kda_last_error().decode()})")


def release():
    """kda_release: destroy the streams and events the library keeps between
    calls (all devices and threads; call with no library call in flight)."""
    _check("kda_release", lib().kda_release())


def wait_timeouts():
    """kda_wait_timeouts: the bounded in-kernel waits of pipelined prefill
    calls that expired on the current device since the library was loaded
    (each stopped workgroup was finished by the call's second launch).  Waits
    for the device's work to finish."""
    n = ctypes.c_uint(0)
    _check("kda_wait_timeouts", lib().kda_wait_timeouts(ctypes.byref(n)))
    return n.value


def debug_pipeline(wait_limit_us=0, withhold_slab=-1):
    """kda_debug_pipeline: test aid for the stop-and-resume path of pipelined
    prefill (defaults restore normal operation)."""
    _check("kda_debug_pipeline", lib().kda_debug_pipeline(wait_limit_us, withhold_slab))


def _torch():
    import torch
    return torch


def _dt(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _decay(A):
    """(decay_form, A pointer): K3's logits when A is given, else g and beta themselves."""
    return (KDA_DECAY_DIRECT, None) if A is None else (KDA_DECAY_K3, _ptr(A))


def _stream(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def prefill(q, k, v, conv_w, g, beta, gate, S0=None, conv_in=None, chunk=64, out_dtype=None,
            o=None, S_T=None, conv_out=None, want_state=True, want_conv=True, workspace="auto", A=None):
    """Chunkwise KDA prefill (kda_prefill).  Shapes as in include/kda.h.

    Returns (o, S_T, conv_out); S_T / conv_out are None when not wanted.
    Passing S_T=S0 / conv_out=conv_in updates the carry in place.
    workspace: "auto" allocates what kda_prefill_workspace_bytes asks for (the
    two-kernel path where the sizes have one), None passes no workspace (the
    single-kernel path), a uint8 device tensor to use, or "noalloc": call
    kda_prefill_noalloc, whose workspace is the library's own device scratch
    (pass o / S_T / conv_out as well for a call that allocates nothing).
    """
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_out is None and want_conv:
        conv_out = torch.empty((B, 3, H * (2 * dk + dv)), dtype=q.dtype, device=dev)
    a = PrefillArgs(B, T, H, dk, dv, chunk, _dt(q), _dt(o), _ptr(q), _ptr(k), _ptr(v),
                    _ptr(conv_w), _ptr(g), _ptr(beta), _ptr(gate), _ptr(S0), _ptr(conv_in),
                    _ptr(o), _ptr(S_T), _ptr(conv_out), None, 0, *_decay(A))
    if isinstance(workspace, str) and workspace == "noalloc":
        _check("kda_prefill_noalloc", lib().kda_prefill_noalloc(ctypes.byref(a), _stream(dev)))
        return o, S_T, conv_out
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', 'noalloc', None or a uint8 tensor")
        nbytes = lib().kda_prefill_workspace_bytes(ctypes.byref(a))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    if workspace is not None:
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check("kda_prefill", lib().kda_prefill(ctypes.byref(a), _stream(dev)))
    return o, S_T, conv_out


def workspace_bytes(B, T, H, dk, dv, chunk=64, in_dtype=KDA_BF16, out_dtype=KDA_F32, minimum=False):
    """kda_prefill_workspace_bytes (or _min_bytes) for these sizes (0: no two-kernel path)."""
    a = PrefillArgs(B, T, H, dk, dv, chunk, in_dtype, out_dtype)
    fn = lib().kda_prefill_workspace_min_bytes if minimum else lib().kda_prefill_workspace_bytes
    return int(fn(ctypes.byref(a)))


def decode_step(q, k, v, conv_w, g, beta, gate, S, conv_state, o=None, out_dtype=None, A=None):
    """One KDA decode step (kda_decode_step); S and conv_state are updated in place."""
    torch = _torch()
    N, H, dk = q.shape
    dv = v.shape[-1]
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=q.device)
    a = DecodeArgs(N, H, dk, dv, _dt(q), _dt(o), _ptr(q), _ptr(k), _ptr(v), _ptr(conv_w),
                   _ptr(g), _ptr(beta), _ptr(gate), _ptr(S), _ptr(conv_state), _ptr(o), *_decay(A))
    _check("kda_decode_step", lib().kda_decode_step(ctypes.byref(a), _stream(q.device)))
    return o


def decode_multi(q, k, v, conv_w, g, beta, gate, S, conv_state, o=None, out_dtype=None, accept=None,
                 A=None):
    """M tokens per sequence in one call (kda_decode_multi): inputs [N, M, H, .].

    Returns o [N, M, H, dv] for every token.  S and conv_state are updated in place
    to the state after the first accept[n] tokens (accept: int32 [N] device tensor,
    or None for all M)."""
    torch = _torch()
    N, M, H, dk = q.shape
    dv = v.shape[-1]
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, M, H, dv), dtype=out_dtype, device=q.device)
    if accept is not None and accept.dtype != torch.int32:
        raise TypeError("accept must be an int32 tensor")
    a = DecodeMultiArgs(N, M, H, dk, dv, _dt(q), _dt(o), _ptr(q), _ptr(k), _ptr(v), _ptr(conv_w),
                        _ptr(g), _ptr(beta), _ptr(gate), _ptr(S), _ptr(conv_state), _ptr(o),
                        _ptr(accept), *_decay(A))
    _check("kda_decode_multi", lib().kda_decode_multi(ctypes.byref(a), _stream(q.device)))
    return o


def prep(q, k, v, conv_w, g, conv_in=None, chunk=64, A=None):
    """Stage 1 on its own (kda_prep): returns fp32 (q^, k^, v^, G)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    f = dict(dtype=torch.float32, device=q.device)
    qo, ko, vo = torch.empty((B, T, H, dk), **f), torch.empty((B, T, H, dk), **f), torch.empty((B, T, H, dv), **f)
    Go = torch.empty((B, T, H, dk), **f)
    a = PrepArgs(B, T, H, dk, dv, chunk, _dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(conv_w), _ptr(g),
                 _ptr(conv_in), _ptr(qo), _ptr(ko), _ptr(vo), _ptr(Go), *_decay(A))
    _check("kda_prep", lib().kda_prep(ctypes.byref(a), _stream(q.device)))
    return qo, ko, vo, Go


def prefill_cp(q, k, v, conv_w, g, beta, gate, segments, S0=None, conv_in=None, chunk=64, out_dtype=None,
               o=None, S_T=None, conv_out=None, want_state=True, want_conv=True, workspace=None, A=None):
    """Context-parallel prefill on one device (kda_prefill_cp): the results of
    `prefill`, computed from `segments` equal segments per sequence, each formed
    from S = 0 and S = I, composed, and run again from its entering state.
    workspace: None allocates kda_prefill_cp_workspace_bytes, or a uint8 tensor."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_out is None and want_conv:
        conv_out = torch.empty((B, 3, H * (2 * dk + dv)), dtype=q.dtype, device=dev)
    pa = PrefillArgs(B, T, H, dk, dv, chunk, _dt(q), _dt(o), _ptr(q), _ptr(k), _ptr(v),
                     _ptr(conv_w), _ptr(g), _ptr(beta), _ptr(gate), _ptr(S0), _ptr(conv_in),
                     _ptr(o), _ptr(S_T), _ptr(conv_out), None, 0, *_decay(A))
    a = PrefillCpArgs(pa, int(segments), None, 0)
    if workspace is None:
        nbytes = lib().kda_prefill_cp_workspace_bytes(ctypes.byref(a))
        if nbytes == 0 and T > 0:
            raise ValueError(f"no context-parallel split of T={T} into {segments} segments for these sizes")
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check("kda_prefill_cp", lib().kda_prefill_cp(ctypes.byref(a), _stream(dev)))
    return o, S_T, conv_out


def cp_workspace_bytes(B, T, H, dk, dv, segments, chunk=64, in_dtype=KDA_BF16, out_dtype=KDA_F32):
    """kda_prefill_cp_workspace_bytes for these sizes (0: invalid)."""
    a = PrefillCpArgs(PrefillArgs(B, T, H, dk, dv, chunk, in_dtype, out_dtype), int(segments), None, 0)
    return int(lib().kda_prefill_cp_workspace_bytes(ctypes.byref(a)))


def cp_compose(N, P, S0=None, B=1, S_start=None, S_T=None, want_state=True):
    """Prefix composition of segment fragments (kda_cp_compose).  N, P: fp32
    [B*R, H, d, d] final states of each segment from S = 0 and from S = I;
    S0 [B, H, d, d] or None.  Returns (S_start [B*R, H, d, d], S_T [B, H, d, d])."""
    torch = _torch()
    BR, H, d, _ = N.shape
    if BR % B:
        raise ValueError("N's first dimension must be B * R")
    if S_start is None:
        S_start = torch.empty_like(N)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, d, d), dtype=torch.float32, device=N.device)
    a = CpComposeArgs(B, BR // B, H, d, _ptr(N), _ptr(P), _ptr(S0), _ptr(S_start), _ptr(S_T))
    _check("kda_cp_compose", lib().kda_cp_compose(ctypes.byref(a), _stream(N.device)))
    return S_start, S_T


def cp_rank_workspace_bytes(B, T, H, dk, dv, chunk=64, in_dtype=KDA_BF16, out_dtype=KDA_F32):
    """kda_cp_rank_workspace_bytes for these sizes (0: invalid)."""
    a = PrefillArgs(B, T, H, dk, dv, chunk, in_dtype, out_dtype)
    return int(lib().kda_cp_rank_workspace_bytes(ctypes.byref(a)))


def _rank_args(q, k, v, conv_w, g, beta, gate, S0, conv_in, chunk, o, S_T, conv_out, workspace, A):
    B, T, H, dk = q.shape
    a = PrefillArgs(B, T, H, dk, v.shape[-1], chunk, _dt(q), _dt(o), _ptr(q), _ptr(k), _ptr(v),
                    _ptr(conv_w), _ptr(g), _ptr(beta), _ptr(gate), _ptr(S0), _ptr(conv_in),
                    _ptr(o), _ptr(S_T), _ptr(conv_out), _ptr(workspace),
                    workspace.numel() * workspace.element_size(), *_decay(A))
    return a


def cp_fragments(q, k, v, conv_w, g, beta, gate, conv_in=None, chunk=64, N=None, P=None, workspace=None,
                 o=None, out_dtype=None, A=None):
    """One rank's segment, part 1 (kda_cp_fragments): its final states from
    S = 0 (N) and from S = I (P), fp32 [B, H, dk, dv].  conv_in: the three raw
    tokens before the segment.  Returns (workspace, N, P); pass the workspace
    unchanged to cp_finish.  o (the [B, T, H, dv] output buffer cp_finish will
    fill) serves as scratch on sizes without the two-kernel path."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32 if out_dtype is None else out_dtype, device=dev)
    if workspace is None:
        nbytes = cp_rank_workspace_bytes(B, T, H, dk, dv, chunk, _dt(q), _dt(o))
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    if N is None:
        N = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if P is None:
        P = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    a = _rank_args(q, k, v, conv_w, g, beta, gate, None, conv_in, chunk, o, None, None, workspace, A)
    _check("kda_cp_fragments", lib().kda_cp_fragments(ctypes.byref(a), _ptr(N), _ptr(P), _stream(dev)))
    return workspace, N, P


def cp_finish(workspace, q, k, v, conv_w, g, beta, gate, S_start, conv_in=None, chunk=64, o=None,
              S_T=None, conv_out=None, want_state=True, want_conv=True, out_dtype=None, A=None):
    """One rank's segment, part 2 (kda_cp_finish): the segment from its
    entering state S_start with the workspace of cp_fragments and the same
    inputs.  Returns (o, S_T, conv_out) as prefill."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32 if out_dtype is None else out_dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_out is None and want_conv:
        conv_out = torch.empty((B, 3, H * (2 * dk + dv)), dtype=q.dtype, device=dev)
    a = _rank_args(q, k, v, conv_w, g, beta, gate, S_start, conv_in, chunk, o, S_T, conv_out, workspace, A)
    _check("kda_cp_finish", lib().kda_cp_finish(ctypes.byref(a), _stream(dev)))
    return o, S_T, conv_out


def backward_workspace_bytes(B, T, H, dk, dv, in_dtype=KDA_BF16):
    """kda_prefill_backward_workspace_bytes for these sizes (0: invalid)."""
    a = PrefillBackwardArgs(B, T, H, dk, dv, in_dtype)
    return int(lib().kda_prefill_backward_workspace_bytes(ctypes.byref(a)))


def prefill_backward(q, k, v, conv_w, g, beta, gate, grad_o, S0=None, conv_in=None, grad_S_T=None,
                     grad_conv_out=None, want_state_grad=True, want_conv_grad=True, workspace=None):
    """Gradients of <grad_o, o> + <grad_S_T, S_T> + <grad_conv_out, conv_out> of
    `prefill` (kda_prefill_backward).
    Returns a dict of fp32 tensors: q, k, v, g, beta, gate (the inputs' shapes),
    S0 [B,H,dk,dv] and conv_in [B,3,Cch] (None when not wanted)."""
    torch = _torch()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    f = dict(dtype=torch.float32, device=dev)
    out = {x: torch.empty(t.shape, **f) for x, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                                                     ("gate", gate))}
    out["S0"] = torch.empty((B, H, dk, dv), **f) if want_state_grad else None
    out["conv_in"] = torch.empty((B, 3, H * (2 * dk + dv)), **f) if want_conv_grad else None
    a = PrefillBackwardArgs(B, T, H, dk, dv, _dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(conv_w), _ptr(g),
                            _ptr(beta), _ptr(gate), _ptr(S0), _ptr(conv_in), _ptr(grad_o), _ptr(grad_S_T),
                            _ptr(grad_conv_out), _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["g"]),
                            _ptr(out["beta"]), _ptr(out["gate"]), _ptr(out["S0"]), _ptr(out["conv_in"]), None, 0,
                            KDA_DECAY_DIRECT, None)
    if workspace is None:
        workspace = torch.empty(max(int(lib().kda_prefill_backward_workspace_bytes(ctypes.byref(a))), 16),
                                dtype=torch.uint8, device=dev)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check("kda_prefill_backward", lib().kda_prefill_backward(ctypes.byref(a), _stream(dev)))
    return out
