"""MI355X (gfx950) gated delta-rule / Kimi Delta Attention library: Python binding.

A thin ctypes layer over ``libkda.so`` (the C ABI in ``include/kda.h``): every
function has the C entry point's name, checks tensor shapes and dtypes, and
passes device pointers and the current HIP stream.  All computation happens
in the library's HIP kernels; PyTorch only supplies device memory and streams.
If the library is missing the calls raise; there is no fallback.

Build the library first:  ``python -m gated_delta_rule_08_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KdaError", "load_library", "kda_abi_version", "kda_chunk_fwd", "kda_chunk_fwd_supported",
    "kda_chunk_fwd_workspace_bytes", "kda_decode_step", "kda_state_init", "kda_state_load",
    "kda_state_store", "KDA_READ_INITIAL_STATE", "KDA_WRITE_FINAL_STATE", "kda_chunk_fwd_raw",
    "kda_decode_step_raw", "kda_state_affine", "kda_chunk_bwd",
    "kda_chunk_bwd_raw", "launch_timer", "KDA_LAUNCH_TIMER_MAX", "kda_chunk_fwd_noalloc",
    "KDA_NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK = 0
KDA_FP32, KDA_BF16 = 0, 1
KDA_READ_INITIAL_STATE = 1
KDA_WRITE_FINAL_STATE = 2
KDA_GATE_SCALAR = 4
KDA_GATE_NONE = 8
KDA_ADDITIVE = 16
KDA_LAUNCH_TIMER_MAX = 16
KDA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_WORKSPACE_TOO_SMALL", 4: "KDA_ERR_HIP"}


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32)]


_lib = None


def load_library(path: str | None = None):
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_delta_rule_08_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, U32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    SH = ctypes.POINTER(_Shape)
    lib.kda_abi_version.restype = I32
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_supported.argtypes = [I32, I32, I32, I32]
    lib.kda_chunk_fwd_supported.restype = I32
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [SH, I32, I32, I32]
    lib.kda_chunk_fwd_workspace_bytes.restype = SZ
    lib.kda_chunk_fwd.argtypes = [SH, I32, I32, I32, P, P, P, P, P, P, P, I32, P, U32, P, P, SZ, P]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [SH, I32, I32, I32, P, P, P, P, P, P, P, I32, P, U32, P,
                                          P]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [SH, I32, P, P, P, P, P, P, I32, P, P, P]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step_ex.argtypes = [SH, I32, P, P, P, P, P, P, I32, P, U32, P, P]
    lib.kda_decode_step_ex.restype = ctypes.c_int
    F32 = ctypes.c_float
    lib.kda_chunk_fwd_raw.argtypes = [SH, I32, I32, I32, P, P, P, P, P, P, F32, P, I32, P, U32, P,
                                      P, SZ, P]
    lib.kda_chunk_fwd_raw.restype = ctypes.c_int
    lib.kda_decode_step_raw.argtypes = [SH, I32, P, P, P, P, P, F32, P, I32, P, U32, P, P]
    lib.kda_decode_step_raw.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [SH, I32, I32, I32]
    lib.kda_chunk_bwd_workspace_bytes.restype = SZ
    lib.kda_chunk_bwd.argtypes = [SH, I32, I32, I32, P, P, P, P, P, P, P, I32, P, U32, P, P, P, P,
                                  P, P, P, P, P, SZ, P]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd_raw_workspace_bytes.argtypes = [SH, I32, I32, I32]
    lib.kda_chunk_bwd_raw_workspace_bytes.restype = SZ
    lib.kda_chunk_bwd_raw.argtypes = [SH, I32, I32, I32, P, P, P, P, P, P, ctypes.c_float, P, I32,
                                      P, U32, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.kda_chunk_bwd_raw.restype = ctypes.c_int
    lib.kda_state_affine.argtypes = [SH, I32, P, P, P, P, P]
    lib.kda_state_affine.restype = ctypes.c_int
    lib.kda_state_init.argtypes = [SH, P, I32, P]
    lib.kda_state_init.restype = ctypes.c_int
    lib.kda_state_load.argtypes = [SH, P, I32, P, I32, P, P]
    lib.kda_state_load.restype = ctypes.c_int
    lib.kda_state_store.argtypes = [SH, P, I32, P, I32, P, P]
    lib.kda_state_store.restype = ctypes.c_int
    lib.kda_launch_timer_begin.argtypes = [P]
    lib.kda_launch_timer_begin.restype = ctypes.c_int
    lib.kda_launch_timer_end.argtypes = [ctypes.POINTER(ctypes.c_float),
                                         ctypes.POINTER(ctypes.c_char_p), I32,
                                         ctypes.POINTER(ctypes.c_int32)]
    lib.kda_launch_timer_end.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != KDA_OK:
        raise KdaError(status, load_library().kda_last_error().decode())


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_FP32
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


GATES = ("channel", "scalar", "none")


def _variant_flags(gate: str, additive: bool) -> int:
    if gate not in GATES:
        raise ValueError(f"gate must be one of {GATES}, got {gate!r}")
    return ({"channel": 0, "scalar": KDA_GATE_SCALAR, "none": KDA_GATE_NONE}[gate]
            | (KDA_ADDITIVE if additive else 0))


def _need_gate_beta(g, beta, lead, dk, gate, additive):
    """g and beta as the variant reads them (see the flags in include/kda.h)."""
    if gate == "channel":
        _need(g, "g", lead + (dk,), torch.float32)
    elif gate == "scalar":
        _need(g, "g", lead, torch.float32)
    elif g is not None:
        raise ValueError("gate='none' reads no g: pass g=None")
    if not additive:
        _need(beta, "beta", lead, torch.float32)
    elif beta is not None:
        raise ValueError("additive=True reads no beta: pass beta=None")


def kda_abi_version() -> int:
    return int(load_library().kda_abi_version())


def kda_chunk_fwd_supported(dk: int, dv: int, chunk: int, io_dtype: torch.dtype) -> bool:
    code = KDA_BF16 if io_dtype == torch.bfloat16 else KDA_FP32
    return bool(load_library().kda_chunk_fwd_supported(dk, dv, chunk, code))


def kda_chunk_fwd_workspace_bytes(num_heads: int, dk: int, dv: int, io_dtype: torch.dtype,
                                  chunk: int, total_tokens: int, num_seqs: int) -> int:
    sh = _Shape(num_heads, dk, dv, KDA_BF16 if io_dtype == torch.bfloat16 else KDA_FP32)
    return int(load_library().kda_chunk_fwd_workspace_bytes(ctypes.byref(sh), chunk,
                                                            total_tokens, num_seqs))


def kda_chunk_bwd_workspace_bytes(num_heads: int, dk: int, dv: int, io_dtype: torch.dtype,
                                  chunk: int, total_tokens: int, num_seqs: int) -> int:
    sh = _Shape(num_heads, dk, dv, KDA_BF16 if io_dtype == torch.bfloat16 else KDA_FP32)
    return int(load_library().kda_chunk_bwd_workspace_bytes(ctypes.byref(sh), chunk,
                                                            total_tokens, num_seqs))


def kda_chunk_bwd_raw_workspace_bytes(num_heads: int, dk: int, dv: int, io_dtype: torch.dtype,
                                      chunk: int, total_tokens: int, num_seqs: int) -> int:
    sh = _Shape(num_heads, dk, dv, KDA_BF16 if io_dtype == torch.bfloat16 else KDA_FP32)
    return int(load_library().kda_chunk_bwd_raw_workspace_bytes(ctypes.byref(sh), chunk,
                                                                total_tokens, num_seqs))


def kda_chunk_fwd(q, k, v, g, beta, cu_seqlens, chunk: int = 64, states=None, state_slots=None,
                  read_initial: bool = False, write_final: bool = False, o=None, workspace=None,
                  stream=None, gate: str = "channel", additive: bool = False):
    """Chunked prefill over packed sequences (see kda_chunk_fwd in include/kda.h).

    q, k: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; cu_seqlens: int32 [N+1] on
    the device; states: fp32 pool [S, H, dk, dv]; state_slots: int32 [N] or None.
    g: [T, H, dk] (gate="channel"), [T, H] (gate="scalar") or None (gate="none").
    additive=True drops the delta correction (u = v) and takes beta=None.
    Returns o [T, H, dv] in the dtype of q.  ``workspace`` (uint8, device) is
    allocated here when not given.
    """
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    io = _io_dtype(q)
    _need(q, "q", (T, H, dk), q.dtype)
    _need(k, "k", (T, H, dk), q.dtype)
    _need(v, "v", (T, H, dv), q.dtype)
    _need_gate_beta(g, beta, (T, H), dk, gate, additive)
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)
    flags = ((KDA_READ_INITIAL_STATE if read_initial else 0)
             | (KDA_WRITE_FINAL_STATE if write_final else 0) | _variant_flags(gate, additive))
    num_slots = 0
    if states is not None:
        _need(states, "states", (states.shape[0], H, dk, dv), torch.float32)
        num_slots = states.shape[0]
    if state_slots is not None:
        _need(state_slots, "state_slots", (N,), torch.int32)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=q.device)
    else:
        _need(o, "o", (T, H, dv), q.dtype)
    sh = _Shape(H, dk, dv, io)
    need = int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(sh), chunk, T, N))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kda_chunk_fwd(ctypes.byref(sh), chunk, T, N, _ptr(cu_seqlens), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(g), _ptr(beta), _ptr(states), num_slots,
                             _ptr(state_slots), flags, _ptr(o), _ptr(workspace), ws_bytes,
                             _stream(stream)))
    return o


def kda_chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, o, chunk: int = 64, states=None,
                          state_slots=None, read_initial: bool = False, write_final: bool = False,
                          stream=None, gate: str = "channel", additive: bool = False):
    """kda_chunk_fwd with the library's own scratch (see kda_chunk_fwd_noalloc in
    include/kda.h): the call allocates no device memory, so the output ``o`` [T, H, dv]
    must be given.  Calls needing more than KDA_NOALLOC_SCRATCH_BYTES of scratch raise
    KDA_ERR_WORKSPACE_TOO_SMALL; calls that overlap on one GPU race on the scratch."""
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    io = _io_dtype(q)
    _need(q, "q", (T, H, dk), q.dtype)
    _need(k, "k", (T, H, dk), q.dtype)
    _need(v, "v", (T, H, dv), q.dtype)
    _need_gate_beta(g, beta, (T, H), dk, gate, additive)
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)
    _need(o, "o", (T, H, dv), q.dtype)
    flags = ((KDA_READ_INITIAL_STATE if read_initial else 0)
             | (KDA_WRITE_FINAL_STATE if write_final else 0) | _variant_flags(gate, additive))
    num_slots = 0
    if states is not None:
        _need(states, "states", (states.shape[0], H, dk, dv), torch.float32)
        num_slots = states.shape[0]
    if state_slots is not None:
        _need(state_slots, "state_slots", (N,), torch.int32)
    sh = _Shape(H, dk, dv, io)
    _check(lib.kda_chunk_fwd_noalloc(ctypes.byref(sh), chunk, T, N, _ptr(cu_seqlens), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(states),
                                     num_slots, _ptr(state_slots), flags, _ptr(o),
                                     _stream(stream)))
    return o


def kda_chunk_bwd(q, k, v, g, beta, cu_seqlens, d_o, chunk: int = 64, states=None,
                  state_slots=None, read_initial: bool = False, d_final=None,
                  want_d_initial: bool = False, workspace=None, stream=None, out=None,
                  gate: str = "channel", additive: bool = False):
    """Gradients through kda_chunk_fwd (see kda_chunk_bwd in include/kda.h).

    Same inputs and variant arguments as the forward call plus d_o [T, H, dv] and,
    optionally, d_final: fp32 [N, H, dk, dv] (dL/dS_final).  Returns a dict with
    dq, dk, dv (dtype of q), dg (fp32, shaped like g; None for gate="none"), dbeta
    (fp32; None when additive) and d_initial (fp32 [N, H, dk, dv], dL/dS0) when
    want_d_initial; ``out`` may hold those tensors already (they are checked and
    overwritten).
    """
    lib = load_library()
    T, H, dk = q.shape
    dv = v.shape[2]
    io = _io_dtype(q)
    for t, name, d in ((q, "q", dk), (k, "k", dk), (v, "v", dv), (d_o, "d_o", dv)):
        _need(t, name, (T, H, d), q.dtype)
    _need_gate_beta(g, beta, (T, H), dk, gate, additive)
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)
    num_slots = 0
    if states is not None:
        _need(states, "states", (states.shape[0], H, dk, dv), torch.float32)
        num_slots = states.shape[0]
    if state_slots is not None:
        _need(state_slots, "state_slots", (N,), torch.int32)
    if d_final is not None:
        _need(d_final, "d_final", (N, H, dk, dv), torch.float32)
    g_shape = {"channel": (T, H, dk), "scalar": (T, H), "none": None}[gate]
    if out is None:
        out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                   dg=None if g_shape is None else torch.empty(g_shape, dtype=torch.float32,
                                                               device=q.device),
                   dbeta=None if additive else torch.empty((T, H), dtype=torch.float32,
                                                           device=q.device))
        out["d_initial"] = (torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
                            if want_d_initial else None)
    else:
        for name, shape, dt in (("dq", (T, H, dk), q.dtype), ("dk", (T, H, dk), q.dtype),
                                ("dv", (T, H, dv), q.dtype), ("dg", g_shape, torch.float32),
                                ("dbeta", None if additive else (T, H), torch.float32)):
            if shape is not None:
                _need(out.get(name), name, shape, dt)
        if out.get("d_initial") is not None:
            _need(out["d_initial"], "d_initial", (N, H, dk, dv), torch.float32)
    sh = _Shape(H, dk, dv, io)
    need = int(lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(sh), chunk, T, N))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = (KDA_READ_INITIAL_STATE if read_initial else 0) | _variant_flags(gate, additive)
    _check(lib.kda_chunk_bwd(ctypes.byref(sh), chunk, T, N, _ptr(cu_seqlens), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(g), _ptr(beta), _ptr(states), num_slots,
                             _ptr(state_slots), flags, _ptr(d_o), _ptr(d_final), _ptr(out["dq"]),
                             _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out.get("dg")),
                             _ptr(out.get("dbeta")), _ptr(out.get("d_initial")), _ptr(workspace),
                             ws_bytes, _stream(stream)))
    return out


def kda_chunk_bwd_raw(q_raw, k_raw, v, gate_logits, beta_logits, cu_seqlens, d_o, chunk: int = 64,
                      gate_min: float = float("-inf"), states=None, state_slots=None,
                      read_initial: bool = False, d_final=None, want_d_initial: bool = False,
                      workspace=None, stream=None, gate: str = "channel", additive: bool = False):
    """Gradients through kda_chunk_fwd_raw (see kda_chunk_bwd_raw in include/kda.h).

    Returns a dict with dq_raw, dk_raw, dv, dgate_logits (None for gate="none"),
    dbeta_logits (None when additive), all bf16, and d_initial (fp32) when
    want_d_initial.
    """
    lib = load_library()
    T, H, dk = q_raw.shape
    dv = v.shape[2]
    for t, name, d in ((q_raw, "q_raw", dk), (k_raw, "k_raw", dk), (v, "v", dv), (d_o, "d_o", dv)):
        _need(t, name, (T, H, d), torch.bfloat16)
    _need_raw_gate_beta(gate_logits, beta_logits, (T, H), dk, gate, additive)
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)
    num_slots = 0
    if states is not None:
        _need(states, "states", (states.shape[0], H, dk, dv), torch.float32)
        num_slots = states.shape[0]
    if state_slots is not None:
        _need(state_slots, "state_slots", (N,), torch.int32)
    if d_final is not None:
        _need(d_final, "d_final", (N, H, dk, dv), torch.float32)
    out = dict(dq_raw=torch.empty_like(q_raw), dk_raw=torch.empty_like(k_raw),
               dv=torch.empty_like(v),
               dgate_logits=None if gate == "none" else torch.empty_like(gate_logits),
               dbeta_logits=None if additive else torch.empty_like(beta_logits),
               d_initial=(torch.empty((N, H, dk, dv), dtype=torch.float32, device=v.device)
                          if want_d_initial else None))
    sh = _Shape(H, dk, dv, KDA_BF16)
    need = int(lib.kda_chunk_bwd_raw_workspace_bytes(ctypes.byref(sh), chunk, T, N))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = (KDA_READ_INITIAL_STATE if read_initial else 0) | _variant_flags(gate, additive)
    _check(lib.kda_chunk_bwd_raw(ctypes.byref(sh), chunk, T, N, _ptr(cu_seqlens), _ptr(q_raw),
                                 _ptr(k_raw), _ptr(v), _ptr(gate_logits), _ptr(beta_logits),
                                 float(gate_min), _ptr(states), num_slots, _ptr(state_slots), flags,
                                 _ptr(d_o), _ptr(d_final), _ptr(out["dq_raw"]),
                                 _ptr(out["dk_raw"]), _ptr(out["dv"]), _ptr(out["dgate_logits"]),
                                 _ptr(out["dbeta_logits"]), _ptr(out["d_initial"]),
                                 _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def kda_decode_step(q, k, v, g, beta, states, state_slots=None, o=None, stream=None,
                    gate: str = "channel", additive: bool = False):
    """One token per sequence against resident states, updated in place.

    q, k: [B, H, dk]; v: [B, H, dv]; beta: [B, H]; states: fp32 pool
    [S, H, dk, dv]; state_slots: int32 [B] or None.  g: [B, H, dk]
    (gate="channel"), [B, H] (gate="scalar") or None (gate="none");
    additive=True drops the delta correction and takes beta=None.
    Returns o [B, H, dv].
    """
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[2]
    io = _io_dtype(q)
    _need(q, "q", (B, H, dk), q.dtype)
    _need(k, "k", (B, H, dk), q.dtype)
    _need(v, "v", (B, H, dv), q.dtype)
    _need_gate_beta(g, beta, (B, H), dk, gate, additive)
    _need(states, "states", (states.shape[0], H, dk, dv), torch.float32)
    if state_slots is not None:
        _need(state_slots, "state_slots", (B,), torch.int32)
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    else:
        _need(o, "o", (B, H, dv), q.dtype)
    sh = _Shape(H, dk, dv, io)
    _check(lib.kda_decode_step_ex(ctypes.byref(sh), B, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(states), states.shape[0], _ptr(state_slots),
                                  _variant_flags(gate, additive), _ptr(o), _stream(stream)))
    return o


def _need_raw_gate_beta(gate_logits, beta_logits, lead, dk, gate, additive):
    """bf16 logits as the variant reads them (see kda_chunk_fwd_raw in include/kda.h)."""
    if gate == "channel":
        _need(gate_logits, "gate_logits", lead + (dk,), torch.bfloat16)
    elif gate == "scalar":
        _need(gate_logits, "gate_logits", lead, torch.bfloat16)
    elif gate_logits is not None:
        raise ValueError("gate='none' reads no gate: pass gate_logits=None")
    if not additive:
        _need(beta_logits, "beta_logits", lead, torch.bfloat16)
    elif beta_logits is not None:
        raise ValueError("additive=True reads no beta: pass beta_logits=None")


def kda_chunk_fwd_raw(q_raw, k_raw, v, gate_logits, beta_logits, cu_seqlens, chunk: int = 64,
                      gate_min: float = float("-inf"), states=None, state_slots=None,
                      read_initial: bool = False, write_final: bool = False, o=None,
                      workspace=None, stream=None, gate: str = "channel", additive: bool = False):
    """Prefill from raw bf16 projections with the input preparation fused in
    (see kda_chunk_fwd_raw in include/kda.h): q = normalize(silu(q_raw)),
    k = normalize(silu(k_raw)), beta = sigmoid(beta_logits),
    g = max(log sigmoid(gate_logits), gate_min).  Returns o [T, H, dv] (bf16)."""
    lib = load_library()
    T, H, dk = q_raw.shape
    dv = v.shape[2]
    for t, name, shp in ((q_raw, "q_raw", (T, H, dk)), (k_raw, "k_raw", (T, H, dk)),
                         (v, "v", (T, H, dv))):
        _need(t, name, shp, torch.bfloat16)
    _need_raw_gate_beta(gate_logits, beta_logits, (T, H), dk, gate, additive)
    N = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32)
    flags = ((KDA_READ_INITIAL_STATE if read_initial else 0)
             | (KDA_WRITE_FINAL_STATE if write_final else 0) | _variant_flags(gate, additive))
    num_slots = 0
    if states is not None:
        _need(states, "states", (states.shape[0], H, dk, dv), torch.float32)
        num_slots = states.shape[0]
    if state_slots is not None:
        _need(state_slots, "state_slots", (N,), torch.int32)
    if o is None:
        o = torch.empty((T, H, dv), dtype=torch.bfloat16, device=q_raw.device)
    else:
        _need(o, "o", (T, H, dv), torch.bfloat16)
    sh = _Shape(H, dk, dv, KDA_BF16)
    need = int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(sh), chunk, T, N))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_raw.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.kda_chunk_fwd_raw(ctypes.byref(sh), chunk, T, N, _ptr(cu_seqlens), _ptr(q_raw),
                                 _ptr(k_raw), _ptr(v), _ptr(gate_logits), _ptr(beta_logits),
                                 float(gate_min), _ptr(states), num_slots, _ptr(state_slots),
                                 flags, _ptr(o), _ptr(workspace), ws_bytes, _stream(stream)))
    return o


def kda_decode_step_raw(q_raw, k_raw, v, gate_logits, beta_logits, states, gate_min=float("-inf"),
                        state_slots=None, o=None, stream=None, gate: str = "channel",
                        additive: bool = False):
    """kda_decode_step from raw bf16 projections (see kda_decode_step_raw)."""
    lib = load_library()
    B, H, dk = q_raw.shape
    dv = v.shape[2]
    for t, name, shp in ((q_raw, "q_raw", (B, H, dk)), (k_raw, "k_raw", (B, H, dk)),
                         (v, "v", (B, H, dv))):
        _need(t, name, shp, torch.bfloat16)
    _need_raw_gate_beta(gate_logits, beta_logits, (B, H), dk, gate, additive)
    _need(states, "states", (states.shape[0], H, dk, dv), torch.float32)
    if state_slots is not None:
        _need(state_slots, "state_slots", (B,), torch.int32)
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.bfloat16, device=q_raw.device)
    else:
        _need(o, "o", (B, H, dv), torch.bfloat16)
    sh = _Shape(H, dk, dv, KDA_BF16)
    _check(lib.kda_decode_step_raw(ctypes.byref(sh), B, _ptr(q_raw), _ptr(k_raw), _ptr(v),
                                   _ptr(gate_logits), _ptr(beta_logits), float(gate_min),
                                   _ptr(states), states.shape[0], _ptr(state_slots),
                                   _variant_flags(gate, additive), _ptr(o), _stream(stream)))
    return o


def kda_state_affine(M, S_in, B, out=None, stream=None):
    """out[i] = M[i] @ S_in[i] + B[i] per head (see kda_state_affine in include/kda.h).

    M: fp32 [n, H, dk, dk]; S_in, B: fp32 [n, H, dk, dv].  ``out`` may be B."""
    lib = load_library()
    n, H, dk, dv = S_in.shape
    _need(M, "M", (n, H, dk, dk), torch.float32)
    _need(S_in, "S_in", (n, H, dk, dv), torch.float32)
    _need(B, "B", (n, H, dk, dv), torch.float32)
    if out is None:
        out = torch.empty_like(B)
    else:
        _need(out, "out", (n, H, dk, dv), torch.float32)
    sh = _Shape(H, dk, dv, KDA_FP32)
    _check(lib.kda_state_affine(ctypes.byref(sh), n, _ptr(M), _ptr(S_in), _ptr(B), _ptr(out),
                                _stream(stream)))
    return out


def _pool_shape(states):
    _need(states, "states", tuple(states.shape), torch.float32)
    if states.dim() != 4:
        raise ValueError("states must be [num_slots, H, dk, dv]")
    S, H, dk, dv = states.shape
    return S, _Shape(H, dk, dv, KDA_FP32)


def kda_state_init(states, stream=None):
    """Zero a state pool [num_slots, H, dk, dv]."""
    S, sh = _pool_shape(states)
    _check(load_library().kda_state_init(ctypes.byref(sh), _ptr(states), S, _stream(stream)))
    return states


def kda_state_load(states, src, slots=None, stream=None):
    """Copy dense src [n, H, dk, dv] into pool slots (slots[i], or i)."""
    S, sh = _pool_shape(states)
    n = src.shape[0]
    _need(src, "src", (n,) + tuple(states.shape[1:]), torch.float32)
    if slots is not None:
        _need(slots, "slots", (n,), torch.int32)
    _check(load_library().kda_state_load(ctypes.byref(sh), _ptr(states), S, _ptr(slots), n,
                                         _ptr(src), _stream(stream)))
    return states


def kda_state_store(states, slots=None, n=None, dst=None, stream=None):
    """Copy pool slots (slots[i], or i for i < n) into a dense [n, H, dk, dv] tensor."""
    S, sh = _pool_shape(states)
    if slots is not None:
        n = slots.numel()
        _need(slots, "slots", (n,), torch.int32)
    if n is None:
        n = S
    if dst is None:
        dst = torch.empty((n,) + tuple(states.shape[1:]), dtype=torch.float32, device=states.device)
    else:
        _need(dst, "dst", (n,) + tuple(states.shape[1:]), torch.float32)
    _check(load_library().kda_state_store(ctypes.byref(sh), _ptr(states), S, _ptr(slots), n,
                                          _ptr(dst), _stream(stream)))
    return dst


class launch_timer:
    """Per-launch timing of the library's kernels (kda_launch_timer_begin/end):

        with launch_timer(stream) as lt:
            kda_chunk_fwd(..., stream=stream)
        lt.launches  # [(kernel name, milliseconds), ...] in launch order

    Every library call inside the block must use `stream`; leaving the block
    waits for the last launch."""

    def __init__(self, stream=None):
        self.stream = stream
        self.launches = []

    def __enter__(self):
        _check(load_library().kda_launch_timer_begin(_stream(self.stream)))
        return self

    def __exit__(self, exc_type, exc, tb):
        cap = KDA_LAUNCH_TIMER_MAX
        ms = (ctypes.c_float * cap)()
        names = (ctypes.c_char_p * cap)()
        n = ctypes.c_int32(0)
        st = load_library().kda_launch_timer_end(ms, names, cap, ctypes.byref(n))
        if exc_type is None:
            _check(st)
            self.launches = [(names[i].decode(), float(ms[i])) for i in range(min(n.value, cap))]
        return False
