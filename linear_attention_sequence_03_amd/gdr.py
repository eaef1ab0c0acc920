"""Thin ctypes binding of libgdr.so (argument marshalling only).

Every computation happens in the HIP kernels behind the C ABI of
``include/gdr.h``; this module checks tensor dtypes/devices, allocates outputs
and the workspace with torch (device memory), passes raw pointers and the
current HIP stream, and turns error codes into exceptions.  There is no CPU
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libgdr.so")

GDR_OK, GDR_ERR_INVALID_ARG, GDR_ERR_UNSUPPORTED, GDR_ERR_HIP = 0, 1, 2, 3
GDR_F32, GDR_BF16 = 0, 1
GDR_GATE_SCALAR, GDR_GATE_CHANNEL = 0, 1
GDR_PROLOGUE_L2NORM_QK, GDR_PROLOGUE_BETA_SIGMOID, GDR_PROLOGUE_DECAY_SOFTPLUS = 1, 2, 4
GDR_NOALLOC_SCRATCH_BYTES = 64 << 20   # the fixed scratch of gdr_chunk_fwd_noalloc

# Every symbol include/gdr.h declares.
EXPORTS = ("gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd", "gdr_chunk_fwd_noalloc",
           "gdr_decode_step", "gdr_decode_multi", "gdr_decode_tree", "gdr_decode_tree_commit",
           "gdr_chunk_fwd_prologue", "gdr_chunk_fwd_prologue_workspace_size", "gdr_decode_step_prologue",
           "gdr_fg2_chunk_fwd_workspace_size", "gdr_fg2_chunk_fwd", "gdr_fg2_decode_step",
           "gdr_gdn2_fwd", "gdr_gdn2_chunk_fwd_workspace_size", "gdr_gdn2_chunk_fwd",
           "gdr_status_string", "gdr_last_error")

_lib = None


class GdrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: Optional[str] = None):
    """Load libgdr.so (built in-tree by ``build.py``).  Raises if it is absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIBRARY_PATH
    if not os.path.exists(p):
        raise ImportError("libgdr.so not built (%s); run "
                          "`python -m linear_attention_sequence_03_amd.build`" % p)
    lib = ctypes.CDLL(p)
    vp, i64, f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.gdr_status_string.argtypes = [f]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, f, f,
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_fwd_workspace_size.restype = f
    lib.gdr_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                  i64, i64, i64, i64, i64, i64, f, f,
                                  vp, ctypes.c_size_t, vp]
    lib.gdr_chunk_fwd.restype = f
    lib.gdr_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                          i64, i64, i64, i64, i64, i64, f, f, vp]
    lib.gdr_chunk_fwd_noalloc.restype = f
    lib.gdr_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                    i64, i64, i64, i64, f, f, vp]
    lib.gdr_decode_step.restype = f
    lib.gdr_chunk_fwd_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                           i64, i64, i64, i64, i64, i64, f, f,
                                           vp, ctypes.c_size_t, ctypes.c_uint, vp]
    lib.gdr_chunk_fwd_prologue.restype = f
    lib.gdr_chunk_fwd_prologue_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, f, f,
                                                          ctypes.c_uint, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_fwd_prologue_workspace_size.restype = f
    lib.gdr_decode_step_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp,
                                             i64, i64, i64, i64, f, f, ctypes.c_uint, vp]
    lib.gdr_decode_step_prologue.restype = f
    lib.gdr_gdn2_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 i64, i64, i64, i64, i64, f, f, vp]
    lib.gdr_gdn2_fwd.restype = f
    lib.gdr_gdn2_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, f, f,
                                                      ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_gdn2_chunk_fwd_workspace_size.restype = f
    lib.gdr_gdn2_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       i64, i64, i64, i64, i64, i64, f, f,
                                       vp, ctypes.c_size_t, vp]
    lib.gdr_gdn2_chunk_fwd.restype = f
    lib.gdr_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     i64, i64, i64, i64, i64, f, f, vp]
    lib.gdr_decode_multi.restype = f
    lib.gdr_decode_tree.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    i64, i64, i64, i64, i64, f, f, vp]
    lib.gdr_decode_tree.restype = f
    lib.gdr_decode_tree_commit.argtypes = [vp, vp, vp, vp, vp, vp, vp,
                                           i64, i64, i64, i64, i64, f, f, vp]
    lib.gdr_decode_tree_commit.restype = f
    lib.gdr_fg2_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, f, f,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_fg2_chunk_fwd_workspace_size.restype = f
    lib.gdr_fg2_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      i64, i64, i64, i64, i64, i64, f, f,
                                      vp, ctypes.c_size_t, vp]
    lib.gdr_fg2_chunk_fwd.restype = f
    lib.gdr_fg2_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        i64, i64, i64, i64, f, f, vp]
    lib.gdr_fg2_decode_step.restype = f
    if path is None:
        _lib = lib
    return lib


def gdr_status_string(status: int) -> str:
    return load_library().gdr_status_string(int(status)).decode()


def _raise(status: int):
    lib = load_library()
    detail = lib.gdr_last_error().decode()
    raise GdrError(status, "%s: %s" % (lib.gdr_status_string(status).decode(), detail))


def _io_code(dtype) -> int:
    import torch
    if dtype == torch.float32:
        return GDR_F32
    if dtype == torch.bfloat16:
        return GDR_BF16
    raise TypeError("q/k/v must be float32 or bfloat16, got %s" % dtype)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(name, t, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.device != device:
        raise ValueError("%s: on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device, stream):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def gdr_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().gdr_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate,
                                                     ctypes.byref(out))
    if st != GDR_OK:
        _raise(st)
    return int(out.value)


def gdr_chunk_fwd_prologue_workspace_size(B, T, H, dk, dv, chunk, io, gate, flags) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().gdr_chunk_fwd_prologue_workspace_size(B, T, H, dk, dv, chunk, io, gate,
                                                              int(flags), ctypes.byref(out))
    if st != GDR_OK:
        _raise(st)
    return int(out.value)


def _chunk_io(q, k, v, log_alpha, beta, S0, o, S_T, want_state):
    """Check the prefill tensors; allocate o and S_T when not given."""
    import torch
    dev = q.device
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 4 else GDR_GATE_SCALAR
    _need("q", q, q.dtype, (B, T, H, dk), dev)
    _need("k", k, q.dtype, (B, T, H, dk), dev)
    _need("v", v, q.dtype, (B, T, H, dv), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, T, H, dk) if gate == GDR_GATE_CHANNEL else (B, T, H), dev)
    _need("beta", beta, torch.float32, (B, T, H), dev)
    if S0 is not None:
        _need("S0", S0, torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _need("o", o, q.dtype, (B, T, H, dv), dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if S_T is not None:
        _need("S_T", S_T, torch.float32, (B, H, dv, dk), dev)
    return (B, T, H, dk, dv, _io_code(q.dtype), gate), o, S_T


def gdr_chunk_fwd(q, k, v, log_alpha, beta, S0=None, chunk: int = 64, o=None, S_T=None,
                  workspace=None, want_state: bool = True, stream=None, prologue: int = 0) -> Tuple:
    """Whole-sequence forward.  q,k: [B,T,H,dk]; v: [B,T,H,dv] (fp32 or bf16);
    log_alpha: [B,T,H] (scalar gate) or [B,T,H,dk] (channel gate), fp32;
    beta: [B,T,H] fp32; S0: [B,H,dv,dk] fp32 or None.
    Returns (o [B,T,H,dv] in the io dtype, S_T [B,H,dv,dk] fp32 or None).
    ``prologue`` (GDR_PROLOGUE_* flags) normalises q, k and / or maps beta and
    decay logits inside the library."""
    import torch
    (B, T, H, dk, dv, io, gate), o, S_T = _chunk_io(q, k, v, log_alpha, beta, S0, o, S_T, want_state)
    dev = q.device
    nbytes = gdr_chunk_fwd_prologue_workspace_size(B, T, H, dk, dv, chunk, io, gate, prologue)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if prologue:
        st = load_library().gdr_chunk_fwd_prologue(
            _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T),
            B, T, H, dk, dv, chunk, io, gate, _ptr(workspace), wbytes, int(prologue),
            _stream(dev, stream))
    else:
        st = load_library().gdr_chunk_fwd(
            _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T),
            B, T, H, dk, dv, chunk, io, gate, _ptr(workspace), wbytes, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return o, S_T


def gdr_chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0=None, chunk: int = 64, o=None, S_T=None,
                          want_state: bool = True, stream=None) -> Tuple:
    """:func:`gdr_chunk_fwd` with the library's fixed device scratch in place of
    a workspace (at most GDR_NOALLOC_SCRATCH_BYTES of it).  Pass ``o`` (and
    ``S_T``) to keep this call free of allocations too; calls that overlap on
    one GPU race on the shared scratch."""
    (B, T, H, dk, dv, io, gate), o, S_T = _chunk_io(q, k, v, log_alpha, beta, S0, o, S_T, want_state)
    st = load_library().gdr_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S_T),
        B, T, H, dk, dv, chunk, io, gate, _stream(q.device, stream))
    if st != GDR_OK:
        _raise(st)
    return o, S_T


def gdr_decode_step(q, k, v, log_alpha, beta, S, S_out=None, o=None, inplace: bool = False,
                    stream=None, prologue: int = 0) -> Tuple:
    """One decode step.  q,k: [B,H,dk]; v: [B,H,dv]; log_alpha: [B,H] or [B,H,dk];
    beta: [B,H]; S: [B,H,dv,dk] fp32.  ``inplace=True`` writes the new state into
    S.  Returns (o [B,H,dv], S_out)."""
    import torch
    dev = q.device
    B, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_code(q.dtype)
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 3 else GDR_GATE_SCALAR
    _need("q", q, q.dtype, (B, H, dk), dev)
    _need("k", k, q.dtype, (B, H, dk), dev)
    _need("v", v, q.dtype, (B, H, dv), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, H, dk) if gate == GDR_GATE_CHANNEL else (B, H), dev)
    _need("beta", beta, torch.float32, (B, H), dev)
    _need("S", S, torch.float32, (B, H, dv, dk), dev)
    if inplace:
        S_out = S
    elif S_out is None:
        S_out = torch.empty_like(S)
    _need("S_out", S_out, torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    _need("o", o, q.dtype, (B, H, dv), dev)
    if prologue:
        st = load_library().gdr_decode_step_prologue(
            _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(S_out), _ptr(o),
            B, H, dk, dv, io, gate, int(prologue), _stream(dev, stream))
    else:
        st = load_library().gdr_decode_step(
            _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(S_out), _ptr(o),
            B, H, dk, dv, io, gate, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return o, S_out


def gdr_fg2_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().gdr_fg2_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate,
                                                         ctypes.byref(out))
    if st != GDR_OK:
        _raise(st)
    return int(out.value)


def gdr_fg2_chunk_fwd(q, k, v, log_alpha, beta_k, beta_v=None, S0=None, chunk: int = 64, o=None,
                      S_T=None, workspace=None, want_state: bool = True, stream=None) -> Tuple:
    """Whole-sequence forward with channel-wise write rates (FG2-GDN; FG2-GDN+
    when ``beta_v`` is given).  beta_k: [B,T,H,dk] fp32; beta_v: [B,T,H,dv] fp32 or
    None (= beta_k).  Other arguments as in :func:`gdr_chunk_fwd`."""
    import torch
    dev = q.device
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_code(q.dtype)
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 4 else GDR_GATE_SCALAR
    _need("q", q, q.dtype, (B, T, H, dk), dev)
    _need("k", k, q.dtype, (B, T, H, dk), dev)
    _need("v", v, q.dtype, (B, T, H, dv), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, T, H, dk) if gate == GDR_GATE_CHANNEL else (B, T, H), dev)
    _need("beta_k", beta_k, torch.float32, (B, T, H, dk), dev)
    if beta_v is not None:
        _need("beta_v", beta_v, torch.float32, (B, T, H, dv), dev)
    if S0 is not None:
        _need("S0", S0, torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _need("o", o, q.dtype, (B, T, H, dv), dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if S_T is not None:
        _need("S_T", S_T, torch.float32, (B, H, dv, dk), dev)
    nbytes = gdr_fg2_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().gdr_fg2_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta_k), _ptr(beta_v), _ptr(S0), _ptr(o),
        _ptr(S_T), B, T, H, dk, dv, chunk, io, gate, _ptr(workspace), wbytes, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return o, S_T


def gdr_fg2_decode_step(q, k, v, log_alpha, beta_k, beta_v, S, S_out=None, o=None,
                        inplace: bool = False, stream=None) -> Tuple:
    """One decode step with channel-wise write rates.  beta_k: [B,H,dk]; beta_v:
    [B,H,dv] or None (= beta_k).  Other arguments as in :func:`gdr_decode_step`."""
    import torch
    dev = q.device
    B, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_code(q.dtype)
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 3 else GDR_GATE_SCALAR
    _need("q", q, q.dtype, (B, H, dk), dev)
    _need("k", k, q.dtype, (B, H, dk), dev)
    _need("v", v, q.dtype, (B, H, dv), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, H, dk) if gate == GDR_GATE_CHANNEL else (B, H), dev)
    _need("beta_k", beta_k, torch.float32, (B, H, dk), dev)
    if beta_v is not None:
        _need("beta_v", beta_v, torch.float32, (B, H, dv), dev)
    _need("S", S, torch.float32, (B, H, dv, dk), dev)
    if inplace:
        S_out = S
    elif S_out is None:
        S_out = torch.empty_like(S)
    _need("S_out", S_out, torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    _need("o", o, q.dtype, (B, H, dv), dev)
    st = load_library().gdr_fg2_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta_k), _ptr(beta_v), _ptr(S),
        _ptr(S_out), _ptr(o), B, H, dk, dv, io, gate, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return o, S_out


def gdr_decode_multi(q, k, v, log_alpha, beta, S, S_out=None, accepted=None, o=None,
                     want_o: bool = True, inplace: bool = False, stream=None) -> Tuple:
    """Td tokens per sequence in one pass over the state.  q,k: [B,Td,H,dk];
    v: [B,Td,H,dv]; log_alpha: [B,Td,H] or [B,Td,H,dk]; beta: [B,Td,H];
    S: [B,H,dv,dk] fp32 (read only unless ``inplace``).  ``S_out`` (or S itself
    with ``inplace=True``) receives the state after ``accepted[b]`` tokens
    (int32 [B] on the device; None = all Td); with neither, no state is
    written.  Returns (o [B,Td,H,dv] or None, S_out or None)."""
    import torch
    dev = q.device
    B, Td, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_code(q.dtype)
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 4 else GDR_GATE_SCALAR
    _need("q", q, q.dtype, (B, Td, H, dk), dev)
    _need("k", k, q.dtype, (B, Td, H, dk), dev)
    _need("v", v, q.dtype, (B, Td, H, dv), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, Td, H, dk) if gate == GDR_GATE_CHANNEL else (B, Td, H), dev)
    _need("beta", beta, torch.float32, (B, Td, H), dev)
    _need("S", S, torch.float32, (B, H, dv, dk), dev)
    if inplace:
        S_out = S
    if S_out is not None:
        _need("S_out", S_out, torch.float32, (B, H, dv, dk), dev)
    if accepted is not None:
        _need("accepted", accepted, torch.int32, (B,), dev)
    if o is None and want_o:
        o = torch.empty((B, Td, H, dv), dtype=q.dtype, device=dev)
    if o is not None:
        _need("o", o, q.dtype, (B, Td, H, dv), dev)
    st = load_library().gdr_decode_multi(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(S_out),
        _ptr(accepted), _ptr(o), B, Td, H, dk, dv, io, gate, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return o, S_out


def gdr_gdn2_fwd(q, k, v, log_alpha, erase, write, S0=None, o=None, S_T=None,
                 want_state: bool = True, stream=None) -> Tuple:
    """Whole-sequence forward with decoupled erase / write gates (Gated
    DeltaNet-2).  erase: [B,T,H,dk] fp32; write: [B,T,H,dv] fp32; other
    arguments as in :func:`gdr_chunk_fwd`.  Returns (o, S_T)."""
    import torch
    dev = q.device
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_code(q.dtype)
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 4 else GDR_GATE_SCALAR
    _need("q", q, q.dtype, (B, T, H, dk), dev)
    _need("k", k, q.dtype, (B, T, H, dk), dev)
    _need("v", v, q.dtype, (B, T, H, dv), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, T, H, dk) if gate == GDR_GATE_CHANNEL else (B, T, H), dev)
    _need("erase", erase, torch.float32, (B, T, H, dk), dev)
    _need("write", write, torch.float32, (B, T, H, dv), dev)
    if S0 is not None:
        _need("S0", S0, torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _need("o", o, q.dtype, (B, T, H, dv), dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if S_T is not None:
        _need("S_T", S_T, torch.float32, (B, H, dv, dk), dev)
    st = load_library().gdr_gdn2_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(erase), _ptr(write), _ptr(S0), _ptr(o),
        _ptr(S_T), B, T, H, dk, dv, io, gate, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return o, S_T


def gdr_gdn2_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().gdr_gdn2_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate,
                                                          ctypes.byref(out))
    if st != GDR_OK:
        _raise(st)
    return int(out.value)


def gdr_gdn2_chunk_fwd(q, k, v, log_alpha, erase, write, S0=None, chunk: int = 64, o=None,
                       S_T=None, workspace=None, want_state: bool = True, stream=None) -> Tuple:
    """Chunkwise form of :func:`gdr_gdn2_fwd` (bf16 io, chunk 64).  The
    workspace is allocated here when not given.  Returns (o, S_T)."""
    import torch
    dev = q.device
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_code(q.dtype)
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 4 else GDR_GATE_SCALAR
    _need("q", q, q.dtype, (B, T, H, dk), dev)
    _need("k", k, q.dtype, (B, T, H, dk), dev)
    _need("v", v, q.dtype, (B, T, H, dv), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, T, H, dk) if gate == GDR_GATE_CHANNEL else (B, T, H), dev)
    _need("erase", erase, torch.float32, (B, T, H, dk), dev)
    _need("write", write, torch.float32, (B, T, H, dv), dev)
    if S0 is not None:
        _need("S0", S0, torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    _need("o", o, q.dtype, (B, T, H, dv), dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    if S_T is not None:
        _need("S_T", S_T, torch.float32, (B, H, dv, dk), dev)
    nbytes = gdr_gdn2_chunk_fwd_workspace_size(B, T, H, dk, dv, chunk, io, gate)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load_library().gdr_gdn2_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(erase), _ptr(write), _ptr(S0), _ptr(o),
        _ptr(S_T), B, T, H, dk, dv, chunk, io, gate, _ptr(workspace), wbytes, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return o, S_T


def gdr_decode_tree(q, k, v, log_alpha, beta, S, parent, o=None, D=None, want_o: bool = True,
                    want_D: bool = True, stream=None) -> Tuple:
    """Verify a tree of draft tokens: q,k: [B,Td,H,dk]; v: [B,Td,H,dv];
    log_alpha: [B,Td,H] or [B,Td,H,dk]; beta: [B,Td,H]; S: [B,H,dv,dk] fp32
    (read only); parent: [B,Td] int32 (-1 or an earlier node).  Returns
    (o [B,Td,H,dv] io dtype, D [B,Td,H,dv] fp32 written values), either None
    when not wanted."""
    import torch
    dev = q.device
    B, Td, H, dk = q.shape
    dv = v.shape[-1]
    io = _io_code(q.dtype)
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 4 else GDR_GATE_SCALAR
    _need("q", q, q.dtype, (B, Td, H, dk), dev)
    _need("k", k, q.dtype, (B, Td, H, dk), dev)
    _need("v", v, q.dtype, (B, Td, H, dv), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, Td, H, dk) if gate == GDR_GATE_CHANNEL else (B, Td, H), dev)
    _need("beta", beta, torch.float32, (B, Td, H), dev)
    _need("S", S, torch.float32, (B, H, dv, dk), dev)
    _need("parent", parent, torch.int32, (B, Td), dev)
    if o is None and want_o:
        o = torch.empty((B, Td, H, dv), dtype=q.dtype, device=dev)
    if o is not None:
        _need("o", o, q.dtype, (B, Td, H, dv), dev)
    if D is None and want_D:
        D = torch.empty((B, Td, H, dv), dtype=torch.float32, device=dev)
    if D is not None:
        _need("D", D, torch.float32, (B, Td, H, dv), dev)
    st = load_library().gdr_decode_tree(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(parent), _ptr(o), _ptr(D),
        B, Td, H, dk, dv, io, gate, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return o, D


def gdr_decode_tree_commit(k, log_alpha, parent, D, accepted, S, S_out=None, inplace: bool = False,
                           stream=None):
    """The state after the accepted node of every sequence (accepted: [B]
    int32; -1 keeps S), from gdr_decode_tree's written values D.
    ``inplace=True`` writes it into S.  Returns S_out."""
    import torch
    dev = k.device
    B, Td, H, dk = k.shape
    dv = D.shape[-1]
    io = _io_code(k.dtype)
    gate = GDR_GATE_CHANNEL if log_alpha.dim() == 4 else GDR_GATE_SCALAR
    _need("k", k, k.dtype, (B, Td, H, dk), dev)
    _need("log_alpha", log_alpha, torch.float32,
          (B, Td, H, dk) if gate == GDR_GATE_CHANNEL else (B, Td, H), dev)
    _need("parent", parent, torch.int32, (B, Td), dev)
    _need("D", D, torch.float32, (B, Td, H, dv), dev)
    _need("accepted", accepted, torch.int32, (B,), dev)
    _need("S", S, torch.float32, (B, H, dv, dk), dev)
    if inplace:
        S_out = S
    elif S_out is None:
        S_out = torch.empty_like(S)
    _need("S_out", S_out, torch.float32, (B, H, dv, dk), dev)
    st = load_library().gdr_decode_tree_commit(
        _ptr(k), _ptr(log_alpha), _ptr(parent), _ptr(D), _ptr(accepted), _ptr(S), _ptr(S_out),
        B, Td, H, dk, dv, io, gate, _stream(dev, stream))
    if st != GDR_OK:
        _raise(st)
    return S_out
