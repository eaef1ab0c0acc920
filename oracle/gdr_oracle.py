"""ctypes front end of the fp64 C oracle (test infrastructure only).

The oracle computes, token by token and in fp64, the gated delta rule

    S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,

with ``S`` stored ``[d_v, d_k]`` per head (see ``gdr_oracle.c`` for the page
citations).  Inputs are converted to fp64 exactly (they are fp32 arrays whose
values already carry the storage rounding of the GPU inputs), so the comparison
measures only the GPU path's own error.

``build()`` compiles ``gdr_oracle.c`` with gcc into ``libgdr_oracle.so`` next to
it; ``chunk_fwd`` / ``decode_step`` build on first use if the library is absent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build(src=None, out=None) -> str:
    """Compile the C oracle (always recompiles).  Returns the library path."""
    out = out or _LIB
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", src or _SRC,
           "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path=None):
    """Load the oracle library (the default one unless ``path`` is given)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    if path is None and not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(path or _LIB)
    d = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.gdr_oracle_chunk_fwd.argtypes = [d, d, d, d, d, d, d, d,
                                         i64, i64, i64, i64, i64,
                                         ctypes.c_int, ctypes.c_int]
    lib.gdr_oracle_chunk_fwd.restype = ctypes.c_int
    lib.gdr_oracle_decode_step.argtypes = [d, d, d, d, d, d, d, d,
                                           i64, i64, i64, i64, ctypes.c_int]
    lib.gdr_oracle_decode_step.restype = ctypes.c_int
    lib.gdr_oracle_fg2_chunk_fwd.argtypes = [d, d, d, d, d, d, d, d, d,
                                             i64, i64, i64, i64, i64,
                                             ctypes.c_int, ctypes.c_int]
    lib.gdr_oracle_fg2_chunk_fwd.restype = ctypes.c_int
    lib.gdr_oracle_fg2_decode_step.argtypes = [d, d, d, d, d, d, d, d, d,
                                               i64, i64, i64, i64, ctypes.c_int]
    lib.gdr_oracle_fg2_decode_step.restype = ctypes.c_int
    lib.gdr_oracle_gdn2_chunk_fwd.argtypes = [d, d, d, d, d, d, d, d, d,
                                              i64, i64, i64, i64, i64,
                                              ctypes.c_int, ctypes.c_int]
    lib.gdr_oracle_gdn2_chunk_fwd.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, threads=None, lib=None):
    """Whole-sequence forward.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; log_alpha: [B,T,H] (scalar gate) or
    [B,T,H,dk] (channel gate); beta: [B,T,H]; S0: [B,H,dv,dk] or None (zeros).
    Returns (o [B,T,H,dv], S_T [B,H,dv,dk]) as fp64 arrays.
    """
    q, k, v, la, be = (_f64(a) for a in (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    channel = la.ndim == 4
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or be.shape != (B, T, H):
        raise ValueError("shape mismatch")
    if la.shape != ((B, T, H, dk) if channel else (B, T, H)):
        raise ValueError("log_alpha shape mismatch")
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None and s0.shape != (B, H, dv, dk):
        raise ValueError("S0 shape mismatch")
    o = np.zeros((B, T, H, dv), np.float64)
    st = np.zeros((B, H, dv, dk), np.float64)
    n = default_threads() if threads is None else int(threads)
    rc = (lib or load()).gdr_oracle_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be),
                                      _ptr(s0), _ptr(o), _ptr(st),
                                      B, T, H, dk, dv, int(channel), n)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, st


def decode_step(q, k, v, log_alpha, beta, S, lib=None):
    """One recurrent step.  q,k: [B,H,dk]; v: [B,H,dv]; log_alpha: [B,H] or
    [B,H,dk]; beta: [B,H]; S: [B,H,dv,dk].  Returns (o [B,H,dv], S' [B,H,dv,dk])."""
    q, k, v, la, be, s = (_f64(a) for a in (q, k, v, log_alpha, beta, S))
    B, H, dk = q.shape
    dv = v.shape[2]
    channel = la.ndim == 3
    if la.shape != ((B, H, dk) if channel else (B, H)) or s.shape != (B, H, dv, dk):
        raise ValueError("shape mismatch")
    o = np.zeros((B, H, dv), np.float64)
    s_out = s.copy()
    rc = (lib or load()).gdr_oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be),
                                        _ptr(s_out), _ptr(s_out), _ptr(o),
                                        B, H, dk, dv, int(channel))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, s_out


def fg2_chunk_fwd(q, k, v, log_alpha, beta_k, beta_v=None, S0=None, threads=None, lib=None):
    """Whole-sequence forward with channel-wise write rates (FG2-GDN / FG2-GDN+).

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; log_alpha: [B,T,H] or [B,T,H,dk];
    beta_k: [B,T,H,dk]; beta_v: [B,T,H,dv] or None (= beta_k, needs dk == dv);
    S0: [B,H,dv,dk] or None.  Returns (o, S_T) as fp64 arrays.
    """
    q, k, v, la, bk = (_f64(a) for a in (q, k, v, log_alpha, beta_k))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    channel = la.ndim == 4
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or bk.shape != (B, T, H, dk):
        raise ValueError("shape mismatch")
    if la.shape != ((B, T, H, dk) if channel else (B, T, H)):
        raise ValueError("log_alpha shape mismatch")
    bv = None if beta_v is None else _f64(beta_v)
    if bv is not None and bv.shape != (B, T, H, dv):
        raise ValueError("beta_v shape mismatch")
    s0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, dv), np.float64)
    st = np.zeros((B, H, dv, dk), np.float64)
    n = default_threads() if threads is None else int(threads)
    rc = (lib or load()).gdr_oracle_fg2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(bk),
                                                  _ptr(bv), _ptr(s0), _ptr(o), _ptr(st),
                                                  B, T, H, dk, dv, int(channel), n)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, st


def fg2_decode_step(q, k, v, log_alpha, beta_k, beta_v, S, lib=None):
    """One recurrent step with channel-wise write rates.  q,k: [B,H,dk]; v: [B,H,dv];
    log_alpha: [B,H] or [B,H,dk]; beta_k: [B,H,dk]; beta_v: [B,H,dv] or None;
    S: [B,H,dv,dk].  Returns (o [B,H,dv], S')."""
    q, k, v, la, bk, s = (_f64(a) for a in (q, k, v, log_alpha, beta_k, S))
    B, H, dk = q.shape
    dv = v.shape[2]
    channel = la.ndim == 3
    bv = None if beta_v is None else _f64(beta_v)
    o = np.zeros((B, H, dv), np.float64)
    s_out = s.copy()
    rc = (lib or load()).gdr_oracle_fg2_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(bk),
                                                    _ptr(bv), _ptr(s_out), _ptr(s_out), _ptr(o),
                                                    B, H, dk, dv, int(channel))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, s_out


def decode_multi(q, k, v, log_alpha, beta, S, accepted=None, lib=None):
    """Td tokens per sequence applied to the state S in order, as Td decode
    steps would (speculative-decoding verify / commit).  q,k: [B,Td,H,dk];
    v: [B,Td,H,dv]; log_alpha: [B,Td,H] or [B,Td,H,dk]; beta: [B,Td,H];
    S: [B,H,dv,dk]; accepted: B integers (clamped to [0, Td]) or None (= Td).
    Returns (o [B,Td,H,dv] from every token, S_out [B,H,dv,dk] = the state after
    the first accepted[b] tokens of sequence b).  A composition of the
    whole-sequence recurrence above, with no arithmetic of its own."""
    q, k, v, la, be, s = (_f64(a) for a in (q, k, v, log_alpha, beta, S))
    B, Td = q.shape[:2]
    o, _ = chunk_fwd(q, k, v, la, be, s, lib=lib)
    s_out = s.copy()
    for b in range(B):
        n = Td if accepted is None else int(min(max(int(accepted[b]), 0), Td))
        sl = lambda a: a[b:b + 1, :n]  # noqa: E731
        _, st = chunk_fwd(sl(q), sl(k), sl(v), sl(la), sl(be), s[b:b + 1], lib=lib)
        s_out[b] = st[0]
    return o, s_out


def decode_tree(q, k, v, log_alpha, beta, S, parent):
    """A tree of draft tokens applied to the committed state S (speculative
    decoding with branching drafts; the TreeWY note on the mindpattern "Gated
    DeltaNet-2" page verifies every node of such a tree at once and keeps a
    pseudo-value per node in place of per-node state snapshots).

    Node i of sequence b follows parent[b][i] (a node with a smaller index) or,
    for parent -1, the committed state itself.  Its state is the delta rule
    applied along its root path, one token per node:
        S_pre = S_parent Diag(alpha_i),  u_i = beta_i (v_i - S_pre k_i),
        S_i = S_pre + u_i k_i^T,         o_i = S_i q_i.
    Returns (o [B,Td,H,dv], u [B,Td,H,dv] (the written value of every node),
    states {(b, i): [H,dv,dk]}).  Plain fp64 numpy, node by node in index
    order (parents come first), every state kept; for test sizes."""
    q, k, v, la, be, s = (_f64(a) for a in (q, k, v, log_alpha, beta, S))
    B, Td, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, Td, H, dv))
    u = np.zeros((B, Td, H, dv))
    states = {}
    for b in range(B):
        for i in range(Td):
            p = int(parent[b][i])
            if not -1 <= p < i:
                raise ValueError("parent[%d][%d] = %d is not -1 or an earlier node" % (b, i, p))
            prev = s[b] if p < 0 else states[(b, p)]
            a = np.exp(la[b, i]) if la.ndim == 4 else np.exp(la[b, i])[:, None]
            pre = prev * a[:, None, :]                       # S Diag(alpha), per head
            pred = np.einsum("hvc,hc->hv", pre, k[b, i])
            u[b, i] = be[b, i][:, None] * (v[b, i] - pred)
            st = pre + u[b, i][:, :, None] * k[b, i][:, None, :]
            states[(b, i)] = st
            o[b, i] = np.einsum("hvc,hc->hv", st, q[b, i])
    return o, u, states


def decode_tree_commit(S, states, accepted):
    """The state after the accepted node of every sequence (accepted[b] = -1
    keeps S[b]), from decode_tree's states."""
    out = _f64(S).copy()
    for b, a in enumerate(accepted):
        if int(a) >= 0:
            out[b] = states[(b, int(a))]
    return out


def gdn2_chunk_fwd(q, k, v, log_alpha, erase, write, S0=None, threads=None, lib=None):
    """Whole-sequence forward with decoupled erase and write gates (Gated
    DeltaNet-2 reading, see gdr_oracle.c).  q, k: [B,T,H,dk]; v: [B,T,H,dv];
    log_alpha: [B,T,H] or [B,T,H,dk]; erase: [B,T,H,dk]; write: [B,T,H,dv];
    S0: [B,H,dv,dk] or None.  Returns (o, S_T) as fp64 arrays."""
    q, k, v, la, eb, ww = (_f64(a) for a in (q, k, v, log_alpha, erase, write))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    channel = la.ndim == 4
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or eb.shape != (B, T, H, dk) \
            or ww.shape != (B, T, H, dv):
        raise ValueError("shape mismatch")
    if la.shape != ((B, T, H, dk) if channel else (B, T, H)):
        raise ValueError("log_alpha shape mismatch")
    s0 = None if S0 is None else _f64(S0)
    o = np.zeros((B, T, H, dv), np.float64)
    st = np.zeros((B, H, dv, dk), np.float64)
    n = default_threads() if threads is None else int(threads)
    rc = (lib or load()).gdr_oracle_gdn2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(eb),
                                                   _ptr(ww), _ptr(s0), _ptr(o), _ptr(st),
                                                   B, T, H, dk, dv, int(channel), n)
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return o, st


PROLOGUE_L2NORM_QK = 1
PROLOGUE_BETA_SIGMOID = 2
PROLOGUE_DECAY_SOFTPLUS = 4
PROLOGUE_EPS = 1e-6


def prologue_inputs(q, k, beta, flags, eps=PROLOGUE_EPS):
    """The gate prologue ("FG2-GDN" page, section 3.5: queries and keys are
    L2-normalised; the write rate is the sigmoid of its projection), applied to
    raw inputs in fp64: q / sqrt(sum q^2 + eps) and likewise k per token and
    head (flag 1), beta = 1 / (1 + e^{-x}) (flag 2).  eps = 1e-6 is this build's
    choice (the page gives none); it only matters for near-zero rows."""
    q, k, be = (_f64(a) for a in (q, k, beta))
    if flags & PROLOGUE_L2NORM_QK:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    if flags & PROLOGUE_BETA_SIGMOID:
        be = 1.0 / (1.0 + np.exp(-be))
    return q, k, be


def prologue_decay(log_alpha, flags):
    """The decay from its logit (flag 4): log alpha = -softplus(x) = -ln(1 + e^x),
    so alpha = 1 / (1 + e^x) lies in (0, 1) for every finite x.  The "FG2-GDN"
    page (section 3.5) feeds channel-wise projections to KDA's gated-decay
    transform, which yields alpha in (0, 1), without printing it; the NVFP4
    abstract on the "Daily Papers" DeltaNet search page (finding ii) names
    softplus / exponential parameterisations for the decay gate.  This reading
    takes the plainest such map: a softplus, negated, then the exponential that
    every call already applies to log alpha.  In fp64 through logaddexp (no
    overflow for large |x|)."""
    x = _f64(log_alpha)
    if flags & PROLOGUE_DECAY_SOFTPLUS:
        return -np.logaddexp(0.0, x)
    return x


def chunk_fwd_prologue(q, k, v, log_alpha, beta, S0=None, flags=0, threads=None, lib=None):
    """The whole-sequence forward on raw q, k, beta and decay logits: the
    prologue above, then the recurrence (a composition, no arithmetic of its own)."""
    q2, k2, be2 = prologue_inputs(q, k, beta, flags)
    return chunk_fwd(q2, k2, v, prologue_decay(log_alpha, flags), be2, S0, threads=threads, lib=lib)


def decode_step_prologue(q, k, v, log_alpha, beta, S, flags=0, lib=None):
    q2, k2, be2 = prologue_inputs(q, k, beta, flags)
    return decode_step(q2, k2, v, prologue_decay(log_alpha, flags), be2, S, lib=lib)
