"""Seeded synthetic inputs for the gated delta rule (shared by tests and bench).

This module holds no arithmetic of the method itself: it only draws random
tensors with the distributions of the workloads and rounds them to their storage
type.  Both the GPU path and the CPU oracle consume exactly the arrays returned
here (the oracle after an exact widening to fp64).

Distributions (the workloads' recipe):
  q, k   ~ N(0,1), then scaled to unit L2 norm over d_k per (b,t,h)
  v      ~ N(0,1)
  beta   = sigmoid(N(0,1))
  log_alpha ~ U(-0.1, -0.001)      per (b,t,h), or per (b,t,h,channel)
  S0 / S ~ N(0, std^2)              when present
Draw order: q, k, v, beta logits, log_alpha, then S0 / S, from
``numpy.random.Generator(PCG64(seed))``.  q, k, v are rounded to the storage
type (bf16 round-to-nearest-even, or fp32); the gates and states are fp32.
The returned arrays are float32 whose values are exactly representable in the
storage type, so a cast to bf16 on the device is exact.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    call: str            # "chunk" or "decode"
    gate: str            # "scalar" (Gated DeltaNet) or "channel" (KDA)
    io: str              # "f32" or "bf16": storage type of q, k, v and o
    B: int
    H: int
    T: int
    d: int               # d_k = d_v
    chunk: int
    s0_std: Optional[float]
    tol: float           # normwise relative tolerance of o and of the state
    seed: int


# The five workloads (tokens/s of #1 is the headline number; #4 is the decode step).
WORKLOADS = [
    Workload("gdn_chunk_f32_B1_H2_T256_d64", "chunk", "scalar", "f32",
             1, 2, 256, 64, 64, None, 1e-4, 1000),
    Workload("gdn_prefill_bf16_B4_H16_T4096_d128", "chunk", "scalar", "bf16",
             4, 16, 4096, 128, 64, None, 2e-2, 1001),
    Workload("kda_prefill_bf16_B2_H32_T8192_d128", "chunk", "channel", "bf16",
             2, 32, 8192, 128, 64, None, 2e-2, 1002),
    Workload("gdn_prefill_s0_bf16_B1_H32_T32768_d128", "chunk", "scalar", "bf16",
             1, 32, 32768, 128, 64, 0.02, 2e-2, 1003),
    Workload("gdn_decode_f32_B256_H32_d128", "decode", "scalar", "f32",
             256, 32, 1, 128, 0, 0.05, 1e-4, 1004),
]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even); return float32 holding it."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def _store(x: np.ndarray, io: str) -> np.ndarray:
    if io == "bf16":
        return round_bf16(x)
    if io == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(io)


def _unit_rows(rng, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x


def chunk_inputs(B, T, H, dk, dv, gate="scalar", io="bf16", seed=0,
                 s0_std=None, log_alpha_range=(-0.1, -0.001)):
    """Inputs of one whole-sequence call, as a dict of float32 numpy arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _store(_unit_rows(rng, (B, T, H, dk)), io)
    k = _store(_unit_rows(rng, (B, T, H, dk)), io)
    v = _store(rng.standard_normal((B, T, H, dv)), io)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    la_shape = (B, T, H, dk) if gate == "channel" else (B, T, H)
    lo, hi = log_alpha_range
    log_alpha = rng.uniform(lo, hi, la_shape).astype(np.float32)
    S0 = None
    if s0_std is not None:
        S0 = (rng.standard_normal((B, H, dv, dk)) * s0_std).astype(np.float32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, S0=S0)


def decode_inputs(B, H, dk, dv, gate="scalar", io="f32", seed=0, s_std=0.05,
                  log_alpha_range=(-0.1, -0.001)):
    """Inputs of one decode step, as a dict of float32 numpy arrays."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _store(_unit_rows(rng, (B, H, dk)), io)
    k = _store(_unit_rows(rng, (B, H, dk)), io)
    v = _store(rng.standard_normal((B, H, dv)), io)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, H))))).astype(np.float32)
    la_shape = (B, H, dk) if gate == "channel" else (B, H)
    lo, hi = log_alpha_range
    log_alpha = rng.uniform(lo, hi, la_shape).astype(np.float32)
    S = (rng.standard_normal((B, H, dv, dk)) * s_std).astype(np.float32)
    return dict(q=q, k=k, v=v, log_alpha=log_alpha, beta=beta, S=S)


def workload_inputs(w: Workload):
    if w.call == "chunk":
        return chunk_inputs(w.B, w.T, w.H, w.d, w.d, w.gate, w.io, w.seed, w.s0_std)
    return decode_inputs(w.B, w.H, w.d, w.d, w.gate, w.io, w.seed, w.s0_std)


def write_rates(shape_k, dv=None, seed=0):
    """Channel-wise write rates for the FG2 calls: beta^k = sigmoid(N(0,1)) of
    shape ``shape_k`` (leading dims + [dk]) and, when ``dv`` is given, a separate
    beta^v = sigmoid(N(0,1)) with last dim dv.  Drawn from their own seeded
    stream, so the other inputs of a workload do not change."""
    rng = np.random.Generator(np.random.PCG64(seed + 5000))
    bk = (1.0 / (1.0 + np.exp(-rng.standard_normal(shape_k)))).astype(np.float32)
    bv = None
    if dv is not None:
        bv = (1.0 / (1.0 + np.exp(-rng.standard_normal(tuple(shape_k[:-1]) + (dv,))))).astype(np.float32)
    return bk, bv


def gdn2_gates(B, T, H, dk, dv, seed=0):
    """Decoupled erase / write gates for the Gated DeltaNet-2 call:
    b = sigmoid(N(0,1)) of shape [B,T,H,dk], w = sigmoid(N(0,1)) of shape
    [B,T,H,dv], from their own seeded stream."""
    rng = np.random.Generator(np.random.PCG64(seed + 7000))
    b = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, dk))))).astype(np.float32)
    w = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, dv))))).astype(np.float32)
    return b, w


def raw_prologue_inputs(inp, io="bf16", seed=0, decay_logits=False):
    """Raw inputs for the gate prologue from a workload's inputs: q and k rows
    scaled by factors U(1, 8) per token and head (then stored in the io type),
    beta replaced by logits N(0, 1.5^2).  With ``decay_logits`` log_alpha
    (same shape) is replaced by decay logits U(-8, 2): alpha = 1 / (1 + e^x)
    from 0.9997 (x = -8) down to 0.12 (x = 2), the workloads' range of weak
    decays plus strong ones.  Own seeded stream."""
    rng = np.random.Generator(np.random.PCG64(seed + 9000))
    out = dict(inp)
    for n in ("q", "k"):
        x = inp[n].astype(np.float64)
        out[n] = _store(x * rng.uniform(1.0, 8.0, x.shape[:-1] + (1,)), io)
    out["beta"] = (rng.standard_normal(inp["beta"].shape) * 1.5).astype(np.float32)
    if decay_logits:
        out["log_alpha"] = rng.uniform(-8.0, 2.0, inp["log_alpha"].shape).astype(np.float32)
    return out


DRAFT_TREES = ("chain", "star", "binary", "random")


def draft_tree(kind, B, Td, seed=0):
    """Parent indices [B, Td] (int32) of a draft tree per sequence, nodes in
    topological order: parent -1 hangs a node off the committed state, any
    other parent is an earlier node.
      chain   one linear draft (parent i - 1)
      star    Td alternatives for the next token (all -1)
      binary  a complete binary tree under node 0
      random  each node's parent uniform over -1 .. i - 1 (own seeded stream)"""
    if kind == "chain":
        p = np.arange(Td) - 1
        return np.ascontiguousarray(np.broadcast_to(p, (B, Td)), dtype=np.int32)
    if kind == "star":
        return np.full((B, Td), -1, dtype=np.int32)
    if kind == "binary":
        p = (np.arange(Td) - 1) // 2
        p[0] = -1
        return np.ascontiguousarray(np.broadcast_to(p, (B, Td)), dtype=np.int32)
    if kind == "random":
        rng = np.random.Generator(np.random.PCG64(seed + 13000))
        p = np.stack([np.array([rng.integers(-1, i) if i > 0 else -1 for i in range(Td)]) for _ in range(B)])
        return p.astype(np.int32)
    raise ValueError(kind)


EDGE_KEYS = ("repeated", "antiparallel", "near_collinear", "plane", "cyclic3")


def edge_key_inputs(kind, B, T, H, d, io="bf16", seed=0, key_norm=1.0, beta=1.0,
                    log_alpha=0.0, s0_std=0.1):
    """Valid but adversarial inputs for the chunk solve: keys of norm
    ``key_norm`` with a degenerate Gram structure, a constant write rate
    ``beta`` and a constant ``log_alpha`` (0 = no decay).  Key patterns, per
    (b, h), from one random unit direction u (and a second one w):
      repeated        every token has key u
      antiparallel    keys alternate u, -u, u, ...
      near_collinear  u plus N(0, 0.01^2) noise, renormalised
      plane           random directions inside span{u, w}
      cyclic3         keys cycle through three orthonormal directions
    q, v and S0 are drawn as in chunk_inputs.  Own seeded stream."""
    if kind not in EDGE_KEYS:
        raise ValueError(kind)
    rng = np.random.Generator(np.random.PCG64(seed + 11000))
    q = _store(_unit_rows(rng, (B, T, H, d)), io)
    v = _store(rng.standard_normal((B, T, H, d)), io)
    u = _unit_rows(rng, (B, 1, H, d))
    w = rng.standard_normal((B, 1, H, d))
    w -= np.sum(w * u, axis=-1, keepdims=True) * u
    w /= np.linalg.norm(w, axis=-1, keepdims=True)
    t = np.arange(T).reshape(1, T, 1, 1)
    if kind == "repeated":
        k = np.broadcast_to(u, (B, T, H, d)).copy()
    elif kind == "antiparallel":
        k = np.where(t % 2 == 0, 1.0, -1.0) * u
    elif kind == "near_collinear":
        k = u + 0.01 * rng.standard_normal((B, T, H, d))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    elif kind == "plane":
        th = rng.uniform(0.0, 2.0 * np.pi, (B, T, H, 1))
        k = np.cos(th) * u + np.sin(th) * w
    else:
        x = w - np.sum(w * u, axis=-1, keepdims=True) * u
        z = rng.standard_normal((B, 1, H, d))
        z -= np.sum(z * u, axis=-1, keepdims=True) * u + np.sum(z * x, axis=-1, keepdims=True) * x
        z /= np.linalg.norm(z, axis=-1, keepdims=True)
        k = np.where(t % 3 == 0, u, np.where(t % 3 == 1, x, z))
    k = _store(key_norm * k, io)
    S0 = None if s0_std is None else (rng.standard_normal((B, H, d, d)) * s0_std).astype(np.float32)
    return dict(q=q, k=k, v=v,
                log_alpha=np.full((B, T, H), log_alpha, np.float32),
                beta=np.full((B, T, H), beta, np.float32), S0=S0)
