"""Pins of the oracle's decoupled erase / write gate variant (Gated DeltaNet-2).

Reading (the pages describe the update in words only: "Daily Papers" pages,
Gated DeltaNet-2 abstract and citation notes): a channel-wise erase gate
b_t in R^{d_k} on the key side and a channel-wise write gate w_t in R^{d_v} on
the value side replace the tied scalar beta_t,
    S_t = S_{t-1} Diag(alpha_t)(I - k_t (b_t * k_t)^T) + (w_t * v_t) k_t^T,
    o_t = S_t q_t.
Checks use independent routes: exact rational brute force over explicit
transition matrices, the stated reduction to KDA / Gated DeltaNet when both
gates collapse to the same scalar, the closed form with no erase (gated linear
attention), the exact-write invariant, and planted mistakes.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _inputs(seed, B=2, T=23, H=2, dk=5, dv=4, channel=True):
    r = _rng(seed)
    q = _unit(r, (B, T, H, dk))
    k = _unit(r, (B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    la = r.uniform(-0.5, -0.001, (B, T, H, dk) if channel else (B, T, H))
    eb = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dk))))
    ww = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dv))))
    S0 = r.standard_normal((B, H, dv, dk)) * 0.3
    return q, k, v, la, eb, ww, S0


def _rational_case(seed, T, dk, dv, channel):
    r = _rng(seed)
    fr = lambda lo, hi, den: Fraction(int(r.integers(lo, hi)), den)  # noqa: E731
    q = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    k = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    v = [[fr(-8, 9, 4) for _ in range(dv)] for _ in range(T)]
    alpha = ([[fr(1, 9, 8) for _ in range(dk)] for _ in range(T)] if channel
             else [[fr(1, 9, 8)] * dk for _ in range(T)])
    eb = [[fr(0, 9, 8) for _ in range(dk)] for _ in range(T)]
    ww = [[fr(0, 9, 8) for _ in range(dv)] for _ in range(T)]
    S0 = [[fr(-4, 5, 4) for _ in range(dk)] for _ in range(dv)]
    return q, k, v, alpha, eb, ww, S0


def _run_rational(case, channel, lib=None):
    q, k, v, alpha, eb, ww, S0 = case
    T, dk, dv = len(q), len(q[0]), len(v[0])
    f = lambda x: np.array([[float(a) for a in row] for row in x])  # noqa: E731
    la = np.log(f(alpha))
    la = la.reshape(1, T, 1, dk) if channel else la[:, 0].reshape(1, T, 1)
    return oracle.gdn2_chunk_fwd(f(q).reshape(1, T, 1, dk), f(k).reshape(1, T, 1, dk),
                                 f(v).reshape(1, T, 1, dv), la, f(eb).reshape(1, T, 1, dk),
                                 f(ww).reshape(1, T, 1, dv), f(S0).reshape(1, 1, dv, dk), lib=lib)


def _exact_close(case, channel, lib=None):
    o_ex, s_ex = exact.run_gdn2(*case)
    o, st = _run_rational(case, channel, lib)
    o_ex = np.array([[float(x) for x in r] for r in o_ex])
    s_ex = np.array([[float(x) for x in r] for r in s_ex])
    scale = max(1.0, np.abs(o_ex).max(), np.abs(s_ex).max())
    return (np.allclose(o[0, :, 0, :], o_ex, rtol=0, atol=1e-12 * scale)
            and np.allclose(st[0, 0], s_ex, rtol=0, atol=1e-12 * scale))


@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("seed,T,dk,dv", [(1, 1, 1, 1), (2, 6, 3, 2), (3, 7, 4, 4), (4, 5, 2, 3)])
def test_gdn2_bruteforce_exact(seed, T, dk, dv, channel):
    assert _exact_close(_rational_case(seed, T, dk, dv, channel), channel)


@pytest.mark.parametrize("channel", [False, True])
def test_gdn2_tied_gates_are_kda(channel):
    """b_t = beta_t 1 and w_t = beta_t 1: exactly KDA (Gated DeltaNet for a
    scalar decay) with rate beta_t."""
    q, k, v, la, eb, _, S0 = _inputs(31, channel=channel)
    beta = eb[..., 0]
    o, st = oracle.gdn2_chunk_fwd(q, k, v, la, np.repeat(beta[..., None], k.shape[-1], -1),
                                  np.repeat(beta[..., None], v.shape[-1], -1), S0)
    o_ref, st_ref = oracle.chunk_fwd(q, k, v, la, beta, S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(st, st_ref, rtol=0, atol=1e-12)


def test_gdn2_no_erase_is_gated_linear_attention():
    """b = 0: nothing is erased, S_T = S0 Diag(prod alpha) + sum_t (w_t v_t) k_t^T
    Diag(prod_{s>t} alpha_s), written out directly."""
    q, k, v, la, _, ww, S0 = _inputs(32, B=1, H=1, T=9)
    o, st = oracle.gdn2_chunk_fwd(q, k, v, la, np.zeros_like(k), ww, S0)
    a = np.exp(la[0, :, 0])                     # [T, dk]
    T = a.shape[0]
    S = S0[0, 0] * np.prod(a, axis=0)
    for t in range(T):
        tail = np.prod(a[t + 1:], axis=0) if t + 1 < T else np.ones(a.shape[1])
        S = S + np.outer(ww[0, t, 0] * v[0, t, 0], k[0, t, 0] * tail)
    np.testing.assert_allclose(st[0, 0], S, rtol=0, atol=1e-12)


def test_gdn2_full_erase_writes_exactly():
    """b = 1 and ||k|| = 1: the new state maps k_t to w_t * v_t whatever the
    decay and the previous state (S~ k - S~ k (k.k) + (w v)(k.k))."""
    q, k, v, la, _, ww, S0 = _inputs(33, T=8)
    eb = np.ones_like(k)
    for T in range(1, 9):
        _, st = oracle.gdn2_chunk_fwd(q[:, :T], k[:, :T], v[:, :T], la[:, :T], eb[:, :T],
                                      ww[:, :T], S0)
        got = np.einsum("bhic,bhc->bhi", st, k[:, T - 1])
        np.testing.assert_allclose(got, ww[:, T - 1] * v[:, T - 1], rtol=0, atol=1e-12)


GDN2_MUTATIONS = {
    "erase_along_k": [("row[c] -= r * eb[c] * k[c];", "row[c] -= r * k[c];")],
    "erase_read_at_gated_key": [("for (int64_t c = 0; c < dk; ++c) r += row[c] * k[c];      /* read at k        */",
                                 "for (int64_t c = 0; c < dk; ++c) r += row[c] * eb[c] * k[c];")],
    "write_gate_dropped": [("const double u = ww[i] * v[i];", "const double u = v[i];")],
    "erase_sign": [("row[c] -= r * eb[c] * k[c];", "row[c] += r * eb[c] * k[c];")],
    "write_gated_on_key": [("const double u = ww[i] * v[i];", "const double u = eb[i] * v[i];")],
}


def _gdn2_checks(lib):
    failed = []
    for channel in (False, True):
        if not _exact_close(_rational_case(41, 6, 3, 3, channel), channel, lib):
            failed.append("brute_%s" % channel)
    return failed


def test_gdn2_unmutated_oracle_passes(tmp_path):
    from test_oracle_mutations import _build_variant
    assert _gdn2_checks(_build_variant(tmp_path, "clean_gdn2", [])) == []


@pytest.mark.parametrize("name", sorted(GDN2_MUTATIONS))
def test_gdn2_planted_mistake_is_caught(tmp_path, name):
    from test_oracle_mutations import _build_variant
    lib = _build_variant(tmp_path, name, GDN2_MUTATIONS[name])
    assert _gdn2_checks(lib), "mutation %s escaped" % name
