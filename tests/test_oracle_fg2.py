"""Pins of the oracle's channel-wise write-rate variant (FG2-GDN, FG2-GDN+).

Reading ("FG2-GDN" page, sections 3.2 and 3.4-3.6; the equations themselves are
not printed): the write rate becomes a vector beta^k_t in R^{d_k} entering
through the scaled key k~ = sqrt(beta^k) * k, the value is scaled by
sqrt(beta^v) (beta^v = beta^k for FG2-GDN, a separate d_v-vector for FG2-GDN+),
and the update is the tied delta rule with unit rate on the scaled vectors:
    S_t = S_{t-1} Diag(alpha_t)(I - k~ k~^T) + v~ k~^T,   o_t = S_t q_t.
Each check below uses a route independent of the oracle: exact rational brute
force over explicit transition matrices, the reduction to KDA / Gated DeltaNet
that the page states, and invariants of the update.
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


def _inputs(seed, B=2, T=29, H=2, dk=5, dv=5, channel=True, sep_v=False):
    r = _rng(seed)
    q = _unit(r, (B, T, H, dk))
    k = _unit(r, (B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    la = r.uniform(-0.5, -0.001, (B, T, H, dk) if channel else (B, T, H))
    bk = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dk))))
    bv = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dv)))) if sep_v else None
    S0 = r.standard_normal((B, H, dv, dk)) * 0.3
    return q, k, v, la, bk, bv, S0


# --------------------------------------------------------------------------
# Exact brute force (rational square roots of the rates).
# --------------------------------------------------------------------------
def _rational_case(seed, T, dk, dv, channel, sep_v):
    r = _rng(seed)
    fr = lambda lo, hi, den: Fraction(int(r.integers(lo, hi)), den)  # noqa: E731
    q = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    k = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    v = [[fr(-8, 9, 4) for _ in range(dv)] for _ in range(T)]
    if channel:
        alpha = [[fr(1, 9, 8) for _ in range(dk)] for _ in range(T)]
    else:
        alpha = [[fr(1, 9, 8)] * dk for _ in range(T)]
    sk = [[fr(0, 9, 8) for _ in range(dk)] for _ in range(T)]
    sv = [[fr(0, 9, 8) for _ in range(dv)] for _ in range(T)] if sep_v else sk
    S0 = [[fr(-4, 5, 4) for _ in range(dk)] for _ in range(dv)]
    return q, k, v, alpha, sk, sv, S0


@pytest.mark.parametrize("sep_v", [False, True])
@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("seed,T,dk,dv", [(1, 1, 1, 1), (2, 6, 3, 3), (3, 7, 4, 4), (4, 5, 3, 2)])
def test_fg2_bruteforce_exact(seed, T, dk, dv, channel, sep_v):
    if dk != dv and not sep_v:
        pytest.skip("beta^v = beta^k needs d_k = d_v")
    q, k, v, alpha, sk, sv, S0 = _rational_case(seed, T, dk, dv, channel, sep_v)
    o_ex, s_ex = exact.run_fg2(q, k, v, alpha, sk, sv, S0)
    f = lambda x: np.array([[float(a) for a in row] for row in x])  # noqa: E731
    la = np.log(f(alpha))
    la = la.reshape(1, T, 1, dk) if channel else la[:, 0].reshape(1, T, 1)
    bk = (f(sk) ** 2).reshape(1, T, 1, dk)
    bv = (f(sv) ** 2).reshape(1, T, 1, dv) if sep_v else None
    o, st = oracle.fg2_chunk_fwd(f(q).reshape(1, T, 1, dk), f(k).reshape(1, T, 1, dk),
                                 f(v).reshape(1, T, 1, dv), la, bk, bv, f(S0).reshape(1, 1, dv, dk))
    o_ex = np.array([[float(x) for x in r] for r in o_ex])
    s_ex = np.array([[float(x) for x in r] for r in s_ex])
    scale = max(1.0, np.abs(o_ex).max(), np.abs(s_ex).max())
    np.testing.assert_allclose(o[0, :, 0, :], o_ex, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(st[0, 0], s_ex, rtol=0, atol=1e-12 * scale)


# --------------------------------------------------------------------------
# The stated reduction: one rate for every channel is KDA (Gated DeltaNet for
# a scalar decay) with that scalar rate.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("channel", [False, True])
def test_fg2_constant_rate_is_kda(channel):
    q, k, v, la, bk, _, S0 = _inputs(11, channel=channel)
    beta = bk[..., 0]
    bk_const = np.repeat(beta[..., None], k.shape[-1], axis=-1)
    o, st = oracle.fg2_chunk_fwd(q, k, v, la, bk_const, None, S0)
    o_ref, st_ref = oracle.chunk_fwd(q, k, v, la, beta, S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(st, st_ref, rtol=0, atol=1e-12)
    # a separate value rate equal to the key rate is the same thing
    o2, st2 = oracle.fg2_chunk_fwd(q, k, v, la, bk_const, bk_const.copy(), S0)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(st2, st)


def test_fg2_value_rate_only_scales_values():
    """With beta^k = 1 everywhere, FG2-GDN+ with value rates beta^v equals the
    unit-rate delta rule on values sqrt(beta^v) * v."""
    q, k, v, la, _, bv, S0 = _inputs(12, sep_v=True)
    ones = np.ones_like(k)
    o, st = oracle.fg2_chunk_fwd(q, k, v, la, ones, bv, S0)
    o_ref, st_ref = oracle.chunk_fwd(q, k, np.sqrt(bv) * v, la, np.ones(k.shape[:3]), S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(st, st_ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Invariants of the update.
# --------------------------------------------------------------------------
def test_fg2_unit_scaled_key_writes_exactly():
    """If ||k~_t|| = 1 the new state maps k~_t to v~_t, whatever the decay and
    the previous state: S_t k~ = S~ k~ - S~ k~ + v~ = v~."""
    r = _rng(13)
    B, T, H, dk, dv = 1, 12, 2, 6, 5
    q = _unit(r, (B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    bk = r.uniform(0.05, 1.0, (B, T, H, dk))
    k = k / np.sqrt(np.sum(bk * k * k, axis=-1, keepdims=True))   # ||sqrt(bk) k|| = 1
    v = r.standard_normal((B, T, H, dv))
    bv = r.uniform(0.05, 1.0, (B, T, H, dv))
    la = r.uniform(-2.0, 0.0, (B, T, H, dk))
    S = r.standard_normal((B, H, dv, dk))
    for t in range(T):
        sl = lambda x: np.ascontiguousarray(x[:, t])  # noqa: E731
        _, S = oracle.fg2_decode_step(sl(q), sl(k), sl(v), sl(la), sl(bk), sl(bv), S)
        ks = np.sqrt(bk[:, t]) * k[:, t]
        got = np.einsum("bhic,bhc->bhi", S, ks)
        np.testing.assert_allclose(got, np.sqrt(bv[:, t]) * v[:, t], rtol=0, atol=1e-12)


def test_fg2_zero_rate_channel_only_decays():
    """A key channel c with beta^k_c = 0 at every step is never erased or
    written: column c of the state only decays, S_T[:, c] = S0[:, c] prod alpha_c."""
    q, k, v, la, bk, _, S0 = _inputs(14, T=17)
    c = 2
    bk[..., c] = 0.0
    _, st = oracle.fg2_chunk_fwd(q, k, v, la, bk, None, S0)
    decay = np.exp(la[..., c].sum(axis=1))     # [B, H]
    np.testing.assert_allclose(st[..., c], S0[..., c] * decay[:, :, None], rtol=1e-12, atol=1e-14)


def test_fg2_chunk_equals_repeated_decode():
    q, k, v, la, bk, bv, S0 = _inputs(15, T=9, sep_v=True)
    o, st = oracle.fg2_chunk_fwd(q, k, v, la, bk, bv, S0)
    S = S0.copy()
    for t in range(q.shape[1]):
        sl = lambda x: np.ascontiguousarray(x[:, t])  # noqa: E731
        ot, S = oracle.fg2_decode_step(sl(q), sl(k), sl(v), sl(la), sl(bk), sl(bv), S)
        np.testing.assert_allclose(ot, o[:, t], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, st, rtol=0, atol=1e-13)


def test_fg2_rejects_missing_value_rate_when_dims_differ():
    q, k, v, la, bk, _, S0 = _inputs(16, dk=5, dv=4, sep_v=False)
    with pytest.raises(ValueError):
        oracle.fg2_chunk_fwd(q, k, v, la, bk, None, None)


# --------------------------------------------------------------------------
# The FG2 pins have teeth: plausible mistakes planted in a copy of the C
# oracle must each be caught by one of them; the real oracle passes all.
# --------------------------------------------------------------------------
FG2_MUTATIONS = {
    "rate_not_rooted_on_key": [("ks[c] = sqrt(bk[c]) * k[c];", "ks[c] = bk[c] * k[c];")],
    "value_not_scaled": [("vs[i] = sqrt(bv[i]) * v[i];", "vs[i] = v[i];")],
    "value_rate_ignored": [("const double *bv = J->beta_v ? J->beta_v + bth * dv : bk;",
                            "const double *bv = bk;")],
    "rate_applied_twice": [("ks, vs, la, J->channel_gate, 1.0,", "ks, vs, la, J->channel_gate, bk[0],")],
    "key_rate_index_shifted": [("ks[c] = sqrt(bk[c]) * k[c];", "ks[c] = sqrt(bk[(c + 1) % dk]) * k[c];")],
}


def _fg2_checks(lib):
    failed = []
    for channel, sep_v in ((True, True), (False, False)):
        q, k, v, alpha, sk, sv, S0 = _rational_case(21, 6, 3, 3, channel, sep_v)
        o_ex, s_ex = exact.run_fg2(q, k, v, alpha, sk, sv, S0)
        f = lambda x: np.array([[float(a) for a in row] for row in x])  # noqa: E731
        T, dk, dv = 6, 3, 3
        la = np.log(f(alpha))
        la = la.reshape(1, T, 1, dk) if channel else la[:, 0].reshape(1, T, 1)
        bv = (f(sv) ** 2).reshape(1, T, 1, dv) if sep_v else None
        o, st = oracle.fg2_chunk_fwd(f(q).reshape(1, T, 1, dk), f(k).reshape(1, T, 1, dk),
                                     f(v).reshape(1, T, 1, dv), la, (f(sk) ** 2).reshape(1, T, 1, dk),
                                     bv, f(S0).reshape(1, 1, dv, dk), lib=lib)
        o_ex = np.array([[float(x) for x in r] for r in o_ex])
        s_ex = np.array([[float(x) for x in r] for r in s_ex])
        if not (np.allclose(o[0, :, 0, :], o_ex, atol=1e-12, rtol=0)
                and np.allclose(st[0, 0], s_ex, atol=1e-12, rtol=0)):
            failed.append("brute_%s_%s" % (channel, sep_v))
    q, k, v, la, bk, _, S0 = _inputs(22, T=7)
    beta = bk[..., 0]
    bk_const = np.repeat(beta[..., None], k.shape[-1], axis=-1)
    o, st = oracle.fg2_chunk_fwd(q, k, v, la, bk_const, None, S0, lib=lib)
    o_ref, st_ref = oracle.chunk_fwd(q, k, v, la, beta, S0)
    if not (np.allclose(o, o_ref, atol=1e-12, rtol=0) and np.allclose(st, st_ref, atol=1e-12, rtol=0)):
        failed.append("kda_reduction")
    return failed


def test_fg2_unmutated_oracle_passes(tmp_path):
    from test_oracle_mutations import _build_variant
    assert _fg2_checks(_build_variant(tmp_path, "clean_fg2", [])) == []


@pytest.mark.parametrize("name", sorted(FG2_MUTATIONS))
def test_fg2_planted_mistake_is_caught(tmp_path, name):
    from test_oracle_mutations import _build_variant
    lib = _build_variant(tmp_path, name, FG2_MUTATIONS[name])
    assert _fg2_checks(lib), "mutation %s escaped every FG2 check" % name
