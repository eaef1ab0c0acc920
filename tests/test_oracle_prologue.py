"""Pins of the oracle's gate prologue (L2-normalised q and k, beta from logits
through a sigmoid; "FG2-GDN" page, section 3.5), checked against routes that do
not share its code: scipy's logistic function, normalisation invariants, and
the plain recurrence on inputs prepared by hand."""
import numpy as np
import pytest
from scipy.special import expit

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _raw(seed, B=2, T=19, H=2, dk=6, dv=5, channel=True):
    r = _rng(seed)
    # raw rows of norm roughly 2..20, where the epsilon of the normalisation
    # changes a row by less than 1e-7 relative
    q = r.standard_normal((B, T, H, dk)) * r.uniform(1.0, 8.0, (B, T, H, 1))
    k = r.standard_normal((B, T, H, dk)) * r.uniform(1.0, 8.0, (B, T, H, 1))
    v = r.standard_normal((B, T, H, dv))
    la = r.uniform(-0.5, -0.001, (B, T, H, dk) if channel else (B, T, H))
    x = r.standard_normal((B, T, H)) * 2
    S0 = r.standard_normal((B, H, dv, dk)) * 0.3
    return q, k, v, la, x, S0


def test_prologue_off_is_the_recurrence():
    q, k, v, la, x, S0 = _raw(1)
    be = expit(x)
    o1, s1 = oracle.chunk_fwd_prologue(q, k, v, la, be, S0, flags=0)
    o2, s2 = oracle.chunk_fwd(q, k, v, la, be, S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_prologue_sigmoid_matches_scipy():
    q, k, v, la, x, S0 = _raw(2)
    o1, s1 = oracle.chunk_fwd_prologue(q, k, v, la, x, S0, flags=oracle.gdr_oracle.PROLOGUE_BETA_SIGMOID)
    o2, s2 = oracle.chunk_fwd(q, k, v, la, expit(x), S0)
    # raw keys are not unit-norm here, so the state grows large: compare relatively
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=0)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=0)


@pytest.mark.parametrize("channel", [False, True])
def test_prologue_norm_is_scale_invariant(channel):
    """Rescaling raw q and k rows by positive factors changes nothing (up to
    the epsilon, negligible at these norms)."""
    q, k, v, la, x, S0 = _raw(3, channel=channel)
    flags = oracle.gdr_oracle.PROLOGUE_L2NORM_QK | oracle.gdr_oracle.PROLOGUE_BETA_SIGMOID
    r = _rng(30)
    o1, s1 = oracle.chunk_fwd_prologue(q, k, v, la, x, S0, flags=flags)
    o2, s2 = oracle.chunk_fwd_prologue(q * r.uniform(0.5, 9, q.shape[:3] + (1,)),
                                       k * r.uniform(0.5, 9, k.shape[:3] + (1,)), v, la, x, S0,
                                       flags=flags)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-6)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-6)


def test_prologue_norm_matches_hand_normalised_inputs():
    q, k, v, la, x, S0 = _raw(4)
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    be = expit(x)
    o1, s1 = oracle.chunk_fwd_prologue(q, k, v, la, be, S0, flags=oracle.gdr_oracle.PROLOGUE_L2NORM_QK)
    o2, s2 = oracle.chunk_fwd(qn, kn, v, la, be, S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-6)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-6)
    q2, k2, _ = oracle.prologue_inputs(q, k, x, oracle.gdr_oracle.PROLOGUE_L2NORM_QK)
    np.testing.assert_allclose(np.linalg.norm(k2, axis=-1), 1.0, rtol=0, atol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(q2, axis=-1), 1.0, rtol=0, atol=1e-6)


def test_prologue_zero_rows_stay_finite():
    q, k, v, la, x, S0 = _raw(5, T=4)
    q[:, 1] = 0.0
    k[:, 2] = 0.0
    o, st = oracle.chunk_fwd_prologue(q, k, v, la, x, S0, flags=3)
    assert np.isfinite(o).all() and np.isfinite(st).all()


def test_decode_prologue_is_one_token_of_chunk():
    q, k, v, la, x, S0 = _raw(6, T=1)
    o, st = oracle.chunk_fwd_prologue(q, k, v, la, x, S0, flags=3)
    od, sd = oracle.decode_step_prologue(q[:, 0], k[:, 0], v[:, 0], la[:, 0], x[:, 0], S0, flags=3)
    np.testing.assert_allclose(od, o[:, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sd, st, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# The decay from its logit (flag 4): log alpha = -softplus(x), alpha = 1/(1+e^x).
# ---------------------------------------------------------------------------
DECAY = oracle.gdr_oracle.PROLOGUE_DECAY_SOFTPLUS


def test_decay_softplus_closed_forms():
    from scipy.special import log_expit
    x = np.array([-600.0, -60.0, -5.0, -1e-3, 0.0, 1e-3, 2.0, 40.0, 800.0])
    la = oracle.prologue_decay(x, DECAY)
    # -softplus(x) = log sigmoid(-x): scipy's log-logistic, a separate routine
    np.testing.assert_allclose(la, log_expit(-x), rtol=1e-15, atol=0)
    assert la[4] == -np.log(2.0)                       # x = 0: alpha = 1/2
    np.testing.assert_allclose(la[0], -np.exp(-600.0), rtol=1e-14)   # alpha -> 1: -e^x
    np.testing.assert_allclose(la[-1], -800.0, rtol=1e-15)   # alpha ~ e^-x
    assert np.all(np.diff(la) < 0)                     # monotone decreasing in x
    assert np.all(la < 0)                              # alpha in (0, 1)
    # flag off: the log decay passes through unchanged
    np.testing.assert_array_equal(oracle.prologue_decay(x, 3), x)


@pytest.mark.parametrize("channel", [False, True])
def test_decay_softplus_inverts_to_the_log_decay(channel):
    """x = ln(e^{-log alpha} - 1) is the logit of a given decay; the prologue on x
    must reproduce the plain recurrence on log alpha."""
    q, k, v, la, _, S0 = _raw(7, channel=channel)
    be = expit(_rng(70).standard_normal(la.shape[:3]))
    x = np.log(np.expm1(-la))
    o1, s1 = oracle.chunk_fwd_prologue(q, k, v, x, be, S0, flags=DECAY)
    o2, s2 = oracle.chunk_fwd(q, k, v, la, be, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-11, atol=1e-12)
    od, sd = oracle.decode_step_prologue(q[:, 0], k[:, 0], v[:, 0], x[:, 0], be[:, 0], S0, flags=DECAY)
    od2, sd2 = oracle.decode_step(q[:, 0], k[:, 0], v[:, 0], la[:, 0], be[:, 0], S0)
    np.testing.assert_allclose(od, od2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sd, sd2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("channel", [False, True])
def test_decay_softplus_exact_rational(channel):
    """Logits x = ln m (m a positive integer) give alpha = 1/(1+m) exactly: the
    prologue against the exact rational recurrence of oracle.exact."""
    from fractions import Fraction
    from oracle import exact
    r = _rng(71)
    T, dk, dv = 6, 3, 2
    fr = lambda lo, hi, den: Fraction(int(r.integers(lo, hi)), den)  # noqa: E731
    q = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    k = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    v = [[fr(-8, 9, 4) for _ in range(dv)] for _ in range(T)]
    m = r.integers(1, 9, (T, dk if channel else 1))
    alpha = [[Fraction(1, 1 + int(m[t, c if channel else 0])) for c in range(dk)] for t in range(T)]
    beta = [fr(0, 9, 8) for _ in range(T)]
    S0 = [[fr(-4, 5, 4) for _ in range(dk)] for _ in range(dv)]
    o_ex, s_ex = exact.run(q, k, v, alpha, beta, S0)
    f = lambda a: np.array([[float(x) for x in row] for row in a])  # noqa: E731
    x = np.log(m.astype(np.float64))
    x = x.reshape(1, T, 1, dk) if channel else x.reshape(1, T, 1)
    o, st = oracle.chunk_fwd_prologue(f(q).reshape(1, T, 1, dk), f(k).reshape(1, T, 1, dk),
                                      f(v).reshape(1, T, 1, dv), x,
                                      np.array([float(b) for b in beta]).reshape(1, T, 1),
                                      f(S0).reshape(1, 1, dv, dk), flags=DECAY)
    np.testing.assert_allclose(o[0, :, 0], f(o_ex), rtol=0, atol=1e-13)
    np.testing.assert_allclose(st[0, 0], f(s_ex), rtol=0, atol=1e-13)
