"""Pins of the fp64 oracle against facts fixed by the method and by mathematics.

None of these compares the oracle with itself: each check uses an independent
route (hand arithmetic, exact rational brute force over explicit transition
matrices, closed forms, invariants, finite differences, linearity).  Sources:
  * the recurrence S_t = S_{t-1} Diag(a_t)(I - b_t k_t k_t^T) + b_t v_t k_t^T,
    o_t = S_t q_t (scalar decay: Gated DeltaNet; channel decay: KDA) --
    "FG2-GDN" page, sections 1 and 5 ("Linear Attention as Recurrent Memory");
  * the delta rule as one SGD step on ||S^T k - v||^2 -- "FG2-GDN" page,
    section 5 ("Delta Rule and Online Learning");
  * KDA collapsing to Gated DeltaNet when the decay is tied across channels --
    "Daily Papers" pages, Gated DeltaNet-2 abstract;
  * forgetting of a state impulse -- "Daily Papers" (DeltaNet search page),
    the NVFP4 quantisation abstract (finding iii).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_inputs(seed, B=2, T=37, H=3, dk=5, dv=4, channel=False, s0=True):
    r = _rng(seed)
    q = _unit(r, (B, T, H, dk))
    k = _unit(r, (B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    la = r.uniform(-0.5, -0.001, (B, T, H, dk) if channel else (B, T, H))
    S0 = r.standard_normal((B, H, dv, dk)) * 0.3 if s0 else None
    return q, k, v, la, beta, S0


# --------------------------------------------------------------------------
# Hand-worked example (closed form, every step written out).
# d_k = d_v = 2, two tokens, channel gate.
#   S0 = [[1,0],[0,2]]
#   t=1: alpha=(1/2,1/4), beta=1/2, k=(3/5,4/5), v=(1,0), q=(1,0)
#        S0 Diag(alpha)            = [[1/2,0],[0,1/2]]
#        read p = S~ k             = (3/10, 2/5)
#        u = beta (v - p)          = (7/20, -1/5)
#        S1 = S~ + u k^T           = [[71/100, 7/25], [-3/25, 17/50]]
#        o1 = S1 q                 = (71/100, -3/25)
#   t=2: alpha=(1,1), beta=1, k=(0,1), v=(0,1), q=(1,1)
#        p = S1 k = (7/25, 17/50); u = (-7/25, 33/50)
#        S2 = [[71/100, 0], [-3/25, 1]];  o2 = (71/100, 22/25)
# The other order (erase, then decay) would give S1 = [[71/100, 17/50],
# [-6/25, 17/50]], so this example also fixes the order of decay and erase.
# --------------------------------------------------------------------------
HAND = dict(
    S0=[[1, 0], [0, 2]],
    alpha=[[Fraction(1, 2), Fraction(1, 4)], [1, 1]],
    beta=[Fraction(1, 2), 1],
    k=[[Fraction(3, 5), Fraction(4, 5)], [0, 1]],
    v=[[1, 0], [0, 1]],
    q=[[1, 0], [1, 1]],
    o=[[Fraction(71, 100), Fraction(-3, 25)], [Fraction(71, 100), Fraction(22, 25)]],
    S_T=[[Fraction(71, 100), 0], [Fraction(-3, 25), 1]],
)


def _hand_arrays():
    f = lambda x: np.array(x, dtype=np.float64)  # noqa: E731
    q = f([[float(a) for a in r] for r in HAND["q"]]).reshape(1, 2, 1, 2)
    k = f([[float(a) for a in r] for r in HAND["k"]]).reshape(1, 2, 1, 2)
    v = f(HAND["v"]).reshape(1, 2, 1, 2)
    la = f([[math.log(float(a)) for a in r] for r in HAND["alpha"]]).reshape(1, 2, 1, 2)
    be = f([float(b) for b in HAND["beta"]]).reshape(1, 2, 1)
    S0 = f(HAND["S0"]).reshape(1, 1, 2, 2)
    return q, k, v, la, be, S0


def test_hand_example_oracle():
    q, k, v, la, be, S0 = _hand_arrays()
    o, st = oracle.chunk_fwd(q, k, v, la, be, S0)
    want_o = np.array([[float(x) for x in r] for r in HAND["o"]])
    want_s = np.array([[float(x) for x in r] for r in HAND["S_T"]])
    np.testing.assert_allclose(o[0, :, 0, :], want_o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(st[0, 0], want_s, rtol=0, atol=1e-15)


def test_hand_example_exact():
    o, st = exact.run(HAND["q"], HAND["k"], HAND["v"], HAND["alpha"], HAND["beta"],
                      HAND["S0"])
    assert o == HAND["o"]
    assert st == HAND["S_T"]


# --------------------------------------------------------------------------
# Exact brute force over explicit transition matrices (tiny shapes).
# --------------------------------------------------------------------------
def _rational_case(seed, T, dk, dv, channel):
    r = _rng(seed)
    fr = lambda lo, hi, den: Fraction(int(r.integers(lo, hi)), den)  # noqa: E731
    q = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    k = [[fr(-8, 9, 8) for _ in range(dk)] for _ in range(T)]
    v = [[fr(-8, 9, 4) for _ in range(dv)] for _ in range(T)]
    if channel:
        alpha = [[fr(1, 9, 8) for _ in range(dk)] for _ in range(T)]
    else:
        alpha = [[fr(1, 9, 8)] * dk for _ in range(T)]
    beta = [fr(0, 9, 8) for _ in range(T)]
    S0 = [[fr(-4, 5, 4) for _ in range(dk)] for _ in range(dv)]
    return q, k, v, alpha, beta, S0


def _to_oracle(q, k, v, alpha, beta, S0, channel):
    T, dk, dv = len(q), len(q[0]), len(v[0])
    f = lambda x: np.array([[float(a) for a in row] for row in x])  # noqa: E731
    qa = f(q).reshape(1, T, 1, dk)
    ka = f(k).reshape(1, T, 1, dk)
    va = f(v).reshape(1, T, 1, dv)
    la = np.log(f(alpha))
    la = la.reshape(1, T, 1, dk) if channel else la[:, 0].reshape(1, T, 1)
    be = np.array([float(b) for b in beta]).reshape(1, T, 1)
    s0 = f(S0).reshape(1, 1, dv, dk)
    return qa, ka, va, la, be, s0


@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("seed,T,dk,dv", [(1, 1, 1, 1), (2, 5, 3, 2), (3, 8, 4, 4),
                                          (4, 7, 2, 3), (5, 6, 4, 1)])
def test_bruteforce_exact(seed, T, dk, dv, channel):
    case = _rational_case(seed, T, dk, dv, channel)
    o_ex, s_ex = exact.run(*case)
    o, st = oracle.chunk_fwd(*_to_oracle(*case, channel))
    o_ex = np.array([[float(x) for x in r] for r in o_ex])
    s_ex = np.array([[float(x) for x in r] for r in s_ex])
    scale = max(1.0, np.abs(o_ex).max(), np.abs(s_ex).max())
    np.testing.assert_allclose(o[0, :, 0, :], o_ex, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(st[0, 0], s_ex, rtol=0, atol=1e-12 * scale)


def test_golden_exact_fixture():
    """Stored exact results (written by tests/golden/make_golden.py from the
    rational brute force) against the fp64 oracle."""
    with open(os.path.join(GOLDEN, "exact_tiny.json")) as fh:
        cases = json.load(fh)
    assert len(cases) >= 4
    for c in cases:
        F = lambda x: [[Fraction(s) for s in row] for row in x]  # noqa: E731
        q, k, v, alpha, S0 = F(c["q"]), F(c["k"]), F(c["v"]), F(c["alpha"]), F(c["S0"])
        beta = [Fraction(s) for s in c["beta"]]
        o, st = oracle.chunk_fwd(*_to_oracle(q, k, v, alpha, beta, S0, c["channel"]))
        want_o = np.array([[float(Fraction(s)) for s in r] for r in c["o"]])
        want_s = np.array([[float(Fraction(s)) for s in r] for r in c["S_T"]])
        scale = max(1.0, np.abs(want_o).max(), np.abs(want_s).max())
        np.testing.assert_allclose(o[0, :, 0, :], want_o, rtol=0, atol=1e-12 * scale)
        np.testing.assert_allclose(st[0, 0], want_s, rtol=0, atol=1e-12 * scale)


# --------------------------------------------------------------------------
# Closed forms and invariants.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("channel", [False, True])
def test_beta0_alpha1_leaves_state(channel):
    q, k, v, la, be, S0 = _rand_inputs(10, channel=channel)
    la[:] = 0.0
    be[:] = 0.0
    o, st = oracle.chunk_fwd(q, k, v, la, be, S0)
    np.testing.assert_array_equal(st, S0)
    want = np.einsum("bhic,bthc->bthi", S0, q)
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("n", [1, 3, 8])
def test_orthonormal_keys_recall(n):
    """alpha=1, beta=1, orthonormal keys, zero start: S k_i = v_i for all i."""
    r = _rng(20 + n)
    dk, dv = 8, 5
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    keys = Qm[:, :n].T                                    # n orthonormal rows
    v = r.standard_normal((1, n, 1, dv))
    q = _unit(r, (1, n, 1, dk))
    la = np.zeros((1, n, 1))
    be = np.ones((1, n, 1))
    o, st = oracle.chunk_fwd(q, keys.reshape(1, n, 1, dk), v, la, be, None)
    S = st[0, 0]
    for i in range(n):
        np.testing.assert_allclose(S @ keys[i], v[0, i, 0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("channel", [False, True])
def test_unit_beta_writes_exactly(channel):
    """beta=1 and |k|=1: after any step, S_t k_t = v_t, for any alpha and S."""
    r = _rng(30)
    B, H, dk, dv = 3, 4, 16, 8
    q = _unit(r, (B, H, dk))
    k = _unit(r, (B, H, dk))
    v = r.standard_normal((B, H, dv))
    la = r.uniform(-3, 0, (B, H, dk) if channel else (B, H))
    be = np.ones((B, H))
    S = r.standard_normal((B, H, dv, dk))
    _, s1 = oracle.decode_step(q, k, v, la, be, S)
    got = np.einsum("bhic,bhc->bhi", s1, k)
    np.testing.assert_allclose(got, v, rtol=0, atol=1e-13)


def test_kda_tied_decay_is_gdn():
    """A channel decay that is the same on every channel is Gated DeltaNet."""
    q, k, v, la, be, S0 = _rand_inputs(40, channel=False)
    la_ch = np.repeat(la[..., None], q.shape[-1], axis=-1)
    o1, s1 = oracle.chunk_fwd(q, k, v, la, be, S0)
    o2, s2 = oracle.chunk_fwd(q, k, v, la_ch, be, S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("channel", [False, True])
def test_linearity_in_values_and_start_state(channel):
    q, k, v1, la, be, S01 = _rand_inputs(50, channel=channel)
    r = _rng(51)
    v2 = r.standard_normal(v1.shape)
    S02 = r.standard_normal(S01.shape)
    c = -0.7
    oa, sa = oracle.chunk_fwd(q, k, v1, la, be, S01)
    ob, sb = oracle.chunk_fwd(q, k, v2, la, be, S02)
    oc, sc = oracle.chunk_fwd(q, k, v1 + c * v2, la, be, S01 + c * S02)
    np.testing.assert_allclose(oc, oa + c * ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sc, sa + c * sb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("channel", [False, True])
def test_full_forgetting_closed_form(channel):
    """alpha -> 0 (log alpha = -800): S_t = beta_t v_t k_t^T and
    o_t = beta_t (k_t . q_t) v_t."""
    q, k, v, la, be, S0 = _rand_inputs(60, channel=channel)
    la[:] = -800.0
    o, st = oracle.chunk_fwd(q, k, v, la, be, S0)
    want_o = (be * np.einsum("bthc,bthc->bth", k, q))[..., None] * v
    np.testing.assert_allclose(o, want_o, rtol=0, atol=1e-14)
    last = np.einsum("bhi,bhc->bhic", be[:, -1, :, None] * v[:, -1], k[:, -1])
    np.testing.assert_allclose(st, last, rtol=0, atol=1e-14)


@pytest.mark.parametrize("channel", [False, True])
def test_beta0_pure_decay_closed_form(channel):
    """beta = 0: S_T = S0 Diag(prod_t alpha_t)."""
    q, k, v, la, be, S0 = _rand_inputs(70, channel=channel)
    be[:] = 0.0
    _, st = oracle.chunk_fwd(q, k, v, la, be, S0)
    tot = la.sum(axis=1)                          # [B,H] or [B,H,dk]
    fac = np.exp(tot) if channel else np.exp(tot)[..., None] * np.ones(q.shape[-1])
    np.testing.assert_allclose(st, S0 * fac[:, :, None, :], rtol=1e-12, atol=0)


@pytest.mark.parametrize("channel", [False, True])
def test_update_is_one_sgd_step(channel):
    """The write equals one gradient step of size beta on 0.5 ||S k - v||^2,
    taken at the decayed state; the gradient is measured by central finite
    differences (exact for a quadratic up to rounding)."""
    r = _rng(80)
    dk, dv = 6, 4
    q = _unit(r, (1, 1, dk))
    k = _unit(r, (1, 1, dk)) * 1.3                # any k, not only unit keys
    v = r.standard_normal((1, 1, dv))
    la = r.uniform(-1, 0, (1, 1, dk) if channel else (1, 1))
    be = np.array([[0.37]])
    S = r.standard_normal((1, 1, dv, dk))
    _, s1 = oracle.decode_step(q, k, v, la, be, S)
    a = np.exp(la[0, 0]) * np.ones(dk)
    Sd = S[0, 0] * a[None, :]                     # decayed state
    loss = lambda M: 0.5 * np.sum((M @ k[0, 0] - v[0, 0]) ** 2)  # noqa: E731
    h = 1e-3
    grad = np.zeros_like(Sd)
    for i in range(dv):
        for c in range(dk):
            E = np.zeros_like(Sd)
            E[i, c] = h
            grad[i, c] = (loss(Sd + E) - loss(Sd - E)) / (2 * h)
    np.testing.assert_allclose(s1[0, 0], Sd - 0.37 * grad, rtol=0, atol=1e-9)


def test_stability_and_impulse_forgetting():
    """|k|=1, alpha,beta in (0,1]: each step is a contraction plus a bounded
    write, so ||S_t|| <= ||S_{t-1}|| + beta ||v||; a start-state impulse decays
    at least as fast as the product of the largest per-step decays."""
    r = _rng(90)
    B, H, dk, dv, T = 1, 2, 16, 16, 300
    q = _unit(r, (B, T, H, dk))
    k = _unit(r, (B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    la = r.uniform(-0.05, -0.001, (B, T, H, dk))
    be = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    S = r.standard_normal((B, H, dv, dk))
    for t in range(T):
        prev = np.linalg.norm(S, axis=(2, 3))
        _, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], la[:, t], be[:, t], S)
        bound = prev + be[:, t] * np.linalg.norm(v[:, t], axis=-1)
        assert np.all(np.linalg.norm(S, axis=(2, 3)) <= bound * (1 + 1e-12))
    imp = r.standard_normal((B, H, dv, dk))
    _, sa = oracle.chunk_fwd(q, k, v, la, be, np.zeros((B, H, dv, dk)))
    _, sb = oracle.chunk_fwd(q, k, v, la, be, imp)
    resp = np.linalg.norm(sb - sa, axis=(2, 3))
    decay = np.exp(la.max(axis=-1).sum(axis=1))   # [B,H]
    assert np.all(resp <= np.linalg.norm(imp, axis=(2, 3)) * decay * (1 + 1e-9))


def test_chunk_equals_repeated_decode():
    q, k, v, la, be, S0 = _rand_inputs(100, channel=True, T=9)
    o, st = oracle.chunk_fwd(q, k, v, la, be, S0)
    S = S0.copy()
    for t in range(q.shape[1]):
        ot, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], la[:, t], be[:, t], S)
        np.testing.assert_array_equal(ot, o[:, t])
    np.testing.assert_array_equal(S, st)


def test_thread_count_does_not_change_result():
    q, k, v, la, be, S0 = _rand_inputs(110, B=3, H=5)
    o1, s1 = oracle.chunk_fwd(q, k, v, la, be, S0, threads=1)
    o2, s2 = oracle.chunk_fwd(q, k, v, la, be, S0, threads=7)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_empty_sequence_returns_start_state():
    q, k, v, la, be, S0 = _rand_inputs(120, T=0)
    o, st = oracle.chunk_fwd(q, k, v, la, be, S0)
    assert o.shape[1] == 0
    np.testing.assert_array_equal(st, S0)


# --------------------------------------------------------------------------
# Several tokens per call (verify a run of drafts, keep an accepted prefix).
# --------------------------------------------------------------------------
def test_decode_multi_is_repeated_decode_steps():
    q, k, v, la, be, S0 = _rand_inputs(400, B=3, T=6, channel=True)
    accepted = [0, 4, 6]
    o, s_out = oracle.decode_multi(q, k, v, la, be, S0, accepted)
    for b in range(3):
        S = S0[b:b + 1].copy()
        for t in range(6):
            sl = lambda a: np.ascontiguousarray(a[b:b + 1, t])  # noqa: E731
            ot, S = oracle.decode_step(sl(q), sl(k), sl(v), sl(la), sl(be), S)
            np.testing.assert_allclose(ot[0], o[b, t], rtol=0, atol=1e-13)
            if t + 1 == accepted[b]:
                np.testing.assert_allclose(S[0], s_out[b], rtol=0, atol=1e-13)
    np.testing.assert_array_equal(s_out[0], S0[0])     # nothing accepted: state kept


def test_decode_multi_clamps_and_defaults():
    q, k, v, la, be, S0 = _rand_inputs(401, B=2, T=5)
    o1, s1 = oracle.decode_multi(q, k, v, la, be, S0, [-3, 99])
    o2, s2 = oracle.decode_multi(q, k, v, la, be, S0, None)
    _, st = oracle.chunk_fwd(q, k, v, la, be, S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1[0], S0[0])
    np.testing.assert_allclose(s1[1], st[1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(s2, st, rtol=0, atol=1e-14)
