"""Pins for the fp64 CPU oracle: each check ties it to something other than itself.

* library routines it does not use (scipy's logsumexp, softmax and entropy),
* brute force at 40 significant digits with mpmath on tiny inputs,
* closed forms (two keys -> Bernoulli KL; uniform student -> ln n - H(P1)),
* invariants (Gibbs, identical models, single visible key, key translation,
  key permutation, zero row sums of dS),
* central finite differences of the forward for both gradient settings,
* the one number the pages print that has a checkable formula (the ~512 GB
  materialisation at 64K context, 32 heads, bf16).
The last group plants plausible mistakes in the oracle and checks that at
least one pin catches each of them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle import streamkl_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, n_q=7, n_k=9, d1=4, d2=4, std=1.0, independent=False):
    r = np.random.default_rng(seed)
    q1 = r.normal(size=(n_q, d1)) * std
    k1 = r.normal(size=(n_k, d1)) * std
    if independent or d1 != d2:
        q2 = r.normal(size=(n_q, d2)) * std
        k2 = r.normal(size=(n_k, d2)) * std
    else:
        q2 = q1 + 0.5 * r.normal(size=(n_q, d2))
        k2 = k1 + 0.5 * r.normal(size=(n_k, d2))
    return q1, k1, q2, k2


def brute_scores(q, k, scale):
    """Logits by explicit loops (independent of numpy matmul)."""
    n_q, n_k = q.shape[0], k.shape[0]
    S = np.empty((n_q, n_k))
    for i in range(n_q):
        for j in range(n_k):
            S[i, j] = scale * sum(float(q[i, t]) * float(k[j, t]) for t in range(q.shape[1]))
    return S


def visible(i, n_q, n_k, causal):
    return [j for j in range(n_k) if (not causal) or j <= i + (n_k - n_q)]


# --------------------------------------------------------------------------- library routines

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_forward_matches_scipy(seed, causal):
    q1, k1, q2, k2 = rand_case(seed, n_q=6, n_k=9, d1=5, d2=3)
    kl, l1, l2 = oracle.head_forward(q1, k1, q2, k2, causal)
    s1, s2 = 1 / math.sqrt(5), 1 / math.sqrt(3)
    S1, S2 = brute_scores(q1, k1, s1), brute_scores(q2, k2, s2)
    for i in range(6):
        js = visible(i, 6, 9, causal)
        assert l1[i] == pytest.approx(scipy.special.logsumexp(S1[i, js]), rel=1e-14, abs=1e-14)
        assert l2[i] == pytest.approx(scipy.special.logsumexp(S2[i, js]), rel=1e-14, abs=1e-14)
        p1 = scipy.special.softmax(S1[i, js])
        p2 = scipy.special.softmax(S2[i, js])
        assert kl[i] == pytest.approx(scipy.stats.entropy(p1, p2), rel=1e-12, abs=1e-15)


# --------------------------------------------------------------------------- 40-digit brute force

Q1_4 = [[1, 0], [0, 1], [1, 1], [-1, 2]]
K1_4 = [[1, 0], [0, 1], [-1, 1], [2, -1]]
Q2_4 = [[1, 1], [0, 1], [1, 0], [0, 2]]
K2_4 = [[1, 0], [1, 1], [-1, 0], [1, -1]]


def mp_forward(q1, k1, q2, k2, causal):
    """Definition of KL, LSE1, LSE2 evaluated in mpmath at the current precision."""
    n_q, n_k = len(q1), len(k1)
    out = []
    for i in range(n_q):
        js = visible(i, n_q, n_k, causal)
        s1 = [mpmath.mpf(sum(a * b for a, b in zip(q1[i], k1[j]))) for j in js]
        s2 = [mpmath.mpf(sum(a * b for a, b in zip(q2[i], k2[j]))) for j in js]
        z1 = mpmath.fsum(mpmath.exp(x) for x in s1)
        z2 = mpmath.fsum(mpmath.exp(x) for x in s2)
        p1 = [mpmath.exp(x) / z1 for x in s1]
        p2 = [mpmath.exp(x) / z2 for x in s2]
        kl = mpmath.fsum(a * mpmath.log(a / b) for a, b in zip(p1, p2))
        out.append((kl, mpmath.log(z1), mpmath.log(z2)))
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_4x4_brute_force_40_digits(causal):
    mpmath.mp.dps = 40
    ref = mp_forward(Q1_4, K1_4, Q2_4, K2_4, causal)
    kl, l1, l2 = oracle.head_forward(np.array(Q1_4), np.array(K1_4), np.array(Q2_4),
                                     np.array(K2_4), causal, scale1=1.0, scale2=1.0)
    for i, (rkl, rl1, rl2) in enumerate(ref):
        assert kl[i] == pytest.approx(float(rkl), rel=1e-13, abs=1e-15)
        assert l1[i] == pytest.approx(float(rl1), rel=1e-14)
        assert l2[i] == pytest.approx(float(rl2), rel=1e-14)


def test_4x4_gradients_40_digits():
    """Setting 1 and 2 gradients of the 4x4 case by 40-digit numerical differentiation."""
    mpmath.mp.dps = 40
    g = [mpmath.mpf(1) / 4] * 4

    def F(q1, k1, q2, k2):
        return mpmath.fsum(gi * r[0] for gi, r in zip(g, mp_forward(q1, k1, q2, k2, False)))

    def grad(which, row, col):
        base = [[[mpmath.mpf(v) for v in r] for r in m] for m in (Q1_4, K1_4, Q2_4, K2_4)]

        def f(x):
            m = [[list(r) for r in mm] for mm in base]
            m[which][row][col] = x
            return F(*m)
        return mpmath.diff(f, base[which][row][col])

    dq2, dk2 = oracle.head_backward(1, np.array(Q1_4), np.array(K1_4), np.array(Q2_4),
                                    np.array(K2_4), False, np.full(4, 0.25), 1.0, 1.0)
    dq1, dk1 = oracle.head_backward(2, np.array(Q1_4), np.array(K1_4), np.array(Q2_4),
                                    np.array(K2_4), False, np.full(4, 0.25), 1.0, 1.0)
    for r in range(4):
        for c in range(2):
            assert dq2[r, c] == pytest.approx(float(grad(2, r, c)), rel=1e-12, abs=1e-14)
            assert dk2[r, c] == pytest.approx(float(grad(3, r, c)), rel=1e-12, abs=1e-14)
            assert dq1[r, c] == pytest.approx(float(grad(0, r, c)), rel=1e-12, abs=1e-14)
            assert dk1[r, c] == pytest.approx(float(grad(1, r, c)), rel=1e-12, abs=1e-14)


# --------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("seed", range(4))
def test_two_keys_bernoulli_closed_form(seed):
    q1, k1, q2, k2 = rand_case(seed, n_q=5, n_k=2, d1=3, d2=3)
    kl, _, _ = oracle.head_forward(q1, k1, q2, k2, False, 1.0, 1.0)
    for i in range(5):
        a1 = float(q1[i] @ (k1[0] - k1[1]))
        a2 = float(q2[i] @ (k2[0] - k2[1]))
        p, q = 1 / (1 + math.exp(-a1)), 1 / (1 + math.exp(-a2))
        ref = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
        assert kl[i] == pytest.approx(ref, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_student_closed_form(causal):
    q1, k1, _, k2 = rand_case(5, n_q=6, n_k=10, d1=4, d2=4)
    q2 = np.zeros_like(q1)
    kl, _, l2 = oracle.head_forward(q1, k1, q2, k2, causal)
    S1 = brute_scores(q1, k1, 0.5)
    for i in range(6):
        js = visible(i, 6, 10, causal)
        ent = scipy.stats.entropy(scipy.special.softmax(S1[i, js]))
        assert kl[i] == pytest.approx(math.log(len(js)) - ent, rel=1e-12, abs=1e-14)
        assert l2[i] == pytest.approx(math.log(len(js)), rel=1e-14)


# --------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_gibbs_nonnegative(causal):
    for seed in range(10):
        q1, k1, q2, k2 = rand_case(seed, n_q=8, n_k=11, d1=6, d2=6, std=2.0, independent=True)
        kl, _, _ = oracle.head_forward(q1, k1, q2, k2, causal)
        assert (kl >= -1e-15).all()


@pytest.mark.parametrize("causal", [False, True])
def test_identical_models_give_zero(causal):
    q1, k1, _, _ = rand_case(3, n_q=6, n_k=8)
    kl, l1, l2 = oracle.head_forward(q1, k1, q1, k1, causal)
    assert np.abs(kl).max() < 1e-15 and np.array_equal(l1, l2)
    for s in (1, 2):
        dq, dk = oracle.head_backward(s, q1, k1, q1, k1, causal, np.ones(6))
        assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15


def test_causal_first_row_single_key():
    q1, k1, q2, k2 = rand_case(4, n_q=6, n_k=6)
    kl, l1, l2 = oracle.head_forward(q1, k1, q2, k2, True)
    assert kl[0] == 0.0
    assert l1[0] == pytest.approx(float(q1[0] @ k1[0]) / 2, rel=1e-15)
    assert l2[0] == pytest.approx(float(q2[0] @ k2[0]) / 2, rel=1e-15)
    for s in (1, 2):
        dq, _ = oracle.head_backward(s, q1, k1, q2, k2, True, np.ones(6))
        assert np.abs(dq[0]).max() == 0.0


@pytest.mark.parametrize("causal", [False, True])
def test_key_translation_invariance(causal):
    q1, k1, q2, k2 = rand_case(6, n_q=5, n_k=7, d1=4, d2=3)
    r = np.random.default_rng(9)
    u1, u2 = 3.0 * r.normal(size=4), 3.0 * r.normal(size=3)
    g = r.normal(size=5)
    kl, l1, l2 = oracle.head_forward(q1, k1, q2, k2, causal)
    klt, l1t, l2t = oracle.head_forward(q1, k1 + u1, q2, k2 + u2, causal)
    np.testing.assert_allclose(klt, kl, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l1t, l1 + (q1 @ u1) / 2, rtol=1e-12)
    np.testing.assert_allclose(l2t, l2 + (q2 @ u2) / math.sqrt(3), rtol=1e-12)
    for s in (1, 2):
        dq, dk = oracle.head_backward(s, q1, k1, q2, k2, causal, g)
        dqt, dkt = oracle.head_backward(s, q1, k1 + u1, q2, k2 + u2, causal, g)
        np.testing.assert_allclose(dqt, dq, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(dkt, dk, rtol=1e-9, atol=1e-12)


def test_key_permutation_noncausal():
    q1, k1, q2, k2 = rand_case(7, n_q=5, n_k=9)
    perm = np.random.default_rng(1).permutation(9)
    g = np.arange(1, 6) / 5
    kl, _, _ = oracle.head_forward(q1, k1, q2, k2, False)
    klp, _, _ = oracle.head_forward(q1, k1[perm], q2, k2[perm], False)
    np.testing.assert_allclose(klp, kl, rtol=1e-12, atol=1e-15)
    for s in (1, 2):
        _, dk = oracle.head_backward(s, q1, k1, q2, k2, False, g)
        _, dkp = oracle.head_backward(s, q1, k1[perm], q2, k2[perm], False, g)
        np.testing.assert_allclose(dkp, dk[perm], rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("setting", [1, 2])
def test_dk_columns_sum_to_zero(setting, causal):
    """Every row of dS sums to zero, hence sum_j dK[j] = 0 exactly (up to rounding)."""
    q1, k1, q2, k2 = rand_case(8, n_q=9, n_k=12, d1=5, d2=5)
    g = np.random.default_rng(2).normal(size=9)
    _, dk = oracle.head_backward(setting, q1, k1, q2, k2, causal, g)
    assert np.abs(dk.sum(axis=0)).max() < 1e-14 * max(1.0, np.abs(dk).max()) * 12


# --------------------------------------------------------------------------- finite differences

def fd_check(setting, causal, seed=11, n_q=6, n_k=9, d1=4, d2=3, h=1e-6):
    """Max relative error of the oracle's gradients against central differences."""
    q1, k1, q2, k2 = rand_case(seed, n_q=n_q, n_k=n_k, d1=d1, d2=d2)
    g = np.random.default_rng(seed + 1).normal(size=n_q)
    mats = [q1, k1, q2, k2]

    def F(ms):
        kl, _, _ = oracle.head_forward(*ms, causal)
        return float(g @ kl)

    dq, dk = oracle.head_backward(setting, *mats, causal, g)
    iq, ik = (2, 3) if setting == 1 else (0, 1)
    worst = 0.0
    for idx, ana in ((iq, dq), (ik, dk)):
        num = np.zeros_like(mats[idx])
        for pos in np.ndindex(*mats[idx].shape):
            plus = [m.copy() for m in mats]
            minus = [m.copy() for m in mats]
            plus[idx][pos] += h
            minus[idx][pos] -= h
            num[pos] = (F(plus) - F(minus)) / (2 * h)
        worst = max(worst, float(np.abs(num - ana).max() / max(np.abs(num).max(), 1e-30)))
    return worst


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("setting", [1, 2])
def test_finite_differences(setting, causal):
    assert fd_check(setting, causal) < 1e-6


def test_rows_and_dk_rows_consistent_with_full():
    q1, k1, q2, k2 = rand_case(12, n_q=10, n_k=10)
    g = np.linspace(-1, 1, 10)
    rows = np.array([0, 3, 9])
    kl, l1, l2 = oracle.head_forward(q1, k1, q2, k2, True)
    klr, l1r, l2r = oracle.head_forward(q1, k1, q2, k2, True, rows=rows)
    np.testing.assert_array_equal(klr, kl[rows])
    for s in (1, 2):
        dq, dk = oracle.head_backward(s, q1, k1, q2, k2, True, g, block=3)
        dqr, _ = oracle.head_backward(s, q1, k1, q2, k2, True, g, rows=rows)
        np.testing.assert_allclose(dqr, dq[rows], rtol=1e-13, atol=1e-16)
        dkt = oracle.head_backward_dk_rows(s, q1, k1, q2, k2, True, g, key_rows=[7, 8, 9])
        np.testing.assert_allclose(dkt, dk[[7, 8, 9]], rtol=1e-12, atol=1e-16)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("setting", [1, 2])
@pytest.mark.parametrize("dims", [(4, 4), (6, 3)])
def test_dk_keys_equals_full_dk(setting, causal, dims):
    """head_dk_keys (selected key columns, row statistics over all keys) gives
    the same dK rows as the full materialised backward, which the finite
    differences pin; with row statistics that are off by a constant it does not."""
    d1, d2 = dims
    q1, k1, q2, k2 = rand_case(20 + setting, n_q=9, n_k=13, d1=d1, d2=d2)
    g = np.random.default_rng(5).normal(size=9)
    stats = oracle.head_forward(q1, k1, q2, k2, causal)
    _, dk = oracle.head_backward(setting, q1, k1, q2, k2, causal, g)
    keys = np.array([12, 0, 5, 4, 12])
    got = oracle.head_dk_keys(setting, q1, k1, q2, k2, causal, g, keys, stats, block=4)
    np.testing.assert_allclose(got, dk[keys], rtol=1e-12, atol=1e-15)
    kl, l1, l2 = stats
    off = oracle.head_dk_keys(setting, q1, k1, q2, k2, causal, g, keys, (kl, l1 + 0.01, l2), block=4)
    assert np.abs(off - dk[keys]).max() > 1e-6


# --------------------------------------------------------------------------- setting-2 stability

def test_setting2_underflow_gives_zero_not_nan():
    """A P1 entry that underflows to exactly 0 yields dS1 = 0 with no NaN.

    Forming log P instead of logit differences would give -inf there (and NaN
    once multiplied by the zero probability), the failure the pages warn of.
    """
    q1 = np.array([[40.0, 0.0]])
    k1 = np.array([[1.0, 0.0], [-1.0, 0.0], [0.0, 0.0]])
    q2 = np.array([[0.0, 40.0]])
    k2 = np.array([[0.0, 1.0], [0.0, -1.0], [0.0, 0.0]])
    kl, _, _ = oracle.head_forward(q1, k1, q2, k2, False, 30.0, 30.0)
    assert np.isfinite(kl).all()
    dq, dk = oracle.head_backward(2, q1, k1, q2, k2, False, np.ones(1), 30.0, 30.0)
    assert np.isfinite(dq).all() and np.isfinite(dk).all()
    p1 = np.exp(30.0 * (q1 @ k1.T) - scipy.special.logsumexp(30.0 * (q1 @ k1.T)))
    assert p1[0, 1] == 0.0  # the underflowed entry really is zero
    # the key whose probability underflowed receives exactly zero gradient
    assert dk[1].tolist() == [0.0, 0.0]


# --------------------------------------------------------------------------- the pages' printed number

def test_materialised_bytes_matches_printed_figure():
    with open(os.path.join(GOLDEN, "materialised_64k_h32_bf16.json")) as f:
        fx = json.load(f)
    got = oracle.materialised_bytes(1, fx["heads"], fx["context"], fx["context"],
                                    fx["bytes_per_element"], 2)
    # the page prints "about 512 GB" and compares it with a 141 GB GPU
    assert got == 2 ** 39
    assert abs(got / 2 ** 30 - fx["printed_gb"]) / fx["printed_gb"] < 0.01
    assert got > fx["printed_gpu_capacity_gb"] * 1e9


def test_pair_count():
    assert oracle.pair_count(1, 1, 4, 4, False) == 16
    assert oracle.pair_count(1, 1, 4, 4, True) == 10
    assert oracle.pair_count(1, 2, 2, 5, True) == 2 * (3 + 2 * 3)
    m = oracle.valid_mask(np.arange(3), 3, 5, True)
    assert m.sum() == oracle.pair_count(1, 1, 3, 5, True)


# --------------------------------------------------------------------------- planted mistakes

def _mut_sign_setting1(setting, p1, p2, logp1, logp2, kl_rows, g_rows, mask):
    dS = g_rows[:, None] * (p1 - p2) if setting == 1 else _ORIG_DS(setting, p1, p2, logp1, logp2, kl_rows, g_rows, mask)
    return np.where(mask, dS, 0.0)


def _mut_drop_kl_setting2(setting, p1, p2, logp1, logp2, kl_rows, g_rows, mask):
    if setting == 2:
        return np.where(mask, g_rows[:, None] * p1 * np.where(mask, logp1 - logp2, 0.0), 0.0)
    return _ORIG_DS(setting, p1, p2, logp1, logp2, kl_rows, g_rows, mask)


def _mut_g_by_column(setting, p1, p2, logp1, logp2, kl_rows, g_rows, mask):
    dS = _ORIG_DS(setting, p1, p2, logp1, logp2, kl_rows, np.ones_like(g_rows), mask)
    n = dS.shape[1]
    gcol = np.resize(g_rows, n)
    return dS * gcol[None, :]


def _mut_row_stats_unmasked(S, mask):
    m = S.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]
    return lse, np.where(mask, S, -np.inf) - lse[:, None]


def _mut_mask_top_left(rows, n_q, n_k, causal):
    cols = np.arange(n_k)[None, :]
    return np.ones((len(rows), n_k), bool) if not causal else cols <= np.asarray(rows)[:, None]


_ORIG_DS = so._dS


def _pins_pass():
    """Run a compact set of the pins above; True if all pass."""
    try:
        for causal in (False, True):
            for s in (1, 2):
                if fd_check(s, causal, n_q=4, n_k=6, d1=3, d2=3) >= 1e-6:
                    return False
        test_causal_first_row_single_key()
        test_uniform_student_closed_form(True)
        # bottom-right alignment: with more keys than queries, row 0 sees n_k-n_q+1 keys
        q1, k1, q2, k2 = rand_case(1, n_q=3, n_k=5)
        kl, l1, _ = oracle.head_forward(q1, k1, q2 * 0, k2, True)
        if abs(kl[0] - (math.log(3) - scipy.stats.entropy(scipy.special.softmax(
                brute_scores(q1[:1], k1[:3], 0.5)[0])))) > 1e-12:
            return False
    except AssertionError:
        return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("target,mutant", [
    ("_dS", _mut_sign_setting1),
    ("_dS", _mut_drop_kl_setting2),
    ("_dS", _mut_g_by_column),
    ("_row_stats", _mut_row_stats_unmasked),
    ("valid_mask", _mut_mask_top_left),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(so, target, mutant)
    if target == "valid_mask":
        monkeypatch.setattr(oracle, "valid_mask", mutant)
    assert not _pins_pass()
