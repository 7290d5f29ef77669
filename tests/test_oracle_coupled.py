"""Pins of the coupled-noise acceptance oracle.

Source: the SPOT page's "how to use it" section (one shared Gumbel noise
table per absolute output position, Proposition 2: given the noise the
target's transition is a deterministic argmax, marginalised it is a sample
from the target distribution) and the SimSD page, section 4 (walk in the
drafted temporal order, longest accepted prefix).

Pins: the Gumbel-max law (stage-1 target tokens over many noise draws are
distributed as p: chi-square), exact rational brute force, ties to the
smaller index, the noiseless limit (plain argmax), zero target mass, the
prefix semantics with planted drafts, and invariance of the accepted length
under a joint permutation of positions and tau.
"""
from fractions import Fraction

import numpy as np
from scipy import stats

from oracle.coupled import accept_coupled_ref, target_token_ref, target_tokens_ref


def _exact_argmax(p_row, e_row):
    best, bval = -1, None
    for v, (pv, ev) in enumerate(zip(p_row, e_row)):
        if not float(pv) > 0.0:
            continue
        val = Fraction(float(np.float32(pv))) / Fraction(float(np.float32(ev)))
        if bval is None or val > bval:
            best, bval = v, val
    return best


def test_gumbel_max_law():
    # argmax_v p_v / E_v with E_v ~ Exp(1) i.i.d. picks v with probability p_v
    rng = np.random.default_rng(11)
    p = np.array([0.05, 0.1, 0.15, 0.3, 0.4], dtype=np.float32)
    n = 20000
    e = rng.exponential(size=(n, p.size)).astype(np.float32)
    picks = target_tokens_ref(np.broadcast_to(p, e.shape), e)
    counts = np.bincount(picks, minlength=p.size)
    _, pval = stats.chisquare(counts, n * p / p.sum())
    assert pval > 1e-4, (counts, pval)


def test_against_exact_rationals():
    rng = np.random.default_rng(5)
    for trial in range(40):
        V = int(rng.integers(1, 40))
        p = rng.random(V).astype(np.float32)
        p[rng.random(V) < 0.2] = 0.0
        e = rng.exponential(size=V).astype(np.float32)
        if trial % 5 == 0:  # planted exact ties of the ratio
            j = int(rng.integers(0, V))
            p[j] = np.float32(0.5)
            e[j] = np.float32(2.0)
            p[(j + 3) % V] = np.float32(0.25)
            e[(j + 3) % V] = np.float32(1.0)
        want = _exact_argmax(p, e)
        assert target_token_ref(p, e) == want
        assert int(target_tokens_ref(p, e)) == want


def test_ties_go_to_the_smaller_index():
    p = np.array([0.25, 0.5, 0.5], dtype=np.float32)
    e = np.array([0.5, 1.0, 1.0], dtype=np.float32)
    assert target_token_ref(p, e) == 0
    assert int(target_tokens_ref(p, e)) == 0


def test_noiseless_limit_is_plain_argmax():
    rng = np.random.default_rng(3)
    p = rng.random((20, 300)).astype(np.float32)
    e = np.ones_like(p)
    np.testing.assert_array_equal(target_tokens_ref(p, e), np.argmax(p, axis=-1))


def test_zero_mass_row_has_no_target():
    p = np.zeros(10, dtype=np.float32)
    e = np.ones(10, dtype=np.float32)
    assert target_token_ref(p, e) == -1
    assert int(target_tokens_ref(p, e)) == -1


def _inputs(rng, NB, B, V):
    lp = rng.normal(0, np.sqrt(2.0), (NB, B, V))
    p = np.exp(lp - lp.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    e = rng.exponential(size=(NB, B, V)).astype(np.float32)
    tau = np.stack([rng.permutation(B) + 1 for _ in range(NB)]).astype(np.int32)
    return p, e, tau


def test_prefix_semantics_with_planted_drafts():
    rng = np.random.default_rng(9)
    NB, B, V = 6, 5, 64
    p, e, tau = _inputs(rng, NB, B, V)
    a = target_tokens_ref(p, e)  # [NB][B] target token of every position
    gamma = 4
    for m in range(gamma + 1):
        draft = (a + 1) % V  # every draft wrong ...
        for b in range(NB):
            kinv = {int(t): k for k, t in enumerate(tau[b])}
            for t in range(1, m + 1):  # ... except the first m stages
                draft[b, kinv[t]] = a[b, kinv[t]]
        n, nx, st = accept_coupled_ref(p, e, draft.astype(np.int32), tau, gamma)
        assert (st == 0).all()
        assert (n == m).all()
        for b in range(NB):
            kinv = {int(t): k for k, t in enumerate(tau[b])}
            assert nx[b] == (-1 if m == gamma else a[b, kinv[m + 1]])


def test_committed_positions_reduce_to_the_open_walk():
    # Positions committed in an earlier round (label 0) are not walked, and
    # their drafts are not checked: the result equals the walk over the open
    # positions alone.
    rng = np.random.default_rng(23)
    NB, B, V, c = 7, 6, 40, 2
    p, e, _ = _inputs(rng, NB, B, V)
    a = target_tokens_ref(p, e)
    tau = np.zeros((NB, B), np.int32)
    sel = np.zeros((NB, B - c), int)
    for b in range(NB):
        sel[b] = np.sort(rng.permutation(B)[: B - c])
        tau[b, sel[b]] = rng.permutation(B - c) + 1
    draft = np.where(rng.random((NB, B)) < 0.8, a, (a + 3) % V).astype(np.int32)
    draft[tau == 0] = -5  # never checked
    take = lambda x: np.stack([x[b, sel[b]] for b in range(NB)])
    for gamma in (1, B - c, B):
        n, nx, st = accept_coupled_ref(p, e, draft, tau, gamma)
        n2, nx2, st2 = accept_coupled_ref(take(p), take(e), take(draft), take(tau), min(gamma, B - c))
        assert not st.any() and not st2.any()
        np.testing.assert_array_equal(n, n2)
        np.testing.assert_array_equal(nx, nx2)


def test_joint_permutation_invariance():
    rng = np.random.default_rng(21)
    NB, B, V = 5, 6, 48
    p, e, tau = _inputs(rng, NB, B, V)
    a = target_tokens_ref(p, e)
    draft = np.where(rng.random((NB, B)) < 0.7, a, (a + 7) % V).astype(np.int32)
    n0, nx0, _ = accept_coupled_ref(p, e, draft, tau, B)
    perm = rng.permutation(B)
    n1, nx1, _ = accept_coupled_ref(p[:, perm], e[:, perm], draft[:, perm], tau[:, perm], B)
    np.testing.assert_array_equal(n0, n1)
    np.testing.assert_array_equal(nx0, nx1)
