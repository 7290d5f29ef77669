"""Pins of the oracle's tau-ordered acceptance walk.

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models", section 4 (pipeline, acceptance bullet): standard rejection sampling
in the drafted temporal order, committing the longest accepted prefix.  The
SPOT page's "how to use it" section supplies the greedy special case: at
temperature 0 a draft is accepted exactly when it equals the target's own
next state.

Pins: greedy state equality (one-hot targets, RNG-free), p = q, zero target
mass, joint permutation invariance, and the distributional facts of textbook
rejection sampling over many seeds: P(accept stage 1) = sum_v min(p_v, q_v),
the committed token at stage 1 is distributed as p, and the replacement is
distributed as the normalised residual max(0, p - q).
"""
import numpy as np
import pytest
from scipy import stats

from oracle.acceptance import accept_ref


def _probs(rng, NB, B, V, sigma=np.sqrt(2.0)):
    lp = rng.normal(0, sigma, (NB, B, V))
    lq = rng.normal(0, sigma, (NB, B, V))
    p = np.exp(lp - lp.max(-1, keepdims=True)); p /= p.sum(-1, keepdims=True)
    q = np.exp(lq - lq.max(-1, keepdims=True)); q /= q.sum(-1, keepdims=True)
    return p.astype(np.float32), q.astype(np.float32)


def _draft(rng, q):
    NB, B, V = q.shape
    x = np.zeros((NB, B), dtype=np.int32)
    for b in range(NB):
        for k in range(B):
            qq = q[b, k].astype(np.float64)
            x[b, k] = rng.choice(V, p=qq / qq.sum())
    return x


def _taus(rng, NB, B):
    return np.stack([rng.permutation(B) + 1 for _ in range(NB)]).astype(np.int32)


def test_greedy_state_equality():
    rng = np.random.default_rng(5)
    NB, B, V = 40, 8, 11
    p = np.zeros((NB, B, V), np.float32)
    am = rng.integers(0, V, (NB, B))
    for b in range(NB):
        for k in range(B):
            p[b, k, am[b, k]] = 1.0
    q = np.full((NB, B, V), 1.0 / V, np.float32)
    tau = _taus(rng, NB, B)
    x = np.where(rng.random((NB, B)) < 0.8, am, (am + 1) % V).astype(np.int32)
    for gamma in (0, 3, B):
        n, nxt, st = accept_ref(p, q, x, tau, gamma, seed=9)
        assert not st.any()
        for b in range(NB):
            run = 0
            order = np.argsort(tau[b])          # positions in stage order
            for k in order[:gamma]:
                if x[b, k] != am[b, k]:
                    break
                run += 1
            assert n[b] == run
            if run < gamma:
                assert nxt[b] == am[b, order[run]]   # residual of a one-hot target is that token
            else:
                assert nxt[b] == -1


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(6)
    p, _ = _probs(rng, 16, 6, 50)
    x = _draft(rng, p)
    n, nxt, _ = accept_ref(p, p, x, _taus(rng, 16, 6), 6, seed=3, offset=2)
    assert np.all(n == 6) and np.all(nxt == -1)


def test_zero_target_mass_caps_prefix():
    rng = np.random.default_rng(7)
    NB, B, V = 30, 6, 20
    p, q = _probs(rng, NB, B, V)
    x = _draft(rng, q)
    tau = _taus(rng, NB, B)
    for b in range(NB):
        t = 1 + b % B
        k = int(np.where(tau[b] == t)[0][0])
        p[b, k, x[b, k]] = 0.0
    n, _, _ = accept_ref(p, q, x, tau, B, seed=11)
    for b in range(NB):
        assert n[b] <= b % B


def test_joint_permutation_invariance():
    rng = np.random.default_rng(8)
    NB, B, V = 25, 7, 30
    p, q = _probs(rng, NB, B, V)
    x = _draft(rng, q)
    tau = _taus(rng, NB, B)
    n, nxt, _ = accept_ref(p, q, x, tau, 5, seed=77, offset=1)
    pi = rng.permutation(B)
    n2, nxt2, _ = accept_ref(p[:, pi], q[:, pi], x[:, pi], tau[:, pi], 5, seed=77, offset=1)
    assert np.array_equal(n, n2) and np.array_equal(nxt, nxt2)


def test_status_flags():
    rng = np.random.default_rng(9)
    p, q = _probs(rng, 4, 3, 5)
    x = np.zeros((4, 3), np.int32)
    tau = np.array([[1, 2, 3], [-1, 2, 3], [1, 1, 3], [3, 2, 1]], np.int32)
    x[3, 2] = 5                      # stage 1 of sequence 3 holds an out-of-range token
    n, nxt, st = accept_ref(p, q, x, tau, 3, seed=1)
    assert st.tolist() == [0, 1, 2, 8]
    assert n.tolist()[1:] == [-1, -1, -1] and nxt.tolist()[1:] == [-1, -1, -1]
    # label 0 (committed earlier): the open labels must be exactly 1..m, and a
    # committed position's token is never checked
    tau = np.array([[0, 2, 3], [0, 1, 2], [0, 0, 0], [2, 0, 1]], np.int32)
    x = np.zeros((4, 3), np.int32)
    x[1, 0] = x[2, 1] = x[3, 1] = -7
    n, nxt, st = accept_ref(p, q, x, tau, 3, seed=1)
    assert st.tolist() == [2, 0, 0, 0]
    assert n[2] == 0 and nxt[2] == -1  # nothing left to walk: a full acceptance


def _committed_inputs(rng, NB, B, c):
    """tau with c positions labelled 0 per sequence and the open ones 1..B-c."""
    tau = np.zeros((NB, B), np.int32)
    for b in range(NB):
        open_pos = np.sort(rng.permutation(B)[: B - c])
        tau[b, open_pos] = rng.permutation(B - c) + 1
    return tau


@pytest.mark.parametrize("c", [1, 3, 7])
def test_committed_positions_reduce_to_the_open_walk(c):
    # Positions committed in an earlier round (label 0) are not walked: the
    # result equals the walk over the open positions alone, a batch of B - c
    # positions with the same rows (stage-keyed uniforms keep the draws).
    rng = np.random.default_rng(30 + c)
    NB, B, V = 20, 8, 40
    p, q = _probs(rng, NB, B, V)
    x = _draft(rng, q)
    x[:, :] = np.where(rng.random((NB, B)) < 0.3, x, np.argmax(p, -1))  # some long prefixes
    tau = _committed_inputs(rng, NB, B, c)
    sel = np.stack([np.nonzero(tau[b])[0] for b in range(NB)])  # open positions, in order
    take = lambda a: np.stack([a[b, sel[b]] for b in range(NB)])
    for gamma in (0, 2, B - c, B):
        n, nxt, st = accept_ref(p, q, x, tau, gamma, seed=5, offset=3)
        n2, nxt2, st2 = accept_ref(take(p), take(q), take(x), take(tau), min(gamma, B - c), seed=5, offset=3)
        assert not st.any() and not st2.any()
        np.testing.assert_array_equal(n, n2)
        np.testing.assert_array_equal(nxt, nxt2)
        assert (n <= min(gamma, B - c)).all()


def _many_first_stage(p1, q1, trials, seed):
    """Run ``trials`` one-position sequences (B = gamma = 1) sharing p1 / q1."""
    rng = np.random.default_rng(seed)
    V = p1.size
    p = np.broadcast_to(p1, (trials, 1, V))
    q = np.broadcast_to(q1, (trials, 1, V))
    q64 = q1.astype(np.float64)
    x = rng.choice(V, size=(trials, 1), p=q64 / q64.sum()).astype(np.int32)
    tau = np.ones((trials, 1), np.int32)
    n, nxt, _ = accept_ref(p, q, x, tau, 1, seed=seed)
    return x[:, 0], n, nxt


def test_rejection_sampling_distribution():
    # The sequence index is part of the Philox counter, so each trial draws fresh uniforms.
    V = 6
    p1 = np.array([0.30, 0.05, 0.25, 0.10, 0.20, 0.10], np.float32)
    q1 = np.array([0.10, 0.30, 0.20, 0.25, 0.05, 0.10], np.float32)
    trials = 20000
    x, n, nxt = _many_first_stage(p1, q1, trials, seed=2024)
    # acceptance probability sum_v min(p_v, q_v)
    acc = np.minimum(p1.astype(np.float64), q1).sum()
    k = int((n == 1).sum())
    assert abs(k / trials - acc) < 4 * np.sqrt(acc * (1 - acc) / trials)
    # committed token ~ p
    committed = np.where(n == 1, x, nxt)
    counts = np.bincount(committed, minlength=V)
    p64 = p1.astype(np.float64)
    _, pval = stats.chisquare(counts, trials * p64 / p64.sum())
    assert pval > 1e-3
    # replacement ~ normalised residual
    res = np.maximum(0.0, p1.astype(np.float64) - q1)
    res /= res.sum()
    rc = np.bincount(nxt[n == 0], minlength=V)
    assert rc[res == 0].sum() == 0
    nz = res > 0
    _, pval = stats.chisquare(rc[nz], rc.sum() * res[nz])
    assert pval > 1e-3


def test_residual_falls_back_to_target_when_empty():
    # q dominates p everywhere except where p also vanishes: residual sum 0 is
    # impossible for normalised p, q unless p == q, which always accepts; with
    # unnormalised inputs (p <= q) the walk rejects and draws from p itself.
    p = np.array([[[0.0, 0.2, 0.0, 0.1]]], np.float32)
    q = np.array([[[0.5, 0.4, 0.5, 0.2]]], np.float32)
    x = np.array([[0]], np.int32)
    n, nxt, _ = accept_ref(p, q, x, np.array([[1]], np.int32), 1, seed=0)
    assert n[0] == 0 and nxt[0] in (1, 3)
