"""Pins of the oracle's block visibility (the tau-driven temporal mask).

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models", section 2 (temporal attention mask), plus the data-row convention
tau(j) <= tau(i).  Pins: hand-derived fixtures, closed-form counts, the
identity order, joint permutation equivariance, ties.
"""
import numpy as np
import pytest

from oracle.attention import MASK_FULL, block_visibility
from tests.golden import load_mask_fixture


@pytest.mark.parametrize("name", ["mask_tau_2_3_1.txt", "mask_tau_4_1_3_2.txt"])
def test_hand_derived_fixture(name):
    tau, vis = load_mask_fixture(name)
    assert block_visibility(tau).tolist() == vis


def _perms(seed, count, B):
    rng = np.random.default_rng(seed)
    return [rng.permutation(B) + 1 for _ in range(count)]


@pytest.mark.parametrize("B", [1, 2, 3, 5, 8, 16, 33, 64])
def test_closed_form_counts(B):
    for tau in _perms(B, 5, B):
        vis = block_visibility(tau)
        # each mask row sees exactly one of D_k / D~_k for every k
        for i in range(B):
            r = vis[B + i]
            assert np.all(r[:B] ^ r[B:])
            assert r.sum() == B
        # data row i sees tau_i data tokens and no slot
        assert np.array_equal(vis[:B, :B].sum(1), tau)
        assert not vis[:B, B:].any()
        assert vis.sum() == B * B + B * (B + 1) // 2


@pytest.mark.parametrize("B", [1, 4, 9])
def test_identity_order(B):
    vis = block_visibility(np.arange(1, B + 1))
    tri = np.tril(np.ones((B, B), dtype=bool))
    assert np.array_equal(vis[:B, :B], tri)             # causal incl. diagonal
    assert np.array_equal(vis[B:, :B], np.tril(tri, -1) & tri)   # strictly earlier data
    assert np.array_equal(vis[B:, :B], np.tril(np.ones((B, B), bool), -1))
    assert np.array_equal(vis[B:, B:], np.triu(np.ones((B, B), bool)))  # current/later slots


@pytest.mark.parametrize("B", [2, 5, 12])
def test_joint_permutation_equivariance(B):
    rng = np.random.default_rng(100 + B)
    for tau in _perms(B, 4, B):
        pi = rng.permutation(B)
        tau2 = tau[pi]
        rows = np.concatenate([pi, B + pi])
        assert np.array_equal(block_visibility(tau2), block_visibility(tau)[np.ix_(rows, rows)])


def test_self_visibility_and_no_future_data():
    for tau in _perms(3, 10, 7):
        vis = block_visibility(tau)
        B = 7
        for i in range(B):
            assert vis[i, i] and vis[B + i, B + i]
            assert not vis[B + i, i]          # strict inequality for D_i
            for j in range(B):
                if tau[j] > tau[i]:
                    assert not vis[B + i, j] and not vis[i, j]


def test_ties_all_same_stage():
    B = 6
    vis = block_visibility(np.ones(B, dtype=int))
    assert vis[:B, :B].all() and not vis[:B, B:].any()
    assert not vis[B:, :B].any() and vis[B:, B:].all()


def test_full_mode():
    assert block_visibility([3, 1, 2], MASK_FULL).all()


def test_empty_block():
    assert block_visibility([]).shape == (0, 0)
