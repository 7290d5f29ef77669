"""Pins of the projection oracle (float64, CPU).

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models", section 4: one target forward pass over the paired layout; the
projections around its attention follow the nn.Linear convention (y = x W^T).
The pins do not re-call the oracle's matrix product: a pure-Python triple
loop and exact rationals, selection weights whose result is known by
construction, the identity projection and linearity.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle.projection import linear_ref, o_proj_ref, qkv_proj_ref


def _bf16(a):
    """Round float64 values to bfloat16 (nearest even) and back, for exact inputs."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (1, 1, 1), (4, 2, 16)])
def test_linear_against_triple_loop(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K))
    want = [[sum(float(x[m][k]) * float(w[n][k]) for k in range(K)) for n in range(N)] for m in range(M)]
    np.testing.assert_allclose(linear_ref(x, w), np.array(want), rtol=0, atol=1e-12)


def test_linear_exact_on_bf16_inputs():
    # products of bf16 values are exact in float64, and so is the sum of a
    # few dozen of them at these magnitudes: compare with exact rationals
    rng = np.random.default_rng(7)
    M, N, K = 3, 4, 48
    x = _bf16(rng.standard_normal((M, K)))
    w = _bf16(rng.standard_normal((N, K)))
    got = linear_ref(x, w)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(x[m, k])) * Fraction(float(w[n, k])) for k in range(K))
            assert got[m, n] == float(exact)


def test_qkv_split_order_and_row_layout():
    # selection weights: output channel c of the fused projection reads input
    # feature perm[c], so every q / k / v element names the feature it came from
    NB, B, Hq, Hkv, d = 2, 3, 4, 2, 8
    nout = (Hq + 2 * Hkv) * d
    H = nout + 5
    rng = np.random.default_rng(3)
    perm = rng.permutation(H)[:nout]
    w = np.zeros((nout, H))
    w[np.arange(nout), perm] = 1.0
    # x[b][r][f] = 1000 b + 100 r + f identifies sequence, block row and feature
    b_i, r_i, f_i = np.meshgrid(np.arange(NB), np.arange(2 * B), np.arange(H), indexing="ij")
    x = 1000.0 * b_i + 100.0 * r_i + f_i
    q, k, v = qkv_proj_ref(x, w, Hq, Hkv, d)
    for b in range(NB):
        for r in range(2 * B):
            base = 1000.0 * b + 100.0 * r
            for h in range(Hq):
                np.testing.assert_array_equal(q[b, r, h], base + perm[h * d:(h + 1) * d])
            for h in range(Hkv):
                np.testing.assert_array_equal(k[b, r, h], base + perm[Hq * d + h * d:Hq * d + (h + 1) * d])
                np.testing.assert_array_equal(v[b, r, h], base + perm[(Hq + Hkv) * d + h * d:(Hq + Hkv) * d + (h + 1) * d])


def test_o_proj_identity_and_linearity():
    rng = np.random.default_rng(5)
    NB, twoB, Hq, d = 2, 4, 3, 8
    a1 = rng.standard_normal((NB, twoB, Hq, d))
    a2 = rng.standard_normal((NB, twoB, Hq, d))
    eye = np.eye(Hq * d)
    np.testing.assert_array_equal(o_proj_ref(a1, eye), a1.reshape(NB, twoB, Hq * d))
    w = rng.standard_normal((10, Hq * d))
    lhs = o_proj_ref(2.0 * a1 - 3.0 * a2, w)
    rhs = 2.0 * o_proj_ref(a1, w) - 3.0 * o_proj_ref(a2, w)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-11)
