"""Pins of the oracle's verification attention (float64, CPU).

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models": section 1 (paired D / D~ layout), section 2 (temporal mask, and its
purpose: the logits at a mask slot come from a temporally consistent context,
like the prefix-conditioned distribution of autoregressive verification) and
section 3 (RoPE copy).  The pins tie the oracle to library routines and to
closed forms rather than to itself:

* torch's float64 scaled_dot_product_attention over the state each row is
  meant to see (the "state identity"), with GQA by repeat_interleave;
* the all-visible mode against plain bidirectional attention;
* tau = identity against causal attention (the autoregressive special case);
* joint permutation of positions, tau and pos_d permutes the outputs;
* B = 1, P = 0, B = 0 and all-ties special cases;
* a pure-Python brute force over the explicitly enumerated visible set;
* RoPE against complex multiplication and a hand-worked example.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import MASK_FULL, ROPE_SEQUENTIAL, rope_rotate, verify_attn_ref


def _inputs(seed, NB, Hq, Hkv, d, P, B, p_max=None, ties=False):
    rng = np.random.default_rng(seed)
    p_max = P if p_max is None else p_max
    q = rng.standard_normal((NB, 2 * B, Hq, d))
    kb = rng.standard_normal((NB, 2 * B, Hkv, d))
    vb = rng.standard_normal((NB, 2 * B, Hkv, d))
    kc = rng.standard_normal((NB, Hkv, p_max, d))
    vc = rng.standard_normal((NB, Hkv, p_max, d))
    if ties:
        tau = rng.integers(1, B + 1, size=(NB, B))
    else:
        tau = np.stack([rng.permutation(B) + 1 for _ in range(NB)]) if B else np.zeros((NB, 0), int)
    plen = rng.integers(0, p_max + 1, size=NB) if p_max else np.zeros(NB, int)
    return q, kb, vb, kc, vc, plen, tau


def _sdpa(q, k, v, **kw):
    """torch float64 SDPA for one query vector set q [n][d] over k, v [m][d]."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, None]
    kt = torch.from_numpy(np.ascontiguousarray(k))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(v))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, **kw)[0, 0].numpy()


# ----------------------------------------------------------------------------- RoPE

def test_rope_against_complex_rotation():
    rng = np.random.default_rng(1)
    for d, base in [(4, 100.0), (64, 1e4), (128, 1e6)]:
        x = rng.standard_normal((7, d))
        pos = rng.integers(0, 20000, size=7)
        half = d // 2
        z = x[:, :half] + 1j * x[:, half:]
        ang = pos[:, None] * base ** (-np.arange(0, d, 2) / d)
        zr = z * np.exp(1j * ang)
        ref = np.concatenate([zr.real, zr.imag], axis=1)
        np.testing.assert_allclose(rope_rotate(x, pos, base), ref, rtol=0, atol=1e-12)


def test_rope_hand_example():
    # d = 4, base 100: frequencies 1 and 0.1; position 2 gives angles 2 and 0.2.
    x = np.array([1.0, 2.0, 3.0, 4.0])
    c2, s2, c02, s02 = math.cos(2), math.sin(2), math.cos(0.2), math.sin(0.2)
    want = [1 * c2 - 3 * s2, 2 * c02 - 4 * s02, 3 * c2 + 1 * s2, 4 * c02 + 2 * s02]
    np.testing.assert_allclose(rope_rotate(x, 2, 100.0), want, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(rope_rotate(x, 0, 100.0), x)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(2)
    x, y = rng.standard_normal((2, 128))
    for m, n in [(0, 5), (17, 3), (4100, 4097), (16000, 12)]:
        xm, yn = rope_rotate(x, m, 1e6), rope_rotate(y, n, 1e6)
        assert abs(np.linalg.norm(xm) - np.linalg.norm(x)) < 1e-12
        # <R(m) x, R(n) y> depends on m - n only
        ref = rope_rotate(x, m - n, 1e6) @ y if m >= n else x @ rope_rotate(y, n - m, 1e6)
        assert abs(xm @ yn - ref) < 1e-10


# ----------------------------------------------------------------------------- state identity

def _rot_block(q, kb, P, pos_d, b, base):
    B = q.shape[1] // 2
    pos = (P + np.arange(B)) if pos_d is None else np.asarray(pos_d[b])
    rp = np.concatenate([pos, pos])
    return rope_rotate(q[b], rp[:, None], base), rope_rotate(kb[b], rp[:, None], base)


@pytest.mark.parametrize("seed,NB,Hq,Hkv,d,P,B", [
    (11, 2, 4, 2, 16, 9, 4),
    (12, 1, 6, 3, 8, 0, 5),
    (13, 3, 2, 2, 32, 23, 7),
    (14, 1, 8, 1, 16, 4, 1),
])
def test_state_identity_against_sdpa(seed, NB, Hq, Hkv, d, P, B):
    q, kb, vb, kc, vc, plen, tau = _inputs(seed, NB, Hq, Hkv, d, P, B)
    base = 1e4
    out, lse, st = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, rope_base=base)
    assert not st.any()
    G = Hq // Hkv
    for b in range(NB):
        Pb = int(plen[b])
        qh, kh = _rot_block(q, kb, Pb, None, b, base)
        for i in range(B):
            # mask slot D~_i: prompt, then per position k the revealed token D_k if
            # its stage is earlier, otherwise the still-masked slot D~_k
            sel = [k if tau[b, k] < tau[b, i] else B + k for k in range(B)]
            # data token D_i: prompt plus data tokens of stage <= its own
            dsel = [k for k in range(B) if tau[b, k] <= tau[b, i]]
            for h in range(Hq):
                g = h // G
                keys = np.concatenate([kc[b, g, :Pb], kh[sel, g]])
                vals = np.concatenate([vc[b, g, :Pb], vb[b, sel, g]])
                ref = _sdpa(qh[B + i, h][None], keys, vals)[0]
                np.testing.assert_allclose(out[b, B + i, h], ref, rtol=0, atol=1e-12)
                s = (keys @ qh[B + i, h]) / math.sqrt(d)
                assert abs(lse[b, B + i, h] - torch.logsumexp(torch.from_numpy(s), 0).item()) < 1e-12
                keys = np.concatenate([kc[b, g, :Pb], kh[dsel, g]])
                vals = np.concatenate([vc[b, g, :Pb], vb[b, dsel, g]])
                ref = _sdpa(qh[i, h][None], keys, vals)[0]
                np.testing.assert_allclose(out[b, i, h], ref, rtol=0, atol=1e-12)


def test_gqa_grouping_is_contiguous():
    # Heads 0..G-1 read KV head 0, heads G..2G-1 read KV head 1 (repeat_interleave).
    q, kb, vb, kc, vc, plen, tau = _inputs(21, 1, 4, 2, 8, 6, 3)
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau)
    vc2 = vc.copy(); vc2[:, 1] += 10.0
    vb2 = vb.copy(); vb2[:, :, 1] += 10.0
    out2, _, _ = verify_attn_ref(q, kb, vb2, kc, vc2, plen, tau)
    np.testing.assert_allclose(out2[:, :, :2], out[:, :, :2], atol=1e-12)
    np.testing.assert_allclose(out2[:, :, 2:], out[:, :, 2:] + 10.0, atol=1e-9)


# ----------------------------------------------------------------------------- special cases

@pytest.mark.parametrize("P", [0, 13])
def test_full_mode_is_bidirectional_sdpa(P):
    q, kb, vb, kc, vc, plen, tau = _inputs(31, 2, 4, 2, 16, P, 5)
    plen[:] = P
    out, lse, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, mask_mode=MASK_FULL)
    for b in range(2):
        qh, kh = _rot_block(q, kb, P, None, b, 1e4)
        for h in range(4):
            g = h // 2
            keys = np.concatenate([kc[b, g, :P], kh[:, g]])
            vals = np.concatenate([vc[b, g, :P], vb[b, :, g]])
            ref = _sdpa(qh[:, h], keys, vals)
            np.testing.assert_allclose(out[b, :, h], ref, rtol=0, atol=1e-12)


def test_identity_order_data_rows_are_causal():
    # tau = identity: data rows are autoregressive (causal) verification.
    NB, Hq, Hkv, d, B = 1, 2, 1, 16, 6
    q, kb, vb, kc, vc, plen, tau = _inputs(41, NB, Hq, Hkv, d, 0, B)
    tau[:] = np.arange(1, B + 1)
    plen[:] = 0
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau)
    qh, kh = _rot_block(q, kb, 0, None, 0, 1e4)
    for h in range(Hq):
        ref = _sdpa(qh[:B, h], kh[:B, 0], vb[0, :B, 0], is_causal=True)
        np.testing.assert_allclose(out[0, :B, h], ref, rtol=0, atol=1e-12)


def test_identity_order_with_prompt_uses_prefix_causal_mask():
    NB, Hq, Hkv, d, B, P = 1, 2, 2, 8, 5, 7
    q, kb, vb, kc, vc, plen, tau = _inputs(42, NB, Hq, Hkv, d, P, B)
    tau[:] = np.arange(1, B + 1)
    plen[:] = P
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau)
    qh, kh = _rot_block(q, kb, P, None, 0, 1e4)
    allow = torch.from_numpy(np.concatenate([np.ones((B, P), bool), np.tril(np.ones((B, B), bool))], 1))
    for h in range(Hq):
        keys = np.concatenate([kc[0, h, :P], kh[:B, h]])
        vals = np.concatenate([vc[0, h, :P], vb[0, :B, h]])
        ref = _sdpa(qh[:B, h], keys, vals, attn_mask=allow[None, None])
        np.testing.assert_allclose(out[0, :B, h], ref, rtol=0, atol=1e-12)


def test_joint_permutation_equivariance():
    NB, Hq, Hkv, d, P, B = 2, 4, 2, 16, 11, 6
    q, kb, vb, kc, vc, plen, tau = _inputs(51, NB, Hq, Hkv, d, P, B)
    rng = np.random.default_rng(52)
    pos_d = np.stack([rng.permutation(B) + int(plen[b]) for b in range(NB)])
    out, lse, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, pos_d=pos_d)
    pi = rng.permutation(B)
    rows = np.concatenate([pi, B + pi])
    out2, lse2, _ = verify_attn_ref(q[:, rows], kb[:, rows], vb[:, rows], kc, vc, plen,
                                    tau[:, pi], pos_d=pos_d[:, pi])
    np.testing.assert_allclose(out2, out[:, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse[:, rows], rtol=0, atol=1e-12)


def test_single_position_block():
    q, kb, vb, kc, vc, plen, tau = _inputs(61, 2, 2, 1, 8, 5, 1)
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau)
    for b in range(2):
        Pb = int(plen[b])
        qh, kh = _rot_block(q, kb, Pb, None, b, 1e4)
        for h in range(2):
            for r in (0, 1):     # D_0 sees D_0; D~_0 sees D~_0 only
                keys = np.concatenate([kc[b, 0, :Pb], kh[r:r + 1, 0]])
                vals = np.concatenate([vc[b, 0, :Pb], vb[b, r:r + 1, 0]])
                np.testing.assert_allclose(out[b, r, h], _sdpa(qh[r, h][None], keys, vals)[0], atol=1e-12)


def test_empty_block_is_noop():
    q, kb, vb, kc, vc, plen, tau = _inputs(71, 3, 4, 2, 8, 5, 0)
    out, lse, st = verify_attn_ref(q, kb, vb, kc, vc, plen, tau)
    assert out.shape == (3, 0, 4, 8) and lse.shape == (3, 0, 4) and not st.any()


def test_block_contributes_nothing_when_hidden():
    # With B = 1 and a huge negative block key, every row is textbook attention
    # over the prompt alone.
    q, kb, vb, kc, vc, plen, tau = _inputs(72, 1, 2, 1, 8, 9, 1)
    plen[:] = 9
    q[..., 0] = 1.0 + np.abs(q[..., 0])
    kb[:] = 0.0
    kb[..., 0] = -1e4     # at position 0 RoPE is the identity, so every block score is < -3000
    pos_d = np.zeros((1, 1), int)
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, pos_d=pos_d)
    qh = rope_rotate(q[0], 0, 1e4)
    for r in (0, 1):
        for h in range(2):
            ref = _sdpa(qh[r, h][None], kc[0, 0, :9], vc[0, 0, :9])[0]
            np.testing.assert_allclose(out[0, r, h], ref, atol=1e-12)


def test_all_ties_reduce_to_bidirectional_block_steps():
    NB, Hq, Hkv, d, P, B = 1, 2, 1, 16, 6, 5
    q, kb, vb, kc, vc, plen, tau = _inputs(81, NB, Hq, Hkv, d, P, B)
    tau[:] = 1
    plen[:] = P
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau)
    qh, kh = _rot_block(q, kb, P, None, 0, 1e4)
    for h in range(Hq):
        for rows in (slice(0, B), slice(B, 2 * B)):
            keys = np.concatenate([kc[0, 0, :P], kh[rows, 0]])
            vals = np.concatenate([vc[0, 0, :P], vb[0, rows, 0]])
            np.testing.assert_allclose(out[0, rows, h], _sdpa(qh[rows, h], keys, vals), atol=1e-12)


def test_faulted_sequences_are_zero():
    q, kb, vb, kc, vc, plen, tau = _inputs(91, 4, 2, 1, 8, 6, 3)
    tau[1, 0] = -1                 # stage out of range
    plen[2] = 7                    # beyond P_max
    pos_d = np.stack([int(plen[b]) + np.arange(3) for b in range(4)])
    pos_d[3, 2] = -1               # negative position
    out, lse, st = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, pos_d=pos_d)
    assert st.tolist() == [0, 1, 4, 16]
    assert not out[1:].any() and np.all(np.isneginf(lse[1:]))
    assert np.abs(out[0]).sum() > 0


def _with_committed(rng, tau, c):
    """Label c positions of every sequence 0 (committed in an earlier round)
    and the open ones 1..B-c."""
    NB, B = tau.shape
    tau = np.zeros_like(tau)
    for b in range(NB):
        open_pos = np.sort(rng.permutation(B)[: B - c])
        tau[b, open_pos] = rng.permutation(B - c) + 1
    return tau


@pytest.mark.parametrize("seed,c", [(61, 1), (62, 3), (63, 5)])
def test_committed_positions_are_context_for_every_slot(seed, c):
    # A mask slot of an open position sees the prompt, the tokens committed in
    # earlier rounds, the open data tokens of earlier stages and the open
    # slots of its own or later stages (torch float64 SDPA on that state).
    NB, Hq, Hkv, d, P, B = 2, 4, 2, 16, 7, 6
    q, kb, vb, kc, vc, plen, tau = _inputs(seed, NB, Hq, Hkv, d, P, B)
    rng = np.random.default_rng(seed + 100)
    tau = _with_committed(rng, tau, c)
    out, _, st = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, rope_base=1e4)
    assert not st.any()
    for b in range(NB):
        Pb = int(plen[b])
        qh, kh = _rot_block(q, kb, Pb, None, b, 1e4)
        done = [k for k in range(B) if tau[b, k] == 0]
        for i in [k for k in range(B) if tau[b, k] > 0]:
            s = tau[b, i]
            cols = done + [k for k in range(B) if 0 < tau[b, k] < s] + \
                [B + k for k in range(B) if tau[b, k] >= s]
            for h in range(Hq):
                g = h // (Hq // Hkv)
                keys = np.concatenate([kc[b, g, :Pb], kh[cols, g]])
                vals = np.concatenate([vc[b, g, :Pb], vb[b, cols, g]])
                ref = _sdpa(qh[B + i, h][None], keys, vals)[0]
                np.testing.assert_allclose(out[b, B + i, h], ref, rtol=0, atol=1e-12)


def test_committed_label_acts_as_the_earliest_stages():
    # Relabelling the committed positions 1..c (any order) and shifting the
    # open stages by c leaves every open position's rows unchanged.
    NB, Hq, Hkv, d, P, B, c = 3, 4, 2, 8, 5, 7, 3
    q, kb, vb, kc, vc, plen, tau = _inputs(71, NB, Hq, Hkv, d, P, B)
    rng = np.random.default_rng(72)
    tau = _with_committed(rng, tau, c)
    tau2 = tau.copy()
    for b in range(NB):
        done = np.nonzero(tau[b] == 0)[0]
        tau2[b, tau[b] > 0] += c
        tau2[b, done] = rng.permutation(c) + 1
    out, lse, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau)
    out2, lse2, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau2)
    for b in range(NB):
        rows = [r for r in range(2 * B) if tau[b, r % B] > 0]
        np.testing.assert_allclose(out[b, rows], out2[b, rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b, rows], lse2[b, rows], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- brute force

def _brute_force(q, kb, vb, kc, vc, plen, tau, base, seq=False):
    """Pure-Python loops: enumerate each row's visible set, then softmax with math.exp.
    With ``seq`` the mask slots sit B positions after their data tokens."""
    NB, twoB, Hq, d = q.shape
    B = twoB // 2
    G = Hq // kb.shape[2]
    out = np.zeros_like(q)
    for b in range(NB):
        Pb = int(plen[b])
        pos = [Pb + k for k in range(B)]
        mpos = [p + B for p in pos] if seq else pos
        for h in range(Hq):
            g = h // G
            for r in range(twoB):
                i = r % B
                qr = [float(v) for v in rope_rotate(q[b, r, h], pos[i] if r < B else mpos[i], base)]
                cols = []
                for c in range(Pb):
                    cols.append((list(kc[b, g, c]), list(vc[b, g, c])))
                for j in range(B):
                    if r < B:
                        seen_d, seen_m = tau[b, j] <= tau[b, i], False
                    else:
                        seen_d, seen_m = tau[b, j] < tau[b, i], tau[b, j] >= tau[b, i]
                    if seen_d:
                        cols.append((list(rope_rotate(kb[b, j, g], pos[j], base)), list(vb[b, j, g])))
                    if seen_m:
                        cols.append((list(rope_rotate(kb[b, B + j, g], mpos[j], base)), list(vb[b, B + j, g])))
                scores = [sum(a * c for a, c in zip(qr, k)) / math.sqrt(d) for k, _ in cols]
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for wi, (_, v) in zip(w, cols):
                    for e in range(d):
                        out[b, r, h, e] += wi / tot * v[e]
    return out


@pytest.mark.parametrize("seed,P,B", [(101, 0, 3), (102, 5, 4), (103, 3, 2)])
def test_brute_force_tiny(seed, P, B):
    q, kb, vb, kc, vc, plen, tau = _inputs(seed, 2, 4, 2, 8, P, B)
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, rope_base=1e4)
    np.testing.assert_allclose(out, _brute_force(q, kb, vb, kc, vc, plen, tau, 1e4), rtol=0, atol=1e-12)


def test_brute_force_with_ties():
    q, kb, vb, kc, vc, plen, tau = _inputs(104, 1, 2, 1, 8, 4, 5, ties=True)
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, rope_base=1e4)
    np.testing.assert_allclose(out, _brute_force(q, kb, vb, kc, vc, plen, tau, 1e4), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,P,B", [(105, 0, 3), (106, 5, 4)])
def test_brute_force_without_rope_copy(seed, P, B):
    q, kb, vb, kc, vc, plen, tau = _inputs(seed, 2, 4, 2, 8, P, B)
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, rope_base=1e4, rope_mode=ROPE_SEQUENTIAL)
    want = _brute_force(q, kb, vb, kc, vc, plen, tau, 1e4, seq=True)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)


def _rope_complex(x, pos, base):
    """RoPE as multiplication of (x_f + i x_{f+d/2}) by exp(i pos base^(-2f/d))."""
    d = x.shape[-1]
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    zr = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * base ** (-np.arange(0, d, 2) / d))
    return np.concatenate([zr.real, zr.imag], axis=-1)


@pytest.mark.parametrize("P,with_pos", [(0, False), (11, False), (6, True)])
def test_without_rope_copy_full_mode_is_attention_over_consecutive_positions(P, with_pos):
    # All-visible mask: every block row attends to the prompt and all 2B block
    # rows, which sit at consecutive positions P_b .. P_b + 2B - 1 (or at
    # pos_d then pos_d + B): plain bidirectional attention over that layout.
    NB, Hq, Hkv, d, B = 2, 4, 2, 16, 5
    q, kb, vb, kc, vc, plen, tau = _inputs(33, NB, Hq, Hkv, d, P, B)
    plen[:] = P
    pos_d = np.array([[3, 40, 7, 9, 1], [100, 0, 2, 5, 6]]) if with_pos else None
    out, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, pos_d=pos_d, mask_mode=MASK_FULL,
                                rope_mode=ROPE_SEQUENTIAL)
    for b in range(NB):
        base_pos = np.asarray(pos_d[b]) if with_pos else P + np.arange(B)
        rp = np.concatenate([base_pos, base_pos + B])
        qh = _rope_complex(q[b], rp[:, None], 1e4)
        kh = _rope_complex(kb[b], rp[:, None], 1e4)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = np.concatenate([kc[b, g, :P], kh[:, g]])
            vals = np.concatenate([vc[b, g, :P], vb[b, :, g]])
            np.testing.assert_allclose(out[b, :, h], _sdpa(qh[:, h], keys, vals), rtol=0, atol=1e-12)
    # the two placements differ on the mask rows (the position shift is real)
    copy, _, _ = verify_attn_ref(q, kb, vb, kc, vc, plen, tau, pos_d=pos_d, mask_mode=MASK_FULL)
    assert np.abs(copy[:, B:] - out[:, B:]).max() > 1e-3
