"""Pins of the commit-step oracle (CPU).

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models", section 4 (the accepted prefix is committed and the process
repeats) and "Key contributions" item 3 (KV cache and blockwise decoding).
The pins check hand-worked rounds, counts, permutation invariance, and that
keys appended to the cache reproduce, under torch's float64 SDPA with RoPE
by complex multiplication, the attention over the finished block.
"""
import numpy as np
import torch

from oracle.acceptance import accept_ref
from oracle.attention import block_visibility
from oracle.commit import append_kv_ref, block_done, commit_ref, next_round_ref


def test_commit_hand_example():
    # B = 4, tau = (3, 1, 4, 2): stage 1 -> position 1, 2 -> 3, 3 -> 0, 4 -> 2
    tau = np.array([[3, 1, 4, 2], [3, 1, 4, 2], [3, 1, 4, 2]])
    draft = np.array([[10, 11, 12, 13]] * 3)
    n = np.array([2, 0, -1])
    nxt = np.array([99, 7, 5])
    c0 = np.zeros(3, dtype=np.uint64)
    t0 = np.full((3, 4), -1, dtype=np.int32)
    c, t = commit_ref(tau, draft, n, nxt, c0, t0)
    # sequence 0: stages 1, 2 keep drafts at positions 1, 3; stage 3 (position 0) takes 99
    assert t[0].tolist() == [99, 11, -1, 13] and int(c[0]) == 0b1011
    # sequence 1: nothing accepted; stage 1 (position 1) takes 7
    assert t[1].tolist() == [-1, 7, -1, -1] and int(c[1]) == 0b0010
    # sequence 2: faulted round, unchanged
    assert t[2].tolist() == [-1, -1, -1, -1] and int(c[2]) == 0


def test_commit_counts_and_full_acceptance():
    rng = np.random.default_rng(4)
    NB, B = 50, 8
    tau = np.stack([rng.permutation(B) + 1 for _ in range(NB)])
    draft = rng.integers(0, 1000, size=(NB, B))
    n = rng.integers(0, B + 1, size=NB)
    nxt = np.where(n < B, rng.integers(0, 1000, size=NB), -1)
    c, t = commit_ref(tau, draft, n, nxt, np.zeros(NB, dtype=np.uint64), np.full((NB, B), -1))
    for b in range(NB):
        want = int(n[b]) + (1 if nxt[b] >= 0 else 0)
        assert bin(int(c[b])).count("1") == want
        assert (t[b] >= 0).sum() == want
    full = block_done(c, B)
    assert all(full[b] == (n[b] + (nxt[b] >= 0) == B) for b in range(NB))


def test_commit_joint_permutation_invariance():
    rng = np.random.default_rng(6)
    NB, B = 20, 6
    tau = np.stack([rng.permutation(B) + 1 for _ in range(NB)])
    draft = rng.integers(0, 50, size=(NB, B))
    n = rng.integers(0, B, size=NB)
    nxt = rng.integers(0, 50, size=NB)
    c, t = commit_ref(tau, draft, n, nxt, np.zeros(NB, dtype=np.uint64), np.full((NB, B), -1))
    perm = rng.permutation(B)
    c2, t2 = commit_ref(tau[:, perm], draft[:, perm], n, nxt, np.zeros(NB, dtype=np.uint64), np.full((NB, B), -1))
    np.testing.assert_array_equal(t2, t[:, perm])
    for b in range(NB):
        bits = [(int(c[b]) >> k) & 1 for k in range(B)]
        bits2 = [(int(c2[b]) >> k) & 1 for k in range(B)]
        assert bits2 == [bits[p] for p in perm]


def test_next_round_hand_example():
    # B = 5, positions 1 and 3 committed (tokens 40, 41); the drafter ranks
    # the open positions 0, 2, 4 as 7, 2, 7: position 2 first, then the tie
    # 7 / 7 by position, 0 before 4.
    committed = np.array([0b01010], dtype=np.uint64)
    block_tok = np.array([[-1, 40, -1, 41, -1]])
    rank = np.array([[7, 0, 2, 0, 7]])
    draft = np.array([[10, 11, 12, 13, 14]])
    tau, tok = next_round_ref(committed, block_tok, rank, draft)
    assert tau.tolist() == [[2, 0, 1, 0, 3]]
    assert tok.tolist() == [[10, 40, 12, 41, 14]]
    tau, _ = next_round_ref(committed, block_tok, None, draft)  # no ranks: position order
    assert tau.tolist() == [[1, 0, 2, 0, 3]]


def test_next_round_labels_are_a_stable_sort_of_the_open_positions():
    rng = np.random.default_rng(12)
    NB, B = 40, 16
    committed = rng.integers(0, 1 << B, size=NB).astype(np.uint64)
    block_tok = rng.integers(0, 99, size=(NB, B))
    rank = rng.integers(0, 5, size=(NB, B))
    draft = rng.integers(100, 200, size=(NB, B))
    tau, tok = next_round_ref(committed, block_tok, rank, draft)
    for b in range(NB):
        bits = np.array([(int(committed[b]) >> k) & 1 for k in range(B)], bool)
        assert (tau[b, bits] == 0).all() and (tok[b, bits] == block_tok[b, bits]).all()
        assert (tok[b, ~bits] == draft[b, ~bits]).all()
        open_pos = np.nonzero(~bits)[0]
        order = open_pos[np.argsort(rank[b, open_pos], kind="stable")]
        assert tau[b, order].tolist() == list(range(1, len(open_pos) + 1))


def test_rounds_commit_the_whole_block():
    # Rounds of draft -> walk -> commit -> next labels: every round with an
    # open position commits at least one (the walk's replacement at the
    # first rejection, or every walked stage), so B rounds finish a block;
    # committed positions are visible to every open mask slot.
    rng = np.random.default_rng(13)
    NB, B, V = 16, 6, 12
    committed = np.zeros(NB, dtype=np.uint64)
    block_tok = np.full((NB, B), -1, dtype=np.int32)
    for rnd in range(B):
        lp = rng.normal(0, 1.5, (NB, B, V))
        p = np.exp(lp); p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
        lq = rng.normal(0, 1.5, (NB, B, V))
        q = np.exp(lq); q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
        draft = rng.integers(0, V, size=(NB, B)).astype(np.int32)
        tau, tok = next_round_ref(committed, block_tok, rng.integers(0, 100, size=(NB, B)), draft)
        for b in range(NB):
            vis = block_visibility(tau[b])
            done = tau[b] == 0
            for i in np.nonzero(~done)[0]:
                assert vis[B + i, :B][done].all() and not vis[B + i, B:][done].any()
        before = [bin(int(c)).count("1") for c in committed]
        n, nx, st = accept_ref(p, q, tok, tau, B, seed=3, offset=rnd)
        assert not st.any()
        committed, block_tok = commit_ref(tau, tok, n, nx, committed, block_tok)
        after = [bin(int(c)).count("1") for c in committed]
        for b in range(NB):
            assert after[b] - before[b] == (B - before[b] if before[b] == B else n[b] + (nx[b] >= 0))
            assert after[b] > before[b] or before[b] == B
    assert block_done(committed, B).all() and (block_tok >= 0).all()


def _rope_complex(x, pos, base):
    d = x.shape[-1]
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    zr = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * base ** (-np.arange(0, d, 2) / d))
    return np.concatenate([zr.real, zr.imag], axis=-1)


def test_appended_block_acts_as_prompt():
    # After the append, a query at position P + B attends over the cached
    # prefix, block included, exactly as over the prompt keys followed by the
    # block's keys rotated at P .. P + B - 1 (torch SDPA, complex RoPE).
    rng = np.random.default_rng(8)
    NB, B, Hkv, d, p_max, base = 2, 4, 2, 16, 40, 1e4
    P = np.array([10, 23])
    k_blk = rng.standard_normal((NB, 2 * B, Hkv, d))
    v_blk = rng.standard_normal((NB, 2 * B, Hkv, d))
    kc = rng.standard_normal((NB, Hkv, p_max, d))
    vc = rng.standard_normal((NB, Hkv, p_max, d))
    full = np.full(NB, (1 << B) - 1, dtype=np.uint64)
    kc2, vc2, plen2, st = append_kv_ref(k_blk, v_blk, None, full, P, kc, vc, base)
    assert (st == 0).all() and plen2.tolist() == (P + B).tolist()
    for b in range(NB):
        q = rng.standard_normal((1, d))
        qh = _rope_complex(q, np.array([P[b] + B]), base)
        for h in range(Hkv):
            keys = np.concatenate([kc[b, h, :P[b]], _rope_complex(k_blk[b, :B, h], P[b] + np.arange(B), base)])
            vals = np.concatenate([vc[b, h, :P[b]], v_blk[b, :B, h]])
            tq = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
            want = torch.nn.functional.scaled_dot_product_attention(tq(qh), tq(keys), tq(vals))[0, 0].numpy()
            got = torch.nn.functional.scaled_dot_product_attention(
                tq(qh), tq(kc2[b, h, :plen2[b]]), tq(vc2[b, h, :plen2[b]]))[0, 0].numpy()
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
        # rows past the block are untouched
        np.testing.assert_array_equal(kc2[b, :, plen2[b]:], kc[b, :, plen2[b]:])


def test_append_skips_open_blocks_and_flags_full_caches():
    rng = np.random.default_rng(9)
    NB, B, Hkv, d, p_max = 3, 4, 1, 8, 12
    k_blk = rng.standard_normal((NB, 2 * B, Hkv, d))
    v_blk = rng.standard_normal((NB, 2 * B, Hkv, d))
    kc = rng.standard_normal((NB, Hkv, p_max, d))
    vc = rng.standard_normal((NB, Hkv, p_max, d))
    committed = np.array([0b0111, 0b1111, 0b1111], dtype=np.uint64)
    P = np.array([2, 9, 8])
    kc2, vc2, plen2, st = append_kv_ref(k_blk, v_blk, None, committed, P, kc, vc, 1e4)
    assert plen2.tolist() == [2, 9, 12]           # open block, no room, appended
    assert st.tolist() == [0, 4, 0]
    np.testing.assert_array_equal(kc2[:2], kc[:2])
    np.testing.assert_array_equal(vc2[2, 0, 8:12], v_blk[2, :B, 0])
    # a negative given position is the attention's fault flag (16), and the
    # sequence is left unchanged; both flags together when there is no room
    pos = np.array([[5, 6, 7, 8], [9, 10, -1, 12], [0, 1, 2, -3]])
    full = np.full(NB, 0b1111, dtype=np.uint64)
    P = np.array([0, 2, 9])
    kc3, _, plen3, st3 = append_kv_ref(k_blk, v_blk, pos, full, P, kc, vc, 1e4)
    assert st3.tolist() == [0, 16, 4 | 16] and plen3.tolist() == [4, 2, 9]
    np.testing.assert_array_equal(kc3[1:], kc[1:])
