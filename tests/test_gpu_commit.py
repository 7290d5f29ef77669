"""GPU parity of the commit step between rounds (simsd_commit,
simsd_next_round, simsd_append_kv, through the C ABI) against the oracle.

Commit is integer work and must match bit for bit.  Appended keys are the
rotation of the attention kernels (fp32 from an fp64-reduced angle, rounded
to the cache dtype): within one bf16 ulp of the float64 oracle (fp32: 2e-6),
and bit-identical to the rotated data rows the attention path itself uses
(simsd_debug_rope).  Values, untouched cache rows, lengths and flags are
exact.  The next round's labels and tokens (simsd_next_round) match the
oracle exactly, and a multi-round loop (next labels, accept, commit, until
the block is full, then append) follows the oracle chain round by round.
"""
import numpy as np
import pytest
import torch

import diffusion_lm_speculative_amd as sd
from diffusion_lm_speculative_amd import synth
from oracle.acceptance import accept_ref
from oracle.commit import append_kv_ref, block_done, commit_ref, next_round_ref
from oracle.coupled import accept_coupled_ref, target_tokens_ref
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _masks_np(t):
    return t.cpu().numpy().view(np.uint64)


def test_commit_matches_oracle():
    g = torch.Generator().manual_seed(1)
    for NB, B in ((64, 8), (9, 64), (5, 1), (33, 16)):
        tau = torch.stack([torch.randperm(B, generator=g) + 1 for _ in range(NB)]).to(torch.int32)
        draft = torch.randint(0, 1000, (NB, B), generator=g, dtype=torch.int32)
        n = torch.randint(-1, B + 1, (NB,), generator=g, dtype=torch.int32)
        nx = torch.where(n < B, torch.randint(-1, 1000, (NB,), generator=g, dtype=torch.int32), -1).to(torch.int32)
        c0 = torch.randint(0, 2 ** 62, (NB,), generator=g, dtype=torch.int64)
        if B < 64:
            c0 &= (1 << B) - 1
        t0 = torch.randint(-1, 1000, (NB, B), generator=g, dtype=torch.int32)
        rc, rt = commit_ref(tau.numpy(), draft.numpy(), n.numpy(), nx.numpy(), c0.numpy().view(np.uint64), t0.numpy())
        for with_next in (True, False):
            c, t = c0.clone().to(dev()), t0.clone().to(dev())
            sd.commit(tau.to(dev()), draft.to(dev()), n.to(dev()), nx.to(dev()) if with_next else None, c, t)
            torch.cuda.synchronize()
            if with_next:
                assert np.array_equal(_masks_np(c), rc), (NB, B)
                assert np.array_equal(t.cpu().numpy(), rt), (NB, B)
            else:
                rc2, rt2 = commit_ref(tau.numpy(), draft.numpy(), n.numpy(), None, c0.numpy().view(np.uint64), t0.numpy())
                assert np.array_equal(_masks_np(c), rc2) and np.array_equal(t.cpu().numpy(), rt2)


def _one_ulp(want):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("with_pos", [False, True])
def test_append_matches_oracle(dtype, d, with_pos):
    NB, B, Hkv, p_max, base = 6, 8, 4, 300, 1e6
    g = torch.Generator().manual_seed(d + with_pos)
    k_blk = (torch.randn(NB, 2 * B, Hkv, d, generator=g) * 0.5).to(dtype)
    v_blk = (torch.randn(NB, 2 * B, Hkv, d, generator=g) * 0.5).to(dtype)
    kc = (torch.randn(NB, Hkv, p_max, d, generator=g) * 0.5).to(dtype)
    vc = (torch.randn(NB, Hkv, p_max, d, generator=g) * 0.5).to(dtype)
    plen = torch.tensor([0, 17, 292, 293, 200, 100], dtype=torch.int32)   # 293 + 8 > 300: no room
    full = (1 << B) - 1
    committed = torch.tensor([full, full, full, full, full - 1, full], dtype=torch.int64)  # sequence 4 still open
    pos_d = torch.stack([torch.randperm(B, generator=g) * 3 + 50 for _ in range(NB)]).to(torch.int32) if with_pos else None
    if with_pos:  # negative positions: flagged when finished (alone, and with no room), ignored when open
        pos_d[5, 2], pos_d[3, 0], pos_d[4, 1] = -4, -1, -2
    ref_k, ref_v, ref_len, ref_st = append_kv_ref(synth.to_numpy64(k_blk), synth.to_numpy64(v_blk),
                                                  None if pos_d is None else pos_d.numpy(),
                                                  committed.numpy().view(np.uint64), plen.numpy(),
                                                  synth.to_numpy64(kc), synth.to_numpy64(vc), base)
    kc_g, vc_g, len_g = kc.to(dev()), vc.to(dev()), plen.to(dev())
    st = sd.append_kv(k_blk.to(dev()), v_blk.to(dev()), kc_g, vc_g, len_g, rope_base=base,
                      committed=committed.to(dev()), pos_d=None if pos_d is None else pos_d.to(dev()))
    torch.cuda.synchronize()
    assert np.array_equal(len_g.cpu().numpy(), ref_len) and np.array_equal(st.cpu().numpy(), ref_st)
    assert ref_st.tolist() == ([0, 0, 0, 4 | 16, 0, 16] if with_pos else [0, 0, 0, 4, 0, 0])
    np.testing.assert_array_equal(synth.to_numpy64(vc_g), ref_v)
    got_k = synth.to_numpy64(kc_g)
    diff = np.abs(got_k - ref_k)
    if dtype == torch.float32:
        assert diff.max() < 2e-6
    else:
        assert np.all(diff <= np.maximum(_one_ulp(ref_k) * 1.0001, 1e-6))


def test_appended_keys_equal_the_attention_rotation():
    NB, B, Hq, Hkv, d, p_max, base = 4, 8, 8, 2, 128, 64, 1e6
    g = torch.Generator().manual_seed(3)
    q_blk = (torch.randn(NB, 2 * B, Hq, d, generator=g) * 0.5).to(torch.bfloat16).to(dev())
    k_blk = (torch.randn(NB, 2 * B, Hkv, d, generator=g) * 0.5).to(torch.bfloat16).to(dev())
    v_blk = torch.zeros_like(k_blk)
    plen = torch.tensor([0, 9, 30, 56], dtype=torch.int32, device=dev())
    _, k_rot = sd.debug_rope(q_blk, k_blk, plen, None, rope_base=base, p_max=p_max)
    kc = torch.zeros((NB, Hkv, p_max, d), dtype=torch.bfloat16, device=dev())
    vc = torch.zeros_like(kc)
    before = plen.clone()
    sd.append_kv(k_blk, v_blk, kc, vc, plen, rope_base=base)
    torch.cuda.synchronize()
    for b in range(NB):
        P = int(before[b])
        for h in range(Hkv):
            assert torch.equal(kc[b, h, P:P + B], k_rot[b, :B, h]), (b, h)


def test_next_round_matches_oracle():
    g = torch.Generator().manual_seed(3)
    for NB, B, with_rank in ((64, 8, True), (9, 64, True), (5, 1, False), (33, 16, True), (7, 12, False)):
        c = torch.randint(0, 2 ** 62, (NB,), generator=g, dtype=torch.int64)
        if B < 64:
            c &= (1 << B) - 1
        c[0] = 0
        c[1] = (1 << B) - 1 if B < 64 else -1  # every position committed
        bt = torch.randint(0, 1000, (NB, B), generator=g, dtype=torch.int32)
        x = torch.randint(1000, 2000, (NB, B), generator=g, dtype=torch.int32)
        rank = torch.randint(-3, 4, (NB, B), generator=g, dtype=torch.int32) if with_rank else None  # many ties
        print(f"next_round NB={NB} B={B} rank={with_rank}", flush=True)
        tau, tok = sd.next_round(c.to(dev()), bt.to(dev()), x.to(dev()), None if rank is None else rank.to(dev()))
        rtau, rtok = next_round_ref(c.numpy().view(np.uint64), bt.numpy(), None if rank is None else rank.numpy(),
                                    x.numpy())
        assert np.array_equal(tau.cpu().numpy(), rtau) and np.array_equal(tok.cpu().numpy(), rtok)


@pytest.mark.parametrize("coupled", [False, True])
def test_multi_round_loop_follows_the_oracle_chain(coupled):
    # One block of B positions decoded over rounds: each round labels the
    # committed positions 0 and drafts the open ones in a random order
    # (simsd_next_round), walks them (rejection sampling, or the coupled-noise
    # match) and commits the outcome, until the block is finished.
    NB, B, V, Hkv, d, p_max, base = 12, 8, 500, 2, 64, 64, 1e4
    rng = np.random.default_rng(21 + coupled)
    committed = torch.zeros(NB, dtype=torch.int64, device=dev())
    block_tok = torch.full((NB, B), -1, dtype=torch.int32, device=dev())
    r_c = np.zeros(NB, dtype=np.uint64)
    r_t = np.full((NB, B), -1, dtype=np.int32)
    seed = 77
    rounds = 0
    for rnd in range(B):
        inp = synth.make_accept_inputs(NB, B, V, seed=100 + rnd)
        p, q = inp["p"].numpy(), inp["q"].numpy()
        draft = inp["draft_tok"].numpy()
        rank = rng.integers(0, 4, size=(NB, B)).astype(np.int32)
        tau, tok = sd.next_round(committed, block_tok, torch.from_numpy(draft).to(dev()),
                                 torch.from_numpy(rank).to(dev()))
        rtau, rtok = next_round_ref(r_c, r_t, rank, draft)
        assert np.array_equal(tau.cpu().numpy(), rtau) and np.array_equal(tok.cpu().numpy(), rtok), rnd
        if coupled:
            e = synth.make_noise_exp(NB, B, V, seed=300 + rnd).numpy()
            a = target_tokens_ref(p, e)
            rtok = np.where(rng.random((NB, B)) < 0.7, a, rtok).astype(np.int32)  # mostly right drafts
            rtok[rtau == 0] = r_t[rtau == 0]
            tok = torch.from_numpy(rtok).to(dev())
            n, nx, st = sd.accept_coupled(torch.from_numpy(p).to(dev()), torch.from_numpy(e).to(dev()), tok, tau, B)
            rn, rnx, rst = accept_coupled_ref(p, e, rtok, rtau, B)
            assert np.array_equal(nx.cpu().numpy(), rnx)
        else:
            n, nx, st = sd.accept_prefix(torch.from_numpy(p).to(dev()), torch.from_numpy(q).to(dev()), tok, tau, B,
                                         seed, rnd)
            rn, rnx, rst = accept_ref(p, q, rtok, rtau, B, seed, rnd)
            # the replacement token may differ only at a CDF boundary (tested elsewhere); commit the oracle's
            nx = torch.from_numpy(rnx).to(dev())
        assert np.array_equal(n.cpu().numpy(), rn) and np.array_equal(st.cpu().numpy(), rst), rnd
        sd.commit(tau, tok, n, nx, committed, block_tok)
        r_c, r_t = commit_ref(rtau, rtok, rn, rnx, r_c, r_t)
        torch.cuda.synchronize()
        assert np.array_equal(_masks_np(committed), r_c) and np.array_equal(block_tok.cpu().numpy(), r_t), rnd
        rounds += 1
        if block_done(r_c, B).all():
            break
    assert block_done(r_c, B).all(), "every block completes within B rounds"
    print(f"  blocks finished in {rounds} rounds", flush=True)
    # the finished blocks join the cache
    g = torch.Generator().manual_seed(5)
    k_blk = (torch.randn(NB, 2 * B, Hkv, d, generator=g) * 0.5).to(torch.bfloat16)
    v_blk = (torch.randn(NB, 2 * B, Hkv, d, generator=g) * 0.5).to(torch.bfloat16)
    kc = torch.zeros((NB, Hkv, p_max, d), dtype=torch.bfloat16)
    plen = torch.randint(0, p_max - B + 1, (NB,), generator=g, dtype=torch.int32)
    ref_k, ref_v, ref_len, ref_st = append_kv_ref(synth.to_numpy64(k_blk), synth.to_numpy64(v_blk), None, r_c,
                                                  plen.numpy(), synth.to_numpy64(kc), synth.to_numpy64(kc), base)
    kc_g, vc_g, len_g = kc.to(dev()), kc.clone().to(dev()), plen.to(dev())
    st = sd.append_kv(k_blk.to(dev()), v_blk.to(dev()), kc_g, vc_g, len_g, rope_base=base, committed=committed)
    torch.cuda.synchronize()
    assert np.array_equal(len_g.cpu().numpy(), ref_len) and (st.cpu().numpy() == 0).all()
    np.testing.assert_array_equal(synth.to_numpy64(vc_g), ref_v)
    diff = np.abs(synth.to_numpy64(kc_g) - ref_k)
    assert np.all(diff <= np.maximum(_one_ulp(ref_k) * 1.0001, 1e-6))
