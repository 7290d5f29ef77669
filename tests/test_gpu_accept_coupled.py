"""GPU parity of simsd_accept_coupled (through the C ABI) against the oracle.

Every decision is an exact comparison of fp32 products in fp64 on both
sides, so n_accepted, next_token and status must match bit for bit.  Drafts
are planted from the oracle's own target tokens for the first m stages of each
sequence (m spread over 0..gamma), so the walk's prefix lengths cover the
whole range instead of stopping at stage 1.
"""
import numpy as np
import pytest
import torch

import diffusion_lm_speculative_amd as sd
from diffusion_lm_speculative_amd import synth
from oracle.coupled import accept_coupled_ref, target_tokens_ref
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _plant(p, e, x, tau, gamma, seed):
    """Copy of x whose first m stages (m per sequence, seeded) hold the oracle's target tokens."""
    NB, B = tau.shape
    rng = np.random.default_rng(seed)
    x = x.copy()
    for b in range(NB):
        m = int(rng.integers(0, gamma + 1)) if gamma else 0
        for t in range(1, m + 1):
            hit = np.nonzero(tau[b] == t)[0]
            if not hit.size:  # fewer open positions than stages
                break
            k = int(hit[0])
            a = int(target_tokens_ref(p[b, k], e[b, k]))
            if a >= 0:
                x[b, k] = a
    return x


def _run(p, e, x, tau, gamma, workspace=None):
    NB, B, V = p.shape
    print(f"accept_coupled NB={NB} B={B} V={V} gamma={gamma}", flush=True)
    n, nx, st = sd.accept_coupled(torch.as_tensor(p).to(dev()), torch.as_tensor(e).to(dev()),
                                  torch.as_tensor(x).to(dev()), torch.as_tensor(tau).to(dev()), gamma,
                                  workspace=workspace)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nx.cpu().numpy(), st.cpu().numpy()


def _check(p, e, x, tau, gamma, workspace=None):
    n, nx, st = _run(p, e, x, tau, gamma, workspace)
    rn, rnx, rst = accept_coupled_ref(p, e, x, tau, gamma)
    assert np.array_equal(st, rst), (st, rst)
    assert np.array_equal(n, rn), (n, rn)
    assert np.array_equal(nx, rnx), (nx, rnx)
    print(f"  n histogram {np.bincount(n[n >= 0], minlength=gamma + 1).tolist()}", flush=True)
    return n, nx


def _inputs(NB, B, V, gamma, seed):
    inp = synth.make_accept_inputs(NB, B, V, seed=seed)
    p = inp["p"].numpy()
    e = synth.make_noise_exp(NB, B, V, seed=seed + 1).numpy()
    tau = inp["tau"].numpy()
    x = _plant(p, e, inp["draft_tok"].numpy(), tau, gamma, seed)
    return p, e, x, tau


# several chunks and ragged tails: V = 8193 is two chunks with a one-element
# tail; 4099 and 7 are not multiples of four (the scalar load path)
@pytest.mark.parametrize("NB,B,V,gamma", [(64, 8, 1000, 8), (40, 8, 1000, 3), (16, 4, 7, 4), (8, 64, 300, 64),
                                          (5, 3, 100000, 0), (33, 16, 4099, 16), (12, 8, 8193, 8),
                                          (9, 32, 20000, 32), (3, 1, 1, 1)])
def test_small(NB, B, V, gamma):
    p, e, x, tau = _inputs(NB, B, V, gamma, seed=NB * 100 + B)
    n, _ = _check(p, e, x, tau, gamma)
    if gamma >= 3 and NB >= 8:
        assert len(set(n.tolist())) >= 3  # the planted prefixes spread the lengths


def test_full_size_vocab():
    # batch 64, B = gamma = 16, V = 151936 (19 chunks of a row)
    w = synth.WORKLOADS["sdar8b_var16k_b16_accept"]
    p, e, x, tau = _inputs(w.NB, w.B, w.vocab, w.gamma, seed=1004)
    n, _ = _check(p, e, x, tau, w.gamma)
    assert n.max() >= w.gamma // 2


def test_large_batch():
    # batch 65535 (as the standard acceptance's largest), every sequence checked
    p, e, x, tau = _inputs(65535, 2, 40, 2, seed=2025)
    n, _ = _check(p, e, x, tau, 2)
    assert len(set(n.tolist())) == 3


def test_ties_across_chunks_go_to_the_smaller_index():
    # equal ratios p/E from different (p, E) pairs, placed in different chunks
    NB, B, V = 4, 4, 4 * 8192 + 5
    p = np.full((NB, B, V), 1e-6, dtype=np.float32)
    e = np.ones((NB, B, V), dtype=np.float32)
    for b in range(NB):
        for k in range(B):
            lo, hi = 100 + 8192 * b, 8192 * 2 + 300 + k  # lo < hi except where b == 3
            p[b, k, lo], e[b, k, lo] = 0.5, 1.0
            p[b, k, hi], e[b, k, hi] = 0.25, 0.5
    tau = np.tile(np.arange(1, B + 1, dtype=np.int32), (NB, 1))
    x = np.zeros((NB, B), dtype=np.int32)
    n, nx = _check(p, e, x, tau, B)
    assert nx.tolist() == [100, 100 + 8192, 100 + 8192 * 2, 8192 * 2 + 300]


def test_noiseless_limit_is_plain_argmax():
    NB, B, V = 16, 8, 5000
    inp = synth.make_accept_inputs(NB, B, V, seed=77)
    p = inp["p"].numpy()
    e = np.ones_like(p)
    tau = inp["tau"].numpy()
    am = p.argmax(-1).astype(np.int32)
    x = am.copy()
    x[:, 5] = (x[:, 5] + 1) % V  # position 5 mismatches
    n, nx, st = _run(p, e, x, tau, B)
    assert (st == 0).all()
    for b in range(NB):
        assert n[b] == tau[b, 5] - 1
        assert nx[b] == am[b, 5]


def test_zero_mass_row_has_no_target_token():
    NB, B, V = 6, 4, 999
    p, e, x, tau = _inputs(NB, B, V, B, seed=5)
    for b in range(NB):
        k = int(np.nonzero(tau[b] == 1 + b % B)[0][0])
        p[b, k] = 0.0
        p[b, k, b] = -1.0  # negative entries never win either
    x = _plant(p, e, x, tau, B, seed=6)
    n, nx = _check(p, e, x, tau, B)


@pytest.mark.parametrize("NB,B,V,gamma", [(40, 8, 1000, 8), (17, 16, 8193, 6), (5, 64, 300, 64)])
def test_committed_positions_are_not_walked(NB, B, V, gamma):
    inp = synth.make_accept_inputs(NB, B, V, seed=B + gamma)
    p = inp["p"].numpy()
    e = synth.make_noise_exp(NB, B, V, seed=B + gamma + 1).numpy()
    rng = np.random.default_rng(B * 7 + V)
    tau = np.zeros((NB, B), np.int32)
    for b in range(NB):
        c = b % (B + 1)
        open_pos = rng.permutation(B)[: B - c]
        tau[b, open_pos] = rng.permutation(B - c) + 1
    x = _plant(p, e, inp["draft_tok"].numpy(), tau, min(gamma, B), seed=B)
    x[tau == 0] = -9  # never checked
    n, _ = _check(p, e, x, tau, gamma)
    assert (n >= 0).all()


def test_faults_and_status():
    NB, B, V, gamma = 8, 8, 500, 6
    p, e, x, tau = _inputs(NB, B, V, gamma, seed=9)
    tau[1, 3] = -1           # label out of range
    tau[2, 3] = tau[2, 4]    # not a permutation
    x[3, int(np.nonzero(tau[3] == 2)[0][0])] = V       # drafted token out of range at a walked stage
    x[4, int(np.nonzero(tau[4] == 7)[0][0])] = -5      # ... at a stage beyond gamma: not checked
    n, nx = _check(p, e, x, tau, gamma)
    assert n[1] == n[2] == n[3] == -1 and n[4] >= 0


def test_workspace_reuse_and_shrinking_calls():
    NB, B, V, gamma = 24, 16, 30000, 16
    p, e, x, tau = _inputs(NB, B, V, gamma, seed=11)
    ws = torch.empty(sd.accept_coupled_workspace_bytes(NB, B, V), dtype=torch.uint8, device=dev())
    _check(p, e, x, tau, gamma, workspace=ws)
    p2, e2, x2, tau2 = _inputs(7, 8, 9000, 5, seed=12)
    _check(p2, e2, x2, tau2, 5, workspace=ws)
    _check(p, e, x, tau, gamma, workspace=ws)
