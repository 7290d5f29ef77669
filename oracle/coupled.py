"""Oracle of coupled-noise acceptance (test infrastructure only).

Source: page on SPOT (commit-order drafting for diffusion LMs), "how to use
it" section: the drafter and the target share one Gumbel noise table per
absolute output position (the paper's Proposition 2), so that, given the
noise, the target's next state is a deterministic function again and a draft
is verified by state equality: the candidate at a position is kept exactly
when it equals the target's noised argmax there.  Marginalised over the
noise, that argmax is a sample from the target distribution.  The walk
order and the longest-prefix commit are those of the SimSD page, section 4
(tau is the stage map of its section 2).

Readings:
- The noise enters as its exponential form: for Gumbel noise g_v the table
  holds E_v = exp(-g_v) (an Exp(1) variate, float32, > 0), and
  argmax_v (ln p_v + g_v) = argmax_v p_v / E_v.  The comparison of two
  candidates a, b is taken exactly: p_a * E_b against p_b * E_a, each a
  product of two float32 values and so exact in float64.  Equal scores go to
  the smaller index.
- Target token at position k: a_k = argmax over v of p[b][k][v] / E[b][k][v];
  a row with no positive p_v has no target token (a_k = -1).
- Walk: stages t = 1..gamma, k = tau^-1(t): keep the draft iff it equals
  a_k.  n = number kept; next_token = a_k at the first mismatch, or -1 after
  a full acceptance (no extra slot).  Positions with stage label 0 were
  committed in an earlier round of the block and are not walked; the walk
  covers stages 1..min(gamma, m), m the open positions (as in the
  rejection-sampling walk).

Pins (tests/test_oracle_coupled.py): the Gumbel-max distribution (the
stage-1 target token is distributed as p over many noise draws), brute-force
comparison with exact rational arithmetic, ties to the smaller index, the
noiseless limit (equal E: plain argmax of p), the walk's prefix semantics
with drafts planted from the target tokens, invariance of n under a
joint permutation of positions and tau, and committed positions (label 0)
reducing the walk to the one over the open positions alone.
"""

from __future__ import annotations

import numpy as np

from .acceptance import accept_status_ref, walked_stages


def target_token_ref(p_row, e_row):
    """Exact argmax of p_v / E_v (smallest index on ties); -1 without positive mass."""
    p = np.asarray(p_row, dtype=np.float32).astype(np.float64)
    e = np.asarray(e_row, dtype=np.float32).astype(np.float64)
    best = -1
    bp = be = 0.0
    for v in range(p.shape[0]):
        pv = p[v]
        if not pv > 0.0:
            continue
        ev = e[v]
        # pv / ev > bp / be  <=>  pv * be > bp * ev (exact products, be, ev > 0)
        if best < 0 or pv * be > bp * ev:
            best, bp, be = v, pv, ev
    return best


def target_tokens_ref(p, e):
    """Vectorised form of target_token_ref over the last axis (same decisions).

    The float64 ratio p/E is not used for the decision: among the entries
    whose ratio is within a relative 1e-12 of the row maximum (the only ones
    that can hold the exact maximum, since the ratio's rounding error is far
    below that) the exact pairwise products decide.
    """
    p = np.asarray(p, dtype=np.float32).astype(np.float64)
    e = np.asarray(e, dtype=np.float32).astype(np.float64)
    shp = p.shape[:-1]
    flat_p = p.reshape(-1, p.shape[-1])
    flat_e = e.reshape(-1, e.shape[-1])
    out = np.empty(flat_p.shape[0], dtype=np.int64)
    for i in range(flat_p.shape[0]):
        pr, er = flat_p[i], flat_e[i]
        pos = pr > 0.0
        if not pos.any():
            out[i] = -1
            continue
        r = np.where(pos, pr / er, -np.inf)
        m = r.max()
        cand = np.nonzero(r >= m * (1.0 - 1e-12))[0]
        best = int(cand[0])
        for v in cand[1:]:
            v = int(v)
            if pr[v] * er[best] > pr[best] * er[v]:
                best = v
        out[i] = best
    return out.reshape(shp)


def accept_coupled_ref(p, e, draft_tok, tau, gamma):
    """Walk every sequence in tau order with the coupled-noise match.

    p, e: [NB][B][V] float32 target probabilities and exponential noise;
    draft_tok: [NB][B]; tau: [NB][B] stage labels (0 for committed positions,
    a permutation of 1..m over the open ones).
    Returns (n_accepted, next_token, status) as int32 arrays [NB]; faulted
    sequences get n = next = -1.
    """
    draft_tok = np.asarray(draft_tok)
    tau = np.asarray(tau)
    NB, B = tau.shape
    V = p.shape[2]
    n_out = np.zeros(NB, dtype=np.int32)
    nx_out = np.full(NB, -1, dtype=np.int32)
    st_out = np.zeros(NB, dtype=np.int32)
    for b in range(NB):
        st = accept_status_ref(tau[b], draft_tok[b], gamma, V)
        st_out[b] = st
        if st:
            n_out[b] = -1
            continue
        kinv = [0] * (B + 1)
        for k in range(B):
            kinv[int(tau[b, k])] = k
        g = walked_stages(tau[b], gamma)
        n = g
        for t in range(1, g + 1):
            k = kinv[t]
            a = int(target_tokens_ref(p[b, k], e[b, k]))
            if a != int(draft_tok[b, k]):
                n = t - 1
                nx_out[b] = a
                break
        n_out[b] = n
    return n_out, nx_out, st_out
