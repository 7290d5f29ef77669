"""fp64 oracle of the tau-ordered acceptance walk (test infrastructure only).

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models", section 4 (speculative decoding pipeline), acceptance bullet: the
target applies standard rejection sampling following the temporal order the
draft induced, and commits the longest accepted prefix.  The stage map tau is
the permutation of section 2.

"Standard rejection sampling" is read as the textbook rule: the candidate x
drafted from q at stage t is kept with probability min(1, p(x)/q(x)); at the
first rejection a replacement is drawn from the normalised residual
max(0, p - q).  Uniforms come from Philox4x64-10 (Salmon et al., SC'11):
key = (seed, 0); the acceptance uniform of stage t of sequence b uses
counter (b, t, 0, offset) and keeps the top 24 bits of word 0; the residual
draw uses counter (b, n+1, 1, offset) and keeps the top 53 bits.  Keying by
stage (not by position) makes the accepted length invariant under a joint
permutation of positions and tau.

Stage label 0 marks a position committed in an earlier round of the block
(the process repeats, section 4): no walk visits it.  The other labels must
be exactly 1..m, m the number of open positions, and the walk covers stages
1..min(gamma, m); n = min(gamma, m) is a full acceptance.

The acceptance test ``u * q(x) < p(x)`` is exact in float64: u has 24
significant bits and q is a float32, so the product needs at most 48 bits.
The residual CDF is the sequential float64 prefix sum; ``next_token`` is the
first index whose prefix sum exceeds u' * S.  When every residual is zero the
draw falls back to p itself; when that sum is zero too it is -1.  After a
full acceptance (n = gamma) there is no extra slot, so ``next_token`` = -1.

Pins (tests/test_oracle_accept.py): greedy state equality with one-hot
targets, p = q, zero target mass, the first-stage acceptance probability
sum_v min(p_v, q_v) and the committed-token distribution p (chi-square over
many seeds), the residual distribution, invariance of n under a joint
permutation, and committed positions (label 0) reducing the walk to the one
over the open positions alone.
"""

from __future__ import annotations

import numpy as np

from .philox import philox4x64_10, uniform24, uniform53

ST_TAU_RANGE = 1
ST_TAU_NOT_PERM = 2
ST_TOKEN_RANGE = 8


def accept_status_ref(tau_b, draft_tok_b, gamma, vocab):
    """Fault flags of one sequence (0 = valid)."""
    tau_b = [int(t) for t in tau_b]
    B = len(tau_b)
    st = 0
    if any(t < 0 or t > B for t in tau_b):
        return ST_TAU_RANGE
    open_labels = sorted(t for t in tau_b if t > 0)
    if open_labels != list(range(1, len(open_labels) + 1)):
        return ST_TAU_NOT_PERM
    kinv = {t: k for k, t in enumerate(tau_b)}
    for t in range(1, walked_stages(tau_b, gamma) + 1):
        x = int(draft_tok_b[kinv[t]])
        if x < 0 or x >= vocab:
            st |= ST_TOKEN_RANGE
    return st


def walked_stages(tau_b, gamma):
    """Stages the walk covers: 1..min(gamma, m), m = open positions (label > 0)."""
    return min(int(gamma), sum(1 for t in tau_b if int(t) > 0))


def _draw(cdf_src, u):
    """First index whose sequential fp64 prefix sum exceeds u * total, or -1."""
    c = np.cumsum(cdf_src)
    s = c[-1]
    if not s > 0:
        return None
    return int(np.searchsorted(c, u * s, side="right"))


def accept_ref(p, q, draft_tok, tau, gamma, seed, offset=0):
    """Walk every sequence in tau order.

    p, q: [NB][B][V] float32 target / draft probabilities; row k belongs to
    response position k (p is read at the D~_k slot).
    draft_tok: [NB][B] tokens placed in D_k.  tau: [NB][B] stage labels: 0
    for committed positions, a permutation of 1..m over the m open ones.
    Returns (n_accepted [NB], next_token [NB], status [NB]) as int32 arrays;
    faulted sequences get n = next = -1.
    """
    draft_tok = np.asarray(draft_tok)
    tau = np.asarray(tau)
    NB, B = tau.shape
    V = p.shape[2]
    n_out = np.zeros(NB, dtype=np.int32)
    nx_out = np.full(NB, -1, dtype=np.int32)
    st_out = np.zeros(NB, dtype=np.int32)
    key = (int(seed), 0)
    for b in range(NB):
        st = accept_status_ref(tau[b], draft_tok[b], gamma, V)
        st_out[b] = st
        if st:
            n_out[b] = -1
            nx_out[b] = -1
            continue
        kinv = [0] * (B + 1)
        for k in range(B):
            kinv[int(tau[b, k])] = k
        g = walked_stages(tau[b], gamma)
        n = g
        for t in range(1, g + 1):
            k = kinv[t]
            x = int(draft_tok[b, k])
            u = uniform24(philox4x64_10((b, t, 0, offset), key)[0])
            pv = float(p[b, k, x])
            qv = float(q[b, k, x])
            if not (u * qv < pv):
                n = t - 1
                break
        n_out[b] = n
        if n < g:
            ks = kinv[n + 1]
            u2 = uniform53(philox4x64_10((b, n + 1, 1, offset), key)[0])
            p64 = np.asarray(p[b, ks], dtype=np.float64)
            q64 = np.asarray(q[b, ks], dtype=np.float64)
            pick = _draw(np.maximum(0.0, p64 - q64), u2)
            if pick is None:
                pick = _draw(p64, u2)
            nx_out[b] = -1 if pick is None else pick
    return n_out, nx_out, st_out
