"""fp64 oracle of the SimSD verification attention (test infrastructure only).

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models" (gist.science summary of arXiv 2606.02544):

* section 1 (input layout): after the prompt come two sections of length B,
  the data section D (reference tokens, context) and the mask section D~
  ([MASK] slots whose logits are the prediction targets); D_k and D~_k
  stand for the same response position.
* section 2 (temporal attention mask): a permutation assigns every response
  position a stage tau in {1..B}.  D~_i may attend to D_j only when
  tau(j) < tau(i), and to D~_j when tau(j) >= tau(i) (the current or a
  later, still undecided stage).  Future data tokens stay hidden.
* section 3 (position encoding alignment): D~_k reuses the RoPE index of
  D_k.
* "Experimental results", ablations: dropping that RoPE copy ruins the
  verification.  The page does not say which index the mask slots take
  without the copy; the plainest reading, taken here as ``rope_mode =
  ROPE_SEQUENTIAL``, is that the 2B block rows take consecutive indices in
  layout order, so D~_k sits B past D_k (P_b + B + k by default).

Readings taken where the page is silent (each is also listed in the design
notes):

* every block row sees the whole prompt prefix [0, P_b) (the page composes
  the method with a KV cache; block-diffusion models are causal between
  blocks and bidirectional inside one);
* a data row D_i sees D_j when tau(j) <= tau(i) and sees no D~ column;
* RoPE is the rotate-half (non-interleaved) form with frequencies
  base^(-2f/d); D_k and D~_k sit at pos_d[b][k], by default P_b + k;
  prompt keys are stored already rotated;
* softmax scale 1/sqrt(d); query head h reads KV head h // (Hq/Hkv);
* stage label 0 marks a response position committed in an earlier round of
  the same block (section 4: the process repeats): its token sits in D as
  context and, 0 being below every stage, every mask slot sees it; the open
  positions carry stages 1..m.  The predicates below apply unchanged.

The result is the plain definition: for every (sequence, query head, row)
the softmax over the explicitly constructed visible key set, in float64.
No blocking, splitting or online softmax.

Pins (tests/test_oracle_attention.py, tests/test_oracle_mask.py): torch's
float64 scaled_dot_product_attention on the state each mask row is meant to
reproduce, the all-visible mode against bidirectional attention, causal
attention for tau = identity, joint permutation equivariance, a pure-Python
brute-force enumeration on tiny inputs, RoPE against complex rotation and a
hand-worked example, and hand-derived masks under tests/golden/.  The
ablation's positions are pinned by plain bidirectional attention over the
block laid out at consecutive positions (RoPE by complex multiplication) and
by the brute force with shifted mask-slot indices.
"""

from __future__ import annotations

import numpy as np

MASK_TEMPORAL = 0
MASK_FULL = 1

# RoPE index of the mask slots: the method's copy, or the ablation's
# consecutive indices.
ROPE_COPY = 0
ROPE_SEQUENTIAL = 1

# Per-sequence fault flags (the same values the C-ABI documents).
ST_TAU_RANGE = 1
ST_PROMPT_LEN = 4
ST_POS_NEG = 16


def rope_rotate(x, pos, base):
    """Rotate the last axis of ``x`` (length d, even) by RoPE at ``pos``.

    Rotate-half form: for f in [0, d/2) the pair (x_f, x_{f+d/2}) is turned
    by the angle pos * base**(-2f/d).  ``pos`` broadcasts against
    ``x.shape[:-1]``.  All arithmetic is float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    f = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(base), -2.0 * f / d)
    theta = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c = np.cos(theta)
    s = np.sin(theta)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def block_visibility(tau, mode=MASK_TEMPORAL):
    """Boolean [2B, 2B]: entry [r, c] is True when block row r sees block column c.

    Rows and columns 0..B-1 are D_0..D_{B-1}; B..2B-1 are D~_0..D~_{B-1}.
    ``tau`` holds the stage of each response position (1-based; 0 for a
    position committed in an earlier round).  Ties are allowed: the
    predicates below stay well defined.
    """
    tau = [int(t) for t in tau]
    B = len(tau)
    vis = np.zeros((2 * B, 2 * B), dtype=bool)
    if mode == MASK_FULL:
        vis[:, :] = True
        return vis
    for i in range(B):
        for j in range(B):
            # data row D_i: data tokens decided no later than its own stage
            vis[i, j] = tau[j] <= tau[i]
            vis[i, B + j] = False
            # mask row D~_i: revealed data tokens (strictly earlier stages) ...
            vis[B + i, j] = tau[j] < tau[i]
            # ... and mask slots of the current or a later stage
            vis[B + i, B + j] = tau[j] >= tau[i]
    return vis


def verify_status_ref(tau, prompt_len, pos_d, p_max):
    """Per-sequence fault flags of a verification call (0 = valid)."""
    tau = np.asarray(tau)
    NB, B = tau.shape if tau.ndim == 2 else (tau.shape[0], 0)
    st = np.zeros(NB, dtype=np.int32)
    for b in range(NB):
        if B and (np.any(tau[b] < 0) or np.any(tau[b] > B)):
            st[b] |= ST_TAU_RANGE
        if prompt_len is not None:
            P = int(prompt_len[b])
            if P < 0 or P > p_max:
                st[b] |= ST_PROMPT_LEN
        if pos_d is not None and B and np.any(np.asarray(pos_d[b]) < 0):
            st[b] |= ST_POS_NEG
    return st


def verify_attn_ref(q_blk, k_blk, v_blk, k_cache, v_cache, prompt_len, tau,
                    pos_d=None, rope_base=10000.0, scale=None,
                    mask_mode=MASK_TEMPORAL, rope_mode=ROPE_COPY):
    """Attention of the 2B block rows of every sequence, in float64.

    Shapes (contiguous, any float dtype; values are read exactly):
      q_blk [NB][2B][Hq][d]  rows 0..B-1 are D_k, B..2B-1 are D~_k, unrotated
      k_blk, v_blk [NB][2B][Hkv][d]  (k unrotated)
      k_cache, v_cache [NB][Hkv][P_max][d]  prompt keys already rotated
      prompt_len [NB] or None (None means P_max for every sequence)
      tau [NB][B], pos_d [NB][B] or None (None means P_b + k)

    Returns (out [NB][2B][Hq][d], lse [NB][2B][Hq], status [NB]).  A
    sequence with a nonzero status gets zero output rows and lse = -inf.
    """
    q_blk = np.asarray(q_blk, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    tau = np.asarray(tau).astype(np.int64)
    NB, twoB, Hq, d = q_blk.shape
    B = twoB // 2
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    p_max = k_cache.shape[2]
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((NB, twoB, Hq, d), dtype=np.float64)
    lse = np.full((NB, twoB, Hq), -np.inf, dtype=np.float64)
    status = verify_status_ref(tau.reshape(NB, B), prompt_len, pos_d, p_max)
    if B == 0:
        return out, lse, status
    for b in range(NB):
        if status[b]:
            continue
        P = p_max if prompt_len is None else int(prompt_len[b])
        if pos_d is None:
            pos = P + np.arange(B, dtype=np.int64)
        else:
            pos = np.asarray(pos_d[b], dtype=np.int64)
        # RoPE copy: D~_k takes the position of D_k; without it (the
        # ablation) D~_k follows the data section, B positions later.
        row_pos = np.concatenate([pos, pos + B if rope_mode == ROPE_SEQUENTIAL else pos])
        q_hat = rope_rotate(q_blk[b], row_pos[:, None], rope_base)   # [2B][Hq][d]
        k_hat = rope_rotate(k_blk[b], row_pos[:, None], rope_base)   # [2B][Hkv][d]
        vis = np.concatenate(
            [np.ones((twoB, P), dtype=bool), block_visibility(tau[b], mask_mode)],
            axis=1)
        for h in range(Hq):
            g = h // G
            keys = np.concatenate(
                [np.asarray(k_cache[b, g, :P], dtype=np.float64), k_hat[:, g]], axis=0)
            vals = np.concatenate(
                [np.asarray(v_cache[b, g, :P], dtype=np.float64), v_blk[b, :, g]], axis=0)
            s = scale * (q_hat[:, h] @ keys.T)                        # [2B][P+2B]
            s = np.where(vis, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            e = np.exp(s - m)
            l = np.sum(e, axis=1, keepdims=True)
            out[b, :, h] = (e @ vals) / l
            lse[b, :, h] = (m + np.log(l))[:, 0]
    return out, lse, status
