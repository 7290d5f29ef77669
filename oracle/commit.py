"""Oracle of the commit step between verification rounds (test infrastructure
only).

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models": section 4 (acceptance: the longest accepted prefix is committed and
the process repeats) and "Key contributions" item 3 (the method composes with
a KV cache and blockwise decoding: a finished block's keys and values join the
cached prefix).  Section 3 (RoPE copy) fixes the positions the keys were
rotated at.

Readings taken where the page is silent (also listed in the design notes):

* a round commits, in each sequence, the positions of stages 1..n (their
  drafted tokens) and, when the walk drew a replacement (next >= 0), the
  position of stage n+1 with that token; positions committed earlier keep
  their tokens unless a later round walks them again;
* the block state is a committed mask over the B response positions (bit k
  for position k) and the committed token of each position (-1 while open);
* a block is finished when all B positions are committed; its data rows
  D_0..D_{B-1} then join the cache: key k rotated at its RoPE position
  (pos_d[b][k], by default P_b + k, as in the verification pass) and value k
  as is, at cache rows P_b .. P_b + B - 1, and P_b grows by B; a sequence
  without room (P_b + B > p_max) is flagged and left unchanged, and so is one
  whose given positions hold a negative entry (the attention's fault flag
  for such positions);
* faulted rounds (n < 0) change nothing;
* the next round of the block (section 4: the process repeats; the drafter
  that proposes tokens and their order is outside this oracle) labels the
  committed positions with stage 0 and carries their tokens in D, and gives
  the open positions stages 1..m in the drafter's order (its rank per
  position, ties to the smaller position) with the drafter's tokens.

Pins (tests/test_oracle_commit.py): brute-force expectations on hand-built
rounds, the next round's labels as a stable sort of the open positions, the committed count growing by n (+1 with a replacement), invariance
under a joint permutation of positions and tau, and the appended keys
reproducing, under torch's float64 SDPA with RoPE by complex multiplication,
the attention of a query over the block written into the cache.
"""

from __future__ import annotations

import numpy as np

from .attention import ST_POS_NEG, ST_PROMPT_LEN, rope_rotate


def commit_ref(tau, draft_tok, n_accepted, next_token, committed, block_tok):
    """One round's commit.  tau, draft_tok [NB][B]; n_accepted, next_token [NB];
    committed [NB] (uint64 bit masks), block_tok [NB][B].  Returns the new
    (committed, block_tok) as copies."""
    tau = np.asarray(tau)
    NB, B = tau.shape
    committed = np.array(committed, dtype=np.uint64, copy=True)
    block_tok = np.array(block_tok, dtype=np.int32, copy=True)
    for b in range(NB):
        n = int(n_accepted[b])
        if n < 0:
            continue
        pos_of = {int(tau[b, k]): k for k in range(B)}
        for t in range(1, n + 1):
            k = pos_of[t]
            block_tok[b, k] = int(draft_tok[b, k])
            committed[b] |= np.uint64(1) << np.uint64(k)
        nx = int(next_token[b]) if next_token is not None else -1
        if nx >= 0 and (n + 1) in pos_of:
            k = pos_of[n + 1]
            block_tok[b, k] = nx
            committed[b] |= np.uint64(1) << np.uint64(k)
    return committed, block_tok


def next_round_ref(committed, block_tok, rank, draft_tok):
    """Stage labels and data tokens of the block's next round.

    committed [NB] masks, block_tok [NB][B]; rank [NB][B] (the drafter's
    order of the open positions, smaller first; None = position order);
    draft_tok [NB][B] (the drafter's tokens, read at open positions).
    Returns (tau [NB][B], tok [NB][B]) as int32 arrays.
    """
    block_tok = np.asarray(block_tok)
    NB, B = block_tok.shape
    tau = np.zeros((NB, B), dtype=np.int32)
    tok = np.zeros((NB, B), dtype=np.int32)
    for b in range(NB):
        c = int(np.uint64(committed[b]))
        open_pos = [k for k in range(B) if not (c >> k) & 1]
        key = (lambda k: (int(rank[b][k]), k)) if rank is not None else (lambda k: k)
        for t, k in enumerate(sorted(open_pos, key=key)):
            tau[b, k] = t + 1
            tok[b, k] = int(draft_tok[b][k])
        for k in range(B):
            if (c >> k) & 1:
                tok[b, k] = int(block_tok[b][k])
    return tau, tok


def block_done(committed, B):
    full = (1 << B) - 1 if B < 64 else (1 << 64) - 1
    return np.array([int(c) == full for c in np.asarray(committed, dtype=np.uint64)], dtype=bool)


def append_kv_ref(k_blk, v_blk, pos_d, committed, prompt_len, k_cache, v_cache, rope_base, done=None):
    """Append the data rows of finished blocks to the cache, in float64.

    k_blk, v_blk [NB][2B][Hkv][d] (rows 0..B-1 are the data rows); pos_d
    [NB][B] or None; committed [NB] masks or None (every block counts as
    finished); prompt_len [NB]; k_cache, v_cache [NB][Hkv][p_max][d].
    Returns (k_cache, v_cache, prompt_len, status) as new arrays.
    """
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    NB, twoB, Hkv, d = k_blk.shape
    B = twoB // 2
    k_cache = np.array(k_cache, dtype=np.float64, copy=True)
    v_cache = np.array(v_cache, dtype=np.float64, copy=True)
    p_max = k_cache.shape[2]
    plen = np.array(prompt_len, dtype=np.int64, copy=True)
    status = np.zeros(NB, dtype=np.int32)
    fin = np.ones(NB, dtype=bool) if committed is None else block_done(committed, B)
    for b in range(NB):
        if not fin[b] or B == 0:
            continue
        P = int(plen[b])
        if P < 0 or P + B > p_max:
            status[b] = ST_PROMPT_LEN
        if pos_d is not None and np.any(np.asarray(pos_d[b]) < 0):
            status[b] |= ST_POS_NEG
        if status[b]:
            continue
        pos = P + np.arange(B) if pos_d is None else np.asarray(pos_d[b], dtype=np.int64)
        kr = rope_rotate(k_blk[b, :B], pos[:, None], rope_base)  # [B][Hkv][d]
        for h in range(Hkv):
            k_cache[b, h, P:P + B] = kr[:, h]
            v_cache[b, h, P:P + B] = v_blk[b, :B, h]
        plen[b] = P + B
    return k_cache, v_cache, plen.astype(np.int32), status
