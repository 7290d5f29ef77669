"""fp64 oracle of the projections around the verification attention (test
infrastructure only).

Source: page "SimSD - Simple Speculative Decoding in Diffusion Language
Models", section 4 (pipeline): the target model runs ONE forward pass over
the paired data / mask layout, and that pass computes the logits of all
candidates.  Around the attention of each layer of that pass sit, as in any
transformer layer, the linear projection of the block rows' hidden states to
queries, keys and values and the projection of the attention output back to
the hidden size.  The pages print no layer shapes; the SDAR-8B-shaped
workloads use hidden size 4096 with 32 query and 8 KV heads of 128.

Readings taken where the pages are silent (also listed in the design notes):

* the nn.Linear convention: y = x W^T with W stored [out][in], no bias;
* the rows of the fused QKV weight are the Hq query heads (d rows each, head
  by head), then the Hkv key heads, then the Hkv value heads;
* the rows of x are the 2B block rows of every sequence in layout order
  (D_0..D_{B-1}, then D~_0..D~_{B-1}), sequence after sequence;
* no RoPE here: the attention's RoPE copy rotates q and k (its inputs are
  unrotated by contract).

The result is the plain definition, a float64 matrix product (the library
routine is the one step), then a reshape.

Pins (tests/test_oracle_projection.py): a pure-Python triple loop and exact
rational arithmetic on small shapes, hand-built selection weights that expose
the q / k / v split order and the row layout, the identity projection, and
linearity.
"""

from __future__ import annotations

import numpy as np


def linear_ref(x, w):
    """y[m][n] = sum_k x[m][k] * w[n][k] in float64 (x [M][K], w [N][K])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ w.T


def qkv_proj_ref(x, w_qkv, Hq, Hkv, d):
    """Block hidden states x [NB][2B][H] -> (q [NB][2B][Hq][d], k, v [NB][2B][Hkv][d])."""
    x = np.asarray(x, dtype=np.float64)
    NB, twoB, H = x.shape
    y = linear_ref(x.reshape(NB * twoB, H), w_qkv)
    nq, nk = Hq * d, Hkv * d
    q = y[:, :nq].reshape(NB, twoB, Hq, d)
    k = y[:, nq:nq + nk].reshape(NB, twoB, Hkv, d)
    v = y[:, nq + nk:nq + 2 * nk].reshape(NB, twoB, Hkv, d)
    return q, k, v


def o_proj_ref(attn, w_o):
    """Attention output attn [NB][2B][Hq][d] -> [NB][2B][H] with w_o [H][Hq*d]."""
    attn = np.asarray(attn, dtype=np.float64)
    NB, twoB, Hq, d = attn.shape
    y = linear_ref(attn.reshape(NB * twoB, Hq * d), w_o)
    return y.reshape(NB, twoB, -1)
