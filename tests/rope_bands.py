"""Band-limited inputs for checking a kernel's own RoPE-copy rotation.

Page "SimSD - Simple Speculative Decoding in Diffusion Language Models",
section 3: D~_k is rotated at D_k's RoPE position.  Rotate-half RoPE turns
frequency pair f (components f and f + d/2) by pos * base^(-2f/d), and no
other component enters that pair.  So when the block queries and keys are
zero outside the pairs of one band [f0, f0 + 8), every score, and so the
whole attention output, depends only on how that band is rotated: a kernel
that reads the wrong RoPE table entry, pairs the wrong granules or skips the
rotation for those pairs moves the output far from the oracle's, whatever it
does to the other pairs.

The positions are large (distinct, permuted, in [15000, 16370]), so every
band turns by many radians, and the amplitude puts the scores at O(1), so
the attention weights, and the outputs, follow the rotation closely.

`criterion` is the check the GPU tests apply: the kernel output must meet
the bf16 tolerance against the oracle and sit at least 10x closer (mean
absolute difference) to it than to each perturbed oracle that moves the
oracle's own output by at least 10x the bf16 mean tolerance (`strong`):
the block rotation left out, the other RoPE mode, or (P > 0: against the
cached prompt keys) every block position moved by one.  With base 2 every
pair turns by 0.5..1 rad per position, so leaving the rotation out or
moving by one position is plainly visible in every band; at base 1e6 the
low-frequency bands turn by less than a radian even at these positions, so
fewer perturbations qualify there.
"""
from __future__ import annotations

import numpy as np
import torch

from diffusion_lm_speculative_amd.synth import to_numpy64
from oracle.attention import verify_attn_ref

TOL_MAX = 2e-2
TOL_MEAN = 2e-3
BAND = 8           # frequency pairs per band
AMP = 2.0          # amplitude of the nonzero block components (scores of O(1))
POS_LO, POS_HI = 15000, 16370


def bands(d):
    """First pair index of every band of BAND pairs (covering all d/2 pairs)."""
    return list(range(0, d // 2, BAND))


def band_columns(d, f0):
    """Components of the pairs f0..f0+BAND-1: f and f + d/2."""
    f = np.arange(f0, f0 + BAND)
    return np.concatenate([f, f + d // 2])


def make_band_inputs(NB, Hq, Hkv, d, P, B, f0, seed, dtype=torch.bfloat16):
    """Block q/k zero outside band f0, cache keys and all values N(0, 1/4),
    positions a permutation of B distinct values in [POS_LO, POS_HI]."""
    g = torch.Generator().manual_seed(seed)
    cols = torch.as_tensor(band_columns(d, f0))
    mask = torch.zeros(d)
    mask[cols] = 1.0
    q = (torch.randn((NB, 2 * B, Hq, d), generator=g) * AMP * mask).to(dtype)
    kb = (torch.randn((NB, 2 * B, Hkv, d), generator=g) * AMP * mask).to(dtype)
    vb = (torch.randn((NB, 2 * B, Hkv, d), generator=g) * 0.5).to(dtype)
    kc = (torch.randn((NB, Hkv, P, d), generator=g) * AMP).to(dtype)
    vc = (torch.randn((NB, Hkv, P, d), generator=g) * 0.5).to(dtype)
    tau = torch.stack([torch.randperm(B, generator=g) + 1 for _ in range(NB)]).to(torch.int32)
    span = POS_HI - POS_LO + 1
    pos_d = torch.stack([torch.randperm(span, generator=g)[:B] + POS_LO for _ in range(NB)]).to(torch.int32)
    plen = torch.full((NB,), P, dtype=torch.int32)
    return dict(q_blk=q, k_blk=kb, v_blk=vb, k_cache=kc, v_cache=vc, tau=tau, prompt_len=plen, pos_d=pos_d)


def largest_angle(d, f0, base, pos=POS_HI):
    """Largest rotation angle (rad) of band f0 at position `pos`."""
    return pos * float(base) ** (-2.0 * f0 / d)


def criterion(got, good, perturbed):
    """(passed, report): bf16 tolerance against `good`, and at least 10x closer
    to `good` than to each array in `perturbed` (mean absolute difference)."""
    dg = np.abs(got - good)
    mx, mean = float(dg.max()), float(dg.mean())
    seps = [float(np.abs(got - pz).mean()) for pz in perturbed]
    ok = mx <= TOL_MAX and mean <= TOL_MEAN and all(mean * 10 < s for s in seps)
    rep = f"max={mx:.2e} mean={mean:.2e} perturbed_mean=[{', '.join(f'{s:.2e}' for s in seps)}]"
    return ok, rep


def oracle_out(t, base, rope_mode, pos_d):
    """The oracle's output for band inputs `t` (CPU tensors) at positions pos_d."""
    f = to_numpy64
    out, _, _ = verify_attn_ref(f(t["q_blk"]), f(t["k_blk"]), f(t["v_blk"]), f(t["k_cache"]), f(t["v_cache"]),
                                t["prompt_len"].numpy(), t["tau"].numpy(), pos_d=np.asarray(pos_d),
                                rope_base=base, rope_mode=rope_mode)
    return out


def perturbed_oracles(t, base, rope_mode, P):
    """Oracle outputs with the block rotation left out (all block positions
    0), in the other RoPE mode, and (P > 0) with every block position moved
    by one."""
    pos = t["pos_d"].numpy()
    outs = {"unrotated": oracle_out(t, base, rope_mode, np.zeros_like(pos)),
            "other_mode": oracle_out(t, base, 1 - rope_mode, pos)}
    if P > 0:
        outs["pos+1"] = oracle_out(t, base, rope_mode, pos + 1)
    return outs


def strong(perturbed, good):
    """The perturbations that move the oracle output by at least 10x the bf16
    mean tolerance (weaker ones could not separate a correct kernel)."""
    return {k: v for k, v in perturbed.items() if np.abs(v - good).mean() >= 10 * TOL_MEAN}
