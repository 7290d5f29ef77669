"""The band-by-band RoPE check of the GPU tests sees rotation mistakes (CPU).

tests/test_gpu_rope_bands.py passes a kernel when its output meets the bf16
tolerance against the oracle and sits 10x closer to it than to perturbed
oracles.  Here, on the CPU, a stand-in for a correct bf16 kernel (the oracle
on inputs perturbed by half a bf16 unit, output rounded to bf16) passes that
check in every band, and the check fails when a rotation mistake is planted:

* pairs f >= d/4 left unrotated (half of the pairs: the mistake a review
  planted in the oracle, which the tolerance-only tests let through);
* each pair rotated with the upper-half partner of the next pair;
* each pair rotated at a neighbouring frequency.

Both directions are checked: the mistake in the kernel stand-in against the
correct oracle, and in the oracle against the correct stand-in.  At base 2
every mistake is visible in every band it touches; at base 1e6 the check
must fail wherever the mistake moves the oracle's own output by more than
10x the bf16 mean tolerance.
"""
import numpy as np
import pytest
import torch

import oracle.attention as oa
from tests.rope_bands import (TOL_MEAN, band_columns, bands, criterion, make_band_inputs, oracle_out,
                              perturbed_oracles, strong)

SHAPES = [("d128_rows64", 128, 8, 32, 8), ("d64_rows32", 64, 8, 8, 4)]


def _rot(x, pos, base, inv_freq, partner):
    """Rotate-half RoPE with a given frequency per pair and upper-half partner index per pair."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    theta = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(theta), np.sin(theta)
    x1, x2 = x[..., :half], x[..., half:][..., partner]
    out = x.copy()
    out[..., :half] = x1 * c - x2 * s
    out[..., half + partner] = x2 * c + x1 * s
    return out


def mistake(kind):
    """A wrong rotation in the oracle's signature (x, pos, base)."""
    def rot(x, pos, base):
        d = np.asarray(x).shape[-1]
        half = d // 2
        f = np.arange(half, dtype=np.float64)
        inv = np.power(np.float64(base), -2.0 * f / d)
        partner = np.arange(half)
        if kind == "skip_upper_quarter":
            inv = np.where(f >= d // 4, 0.0, inv)
        elif kind == "next_partner":
            partner = (partner + 1) % half
        elif kind == "neighbour_frequency":
            inv = np.power(np.float64(base), -2.0 * np.where(f + 1 < half, f + 1, f - 1) / d)
        return _rot(x, pos, base, inv, partner)
    return rot


def touches(kind, d, f0):
    """Whether the mistake changes the rotation of band f0."""
    return f0 >= d // 4 if kind == "skip_upper_quarter" else True


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32).to(torch.bfloat16).double().numpy()


def kernel_standin(t, base, rope_mode, seed):
    """Oracle on block q/k perturbed by up to half a bf16 unit, output rounded to bf16."""
    rng = np.random.default_rng(seed)
    t2 = dict(t)
    for k in ("q_blk", "k_blk"):
        x = t[k].to(torch.float32)
        e = torch.from_numpy(rng.uniform(-2.0 ** -9, 2.0 ** -9, size=tuple(x.shape)))
        t2[k] = (x.double() * (1.0 + e)).to(torch.float32)
    return _bf16(oracle_out(t2, base, rope_mode, t["pos_d"].numpy()))


def test_band_inputs_are_zero_outside_their_band():
    for d in (64, 128):
        for f0 in bands(d):
            t = make_band_inputs(2, 8, 4, d, 17, 8, f0, seed=f0)
            off = np.setdiff1d(np.arange(d), band_columns(d, f0))
            for k in ("q_blk", "k_blk"):
                x = t[k].float().numpy()
                assert np.all(x[..., off] == 0) and np.all(np.abs(x[..., band_columns(d, f0)]).max() > 0)
        assert sorted(np.concatenate([band_columns(d, f0) for f0 in bands(d)]).tolist()) == list(range(d))


@pytest.mark.parametrize("base", [2.0, 1e6])
@pytest.mark.parametrize("P", [0, 17])
@pytest.mark.parametrize("label,d,B,Hq,Hkv", SHAPES, ids=[s[0] for s in SHAPES])
def test_check_passes_a_correct_kernel_and_fails_planted_mistakes(label, d, B, Hq, Hkv, P, base, monkeypatch):
    rope_mode = oa.ROPE_COPY
    caught = {k: 0 for k in ("skip_upper_quarter", "next_partner", "neighbour_frequency")}
    for f0 in bands(d):
        t = make_band_inputs(2, Hq, Hkv, d, P, B, f0, seed=1000 * d + 10 * B + f0 + P)
        good = oracle_out(t, base, rope_mode, t["pos_d"].numpy())
        pert = strong(perturbed_oracles(t, base, rope_mode, P), good)
        if base == 2.0:  # every pair turns by 0.5..1 rad per position
            assert {"unrotated"} | ({"pos+1"} if P > 0 else set()) <= set(pert), (f0, sorted(pert))
        sim = kernel_standin(t, base, rope_mode, seed=f0)
        ok, rep = criterion(sim, good, list(pert.values()))
        assert ok, ("a correct kernel must pass", f0, rep)
        for kind in caught:
            with monkeypatch.context() as m:
                m.setattr(oa, "rope_rotate", mistake(kind))
                bad = oracle_out(t, base, rope_mode, t["pos_d"].numpy())
                bad_sim = kernel_standin(t, base, rope_mode, seed=f0)
                bad_pert = strong(perturbed_oracles(t, base, rope_mode, P), bad)
            visible = np.abs(bad - good).mean() >= 10 * TOL_MEAN
            if not touches(kind, d, f0):
                assert np.array_equal(bad, good)
                continue
            if base == 2.0:
                assert visible, (kind, f0)
            if not visible:
                continue
            # the mistake in the kernel, the oracle right
            ok_k, rep_k = criterion(bad_sim, good, list(pert.values()))
            # the mistake in the oracle, the kernel right
            ok_o, rep_o = criterion(sim, bad, list(bad_pert.values()))
            assert not ok_k, (kind, f0, rep_k)
            assert not ok_o, (kind, f0, rep_o)
            caught[kind] += 1
    if base == 2.0:
        n = len(bands(d))
        assert caught == {"skip_upper_quarter": n // 2, "next_partner": n, "neighbour_frequency": n}, caught
    else:
        assert caught["skip_upper_quarter"] >= 1 and caught["next_partner"] >= 1, caught
