"""The attention kernels' own RoPE-copy rotation, one frequency band at a time.

Page "SimSD - Simple Speculative Decoding in Diffusion Language Models",
section 3 (D~_k rotated at D_k's position) and "Experimental results"
(the ablation without the copy).  The block queries and keys are zero
outside the 8 frequency pairs of one band (tests/rope_bands.py), so the
output of the kernel depends only on how it rotates those pairs: its RoPE
table entries, its pairing of the two halves (the query rows in registers,
the block keys in LDS) and its positions.  Every band of d = 128 and d = 64
is run on the MFMA kernel (and the VALU kernel), in the 64-row, 128-row and
32-row workgroup forms, with and without a prompt, in both RoPE modes.

Each band must meet the bf16 tolerance against the oracle and sit at least
10x closer to it than to perturbed oracles: the block rotation left out
(all block positions 0, i.e. the band unrotated), the other RoPE mode, and
(with a prompt, whose cached keys fix absolute positions) every block
position moved by one.  A perturbation is used when it moves the oracle's
own output by at least 10x the bf16 mean tolerance; at base 2 (every pair
turns by 0.5..1 rad per position) the first and the last always qualify,
while the other mode's shift of B positions can come close to a whole turn
in some bands.  tests/test_rope_band_criterion.py shows on the CPU
that this check fails when a rotation mistake (pairs f >= d/4 left
unrotated, a wrong partner, a neighbouring frequency) is planted.
"""
import pytest
import torch

import diffusion_lm_speculative_amd as sd
from diffusion_lm_speculative_amd import synth
from tests.gpu_helpers import dev
from tests.rope_bands import bands, criterion, make_band_inputs, oracle_out, perturbed_oracles, strong

pytestmark = pytest.mark.gpu

# (label, d, B, Hq, Hkv): rows per KV head G*2B = 64 (four row waves of one
# tile), 128 (four row waves of two tiles) and 32 (two row waves, d = 64)
SHAPES = [("d128_rows64", 128, 8, 32, 8), ("d128_rows128", 128, 16, 16, 4), ("d64_rows32", 64, 8, 8, 4)]


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
@pytest.mark.parametrize("rope_mode", [sd.ROPE_COPY, sd.ROPE_SEQUENTIAL])
@pytest.mark.parametrize("base", [2.0, 1e6])
@pytest.mark.parametrize("P", [0, 17])
@pytest.mark.parametrize("label,d,B,Hq,Hkv", SHAPES, ids=[s[0] for s in SHAPES])
def test_rope_copy_band_by_band(label, d, B, Hq, Hkv, P, base, rope_mode, impl):
    used_any = False
    for f0 in bands(d):
        t = make_band_inputs(2, Hq, Hkv, d, P, B, f0, seed=1000 * d + 10 * B + f0 + P)
        print(f"case {label} P={P} base={base} rope_mode={rope_mode} impl={impl} band={f0}", flush=True)
        g = {k: v.to(dev()) for k, v in t.items()}
        out, _, st = sd.verify_attn(g["q_blk"], g["k_blk"], g["v_blk"], g["k_cache"], g["v_cache"], g["tau"],
                                    g["prompt_len"], g["pos_d"], rope_base=base, impl=impl, rope_mode=rope_mode)
        torch.cuda.synchronize()
        assert st.cpu().tolist() == [0, 0]
        got = synth.to_numpy64(out)
        good = oracle_out(t, base, rope_mode, t["pos_d"].numpy())
        pert = strong(perturbed_oracles(t, base, rope_mode, P), good)
        if base == 2.0:  # every pair turns by 0.5..1 rad per position
            assert {"unrotated"} | ({"pos+1"} if P > 0 else set()) <= set(pert), sorted(pert)
        used_any |= bool(pert)
        ok, rep = criterion(got, good, list(pert.values()))
        print(f"  {rep} perturbations={sorted(pert)}", flush=True)
        assert ok, (label, f0, rep)
    assert used_any
