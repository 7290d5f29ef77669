"""Shared helpers of the GPU parity tests (inputs, oracle calls, tolerances)."""
import numpy as np
import torch

from diffusion_lm_speculative_amd import synth
from oracle.attention import verify_attn_ref

# Tolerances: fp32 1e-5 max-abs; bf16 inputs with fp32 accumulation 2e-2
# max-abs and 2e-3 mean-abs.
TOL_F32 = 1e-5
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3


def dev():
    return torch.device("cuda:0")


def gpu_inputs(w, seed, NB=None, P=None, on_device=False):
    """Seeded inputs; generated on the CPU (or on the GPU for the large workloads)."""
    where = dev() if on_device else "cpu"
    t = synth.make_verify_inputs(w, seed, device=where, NB=NB, P=P)
    return {k: v.to(dev()) for k, v in t.items()}


def oracle_for(t, w, b_idx=None, pos_d=None, mask_mode=0, scale=None, rope_mode=0):
    """Oracle output for the sequences b_idx (all when None), from the same tensors."""
    sel = slice(None) if b_idx is None else list(b_idx)
    np64 = lambda x: synth.to_numpy64(x[sel])
    out, lse, st = verify_attn_ref(
        np64(t["q_blk"]), np64(t["k_blk"]), np64(t["v_blk"]), np64(t["k_cache"]), np64(t["v_cache"]),
        t["prompt_len"][sel].cpu().numpy(), t["tau"][sel].cpu().numpy(),
        pos_d=None if pos_d is None else pos_d[sel].cpu().numpy(),
        rope_base=w.rope_base, scale=scale, mask_mode=mask_mode, rope_mode=rope_mode)
    return out, lse, st


def compare(got, ref, dtype, label=""):
    """Assert the documented tolerance; returns (max_abs, mean_abs, max_rel)."""
    g = synth.to_numpy64(got)
    diff = np.abs(g - ref)
    mx = float(diff.max()) if diff.size else 0.0
    mean = float(diff.mean()) if diff.size else 0.0
    rel = float((diff / np.maximum(np.abs(ref), 1e-3)).max()) if diff.size else 0.0
    print(f"[{label}] max_abs={mx:.3e} mean_abs={mean:.3e} max_rel={rel:.3e}", flush=True)
    if dtype == torch.float32:
        assert mx <= TOL_F32, (label, mx)
    else:
        assert mx <= TOL_BF16_MAX, (label, mx)
        assert mean <= TOL_BF16_MEAN, (label, mean)
    return mx, mean, rel
