"""GPU parity of the projections around the attention (simsd_linear,
simsd_qkv_proj, through the C ABI) against the float64 oracle.

Tolerance, derived: the kernel rounds an fp32 sum of K bf16 products to
bf16.  Any fp32 summation order is within K * 2^-24 * sum_k |x_k w_k| of the
exact sum, and rounding to bf16 (8 significant bits, nearest even) adds at
most 2^-8 of the magnitude.  Every element must sit inside that bound.
Shapes cover every channel-block width of the kernel (64 for small grids and
N = 4096 at 512 rows, 96 for N = 6144 at 512 rows, 128 for N = 4096 at 1024
rows), row and channel tails, and the SDAR-8B-shaped layer of the benchmark.
"""
import numpy as np
import pytest
import torch

import diffusion_lm_speculative_amd as sd
from diffusion_lm_speculative_amd import synth
from oracle.attention import verify_attn_ref
from oracle.projection import linear_ref, o_proj_ref, qkv_proj_ref
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _bound(x64, w64, ref):
    K = x64.shape[1]
    acc = K * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64).T)
    return 2.0 ** -8 * (np.abs(ref) + acc) + acc


def _check(got, ref, bound, label):
    g = synth.to_numpy64(got).reshape(ref.shape)
    err = np.abs(g - ref)
    worst = float((err / np.maximum(bound, 1e-30)).max()) if err.size else 0.0
    print(f"[{label}] max_abs={err.max():.3e} worst/bound={worst:.3f}", flush=True)
    assert np.all(err <= bound), (label, worst)
    if err.size > 4096:
        assert worst > 0.05, (label, worst)  # the bound is tight enough to see the bf16 rounding


@pytest.mark.parametrize("M,N,K", [(1, 16, 64), (127, 48, 128), (130, 208, 192), (300, 4096, 256),
                                   (512, 6144, 512), (1024, 4096, 256), (1000, 1040, 1024)])
def test_linear(M, N, K):
    print(f"linear M={M} N={N} K={K}", flush=True)
    x, w = synth.make_linear_inputs(M, K, N, seed=M + N + K, device=dev())
    y = sd.linear(x, w)
    torch.cuda.synchronize()
    x64, w64 = synth.to_numpy64(x), synth.to_numpy64(w)
    ref = linear_ref(x64, w64)
    _check(y, ref, _bound(x64, w64, ref), f"linear {M}x{N}x{K}")


def test_output_projection_sdar_shape():
    # attention output of 32 sequences x 16 block rows, 32 heads of 128 -> hidden 4096
    M, H, Hq, d = 512, 4096, 32, 128
    x, w = synth.make_linear_inputs(M, Hq * d, H, seed=77, device=dev())
    y = sd.linear(x, w)
    torch.cuda.synchronize()
    x64, w64 = synth.to_numpy64(x), synth.to_numpy64(w)
    ref = o_proj_ref(x64.reshape(32, 16, Hq, d), w64).reshape(M, H)
    _check(y, ref, _bound(x64, w64, ref), "o_proj 512x4096x4096")


@pytest.mark.parametrize("NB,B,H,Hq,Hkv,d", [(32, 8, 4096, 32, 8, 128), (3, 5, 128, 4, 2, 64), (1, 1, 64, 1, 1, 16)])
def test_qkv_proj(NB, B, H, Hq, Hkv, d):
    print(f"qkv NB={NB} B={B} H={H} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    N = (Hq + 2 * Hkv) * d
    x, w = synth.make_linear_inputs(NB * 2 * B, H, N, seed=NB * 7 + B, device=dev())
    q, k, v = sd.qkv_proj(x.view(NB, 2 * B, H), w, Hq, Hkv, d)
    torch.cuda.synchronize()
    x64, w64 = synth.to_numpy64(x), synth.to_numpy64(w)
    rq, rk, rv = qkv_proj_ref(x64.reshape(NB, 2 * B, H), w64, Hq, Hkv, d)
    full = linear_ref(x64, w64)
    bound = _bound(x64, w64, full)
    nq, nk = Hq * d, Hkv * d
    _check(q, rq, bound[:, :nq].reshape(rq.shape), "q")
    _check(k, rk, bound[:, nq:nq + nk].reshape(rk.shape), "k")
    _check(v, rv, bound[:, nq + nk:].reshape(rv.shape), "v")


def test_layer_composition_matches_the_oracle_chain():
    # hidden states -> QKV projection -> verification attention -> output
    # projection, against the same chain in float64.  Each stage rounds to
    # bf16 on the GPU, so the bound is the attention tests' bf16 tolerance
    # carried through the output projection (scaled by its row norms).
    NB, B, H, Hq, Hkv, d, P = 2, 4, 256, 8, 2, 64, 150
    twoB = 2 * B
    x, w_qkv = synth.make_linear_inputs(NB * twoB, H, (Hq + 2 * Hkv) * d, seed=5, device=dev())
    _, w_o = synth.make_linear_inputs(1, Hq * d, H, seed=6, device=dev())
    g = torch.Generator(device=dev()).manual_seed(7)
    kc = (torch.randn((NB, Hkv, P, d), generator=g, device=dev()) * 0.5).to(torch.bfloat16)
    vc = (torch.randn((NB, Hkv, P, d), generator=g, device=dev()) * 0.5).to(torch.bfloat16)
    tau = torch.stack([torch.randperm(B, generator=g, device=dev()) + 1 for _ in range(NB)]).to(torch.int32)
    q, k, v = sd.qkv_proj(x.view(NB, twoB, H), w_qkv, Hq, Hkv, d)
    attn, _, st = sd.verify_attn(q, k, v, kc, vc, tau, rope_base=1e6)
    y = sd.linear(attn.view(NB * twoB, Hq * d), w_o)
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0
    x64, wq64, wo64 = synth.to_numpy64(x), synth.to_numpy64(w_qkv), synth.to_numpy64(w_o)
    rq, rk, rv = qkv_proj_ref(x64.reshape(NB, twoB, H), wq64, Hq, Hkv, d)
    ra, _, _ = verify_attn_ref(rq, rk, rv, synth.to_numpy64(kc), synth.to_numpy64(vc), None, tau.cpu().numpy(),
                               rope_base=1e6)
    ref = o_proj_ref(ra, wo64).reshape(NB * twoB, H)
    got = synth.to_numpy64(y)
    err = np.abs(got - ref)
    # attention outputs agree within 2e-2 (its documented bf16 tolerance,
    # here on attention inputs that are themselves bf16-rounded projections)
    bound = 2e-2 * np.abs(wo64).sum(axis=1)[None, :] + 2.0 ** -8 * np.abs(ref)
    print(f"[layer] max_abs={err.max():.3e} worst/bound={(err / bound).max():.3f}", flush=True)
    assert np.all(err <= bound)
    assert np.abs(got).max() > 0.05  # not a trivially small output
