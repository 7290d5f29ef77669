"""GPU exports of the in-kernel tau mask and RoPE copy against the oracle.

The mask words come from the same device function the attention kernels use
and must match the oracle bit for bit (every B from 1 to 64, ties, the
all-visible mode).  The rotated block rows must match the oracle's float64
rotation: within 2e-6 for fp32, and within one bf16 unit in the last place
(the kernel rounds the fp32 rotation once) for bf16.
"""
import numpy as np
import pytest
import torch

import diffusion_lm_speculative_amd as sd
from oracle.attention import block_visibility, rope_rotate
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _words(vis, B):
    w = np.zeros((2 * B, 2), dtype=np.uint64)
    for r in range(2 * B):
        for j in range(B):
            if vis[r, j]:
                w[r, 0] |= np.uint64(1) << np.uint64(j)
            if vis[r, B + j]:
                w[r, 1] |= np.uint64(1) << np.uint64(j)
    return w


@pytest.mark.parametrize("B", [1, 2, 3, 4, 7, 8, 16, 31, 32, 33, 63, 64])
@pytest.mark.parametrize("ties", [False, True, "committed"])
def test_mask_bits_exact(B, ties):
    g = torch.Generator().manual_seed(B * 7 + (2 if ties == "committed" else int(ties)))
    NB = 6
    if ties == "committed":  # label 0 for a random share of positions, the open ones 1..m
        tau = torch.zeros(NB, B, dtype=torch.int64)
        for b in range(NB):
            c = int(torch.randint(0, B + 1, (1,), generator=g)) if b else B  # sequence 0: all committed
            open_pos = torch.randperm(B, generator=g)[: B - c]
            tau[b, open_pos] = torch.randperm(B - c, generator=g) + 1
    elif ties:
        tau = torch.randint(1, B + 1, (NB, B), generator=g)
    else:
        tau = torch.stack([torch.randperm(B, generator=g) + 1 for _ in range(NB)])
    tau = tau.to(torch.int32)
    for mode in (sd.MASK_TEMPORAL, sd.MASK_FULL):
        bits = sd.debug_mask(tau.to(dev()), mode).cpu().numpy().view(np.uint64)
        for b in range(NB):
            want = _words(block_visibility(tau[b].tolist(), mode), B)
            assert np.array_equal(bits[b], want), (B, b, mode)


@pytest.mark.parametrize("dtype,d,base", [(torch.float32, 64, 1e4), (torch.float32, 128, 1e6),
                                          (torch.bfloat16, 128, 1e6), (torch.bfloat16, 64, 1e4)])
@pytest.mark.parametrize("seq", [False, True])
def test_rope_copy_rows(dtype, d, base, seq):
    g = torch.Generator().manual_seed(d)
    NB, B, Hq, Hkv = 3, 8, 8, 2
    q = (torch.randn(NB, 2 * B, Hq, d, generator=g) * 0.5).to(dtype)
    k = (torch.randn(NB, 2 * B, Hkv, d, generator=g) * 0.5).to(dtype)
    plen = torch.tensor([0, 4000, 16370], dtype=torch.int32)
    pos_d = None
    qr, kr = sd.debug_rope(q.to(dev()), k.to(dev()), plen.to(dev()), pos_d, rope_base=base, p_max=16384,
                           rope_mode=sd.ROPE_SEQUENTIAL if seq else sd.ROPE_COPY)
    pos = (plen[:, None].long() + torch.arange(B)).numpy()
    # D~_k takes D_k's position, or B past it without the RoPE copy
    rows = np.concatenate([pos, pos + B if seq else pos], axis=1)
    q64 = rope_rotate(q.float().double().numpy(), rows[:, :, None], base)
    k64 = rope_rotate(k.float().double().numpy(), rows[:, :, None], base)
    for got, want in ((qr, q64), (kr, k64)):
        gg = got.float().double().cpu().numpy()
        if dtype == torch.float32:
            assert np.abs(gg - want).max() < 2e-6
        else:
            # one bf16 ulp of the reference value
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
            assert np.all(np.abs(gg - want) <= np.maximum(ulp * 1.0001, 1e-6))
