"""Seeded synthetic inputs for the verification pass (no method arithmetic).

Both the HIP path and the oracle are fed from here.  Shapes follow
SDAR-8B-shaped layers (32 query heads, 8 KV heads, head dim 128) and the
pages' workloads (block sizes B = 4, 8, 16, 32; prompts of 1k..16k tokens);
the pages' own benchmarks (GSM8K, MBPP, TriviaQA, MMLU, ...) are replaced by
random tensors of those shapes.

Recipe (per workload): a torch.Generator on the target device seeded with
``seed``; tensors drawn in the order q_blk, k_blk, v_blk, k_cache, v_cache
from N(0, 1) times ``std`` and rounded to the dtype (bf16 round-to-nearest-
even); then tau = randperm(B) + 1 per sequence; then prompt lengths (uniform
integers in [p_lo, p_hi] for variable-length workloads, else P_max).  For
acceptance: target and draft logits ~ N(0, sigma^2) with sigma = sqrt(2)
(variance 2), p and q their softmaxes in float32, draft tokens sampled from
q, tau = randperm(B) + 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    NB: int
    Hq: int
    Hkv: int
    d: int
    P: int            # P_max (cache capacity)
    B: int
    dtype: torch.dtype
    rope_base: float
    std: float
    p_lo: int = -1    # variable prompt lengths: uniform in [p_lo, P] when p_lo >= 0
    vocab: int = 0    # acceptance vocabulary (0: no acceptance stage)
    gamma: int = 0
    note: str = field(default="", compare=False)

    @property
    def G(self):
        return self.Hq // self.Hkv

    def kv_bytes(self, prompt_len=None):
        """Algorithmic K+V cache bytes read: every key/value of [0, P_b) once."""
        esz = 2 if self.dtype == torch.bfloat16 else 4
        tot = self.NB * self.P if prompt_len is None else int(prompt_len.sum())
        return tot * self.Hkv * self.d * 2 * esz


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 4, 2, 64, 64, 4, torch.float32, 1e4, 1.0,
                          note="batch 1, 4/2 heads, d 64, prompt 64, B 4, fp32"),
    "sdar8b_p1024_b4": Workload("sdar8b_p1024_b4", 16, 32, 8, 128, 1024, 4, torch.bfloat16, 1e6, 0.5,
                                note="batch 16, 32/8 heads, d 128, prompt 1024, B 4, bf16"),
    "sdar8b_p4096_b8": Workload("sdar8b_p4096_b8", 32, 32, 8, 128, 4096, 8, torch.bfloat16, 1e6, 0.5,
                                note="batch 32, 32/8 heads, d 128, prompt 4096, B 8, bf16"),
    "sdar8b_p8192_b32": Workload("sdar8b_p8192_b32", 8, 32, 8, 128, 8192, 32, torch.bfloat16, 1e6, 0.5,
                                 note="batch 8, 32/8 heads, d 128, prompt 8192, B 32, bf16"),
    "sdar8b_var16k_b16_accept": Workload("sdar8b_var16k_b16_accept", 64, 32, 8, 128, 16384, 16, torch.bfloat16,
                                         1e6, 0.5, p_lo=2048, vocab=151936, gamma=16,
                                         note="batch 64, 32/8 heads, d 128, prompt U[2048,16384], B=gamma=16, "
                                              "bf16, then acceptance over V=151936"),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, dtype, g, device):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_verify_inputs(w: Workload, seed: int, device="cpu", NB=None, P=None):
    """Inputs of one verification call as a dict of tensors on ``device``."""
    NB = w.NB if NB is None else NB
    P = w.P if P is None else P
    g = _gen(device, seed)
    twoB = 2 * w.B
    q = _normal((NB, twoB, w.Hq, w.d), w.std, w.dtype, g, device)
    kb = _normal((NB, twoB, w.Hkv, w.d), w.std, w.dtype, g, device)
    vb = _normal((NB, twoB, w.Hkv, w.d), w.std, w.dtype, g, device)
    kc = _normal((NB, w.Hkv, P, w.d), w.std, w.dtype, g, device)
    vc = _normal((NB, w.Hkv, P, w.d), w.std, w.dtype, g, device)
    if w.B and NB:
        tau = torch.stack([torch.randperm(w.B, generator=g, device=device) + 1 for _ in range(NB)])
    else:
        tau = torch.zeros((NB, w.B), dtype=torch.int64, device=device)
    if w.p_lo >= 0:
        plen = torch.randint(w.p_lo, P + 1, (NB,), generator=g, device=device)
    else:
        plen = torch.full((NB,), P, dtype=torch.int64, device=device)
    return dict(q_blk=q, k_blk=kb, v_blk=vb, k_cache=kc, v_cache=vc,
                tau=tau.to(torch.int32).contiguous(), prompt_len=plen.to(torch.int32))


def make_accept_inputs(NB, B, V, seed, device="cpu", sigma=math.sqrt(2.0)):
    """Target / draft probabilities [NB][B][V] float32, draft tokens ~ q, tau."""
    g = _gen(device, seed)
    lp = torch.randn((NB, B, V), generator=g, device=device, dtype=torch.float32).mul_(sigma)
    lq = torch.randn((NB, B, V), generator=g, device=device, dtype=torch.float32).mul_(sigma)
    p = torch.softmax(lp, dim=-1)
    del lp
    q = torch.softmax(lq, dim=-1)
    del lq
    x = torch.multinomial(q.reshape(NB * B, V), 1, generator=g).reshape(NB, B).to(torch.int32)
    tau = torch.stack([torch.randperm(B, generator=g, device=device) + 1 for _ in range(NB)]).to(torch.int32)
    return dict(p=p.contiguous(), q=q.contiguous(), draft_tok=x.contiguous(), tau=tau.contiguous())


def make_noise_exp(NB, B, V, seed, device="cpu"):
    """Shared noise table in exponential form [NB][B][V] float32: Exp(1)
    variates (E = exp(-g) for a Gumbel g), drawn from their own generator and
    kept strictly positive (the smallest normal float32 replaces an
    underflowed zero)."""
    g = _gen(device, seed)
    e = torch.empty((NB, B, V), device=device, dtype=torch.float32).exponential_(1.0, generator=g)
    return e.clamp_min_(torch.finfo(torch.float32).tiny).contiguous()


def make_linear_inputs(M, K, N, seed, device="cpu"):
    """x [M][K] ~ N(0, 1) and w [N][K] ~ N(0, 1/K) (the usual fan-in scale of
    a projection), both rounded to bf16."""
    g = _gen(device, seed)
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32).mul_(K ** -0.5).to(torch.bfloat16)
    return x.contiguous(), w.contiguous()


def to_numpy64(t):
    """Exact float64 copy of a float32 / bfloat16 tensor (for the oracle)."""
    return t.detach().to("cpu").to(torch.float32).double().numpy()
