"""GPU parity of simsd_verify_attn (through the C ABI) against the fp64 oracle.

Small cases cover several key tiles, ragged tails, forced prompt splits,
every MFMA row-tiling variant (up to 256 rows a workgroup), d = 64 and 128,
B = 1 .. 64, variable prompt lengths (including 0), custom RoPE positions,
the all-visible mode and faulted sequences.  The SDAR-shaped workloads run at full size in the
launch configuration the benchmark times, compared on sampled sequences.
Block-dominated cases (P = 0, 1, 17) and fp32 runs at SDAR head shapes make
mask and RoPE mistakes visible despite the bf16 tolerance.
"""
import dataclasses

import numpy as np
import pytest
import torch

import diffusion_lm_speculative_amd as sd
from diffusion_lm_speculative_amd import synth
from tests.gpu_helpers import compare, dev, gpu_inputs, oracle_for

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _w(name=None, **kw):
    base = W[name] if name else W["sdar8b_p1024_b4"]
    return dataclasses.replace(base, **kw)


def _run(t, w, **kw):
    out, lse, st = sd.verify_attn(t["q_blk"], t["k_blk"], t["v_blk"], t["k_cache"], t["v_cache"], t["tau"],
                                  t["prompt_len"], kw.pop("pos_d", None), rope_base=w.rope_base, **kw)
    torch.cuda.synchronize()
    return out, lse, st


def _check(t, w, label, impl=0, kv_chunk=0, pos_d=None, mask_mode=0, b_idx=None, rope_mode=0):
    print(f"case {label}: NB={t['q_blk'].shape[0]} Hq={w.Hq} Hkv={w.Hkv} d={w.d} P={t['k_cache'].shape[2]} "
          f"B={w.B} {w.dtype} impl={impl} kv_chunk={kv_chunk} rope_mode={rope_mode}", flush=True)
    out, lse, st = _run(t, w, impl=impl, kv_chunk=kv_chunk, pos_d=pos_d, mask_mode=mask_mode, rope_mode=rope_mode)
    ref, ref_lse, ref_st = oracle_for(t, w, b_idx=b_idx, pos_d=pos_d, mask_mode=mask_mode, rope_mode=rope_mode)
    sel = slice(None) if b_idx is None else list(b_idx)
    assert np.array_equal(st[sel].cpu().numpy(), ref_st)
    compare(out[sel], ref, w.dtype, label)
    lse_ok = np.isfinite(ref_lse)
    got_lse = lse[sel].double().cpu().numpy()
    tol = 1e-5 if w.dtype == torch.float32 else 2e-2
    assert np.all(np.isneginf(got_lse[~lse_ok]))
    assert np.abs(got_lse[lse_ok] - ref_lse[lse_ok]).max(initial=0.0) <= tol
    return out, lse, ref


# ---------------------------------------------------------------- fp32 (VALU kernel)

def test_tiny_fp32_workload():
    w = W["tiny_fp32"]
    _check(gpu_inputs(w, 1000), w, "tiny_fp32")


@pytest.mark.parametrize("P,B,kv_chunk", [(300, 8, 0), (0, 8, 0), (17, 4, 0), (200, 5, 64)])
def test_fp32_sdar_heads(P, B, kv_chunk):
    w = _w(dtype=torch.float32, B=B, P=P, NB=2)
    _check(gpu_inputs(w, 11 + P), w, f"fp32 sdar P={P} B={B}", kv_chunk=kv_chunk)


# ---------------------------------------------------------------- bf16, both kernels

SMALL = [
    # (label, overrides)
    ("ragged", dict(NB=3, Hq=8, Hkv=2, P=333, B=5)),
    ("block_only", dict(NB=2, P=0, B=8)),
    ("p1", dict(NB=2, P=1, B=8)),
    ("p17", dict(NB=2, P=17, B=8)),
    ("d64_g1", dict(NB=2, Hq=4, Hkv=4, d=64, P=200, B=3)),
    ("b1", dict(NB=3, P=130, B=1)),
    ("b64_g1", dict(NB=1, Hq=2, Hkv=2, P=100, B=64)),
    ("b32_g4", dict(NB=1, Hq=8, Hkv=2, P=150, B=32)),       # 256 rows: one group of eight row waves
    ("b64_g4", dict(NB=1, Hq=4, Hkv=1, P=70, B=64)),        # 512 rows: two row groups
    ("g8_b2", dict(NB=2, Hq=16, Hkv=2, P=64, B=2)),
    ("var_len", dict(NB=6, P=500, B=4, p_lo=0)),
]


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
@pytest.mark.parametrize("label,ov", SMALL, ids=[s[0] for s in SMALL])
def test_bf16_small(label, ov, impl):
    w = _w(**ov)
    _check(gpu_inputs(w, 7 + len(label)), w, f"{label} impl={impl}", impl=impl)


LONG = [
    # (label, overrides): one long split per sequence, so the ring runs its
    # steady state (refills of every stage) and its ragged end
    ("rows16", dict(Hq=8, Hkv=8, B=8)),
    ("rows32", dict(Hq=8, Hkv=2, B=4)),
    ("rows64", dict(Hq=8, Hkv=2, B=8)),
    ("rows128", dict(Hq=8, Hkv=2, B=16)),
    ("rows256", dict(Hq=8, Hkv=2, B=32)),
    ("rows512", dict(Hq=4, Hkv=1, B=64)),
    ("d64", dict(Hq=8, Hkv=2, d=64, B=8)),
]


@pytest.mark.parametrize("label,ov", LONG, ids=[s[0] for s in LONG])
def test_bf16_long_splits(label, ov):
    w = _w(NB=2, P=1000, p_lo=300, **ov)
    t = gpu_inputs(w, 41 + len(label))
    for kv_chunk in (1024, 320):
        _check(t, w, f"long {label} chunk={kv_chunk}", impl=sd.IMPL_MFMA, kv_chunk=kv_chunk)


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
@pytest.mark.parametrize("kv_chunk", [64, 128, 192])
def test_bf16_forced_splits(kv_chunk, impl):
    w = _w(NB=5, Hq=8, Hkv=2, P=450, B=4, p_lo=0)
    t = gpu_inputs(w, 31)
    t["prompt_len"][0] = 0
    t["prompt_len"][1] = 450
    t["prompt_len"][2] = kv_chunk
    _check(t, w, f"split {kv_chunk}", impl=impl, kv_chunk=kv_chunk)


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
def test_custom_positions_and_full_mode(impl):
    w = _w(NB=3, Hq=8, Hkv=2, P=96, B=6)
    t = gpu_inputs(w, 41)
    g = torch.Generator().manual_seed(5)
    pos_d = torch.stack([torch.randperm(6, generator=g) * 3 + 1000 for _ in range(3)]).to(torch.int32).to(dev())
    _check(t, w, "pos_d", impl=impl, pos_d=pos_d)
    _check(t, w, "full mode", impl=impl, mask_mode=sd.MASK_FULL)


# Without the RoPE copy (the ablation): D~_k at pos(D_k) + B.  Block-dominated
# prompts (P = 0, 17) make a wrong position visible; B = 32 at d = 128 runs
# the MFMA kernel with its 2B-entry table beside a 3-stage ring, B = 64 at
# d = 64 a table of 128 entries.
SEQ = [
    ("p0_b8", dict(NB=3, Hq=8, Hkv=2, P=0, p_lo=0, B=8)),
    ("p17_b6", dict(NB=3, Hq=8, Hkv=2, P=17, p_lo=0, B=6)),
    ("p300_b16", dict(NB=2, Hq=8, Hkv=2, P=300, B=16)),
    ("p200_b32", dict(NB=2, Hq=4, Hkv=2, P=200, B=32)),
    ("d64_b64", dict(NB=2, Hq=4, Hkv=1, d=64, P=150, B=64)),
]


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
@pytest.mark.parametrize("label,ov", SEQ, ids=[s[0] for s in SEQ])
def test_without_rope_copy(label, ov, impl):
    w = _w(**ov)
    t = gpu_inputs(w, 91 + len(label))
    _check(t, w, f"seq {label} impl={impl}", impl=impl, rope_mode=sd.ROPE_SEQUENTIAL)
    if label == "p17_b6":
        g = torch.Generator().manual_seed(9)
        pos_d = torch.stack([torch.randperm(w.B, generator=g) * 5 + 77 for _ in range(w.NB)])
        _check(t, w, f"seq pos_d impl={impl}", impl=impl, rope_mode=sd.ROPE_SEQUENTIAL,
               pos_d=pos_d.to(torch.int32).to(dev()))


def test_without_rope_copy_fp32_and_wide_block():
    # fp32 at 1e-5 on a block-dominated case (VALU kernel)
    w = _w(NB=2, Hq=4, Hkv=2, d=128, P=17, p_lo=0, B=8, dtype=torch.float32)
    _check(gpu_inputs(w, 95), w, "seq fp32", rope_mode=sd.ROPE_SEQUENTIAL)
    # d = 128, B = 64: the table of 128 positions does not fit beside the MFMA
    # ring, so AUTO runs the VALU kernel and an explicit MFMA request is refused
    w = _w(NB=1, Hq=4, Hkv=1, P=100, B=64)
    t = gpu_inputs(w, 96)
    _check(t, w, "seq b64 auto", rope_mode=sd.ROPE_SEQUENTIAL)
    with pytest.raises(sd.SimsdError):
        _run(t, w, impl=sd.IMPL_MFMA, rope_mode=sd.ROPE_SEQUENTIAL)


# Stage labels with ties: several positions committed at one step (threshold
# decoding), all positions at stage 1 (a plain bidirectional block step over
# the mask slots), and random repeats.  The mask rules stay defined and the
# oracle applies them literally.
def _tied_tau(kind, NB, B, g):
    if kind == "all1":
        return torch.ones(NB, B, dtype=torch.int32)
    if kind == "steps":
        base = torch.arange(B) // 3 + 1  # 1,1,1,2,2,2,...
        return torch.stack([base[torch.randperm(B, generator=g)] for _ in range(NB)]).to(torch.int32)
    return torch.randint(1, B + 1, (NB, B), generator=g, dtype=torch.int32)


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
@pytest.mark.parametrize("kind", ["all1", "steps", "random"])
@pytest.mark.parametrize("B,P", [(4, 17), (8, 0), (16, 130), (32, 70)])
def test_tied_stage_labels(kind, B, P, impl):
    w = _w(NB=3, Hq=8, Hkv=2, P=P, p_lo=0, B=B)
    t = gpu_inputs(w, 101 + B + P)
    g = torch.Generator().manual_seed(B * 31 + P)
    t["tau"] = _tied_tau(kind, w.NB, B, g).to(dev())
    _check(t, w, f"ties {kind} B={B} P={P} impl={impl}", impl=impl)
    if kind == "steps":
        _check(t, w, f"ties {kind} seq impl={impl}", impl=impl, rope_mode=sd.ROPE_SEQUENTIAL)


def _committed_tau(NB, B, g):
    """Label 0 for positions committed in an earlier round (a different
    count per sequence, all of them in sequence 0), 1..m for the open ones."""
    tau = torch.zeros(NB, B, dtype=torch.int32)
    for b in range(NB):
        c = B if b == 0 else 1 + (b * 5) % B
        open_pos = torch.randperm(B, generator=g)[: B - c]
        tau[b, open_pos] = (torch.randperm(B - c, generator=g) + 1).to(torch.int32)
    return tau


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
@pytest.mark.parametrize("B,P", [(4, 17), (8, 300), (16, 130), (32, 150), (64, 100)])
def test_committed_positions(B, P, impl):
    # later rounds of a block: committed positions carry label 0
    w = _w(NB=4, Hq=8 if B < 64 else 4, Hkv=2 if B < 64 else 1, P=P, p_lo=0, B=B)
    t = gpu_inputs(w, 131 + B + P)
    t["tau"] = _committed_tau(w.NB, B, torch.Generator().manual_seed(B + P)).to(dev())
    _check(t, w, f"committed B={B} P={P} impl={impl}", impl=impl)
    if B == 8:
        _check(t, w, f"committed seq impl={impl}", impl=impl, rope_mode=sd.ROPE_SEQUENTIAL)


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
def test_faulted_sequences(impl):
    w = _w(NB=4, Hq=8, Hkv=2, P=80, B=4)
    t = gpu_inputs(w, 51)
    t["tau"][1, 2] = 9
    t["prompt_len"][2] = 81
    pos_d = (t["prompt_len"][:, None].long() + torch.arange(4, device=dev())).to(torch.int32)
    pos_d[3, 0] = -5
    for kv_chunk in (0, 64):
        _check(t, w, f"faults chunk={kv_chunk}", impl=impl, kv_chunk=kv_chunk, pos_d=pos_d)
    _, _, st = _run(t, w, impl=impl, pos_d=pos_d)
    assert st.cpu().tolist() == [0, sd.ST_TAU_RANGE, sd.ST_PROMPT_LEN, sd.ST_POS_NEG]


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
def test_cache_rows_past_prompt_len_are_never_read(impl):
    # Cache rows at positions >= P_b are not part of the input: fill them with
    # NaN and Inf.  Prompt lengths end inside the first tiles of a split (the
    # rows a kernel may fetch before it knows P_b), on tile edges and at 0.
    w = _w(NB=6, Hq=8, Hkv=2, P=700, B=4)
    t = gpu_inputs(w, 91)
    t["prompt_len"][:] = torch.tensor([0, 1, 63, 64, 130, 700], dtype=torch.int32)
    for b, plen in enumerate(t["prompt_len"].tolist()):
        t["k_cache"][b, :, plen:] = float("nan")
        t["v_cache"][b, :, plen:] = float("inf")
    for kv_chunk in (0, 64, 128):
        out, _, _ = _check(t, w, f"nan tail chunk={kv_chunk}", impl=impl, kv_chunk=kv_chunk)
        assert torch.isfinite(out).all()


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
@pytest.mark.parametrize("big", [12.0, 200.0])
@pytest.mark.parametrize("B", [4, 32])
def test_late_keys_far_above_the_first_tiles(impl, big, B):
    # A few late prompt keys score far above everything before them (by
    # hundreds of log2 units for big=200): probabilities taken relative to an
    # early reference would overflow, so the result must still match.  The
    # block rows sit at RoPE position 0, where the rotation is exact, so the
    # bf16 query operand carries no rounding that keys this long would
    # magnify beyond the bf16 tolerance.  B = 32: 256 rows per workgroup.
    w = _w(NB=2, Hq=8, Hkv=2, P=600, B=B)
    t = gpu_inputs(w, 101)
    t["k_cache"][:, :, 590:593] = big
    t["k_cache"][1, :, 300] = -big
    pos_d = torch.zeros((2, B), dtype=torch.int32, device=dev())
    for kv_chunk in (0, 128, 640):
        out, lse, _ = _check(t, w, f"late big keys {big} B={B} chunk={kv_chunk}", impl=impl, kv_chunk=kv_chunk,
                             pos_d=pos_d)
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("impl", [sd.IMPL_MFMA, sd.IMPL_VALU])
def test_scores_rising_in_steps_across_tiles(impl):
    # keys whose scores climb tile after tile, each step a few tens of log2
    # units: the row's reference has to move up several times within one
    # split, and the rows of the wider blocks (128 and 256 rows per workgroup) too
    for B, Hq in ((4, 8), (16, 8), (32, 8)):
        w = _w(NB=2, Hq=Hq, Hkv=2, P=900, p_lo=800, B=B)
        t = gpu_inputs(w, 111 + B)
        for i in range(1, 9):
            t["k_cache"][:, :, 100 * i + 7] = 1.5 * i
        pos_d = torch.zeros((2, B), dtype=torch.int32, device=dev())
        for kv_chunk in (0, 320):
            out, lse, _ = _check(t, w, f"rising keys B={B} chunk={kv_chunk}", impl=impl, kv_chunk=kv_chunk,
                                 pos_d=pos_d)
            assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def test_mask_mistake_is_visible_in_block_dominated_case():
    # With no prompt the block mask decides the result: the kernel must sit far
    # closer to the temporal-mask oracle than to the all-visible one.
    w = _w(NB=2, P=0, B=8)
    t = gpu_inputs(w, 61)
    out, _, _ = _run(t, w)
    good, _, _ = oracle_for(t, w)
    wrong, _, _ = oracle_for(t, w, mask_mode=sd.MASK_FULL)
    g = synth.to_numpy64(out)
    assert np.abs(g - good).mean() * 10 < np.abs(g - wrong).mean()


def test_mfma_and_valu_agree_and_runs_are_deterministic():
    w = _w(NB=2, Hq=32, Hkv=8, P=700, B=8)
    t = gpu_inputs(w, 71)
    a1, _, _ = _run(t, w, impl=sd.IMPL_MFMA)
    a2, _, _ = _run(t, w, impl=sd.IMPL_MFMA)
    v1, _, _ = _run(t, w, impl=sd.IMPL_VALU)
    assert torch.equal(a1, a2)
    assert (a1.float() - v1.float()).abs().max().item() < 2e-2


@pytest.mark.parametrize("label,ov", [("rows128", dict(NB=64, Hq=8, Hkv=2, B=16)),
                                      ("rows64", dict(NB=64, Hq=8, Hkv=2, B=8)),
                                      ("rows256", dict(NB=64, Hq=16, Hkv=2, B=16)),
                                      ("two_row_groups", dict(NB=32, Hq=16, Hkv=2, B=32))])
def test_longest_first_item_order(label, ov):
    # Ragged prompts (0..2048, ties and empty splits included) in four splits of
    # 512 keys, more workgroups than the CUs hold at once: each workgroup takes
    # the (sequence, split) item of its rank by length, longest first.  Every
    # sequence is checked.
    w = _w(d=128, P=2048, p_lo=0, **ov)
    t = gpu_inputs(w, 141 + w.B + w.Hq)
    plan = sd.verify_plan(sd.make_desc(t["q_blk"], t["k_blk"], t["k_cache"], rope_base=w.rope_base, kv_chunk=512))
    assert plan["lpt"] == 1 and plan["nsplit"] == 4, plan
    _check(t, w, f"longest first {label}", kv_chunk=512)


# 256 rows per workgroup (head dim 128): eight row waves, each over all 64 keys
# of a tile for its 32 rows, and the query rows staged in the two last ring
# stages during the prologue.  Padded rows (160 real), block keys only,
# block-dominated prompts, eight query heads per KV head, two groups of 256, two block tiles,
# forced splits with ragged ends, custom positions and the all-visible mode.
ROWS256 = [
    ("m160", dict(NB=2, Hq=8, Hkv=2, P=200, B=20)),
    ("m256_p0", dict(NB=2, Hq=8, Hkv=2, P=0, p_lo=0, B=32)),
    ("m256_p17", dict(NB=3, Hq=8, Hkv=2, P=17, p_lo=0, B=32)),
    ("m256_g8", dict(NB=3, Hq=16, Hkv=2, P=333, p_lo=0, B=16)),
    ("m512", dict(NB=2, Hq=16, Hkv=2, P=150, B=32)),
    ("m160_b40", dict(NB=2, Hq=4, Hkv=2, P=150, B=40)),    # two block tiles ahead of the prompt
]


@pytest.mark.parametrize("label,ov", ROWS256, ids=[s[0] for s in ROWS256])
def test_rows256_workgroups(label, ov):
    w = _w(**ov)
    t = gpu_inputs(w, 61 + len(label))
    plan = sd.verify_plan(sd.make_desc(t["q_blk"], t["k_blk"], t["k_cache"], rope_base=w.rope_base))
    assert plan["rows_wg"] == 256 and plan["ksplit"] == 1 and plan["qsep"] == 0 and plan["blk_rows"] == 0, plan
    _check(t, w, f"rows256 {label}", impl=sd.IMPL_MFMA)
    if w.P > 64:
        _check(t, w, f"rows256 {label} chunk=64", impl=sd.IMPL_MFMA, kv_chunk=64)
    if label == "m256_p17":
        g = torch.Generator().manual_seed(17)
        pos_d = torch.stack([torch.randperm(w.B, generator=g) * 7 + 15000 for _ in range(w.NB)])
        _check(t, w, f"rows256 {label} pos_d", impl=sd.IMPL_MFMA, pos_d=pos_d.to(torch.int32).to(dev()))
        _check(t, w, f"rows256 {label} full", impl=sd.IMPL_MFMA, mask_mode=sd.MASK_FULL)


@pytest.mark.parametrize("label,ov", [("rows128", dict(Hq=8, Hkv=2, B=16)), ("rows256", dict(Hq=8, Hkv=2, B=32))])
def test_wide_block_tile_counts(label, ov):
    # The wide forms (two row tiles a wave) wait for their tiles in pairs.
    # Prompts of 0 .. 522 keys give 1 to 10 tiles in one split (the block
    # tiles first), odd and even counts with ragged ends, and splits of three
    # tiles give 1 to 4 per split.
    w = _w(NB=9, P=522, p_lo=0, **ov)
    t = gpu_inputs(w, 171 + w.B)
    t["prompt_len"][:] = torch.tensor([0, 1, 64, 65, 128, 190, 256, 300, 522], dtype=torch.int32)
    plan = sd.verify_plan(sd.make_desc(t["q_blk"], t["k_blk"], t["k_cache"], rope_base=w.rope_base))
    assert plan["row_tiles"] == 2 and plan["nstage"] == 4, plan
    for kv_chunk in (0, 192):
        _check(t, w, f"wide tiles {label} chunk={kv_chunk}", impl=sd.IMPL_MFMA, kv_chunk=kv_chunk)


def test_largest_batch_the_grid_takes():
    # The attention kernel's grid is (KV heads, batch x row groups, splits) and
    # its y dimension stops at 65535: a batch of 65535 with one row group per
    # KV head (2 heads per KV head x 2B = 8 rows), ragged prompts including 0,
    # checked on sampled sequences at both ends and in the middle.  Both
    # kernels; the next larger batch is refused on the host.
    w = _w(NB=65535, Hq=2, Hkv=1, d=64, P=128, p_lo=0, B=4)
    t = gpu_inputs(w, 131, on_device=True)
    b_idx = [0, 1, 2, 32767, 65532, 65533, 65534]
    for impl in (sd.IMPL_MFMA, sd.IMPL_VALU):
        _check(t, w, f"batch 65535 impl={impl}", impl=impl, b_idx=b_idx)
    big = dataclasses.replace(w, NB=65536)
    desc = sd.make_desc(torch.empty((65536, 8, 2, 64), dtype=torch.bfloat16),
                        torch.empty((65536, 8, 1, 64), dtype=torch.bfloat16),
                        torch.empty((65536, 1, 128, 64), dtype=torch.bfloat16), rope_base=big.rope_base)
    with pytest.raises(sd.SimsdError):
        sd.verify_workspace_bytes(desc)


def test_empty_inputs_are_noops():
    w = _w(NB=2, P=64, B=0)
    t = gpu_inputs(w, 81)
    out, lse, st = _run(t, w)
    assert out.numel() == 0
    w = _w(NB=0, P=64, B=4)
    t = gpu_inputs(w, 82)
    out, lse, st = _run(t, w)
    assert out.numel() == 0


# ---------------------------------------------------------------- full-size workloads

FULL = [
    ("sdar8b_p1024_b4", None),
    ("sdar8b_p4096_b8", [0, 17, 31]),
    ("sdar8b_p8192_b32", [0, 5]),
    ("sdar8b_var16k_b16_accept", "by_length"),
]


def _by_length(prompt_len):
    """The sequences with the shortest, the median and the longest prompt
    (the extremes of the ragged last splits), plus sequence 0."""
    order = torch.argsort(prompt_len.cpu(), stable=True).tolist()
    return sorted({0, order[0], order[len(order) // 2], order[-1]})


@pytest.mark.parametrize("name,b_idx", FULL, ids=[f[0] for f in FULL])
def test_full_size_workload(name, b_idx):
    w = W[name]
    t = gpu_inputs(w, 1000 + list(W).index(name), on_device=True)
    if b_idx == "by_length":
        b_idx = _by_length(t["prompt_len"])
        print(f"prompt lengths of the checked sequences: {t['prompt_len'][b_idx].tolist()}", flush=True)
    _check(t, w, name, b_idx=b_idx)
    del t
    torch.cuda.empty_cache()
