"""Host checks of the launch plan (simsd_verify_plan_info, no GPU needed).

The MFMA kernel has two ways of handling the 2B block keys: in an LDS region
of their own, loaded with the query rows and done before the first prompt
tile, or streamed through the tile ring ahead of the prompt tiles.  These
tests pin which one the benchmark workloads take, check that the GPU parity
cases reach both, and check the planner's invariants over a sweep of shapes:
every plan fits the LDS, and the block region never costs a workgroup per CU.
"""
import ctypes
import dataclasses
import itertools

import pytest

import diffusion_lm_speculative_amd as sd
from diffusion_lm_speculative_amd import _lib as L
from diffusion_lm_speculative_amd import synth
from tests.test_gpu_verify import LONG, SMALL

LDS_PER_CU = 163840
LDS_RESERVE = 1024  # per workgroup, kept free by the planner


def _desc(NB, Hq, Hkv, d, B, p_max, dtype=L.BF16, impl=L.IMPL_AUTO, rope_mode=L.ROPE_COPY, kv_chunk=0):
    return L.VerifyDesc(NB, Hq, Hkv, d, B, p_max, dtype, L.MASK_TEMPORAL, impl, kv_chunk, 1e6, 0.0, rope_mode)


def _plan_of(w, **kw):
    dt = L.F32 if "float32" in str(w.dtype) else L.BF16
    return sd.verify_plan(_desc(w.NB, w.Hq, w.Hkv, w.d, w.B, w.P, dtype=dt, **kw))


def _lds_without_block_region(p, d):
    return p["lds_bytes"] - 2 * p["blk_rows"] * d * 2


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    L.load()


@pytest.mark.parametrize("name,expect", [
    # workload: (rows per workgroup, row groups, key split, row tiles, stages, qsep, block rows, splits)
    # (1024-key prompts: one split, as splits of fewer than 16 tiles cost more in the merge than
    # they save; the 16k prompts are split at the 8192-key cap)
    ("sdar8b_p1024_b4", (32, 1, 4, 1, 4, 1, 16, 1)),
    ("sdar8b_p4096_b8", (64, 1, 2, 1, 4, 1, 16, 1)),
    ("sdar8b_p8192_b32", (256, 1, 1, 2, 4, 0, 0, 4)),
    ("sdar8b_var16k_b16_accept", (128, 1, 2, 2, 4, 0, 32, 2)),
])
def test_benchmark_workload_plans(name, expect):
    p = _plan_of(synth.WORKLOADS[name])
    got = (p["rows_wg"], p["row_groups"], p["ksplit"], p["row_tiles"], p["nstage"], p["qsep"], p["blk_rows"],
           p["nsplit"])
    assert p["impl"] == L.IMPL_MFMA and got == expect, p
    assert p["lds_bytes"] + LDS_RESERVE <= LDS_PER_CU


def test_headline_plan_lds_layout():
    # 4-stage ring of 64-key K and V tiles, stage labels and positions, 64
    # staged query rows, 16 block K rows + 16 block V rows, RoPE table of B=8
    # positions (d/2 cos/sin pairs each)
    p = _plan_of(synth.WORKLOADS["sdar8b_p4096_b8"])
    d = 128
    assert p["lds_bytes"] == 4 * 2 * 64 * d * 2 + 512 + 64 * d * 2 + 2 * 16 * d * 2 + 8 * (d // 2) * 8


def test_parity_cases_reach_both_block_paths():
    base = synth.WORKLOADS["sdar8b_p1024_b4"]
    kinds = {}
    for label, ov in SMALL + [(f"long_{l}", dict(NB=2, P=1000, p_lo=300, **o)) for l, o in LONG]:
        w = dataclasses.replace(base, **ov)
        p = _plan_of(w, impl=L.IMPL_MFMA)
        kinds.setdefault(p["blk_rows"] > 0, []).append(label)
    assert kinds.get(True) and kinds.get(False), kinds
    assert "block_only" in kinds[True]  # P = 0: only the block keys, from their own region
    assert "b64_g4" in kinds[False] and "long_rows256" in kinds[False]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rope_mode", [L.ROPE_COPY, L.ROPE_SEQUENTIAL])
def test_plan_invariants_over_shapes(d, rope_mode):
    seen = set()
    for B, G, p_max in itertools.product(range(1, 65), (1, 2, 4, 8), (0, 64, 4096)):
        try:
            p = sd.verify_plan(_desc(4, 8 * G, 8, d, B, p_max, rope_mode=rope_mode))
        except L.SimsdError:
            continue  # a table too large for the MFMA kernel with an explicit request only
        if p["impl"] != L.IMPL_MFMA:
            continue
        assert p["lds_bytes"] + LDS_RESERVE <= LDS_PER_CU, (B, G, p)
        r = p["blk_rows"]
        if r:
            assert r % 16 == 0 and 2 * B <= r < 2 * B + 16 and 2 * B <= 64 and p["nstage"] == 4, (B, G, p)
            without = _lds_without_block_region(p, d) + LDS_RESERVE
            assert LDS_PER_CU // (p["lds_bytes"] + LDS_RESERVE) == LDS_PER_CU // without, (B, G, p)
        if p["rows_wg"] == 256:
            assert d == 128 and p["ksplit"] == 1 and p["row_tiles"] == 2 and p["threads"] == 512, (B, G, p)
            assert p["nstage"] == 4 and p["qsep"] == 0 and r == 0, (B, G, p)
        seen.add(r > 0)
    assert seen == {True, False}


def test_rows_per_workgroup():
    # G x 2B rows per KV head: one group of the smallest power-of-two form up to
    # 128 rows; at head dim 128 one group of 256 for 129..256 rows and groups of
    # 256 for multiples of 256, else groups of 128 (no more padded rows than
    # those); groups of 128 where a 256-row group would need a 3-stage ring
    # (the table of the positions without the RoPE copy at B = 32)
    def form(G, B, d=128, **kw):
        p = sd.verify_plan(_desc(4, 8 * G, 8, d, B, 4096, **kw))
        return p["rows_wg"], p["row_groups"]
    assert form(4, 8) == (64, 1)
    assert form(4, 16) == (128, 1)
    assert form(4, 17) == (256, 1)   # 136 rows
    assert form(4, 32) == (256, 1)
    assert form(8, 32) == (256, 2)
    assert form(4, 48) == (128, 3)   # 384 rows
    assert form(2, 64) == (128, 2)   # 256 rows, but the 64-position table leaves only 3 stages
    assert form(4, 32, d=64) == (128, 2)
    assert form(4, 32, rope_mode=L.ROPE_SEQUENTIAL) == (128, 2)


def test_default_splits_keep_at_least_16_tiles():
    for NB, Hkv, p_max in ((16, 8, 1024), (8, 8, 1024), (16, 8, 2048), (1, 2, 8192), (1, 8, 65536), (32, 8, 4096)):
        p = sd.verify_plan(_desc(NB, 4 * Hkv, Hkv, 128, 8, p_max))
        assert p["nsplit"] == 1 or p["chunk"] // 64 >= 16, (NB, Hkv, p_max, p)
        assert p["nsplit"] * p["chunk"] >= p_max
    # an explicit kv_chunk is taken as given
    p = sd.verify_plan(_desc(16, 32, 8, 128, 4, 1024, kv_chunk=256))
    assert p["nsplit"] == 4 and p["chunk"] == 256


@pytest.mark.parametrize("name,expect", [
    ("sdar8b_p1024_b4", 0),           # 67 MB of K/V: fits the last-level cache, kept there between calls
    ("sdar8b_p4096_b8", 1),           # 537 MB
    ("sdar8b_p8192_b32", 1),          # 256 MiB exactly
    ("sdar8b_var16k_b16_accept", 1),  # 4.3 GB of capacity
])
def test_non_temporal_kv_loads_per_workload(name, expect):
    assert _plan_of(synth.WORKLOADS[name])["kv_stream"] == expect


def test_non_temporal_kv_loads_threshold():
    # K and V in bf16: NB * Hkv * p_max * d * 4 bytes against 256 MiB
    at = sd.verify_plan(_desc(8, 32, 8, 128, 8, 8192))      # 2^28 bytes
    below = sd.verify_plan(_desc(8, 32, 8, 128, 8, 8128))   # one tile less per stream
    assert at["kv_stream"] == 1 and below["kv_stream"] == 0
    d64 = sd.verify_plan(_desc(8, 32, 8, 64, 8, 16384))     # the same bytes at head dim 64
    assert d64["kv_stream"] == 1
    valu = sd.verify_plan(_desc(8, 32, 8, 128, 8, 8192, impl=L.IMPL_VALU))
    assert valu["kv_stream"] == 0  # only the MFMA kernel streams through the DMA ring


def test_plan_rejects_like_the_call():
    bad = _desc(1, 3, 2, 128, 4, 64)  # Hq not a multiple of Hkv
    with pytest.raises(L.SimsdError):
        sd.verify_plan(bad)
    p = L.VerifyPlan()
    p.impl = 77
    assert L.load().simsd_verify_plan_info(ctypes.byref(bad), ctypes.byref(p)) == L.ERR_SHAPE
    assert p.impl == 77  # left unchanged
    assert L.load().simsd_verify_plan_info(None, ctypes.byref(p)) == L.ERR_NULL


@pytest.mark.parametrize("G", [1, 4])
def test_sequential_positions_run_on_the_matrix_cores_up_to_b62_at_head_dim_128(G):
    # Without the RoPE copy the table holds 2B positions (2B x 64 pairs x 8 bytes at head dim
    # 128).  Beside a 3-stage ring of 32 KiB tiles and the 512 bytes of labels it fits up to
    # B = 62; B = 63 and 64 go to the VALU kernel under AUTO.
    for B in range(1, 65):
        p = sd.verify_plan(_desc(4, 8 * G, 8, 128, B, 4096, rope_mode=L.ROPE_SEQUENTIAL))
        table = 2 * B * 64 * 8
        fits = 3 * 32768 + 512 + table + LDS_RESERVE <= LDS_PER_CU
        assert fits == (B <= 62), B
        assert p["impl"] == (L.IMPL_MFMA if fits else L.IMPL_VALU), (B, p)


def test_longest_first_only_where_the_grid_takes_several_rounds():
    # the batch-64 ragged workload (1024 workgroups over 256 CUs) ranks its
    # items; the one-round workloads keep the plain dispatch order
    lpt = {name: _plan_of(w)["lpt"] for name, w in synth.WORKLOADS.items()}
    assert lpt == {"tiny_fp32": 0, "sdar8b_p1024_b4": 0, "sdar8b_p4096_b8": 0, "sdar8b_p8192_b32": 0,
                   "sdar8b_var16k_b16_accept": 1}, lpt
    # more than 256 items per KV head: not ranked
    p = sd.verify_plan(_desc(300, 32, 8, 128, 16, 16384, kv_chunk=8192))
    assert p["nsplit"] == 2 and p["lpt"] == 0
