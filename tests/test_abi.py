"""C-ABI checks that need no GPU: the library loads, exports every function
include/simsd.h declares, and rejects invalid arguments on the host before
any HIP call (so nothing is launched).

Calls with made-up pointer values run only where no GPU is visible: they
must never reach a launch, and on a machine without a GPU a launch could not
touch memory anyway.
"""
import ctypes
import subprocess
import sys
import os
import re

import pytest
import torch

from diffusion_lm_speculative_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "simsd.h")

no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="fake-pointer validation calls run only where no GPU is visible")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libsimsd.so is not built (run __graft_entry__.build())")
    return L.load()


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"^\s*(?:int|const char\*)\s+(simsd_\w+)\s*\(", text, flags=re.M))


def test_header_declarations_match_binding():
    decl = _declared()
    assert decl == set(L.SIGNATURES), decl ^ set(L.SIGNATURES)
    assert len(decl) == 21


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    raw = ctypes.CDLL(L.LIB_PATH)
    for name in _declared():
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def test_abi_version_and_strerror(lib):
    assert lib.simsd_abi_version() == 9
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert lib.simsd_strerror(code)
    assert lib.simsd_strerror(-99) == b"unknown error code"


def _desc(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, B=4, p_max=256, dtype=L.BF16,
                mask_mode=L.MASK_TEMPORAL, impl=L.IMPL_AUTO, kv_chunk=0, rope_base=1e6, softmax_scale=0.0,
                rope_mode=L.ROPE_COPY)
    base.update(kw)
    return L.VerifyDesc(*[base[f] for f, _ in L.VerifyDesc._fields_])


def _ws(lib, **kw):
    n = ctypes.c_size_t(12345)
    rc = lib.simsd_verify_attn_workspace(ctypes.byref(_desc(**kw)), ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=6, n_kv_heads=4), L.ERR_SHAPE),
    (dict(head_dim=96), L.ERR_SHAPE),
    (dict(B=65), L.ERR_SHAPE),
    (dict(B=-1), L.ERR_SHAPE),
    (dict(batch=-3), L.ERR_SHAPE),
    (dict(p_max=-1), L.ERR_SHAPE),
    (dict(rope_base=0.0), L.ERR_SHAPE),
    (dict(rope_base=float("nan")), L.ERR_SHAPE),
    (dict(softmax_scale=-1.0), L.ERR_SHAPE),
    (dict(dtype=7), L.ERR_DTYPE),
    (dict(mask_mode=2), L.ERR_DTYPE),
    (dict(impl=3), L.ERR_DTYPE),
    (dict(impl=L.IMPL_MFMA, dtype=L.F32), L.ERR_DTYPE),
    (dict(rope_mode=2), L.ERR_DTYPE),
    (dict(rope_mode=-1), L.ERR_DTYPE),
    # without the RoPE copy the MFMA kernel's table of 2B = 128 positions does
    # not fit beside its ring at head dim 128
    (dict(impl=L.IMPL_MFMA, rope_mode=L.ROPE_SEQUENTIAL, B=64), L.ERR_SHAPE),
    (dict(kv_chunk=100), L.ERR_KV_CHUNK),
    (dict(kv_chunk=-64), L.ERR_KV_CHUNK),
])
def test_workspace_query_rejects(lib, kw, code):
    assert _ws(lib, **kw)[0] == code


def test_mfma_grid_limits(lib):
    # the MFMA grid is (Hkv, batch x row groups, splits): y and z must stay below 2^16
    assert _ws(lib, batch=65535, B=4, n_q_heads=8, n_kv_heads=2, p_max=64)[0] == 0
    assert _ws(lib, batch=65536, B=4, n_q_heads=8, n_kv_heads=2, p_max=64, impl=L.IMPL_MFMA)[0] == L.ERR_SHAPE
    # 256 rows per workgroup: 8 query heads per KV head x 2B = 64 -> 512 rows, 2 row groups
    assert _ws(lib, batch=32767, B=32, n_q_heads=8, n_kv_heads=1, p_max=64, impl=L.IMPL_MFMA)[0] == 0
    assert _ws(lib, batch=32768, B=32, n_q_heads=8, n_kv_heads=1, p_max=64, impl=L.IMPL_MFMA)[0] == L.ERR_SHAPE
    # 128 rows per workgroup: 4 query heads per KV head x 2B = 96 -> 384 rows, 3 row groups
    assert _ws(lib, batch=21845, B=48, n_q_heads=4, n_kv_heads=1, p_max=64, impl=L.IMPL_MFMA)[0] == 0
    assert _ws(lib, batch=21846, B=48, n_q_heads=4, n_kv_heads=1, p_max=64, impl=L.IMPL_MFMA)[0] == L.ERR_SHAPE
    # splits of 64 keys: 65535 of them fit, one more does not
    assert _ws(lib, batch=1, p_max=64 * 65535, kv_chunk=64, impl=L.IMPL_MFMA)[0] == 0
    assert _ws(lib, batch=1, p_max=64 * 65536, kv_chunk=64, impl=L.IMPL_MFMA)[0] == L.ERR_SHAPE
    # many KV heads are fine (x has no such limit), up to the planner's 65536 query heads
    assert _ws(lib, batch=1, n_q_heads=65536, n_kv_heads=65536, p_max=64)[0] == 0
    assert _ws(lib, batch=1, n_q_heads=65537, n_kv_heads=65537, p_max=64)[0] == L.ERR_SHAPE


def test_extreme_shapes_are_rejected_or_sized_without_overflow(lib):
    # sizes whose products overflow 32 or 64 bits must come back as an error
    # (never a wrapped-around size); the host-sanitizer run of this file
    # checks the arithmetic itself
    big = 2 ** 31 - 1
    for kw in (dict(n_q_heads=2 ** 30, n_kv_heads=1, B=64), dict(n_q_heads=big, n_kv_heads=1, B=64),
               dict(batch=big, n_q_heads=big, n_kv_heads=big, p_max=big), dict(batch=big, p_max=big, kv_chunk=64),
               dict(batch=big, n_q_heads=64, n_kv_heads=1, B=64, p_max=big),
               dict(batch=65535, n_q_heads=big, n_kv_heads=big, B=64, p_max=big, kv_chunk=64, impl=L.IMPL_VALU)):
        rc, n = _ws(lib, **kw)
        assert rc == L.ERR_SHAPE or (rc == 0 and 0 <= n < 2 ** 62), (kw, rc, n)
    n = ctypes.c_size_t(0)
    for NB, B, V in ((65535, 64, big), (1, 64, big), (65535, 1, 1)):
        assert lib.simsd_accept_prefix_workspace(NB, B, V, ctypes.byref(n)) == 0 and n.value < 2 ** 62
        assert lib.simsd_accept_coupled_workspace(NB, B, V, ctypes.byref(n)) in (0, L.ERR_SHAPE)
    for M, N, K in ((2 ** 62, 16, 64), (big, big - (big % 16), 64), (1, 16, 2 ** 31 - 64)):
        assert lib.simsd_linear(None, None, M, min(N, big), min(K, big), None, None) in (L.ERR_SHAPE, L.ERR_NULL)


def test_descriptor_layout():
    # int32 x 10, double, float, int32: the C struct is 56 bytes with the
    # double at offset 40
    assert ctypes.sizeof(L.VerifyDesc) == 56
    assert L.VerifyDesc.rope_base.offset == 40
    assert L.VerifyDesc.rope_mode.offset == 52


def test_sequential_positions_plan(lib):
    # AUTO still plans the cases the MFMA table cannot hold (on the VALU kernel)
    assert _ws(lib, rope_mode=L.ROPE_SEQUENTIAL, B=64)[0] == 0
    assert _ws(lib, rope_mode=L.ROPE_SEQUENTIAL, B=32, impl=L.IMPL_MFMA)[0] == 0
    assert _ws(lib, rope_mode=L.ROPE_SEQUENTIAL, B=64, head_dim=64, impl=L.IMPL_MFMA)[0] == 0


def test_workspace_query_sizes(lib):
    # one split: no workspace
    assert _ws(lib, kv_chunk=256) == (0, 0)
    assert _ws(lib, p_max=0) == (0, 0)
    assert _ws(lib, B=0) == (0, 0)
    # two splits of 128 keys: partial o [NB*Hkv*2][M][d] and (m, l) [..][M][2], 256-byte aligned
    NB, Hkv, M, d = 2, 2, 4 * 8, 128
    rc, n = _ws(lib, kv_chunk=128)
    ru = lambda x: (x + 255) // 256 * 256
    assert rc == 0 and n == ru(NB * Hkv * 2 * M * d * 4) + ru(NB * Hkv * 2 * M * 2 * 4)
    # default plan splits a long prompt; the size grows with the split count
    rc1, n1 = _ws(lib, p_max=8192, batch=1)
    assert rc1 == 0 and n1 > 0
    assert lib.simsd_verify_attn_workspace(None, ctypes.byref(ctypes.c_size_t())) == L.ERR_NULL
    assert lib.simsd_accept_prefix_workspace(4, 8, 151936, None) == L.ERR_NULL
    n = ctypes.c_size_t(7)
    # fp64 (residual, target) sums per 1024-entry chunk of a row (149 chunks for V = 151936), then a
    # 32-byte walk record per sequence, each part 256-byte aligned
    assert lib.simsd_accept_prefix_workspace(4, 8, 151936, ctypes.byref(n)) == 0
    assert n.value == ru(4 * 149 * 2 * 8) + ru(4 * 32)
    assert lib.simsd_accept_prefix_workspace(70, 8, 1000, ctypes.byref(n)) == 0
    assert n.value == ru(70 * 1 * 2 * 8) + ru(70 * 32)
    # one grid row per sequence
    assert lib.simsd_accept_prefix_workspace(65536, 8, 1000, ctypes.byref(n)) == L.ERR_SHAPE
    assert lib.simsd_accept_prefix_workspace(4, 0, 151936, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.simsd_accept_prefix_workspace(4, 65, 151936, ctypes.byref(n)) == L.ERR_SHAPE
    assert lib.simsd_accept_prefix_workspace(4, 8, 0, ctypes.byref(n)) == L.ERR_SHAPE


A = 0x10000  # an aligned made-up address; never dereferenced


def _verify(lib, desc, ptrs=None, ws=None, ws_bytes=0):
    p = dict(q=A, k=A, v=A, kc=A, vc=A, plen=None, tau=A, pos=None, out=A, lse=None, st=None)
    if ptrs:
        p.update(ptrs)
    return lib.simsd_verify_attn(ctypes.byref(desc) if desc is not None else None, p["q"], p["k"], p["v"],
                                 p["kc"], p["vc"], p["plen"], p["tau"], p["pos"], p["out"], p["lse"], p["st"],
                                 ws, ctypes.c_size_t(ws_bytes), None)


@no_gpu_only
def test_verify_rejects_on_host(lib):
    d = _desc(kv_chunk=256)
    assert _verify(lib, None) == L.ERR_NULL
    assert _verify(lib, _desc(head_dim=80)) == L.ERR_SHAPE
    for k in ("q", "k", "v", "tau", "out", "kc", "vc"):
        assert _verify(lib, d, {k: None}) == L.ERR_NULL, k
    for k, off in (("q", 8), ("k", 4), ("v", 2), ("kc", 8), ("vc", 8), ("out", 8), ("tau", 2), ("lse", 2),
                   ("st", 1), ("plen", 2), ("pos", 3)):
        assert _verify(lib, d, {k: A + off}) == L.ERR_ALIGN, k
    # two splits need a workspace
    d2 = _desc(kv_chunk=128)
    assert _verify(lib, d2) == L.ERR_WORKSPACE
    assert _verify(lib, d2, ws=A, ws_bytes=64) == L.ERR_WORKSPACE
    rc, need = _ws(lib, kv_chunk=128)
    assert _verify(lib, d2, ws=A + 16, ws_bytes=need) == L.ERR_ALIGN


@no_gpu_only
def test_verify_empty_is_noop(lib):
    # B == 0 or batch == 0: valid, nothing to launch, pointers may be NULL
    assert _verify(lib, _desc(B=0), dict(q=None, k=None, v=None, tau=None, out=None)) == 0
    assert _verify(lib, _desc(batch=0), dict(q=None, k=None, v=None, tau=None, out=None)) == 0
    # no prompt: caches may be NULL (still rejected here for a NULL output)
    assert _verify(lib, _desc(p_max=0), dict(kc=None, vc=None, out=None)) == L.ERR_NULL


@no_gpu_only
def test_accept_rejects_on_host(lib):
    def call(p=A, q=A, x=A, tau=A, NB=4, B=8, gamma=8, V=1000, n=A, nx=None, st=None, ws=None, wsb=0):
        return lib.simsd_accept_prefix(p, q, x, tau, NB, B, gamma, V, 1, 0, n, nx, st, ws,
                                       ctypes.c_size_t(wsb), None)
    assert call(gamma=9) == L.ERR_GAMMA
    assert call(gamma=-1) == L.ERR_GAMMA
    assert call(B=65, gamma=1) == L.ERR_SHAPE
    assert call(V=0) == L.ERR_SHAPE
    assert call(V=1 << 31) == L.ERR_SHAPE
    assert call(NB=-1) == L.ERR_SHAPE
    assert call(NB=0, p=None, q=None, x=None, tau=None, n=None) == 0
    for k in ("p", "q", "x", "tau", "n"):
        assert call(**{k: None}) == L.ERR_NULL, k
    for k in ("p", "q", "x", "tau", "n", "nx", "st"):
        assert call(**{k: A + 2}) == L.ERR_ALIGN, k
    assert call(NB=65536) == L.ERR_SHAPE
    # the residual draw (next_token != NULL, B and gamma > 0) needs the workspace
    assert call(nx=A) == L.ERR_WORKSPACE
    assert call(nx=A, ws=A, wsb=64) == L.ERR_WORKSPACE
    assert call(nx=A, ws=A + 16, wsb=1 << 20) == L.ERR_ALIGN


@no_gpu_only
def test_accept_noalloc_rejects_on_host(lib):
    def call(p=A, q=A, x=A, tau=A, NB=4, B=8, gamma=8, V=1000, n=A, nx=A, st=None):
        return lib.simsd_accept_prefix_noalloc(p, q, x, tau, NB, B, gamma, V, 1, 0, n, nx, st, None)
    # the same checks as simsd_accept_prefix
    assert call(gamma=9) == L.ERR_GAMMA
    assert call(B=65, gamma=1) == L.ERR_SHAPE
    assert call(NB=65536) == L.ERR_SHAPE
    assert call(V=0) == L.ERR_SHAPE
    for k in ("p", "q", "x", "tau", "n"):
        assert call(**{k: None}) == L.ERR_NULL, k
    for k in ("p", "q", "x", "tau", "n", "nx", "st"):
        assert call(**{k: A + 2}) == L.ERR_ALIGN, k
    assert call(NB=0, p=None, q=None, x=None, tau=None, n=None) == 0
    # scratch needed above the fixed 4 MiB: rejected before any HIP call
    n = ctypes.c_size_t(0)
    assert lib.simsd_accept_prefix_workspace(1800, 16, 151936, ctypes.byref(n)) == 0 and n.value > 4 << 20
    assert call(NB=1800, B=16, gamma=16, V=151936) == L.ERR_SCRATCH
    assert call(NB=1, B=2, gamma=2, V=(1 << 31) - 1) == L.ERR_SCRATCH
    assert lib.simsd_strerror(L.ERR_SCRATCH) != b"unknown error code"


@no_gpu_only
def test_stream_probe_rejects_on_host(lib):
    def call(k=A, v=A, sx=8, sy=32, n=4096, d=128, sink=A):
        return lib.simsd_stream_probe(k, v, sx, sy, n, d, sink, None, None, None)
    assert call(n=100) == L.ERR_SHAPE and call(d=96) == L.ERR_SHAPE and call(sy=65536) == L.ERR_SHAPE
    assert call(sx=0) == L.ERR_SHAPE and call(n=-64) == L.ERR_SHAPE
    assert call(n=0, k=None, v=None, sink=None) == 0
    for name in ("k", "v", "sink"):
        assert call(**{name: None}) == L.ERR_NULL, name
    assert call(k=A + 8) == L.ERR_ALIGN and call(sink=A + 2) == L.ERR_ALIGN


@no_gpu_only
def test_mfma_probe_rejects_on_host(lib):
    def call(wgs=256, iters=16, sink=A):
        return lib.simsd_mfma_probe(wgs, iters, sink, None, None, None)
    assert call(wgs=0) == L.ERR_SHAPE and call(wgs=65537) == L.ERR_SHAPE and call(iters=0) == L.ERR_SHAPE
    assert call(sink=None) == L.ERR_NULL
    assert call(sink=A + 2) == L.ERR_ALIGN


@no_gpu_only
def test_read_probe_rejects_on_host(lib):
    def call(k=A, v=A, n=1 << 20, sink=A):
        return lib.simsd_read_probe(k, v, n, sink, None, None, None)
    assert call(n=100) == L.ERR_SHAPE and call(n=-16) == L.ERR_SHAPE
    assert call(n=0, k=None, v=None, sink=None) == 0
    for name in ("k", "v", "sink"):
        assert call(**{name: None}) == L.ERR_NULL, name
    assert call(v=A + 8) == L.ERR_ALIGN and call(sink=A + 2) == L.ERR_ALIGN


@no_gpu_only
def test_commit_and_append_reject_on_host(lib):
    def com(tau=A, x=A, n=A, nx=A, NB=4, B=8, c=A, t=A):
        return lib.simsd_commit(tau, x, n, nx, NB, B, c, t, None)
    assert com(NB=0, tau=None, x=None, n=None, c=None, t=None) == 0
    assert com(B=65) == L.ERR_SHAPE
    assert com(NB=-1) == L.ERR_SHAPE
    for k in ("tau", "x", "n", "c", "t"):
        assert com(**{k: None}) == L.ERR_NULL, k
    for k in ("tau", "x", "n", "nx", "t"):
        assert com(**{k: A + 2}) == L.ERR_ALIGN, k
    assert com(c=A + 4) == L.ERR_ALIGN

    def nxt(c=A, bt=A, r=A, x=A, NB=4, B=8, t=A, o=A):
        return lib.simsd_next_round(c, bt, r, x, NB, B, t, o, None)
    assert nxt(NB=0, c=None, bt=None, x=None, t=None, o=None) == 0
    assert nxt(B=65) == L.ERR_SHAPE and nxt(NB=-2) == L.ERR_SHAPE
    for k in ("c", "bt", "x", "t", "o"):
        assert nxt(**{k: None}) == L.ERR_NULL, k
    for k in ("bt", "r", "x", "t", "o"):
        assert nxt(**{k: A + 2}) == L.ERR_ALIGN, k
    assert nxt(c=A + 4) == L.ERR_ALIGN

    def app(desc=None, kb=A, vb=A, pos=None, c=None, plen=A, kc=A, vc=A, st=None):
        d = desc if desc is not None else _desc()
        return lib.simsd_append_kv(ctypes.byref(d), kb, vb, pos, c, plen, kc, vc, st, None)
    assert lib.simsd_append_kv(None, A, A, None, None, A, A, A, None, None) == L.ERR_NULL
    assert app(desc=_desc(B=65)) == L.ERR_SHAPE
    assert app(desc=_desc(dtype=7)) == L.ERR_DTYPE
    assert app(desc=_desc(batch=65536)) == L.ERR_SHAPE  # one grid row per sequence
    assert app(desc=_desc(batch=0), kb=None, vb=None, plen=None, kc=None, vc=None) == 0
    for k in ("kb", "vb", "plen", "kc", "vc"):
        assert app(**{k: None}) == L.ERR_NULL, k
    for k in ("kb", "vb", "kc", "vc", "plen", "pos", "st"):
        assert app(**{k: A + 1}) == L.ERR_ALIGN, k
    assert app(c=A + 4) == L.ERR_ALIGN


@no_gpu_only
def test_projections_reject_on_host(lib):
    def lin(x=A, w=A, M=512, N=4096, K=4096, y=A):
        return lib.simsd_linear(x, w, M, N, K, y, None)
    assert lin(M=0, x=None, w=None, y=None) == 0
    assert lin(M=-1) == L.ERR_SHAPE
    assert lin(N=8) == L.ERR_SHAPE          # below 16
    assert lin(N=4104) == L.ERR_SHAPE       # not a multiple of 16
    assert lin(K=100) == L.ERR_SHAPE        # not a multiple of 64
    assert lin(K=0) == L.ERR_SHAPE
    assert lin(K=(1 << 24) + 64) == L.ERR_SHAPE
    assert lin(M=65536 * 128) == L.ERR_SHAPE
    for kw in ("x", "w", "y"):
        assert lin(**{kw: None}) == L.ERR_NULL, kw
        assert lin(**{kw: A + 8}) == L.ERR_ALIGN, kw

    def qkv(x=A, w=A, M=512, H=4096, Hq=32, Hkv=8, d=128, q=A, k=A, v=A):
        return lib.simsd_qkv_proj(x, w, M, H, Hq, Hkv, d, q, k, v, None)
    assert qkv(M=0, x=None, w=None, q=None, k=None, v=None) == 0
    assert qkv(d=72) == L.ERR_SHAPE
    assert qkv(Hq=0) == L.ERR_SHAPE
    assert qkv(Hkv=0) == L.ERR_SHAPE
    assert qkv(H=4000) == L.ERR_SHAPE
    for kw in ("x", "w", "q", "k", "v"):
        assert qkv(**{kw: None}) == L.ERR_NULL, kw
        assert qkv(**{kw: A + 4}) == L.ERR_ALIGN, kw


@no_gpu_only
def test_accept_coupled_rejects_on_host(lib):
    WS = 1 << 20
    def call(p=A, e=A, x=A, tau=A, NB=4, B=8, gamma=8, V=1000, n=A, nx=None, st=None, ws=A, wsb=WS):
        return lib.simsd_accept_coupled(p, e, x, tau, NB, B, gamma, V, n, nx, st, ws, ctypes.c_size_t(wsb), None)
    assert call(gamma=9) == L.ERR_GAMMA
    assert call(gamma=-1) == L.ERR_GAMMA
    assert call(B=65, gamma=1) == L.ERR_SHAPE
    assert call(V=0) == L.ERR_SHAPE
    assert call(V=65535 * 8192 + 1) == L.ERR_SHAPE
    assert call(NB=-1) == L.ERR_SHAPE
    assert call(NB=0, p=None, e=None, x=None, tau=None, n=None, ws=None) == 0
    for k in ("p", "e", "x", "tau", "n"):
        assert call(**{k: None}) == L.ERR_NULL, k
    for k in ("x", "tau", "n", "nx", "st"):
        assert call(**{k: A + 2}) == L.ERR_ALIGN, k
    for k in ("p", "e"):  # rows are read in 16-byte pieces
        assert call(**{k: A + 4}) == L.ERR_ALIGN, k
    assert call(ws=None) == L.ERR_WORKSPACE
    assert call(wsb=16) == L.ERR_WORKSPACE
    assert call(ws=A + 64) == L.ERR_ALIGN


def test_accept_coupled_workspace_size(lib):
    n = ctypes.c_size_t(0)
    assert lib.simsd_accept_coupled_workspace(4, 16, 151936, ctypes.byref(n)) == 0
    chunks = -(-151936 // 8192)
    assert n.value == -(-(4 * 16 * chunks * 16) // 256) * 256
    assert lib.simsd_accept_coupled_workspace(4, 65, 100, ctypes.byref(n)) == L.ERR_SHAPE
    assert lib.simsd_accept_coupled_workspace(4, 8, 100, None) == L.ERR_NULL


@no_gpu_only
def test_debug_entry_points_reject_on_host(lib):
    assert lib.simsd_debug_mask(A, 2, 65, 0, A, None) == L.ERR_SHAPE
    assert lib.simsd_debug_mask(A, 2, 4, 5, A, None) == L.ERR_DTYPE
    assert lib.simsd_debug_mask(None, 2, 4, 0, A, None) == L.ERR_NULL
    assert lib.simsd_debug_mask(A, 2, 4, 0, A + 4, None) == L.ERR_ALIGN
    assert lib.simsd_debug_mask(None, 0, 4, 0, None, None) == 0
    d = _desc()
    assert lib.simsd_debug_rope(None, A, A, None, None, A, A, None) == L.ERR_NULL
    assert lib.simsd_debug_rope(ctypes.byref(d), None, A, None, None, A, A, None) == L.ERR_NULL
    assert lib.simsd_debug_rope(ctypes.byref(d), A + 8, A, None, None, A, A, None) == L.ERR_ALIGN


def test_missing_library_raises_and_nothing_falls_back(tmp_path):
    # a fresh interpreter: loading a library that is not there raises, and
    # importing the package pulls in nothing from the oracle
    code = (
        "import sys\n"
        "import diffusion_lm_speculative_amd as sd\n"
        "from diffusion_lm_speculative_amd import _lib\n"
        "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'\n"
        "try:\n"
        f"    _lib.load({str(tmp_path / 'absent.so')!r})\n"
        "except RuntimeError as e:\n"
        "    print('raised', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(3)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr[-2000:])
    assert "is not built" in r.stdout


def test_product_sources_do_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "diffusion_lm_speculative_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
