"""Python binding of the SimSD verification hot path (marshalling only).

Each function checks that the torch tensors it is given match the C ABI of
include/simsd.h (device, dtype, shape, contiguity), allocates outputs and
workspace with torch when the caller does not pass them, and calls the
library on the current HIP stream.  All arithmetic happens in the HIP
kernels; there is no CPU path.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib as L


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_DT = {torch.float32: L.F32, torch.bfloat16: L.BF16}


def make_desc(q_blk, k_blk, k_cache, *, rope_base, softmax_scale=0.0, mask_mode=L.MASK_TEMPORAL,
              impl=L.IMPL_AUTO, kv_chunk=0, p_max=None, rope_mode=L.ROPE_COPY):
    NB, twoB, Hq, d = q_blk.shape
    Hkv = k_blk.shape[2]
    if twoB % 2:
        raise ValueError("q_blk rows must be 2B (D rows then D~ rows)")
    if q_blk.dtype not in _DT:
        raise TypeError("q/k/v must be float32 or bfloat16")
    if p_max is None:
        p_max = 0 if k_cache is None else k_cache.shape[2]
    return L.VerifyDesc(NB, Hq, Hkv, d, twoB // 2, p_max, _DT[q_blk.dtype], int(mask_mode), int(impl),
                        int(kv_chunk), float(rope_base), float(softmax_scale), int(rope_mode))


def verify_workspace_bytes(desc) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.load().simsd_verify_attn_workspace(ctypes.byref(desc), ctypes.byref(n)),
            "simsd_verify_attn_workspace")
    return int(n.value)


def verify_plan(desc) -> dict:
    """How simsd_verify_attn would run `desc` (a VerifyDesc): the fields of
    simsd_verify_plan as a dict.  Host only."""
    p = L.VerifyPlan()
    L.check(L.load().simsd_verify_plan_info(ctypes.byref(desc), ctypes.byref(p)), "simsd_verify_plan_info")
    return {name: int(getattr(p, name)) for name, _ in L.VerifyPlan._fields_}


def verify_attn(q_blk, k_blk, v_blk, k_cache, v_cache, tau, prompt_len=None, pos_d=None, *,
                rope_base=10000.0, softmax_scale=0.0, mask_mode=L.MASK_TEMPORAL, impl=L.IMPL_AUTO,
                kv_chunk=0, rope_mode=L.ROPE_COPY, out=None, lse=None, status=None, workspace=None,
                stream=None, with_lse=True, with_status=True):
    """SimSD verification attention; returns (out, lse, status).

    q_blk [NB][2B][Hq][d], k_blk/v_blk [NB][2B][Hkv][d], k_cache/v_cache
    [NB][Hkv][P_max][d] (float32 or bfloat16, all the same), tau [NB][B]
    int32, prompt_len [NB] int32 or None, pos_d [NB][B] int32 or None.
    """
    lib = L.load()
    dt = q_blk.dtype
    NB, twoB, Hq, d = q_blk.shape
    Hkv = k_blk.shape[2]
    B = twoB // 2
    dev = q_blk.device
    _need(q_blk, "q_blk", dt)
    _need(k_blk, "k_blk", dt, (NB, twoB, Hkv, d), dev)
    _need(v_blk, "v_blk", dt, (NB, twoB, Hkv, d), dev)
    if k_cache is not None or v_cache is not None:
        _need(k_cache, "k_cache", dt, None, dev)
        _need(v_cache, "v_cache", dt, tuple(k_cache.shape), dev)
        if tuple(k_cache.shape[:2]) != (NB, Hkv) or k_cache.shape[3] != d:
            raise ValueError(f"k_cache must be [NB][Hkv][P_max][d], got {tuple(k_cache.shape)}")
    _need(tau, "tau", torch.int32, (NB, B), dev)
    if prompt_len is not None:
        _need(prompt_len, "prompt_len", torch.int32, (NB,), dev)
    if pos_d is not None:
        _need(pos_d, "pos_d", torch.int32, (NB, B), dev)
    desc = make_desc(q_blk, k_blk, k_cache, rope_base=rope_base, softmax_scale=softmax_scale,
                     mask_mode=mask_mode, impl=impl, kv_chunk=kv_chunk, rope_mode=rope_mode)
    if out is None:
        out = torch.empty_like(q_blk)
    _need(out, "out", dt, tuple(q_blk.shape), dev)
    if lse is None and with_lse:
        lse = torch.empty((NB, twoB, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (NB, twoB, Hq), dev)
    if status is None and with_status:
        status = torch.empty((NB,), dtype=torch.int32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, (NB,), dev)
    ws_bytes = verify_workspace_bytes(desc)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.simsd_verify_attn(ctypes.byref(desc), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache),
                               _ptr(v_cache), _ptr(prompt_len), _ptr(tau), _ptr(pos_d), _ptr(out), _ptr(lse),
                               _ptr(status), _ptr(workspace), ctypes.c_size_t(ws_len), _stream_handle(stream))
    L.check(rc, "simsd_verify_attn")
    return out, lse, status


@dataclass
class VerifyCall:
    """A verify_attn call with every pointer bound once (for timing loops).

    `keep` holds the bound tensors so their memory outlives the call object.
    """
    desc: L.VerifyDesc
    args: tuple
    keep: tuple = ()

    def __call__(self):
        rc = L.load().simsd_verify_attn(ctypes.byref(self.desc), *self.args)
        if rc:
            L.check(rc, "simsd_verify_attn")

    def timed(self, start, stop):
        """The same call with `start` / `stop` (torch.cuda.Event with timing,
        each recorded once before so that it exists) bound to the pass's own
        kernels: start of the attention kernel, end of the last kernel."""
        rc = L.load().simsd_verify_attn_timed(ctypes.byref(self.desc), *self.args,
                                              ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event))
        if rc:
            L.check(rc, "simsd_verify_attn_timed")


def bind_verify(q_blk, k_blk, v_blk, k_cache, v_cache, tau, prompt_len=None, pos_d=None, *, out, lse=None,
                status=None, workspace=None, stream=None, **desc_kw) -> VerifyCall:
    desc = make_desc(q_blk, k_blk, k_cache, **desc_kw)
    ws_bytes = verify_workspace_bytes(desc)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        raise ValueError(f"workspace of {ws_bytes} bytes required")
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache), _ptr(v_cache), _ptr(prompt_len), _ptr(tau),
            _ptr(pos_d), _ptr(out), _ptr(lse), _ptr(status), _ptr(workspace), ctypes.c_size_t(ws_len),
            _stream_handle(stream))
    keep = (q_blk, k_blk, v_blk, k_cache, v_cache, tau, prompt_len, pos_d, out, lse, status, workspace)
    return VerifyCall(desc, args, keep)


def accept_workspace_bytes(batch, B, vocab) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.load().simsd_accept_prefix_workspace(int(batch), int(B), int(vocab), ctypes.byref(n)),
            "simsd_accept_prefix_workspace")
    return int(n.value)


def accept_prefix(p_target, q_draft, draft_tok, tau, gamma, seed, offset=0, *, n_accepted=None, next_token=None,
                  status=None, workspace=None, stream=None, with_next=True, with_status=True):
    """tau-ordered rejection-sampling acceptance; returns (n_accepted, next_token, status)."""
    lib = L.load()
    NB, B, V = p_target.shape
    dev = p_target.device
    _need(p_target, "p_target", torch.float32)
    _need(q_draft, "q_draft", torch.float32, (NB, B, V), dev)
    _need(draft_tok, "draft_tok", torch.int32, (NB, B), dev)
    _need(tau, "tau", torch.int32, (NB, B), dev)
    if n_accepted is None:
        n_accepted = torch.empty((NB,), dtype=torch.int32, device=dev)
    _need(n_accepted, "n_accepted", torch.int32, (NB,), dev)
    if next_token is None and with_next:
        next_token = torch.empty((NB,), dtype=torch.int32, device=dev)
    if next_token is not None:
        _need(next_token, "next_token", torch.int32, (NB,), dev)
    if status is None and with_status:
        status = torch.empty((NB,), dtype=torch.int32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, (NB,), dev)
    if next_token is not None and workspace is None:
        ws_bytes = accept_workspace_bytes(NB, B, V)
        if ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.simsd_accept_prefix(_ptr(p_target), _ptr(q_draft), _ptr(draft_tok), _ptr(tau), NB, B, int(gamma),
                                 V, ctypes.c_uint64(int(seed)), ctypes.c_uint64(int(offset)), _ptr(n_accepted),
                                 _ptr(next_token), _ptr(status), _ptr(workspace), ctypes.c_size_t(ws_len),
                                 _stream_handle(stream))
    L.check(rc, "simsd_accept_prefix")
    return n_accepted, next_token, status


def accept_prefix_noalloc(p_target, q_draft, draft_tok, tau, gamma, seed, offset=0, *, n_accepted=None,
                          next_token=None, status=None, stream=None, with_next=True, with_status=True):
    """accept_prefix through the entry point that takes no workspace (its
    scratch is the library's fixed device array); returns (n_accepted,
    next_token, status)."""
    lib = L.load()
    NB, B, V = p_target.shape
    dev = p_target.device
    _need(p_target, "p_target", torch.float32)
    _need(q_draft, "q_draft", torch.float32, (NB, B, V), dev)
    _need(draft_tok, "draft_tok", torch.int32, (NB, B), dev)
    _need(tau, "tau", torch.int32, (NB, B), dev)
    if n_accepted is None:
        n_accepted = torch.empty((NB,), dtype=torch.int32, device=dev)
    _need(n_accepted, "n_accepted", torch.int32, (NB,), dev)
    if next_token is None and with_next:
        next_token = torch.empty((NB,), dtype=torch.int32, device=dev)
    if next_token is not None:
        _need(next_token, "next_token", torch.int32, (NB,), dev)
    if status is None and with_status:
        status = torch.empty((NB,), dtype=torch.int32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, (NB,), dev)
    rc = lib.simsd_accept_prefix_noalloc(_ptr(p_target), _ptr(q_draft), _ptr(draft_tok), _ptr(tau), NB, B,
                                         int(gamma), V, ctypes.c_uint64(int(seed)), ctypes.c_uint64(int(offset)),
                                         _ptr(n_accepted), _ptr(next_token), _ptr(status), _stream_handle(stream))
    L.check(rc, "simsd_accept_prefix_noalloc")
    return n_accepted, next_token, status


def linear(x, w, *, out=None, stream=None):
    """y = x w^T for bf16 x [M][K] and w [N][K] (fp32 accumulation); returns y [M][N] bf16."""
    lib = L.load()
    _need(x, "x", torch.bfloat16)
    M, K = x.shape
    _need(w, "w", torch.bfloat16, None, x.device)
    N = w.shape[0]
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError(f"w must be [N][{K}], got {tuple(w.shape)}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (M, N), x.device)
    L.check(lib.simsd_linear(_ptr(x), _ptr(w), M, N, K, _ptr(out), _stream_handle(stream)), "simsd_linear")
    return out


def qkv_proj(x, w_qkv, Hq, Hkv, d, *, q=None, k=None, v=None, stream=None):
    """Fused QKV projection of block hidden states x [NB][2B][H] (bf16) into
    (q [NB][2B][Hq][d], k, v [NB][2B][Hkv][d])."""
    lib = L.load()
    _need(x, "x", torch.bfloat16)
    NB, twoB, H = x.shape
    dev = x.device
    _need(w_qkv, "w_qkv", torch.bfloat16, ((Hq + 2 * Hkv) * d, H), dev)
    if q is None:
        q = torch.empty((NB, twoB, Hq, d), dtype=torch.bfloat16, device=dev)
    if k is None:
        k = torch.empty((NB, twoB, Hkv, d), dtype=torch.bfloat16, device=dev)
    if v is None:
        v = torch.empty((NB, twoB, Hkv, d), dtype=torch.bfloat16, device=dev)
    _need(q, "q", torch.bfloat16, (NB, twoB, Hq, d), dev)
    _need(k, "k", torch.bfloat16, (NB, twoB, Hkv, d), dev)
    _need(v, "v", torch.bfloat16, (NB, twoB, Hkv, d), dev)
    L.check(lib.simsd_qkv_proj(_ptr(x), _ptr(w_qkv), NB * twoB, H, Hq, Hkv, d, _ptr(q), _ptr(k), _ptr(v),
                               _stream_handle(stream)), "simsd_qkv_proj")
    return q, k, v


def commit(tau, draft_tok, n_accepted, next_token, committed, block_tok, stream=None):
    """Commit one round's accepted prefix (and replacement) into the block state
    (committed [NB] int64 view of the uint64 masks, block_tok [NB][B] int32), in place."""
    lib = L.load()
    _need(tau, "tau", torch.int32)
    NB, B = tau.shape
    dev = tau.device
    _need(draft_tok, "draft_tok", torch.int32, (NB, B), dev)
    _need(n_accepted, "n_accepted", torch.int32, (NB,), dev)
    if next_token is not None:
        _need(next_token, "next_token", torch.int32, (NB,), dev)
    _need(committed, "committed", torch.int64, (NB,), dev)
    _need(block_tok, "block_tok", torch.int32, (NB, B), dev)
    L.check(lib.simsd_commit(_ptr(tau), _ptr(draft_tok), _ptr(n_accepted), _ptr(next_token), NB, B, _ptr(committed),
                             _ptr(block_tok), _stream_handle(stream)), "simsd_commit")
    return committed, block_tok


def next_round(committed, block_tok, draft_tok, rank=None, tau_out=None, tok_out=None, stream=None):
    """Stage labels and data tokens of the block's next round: committed
    positions get stage 0 and their tokens, open ones stages 1..m in the
    drafter's order (rank, ties by position; position order without rank)
    and the drafter's tokens.  Returns (tau, tok) [NB][B] int32."""
    lib = L.load()
    _need(block_tok, "block_tok", torch.int32)
    NB, B = block_tok.shape
    dev = block_tok.device
    _need(committed, "committed", torch.int64, (NB,), dev)
    _need(draft_tok, "draft_tok", torch.int32, (NB, B), dev)
    if rank is not None:
        _need(rank, "rank", torch.int32, (NB, B), dev)
    tau_out = torch.empty((NB, B), dtype=torch.int32, device=dev) if tau_out is None else tau_out
    tok_out = torch.empty((NB, B), dtype=torch.int32, device=dev) if tok_out is None else tok_out
    _need(tau_out, "tau_out", torch.int32, (NB, B), dev)
    _need(tok_out, "tok_out", torch.int32, (NB, B), dev)
    L.check(lib.simsd_next_round(_ptr(committed), _ptr(block_tok), _ptr(rank), _ptr(draft_tok), NB, B, _ptr(tau_out),
                                 _ptr(tok_out), _stream_handle(stream)), "simsd_next_round")
    return tau_out, tok_out


def bind_next_round(committed, block_tok, draft_tok, rank, tau_out, tok_out, stream=None) -> BoundCall:
    NB, B = block_tok.shape
    for t, name in ((block_tok, "block_tok"), (draft_tok, "draft_tok"), (tau_out, "tau_out"), (tok_out, "tok_out")):
        _need(t, name, torch.int32, (NB, B), block_tok.device)
    _need(committed, "committed", torch.int64, (NB,), block_tok.device)
    if rank is not None:
        _need(rank, "rank", torch.int32, (NB, B), block_tok.device)
    return BoundCall("simsd_next_round", (_ptr(committed), _ptr(block_tok), _ptr(rank), _ptr(draft_tok), NB, B,
                                          _ptr(tau_out), _ptr(tok_out), _stream_handle(stream)),
                     (committed, block_tok, draft_tok, rank, tau_out, tok_out))


def append_kv(k_blk, v_blk, k_cache, v_cache, prompt_len, *, rope_base, committed=None, pos_d=None, status=None,
              stream=None):
    """Append finished blocks' data rows to the cache (in place); prompt_len grows by B
    for every appended sequence.  Returns status [NB]."""
    lib = L.load()
    dt = k_blk.dtype
    NB, twoB, Hkv, d = k_blk.shape
    B = twoB // 2
    dev = k_blk.device
    _need(k_blk, "k_blk", dt)
    _need(v_blk, "v_blk", dt, tuple(k_blk.shape), dev)
    _need(k_cache, "k_cache", dt, None, dev)
    _need(v_cache, "v_cache", dt, tuple(k_cache.shape), dev)
    if tuple(k_cache.shape[:2]) != (NB, Hkv) or k_cache.shape[3] != d:
        raise ValueError(f"k_cache must be [NB][Hkv][p_max][d], got {tuple(k_cache.shape)}")
    _need(prompt_len, "prompt_len", torch.int32, (NB,), dev)
    if committed is not None:
        _need(committed, "committed", torch.int64, (NB,), dev)
    if pos_d is not None:
        _need(pos_d, "pos_d", torch.int32, (NB, B), dev)
    if status is None:
        status = torch.empty((NB,), dtype=torch.int32, device=dev)
    _need(status, "status", torch.int32, (NB,), dev)
    desc = L.VerifyDesc(NB, Hkv, Hkv, d, B, k_cache.shape[2], _DT[dt], 0, 0, 0, float(rope_base), 0.0, 0)
    L.check(lib.simsd_append_kv(ctypes.byref(desc), _ptr(k_blk), _ptr(v_blk), _ptr(pos_d), _ptr(committed),
                                _ptr(prompt_len), _ptr(k_cache), _ptr(v_cache), _ptr(status), _stream_handle(stream)),
            "simsd_append_kv")
    return status


@dataclass
class BoundCall:
    """A C-ABI call with every argument marshalled once (for timing loops).
    `keep` holds the bound tensors."""
    fn: str
    args: tuple
    keep: tuple = ()

    def __call__(self):
        rc = getattr(L.load(), self.fn)(*self.args)
        if rc:
            L.check(rc, self.fn)


def bind_commit(tau, draft_tok, n_accepted, next_token, committed, block_tok, stream=None) -> BoundCall:
    NB, B = tau.shape
    for t, name in ((tau, "tau"), (draft_tok, "draft_tok"), (block_tok, "block_tok")):
        _need(t, name, torch.int32, (NB, B), tau.device)
    _need(n_accepted, "n_accepted", torch.int32, (NB,), tau.device)
    _need(committed, "committed", torch.int64, (NB,), tau.device)
    return BoundCall("simsd_commit", (_ptr(tau), _ptr(draft_tok), _ptr(n_accepted), _ptr(next_token), NB, B,
                                      _ptr(committed), _ptr(block_tok), _stream_handle(stream)),
                     (tau, draft_tok, n_accepted, next_token, committed, block_tok))


def bind_append_kv(k_blk, v_blk, k_cache, v_cache, prompt_len, *, rope_base, committed=None, pos_d=None, status=None,
                   stream=None) -> BoundCall:
    dt = k_blk.dtype
    NB, twoB, Hkv, d = k_blk.shape
    _need(v_blk, "v_blk", dt, tuple(k_blk.shape), k_blk.device)
    _need(k_cache, "k_cache", dt, None, k_blk.device)
    _need(v_cache, "v_cache", dt, tuple(k_cache.shape), k_blk.device)
    _need(prompt_len, "prompt_len", torch.int32, (NB,), k_blk.device)
    desc = L.VerifyDesc(NB, Hkv, Hkv, d, twoB // 2, k_cache.shape[2], _DT[dt], 0, 0, 0, float(rope_base), 0.0, 0)
    return BoundCall("simsd_append_kv", (ctypes.byref(desc), _ptr(k_blk), _ptr(v_blk), _ptr(pos_d), _ptr(committed),
                                         _ptr(prompt_len), _ptr(k_cache), _ptr(v_cache), _ptr(status),
                                         _stream_handle(stream)),
                     (desc, k_blk, v_blk, k_cache, v_cache, prompt_len, committed, pos_d, status))


def bind_linear(x, w, out, stream=None) -> BoundCall:
    _need(x, "x", torch.bfloat16)
    M, K = x.shape
    _need(w, "w", torch.bfloat16, None, x.device)
    N = w.shape[0]
    _need(out, "out", torch.bfloat16, (M, N), x.device)
    return BoundCall("simsd_linear", (_ptr(x), _ptr(w), M, N, K, _ptr(out), _stream_handle(stream)), (x, w, out))


def bind_qkv_proj(x, w_qkv, Hq, Hkv, d, q, k, v, stream=None) -> BoundCall:
    _need(x, "x", torch.bfloat16)
    NB, twoB, H = x.shape
    dev = x.device
    _need(w_qkv, "w_qkv", torch.bfloat16, ((Hq + 2 * Hkv) * d, H), dev)
    _need(q, "q", torch.bfloat16, (NB, twoB, Hq, d), dev)
    _need(k, "k", torch.bfloat16, (NB, twoB, Hkv, d), dev)
    _need(v, "v", torch.bfloat16, (NB, twoB, Hkv, d), dev)
    return BoundCall("simsd_qkv_proj", (_ptr(x), _ptr(w_qkv), NB * twoB, H, Hq, Hkv, d, _ptr(q), _ptr(k), _ptr(v),
                                        _stream_handle(stream)), (x, w_qkv, q, k, v))


def accept_coupled_workspace_bytes(batch, B, vocab) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.load().simsd_accept_coupled_workspace(int(batch), int(B), int(vocab), ctypes.byref(n)),
            "simsd_accept_coupled_workspace")
    return int(n.value)


def accept_coupled(p_target, noise_exp, draft_tok, tau, gamma, *, n_accepted=None, next_token=None, status=None,
                   workspace=None, stream=None, with_next=True, with_status=True):
    """Coupled-noise acceptance walked in tau order; returns (n_accepted, next_token, status)."""
    lib = L.load()
    NB, B, V = p_target.shape
    dev = p_target.device
    _need(p_target, "p_target", torch.float32)
    _need(noise_exp, "noise_exp", torch.float32, (NB, B, V), dev)
    _need(draft_tok, "draft_tok", torch.int32, (NB, B), dev)
    _need(tau, "tau", torch.int32, (NB, B), dev)
    if n_accepted is None:
        n_accepted = torch.empty((NB,), dtype=torch.int32, device=dev)
    _need(n_accepted, "n_accepted", torch.int32, (NB,), dev)
    if next_token is None and with_next:
        next_token = torch.empty((NB,), dtype=torch.int32, device=dev)
    if next_token is not None:
        _need(next_token, "next_token", torch.int32, (NB,), dev)
    if status is None and with_status:
        status = torch.empty((NB,), dtype=torch.int32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, (NB,), dev)
    if workspace is None:
        workspace = torch.empty(max(accept_coupled_workspace_bytes(NB, B, V), 256), dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    rc = lib.simsd_accept_coupled(_ptr(p_target), _ptr(noise_exp), _ptr(draft_tok), _ptr(tau), NB, B, int(gamma), V,
                                  _ptr(n_accepted), _ptr(next_token), _ptr(status), _ptr(workspace),
                                  ctypes.c_size_t(ws_len), _stream_handle(stream))
    L.check(rc, "simsd_accept_coupled")
    return n_accepted, next_token, status


@dataclass
class AcceptCall:
    """An accept_prefix call with every pointer bound once (for timing loops);
    call it with (seed, offset).  `keep` holds the bound tensors."""
    args_head: tuple
    args_tail: tuple
    keep: tuple = ()

    def __call__(self, seed, offset=0):
        rc = L.load().simsd_accept_prefix(*self.args_head, ctypes.c_uint64(int(seed)), ctypes.c_uint64(int(offset)),
                                          *self.args_tail)
        if rc:
            L.check(rc, "simsd_accept_prefix")


def bind_accept(p_target, q_draft, draft_tok, tau, gamma, *, n_accepted, next_token=None, status=None,
                workspace=None, stream=None) -> AcceptCall:
    NB, B, V = p_target.shape
    dev = p_target.device
    _need(p_target, "p_target", torch.float32)
    _need(q_draft, "q_draft", torch.float32, (NB, B, V), dev)
    _need(draft_tok, "draft_tok", torch.int32, (NB, B), dev)
    _need(tau, "tau", torch.int32, (NB, B), dev)
    _need(n_accepted, "n_accepted", torch.int32, (NB,), dev)
    if next_token is not None:
        _need(next_token, "next_token", torch.int32, (NB,), dev)
        ws_bytes = accept_workspace_bytes(NB, B, V)
        if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
            raise ValueError(f"workspace of {ws_bytes} bytes required")
    if status is not None:
        _need(status, "status", torch.int32, (NB,), dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    head = (_ptr(p_target), _ptr(q_draft), _ptr(draft_tok), _ptr(tau), NB, B, int(gamma), V)
    tail = (_ptr(n_accepted), _ptr(next_token), _ptr(status), _ptr(workspace), ctypes.c_size_t(ws_len),
            _stream_handle(stream))
    return AcceptCall(head, tail, (p_target, q_draft, draft_tok, tau, n_accepted, next_token, status, workspace))


@dataclass
class CoupledCall:
    """An accept_coupled call with every pointer bound once (for timing loops).
    `keep` holds the bound tensors."""
    args: tuple
    keep: tuple = ()

    def __call__(self):
        rc = L.load().simsd_accept_coupled(*self.args)
        if rc:
            L.check(rc, "simsd_accept_coupled")


def bind_accept_coupled(p_target, noise_exp, draft_tok, tau, gamma, *, n_accepted, next_token=None, status=None,
                        workspace, stream=None) -> CoupledCall:
    NB, B, V = p_target.shape
    dev = p_target.device
    _need(p_target, "p_target", torch.float32)
    _need(noise_exp, "noise_exp", torch.float32, (NB, B, V), dev)
    _need(draft_tok, "draft_tok", torch.int32, (NB, B), dev)
    _need(tau, "tau", torch.int32, (NB, B), dev)
    _need(n_accepted, "n_accepted", torch.int32, (NB,), dev)
    for t, name in ((next_token, "next_token"), (status, "status")):
        if t is not None:
            _need(t, name, torch.int32, (NB,), dev)
    ws_len = workspace.numel() * workspace.element_size()
    if ws_len < accept_coupled_workspace_bytes(NB, B, V):
        raise ValueError(f"workspace of {accept_coupled_workspace_bytes(NB, B, V)} bytes required")
    args = (_ptr(p_target), _ptr(noise_exp), _ptr(draft_tok), _ptr(tau), NB, B, int(gamma), V, _ptr(n_accepted),
            _ptr(next_token), _ptr(status), _ptr(workspace), ctypes.c_size_t(ws_len), _stream_handle(stream))
    return CoupledCall(args, (p_target, noise_exp, draft_tok, tau, n_accepted, next_token, status, workspace))


def stream_probe(k_cache, v_cache, sink, start=None, stop=None, stream=None):
    """The attention kernel's load path alone over a prompt cache [NB][Hkv][P][d]
    (bf16): the streaming ceiling it is compared with.  `start` / `stop`
    (torch.cuda.Event, each recorded once before) take the kernel's own start
    and end."""
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(v_cache, "v_cache", torch.bfloat16, tuple(k_cache.shape), k_cache.device)
    _need(sink, "sink", torch.int32, None, k_cache.device)
    NB, Hkv, P, d = k_cache.shape
    ev = [ctypes.c_void_p(0 if e is None else e.cuda_event) for e in (start, stop)]
    L.check(L.load().simsd_stream_probe(_ptr(k_cache), _ptr(v_cache), Hkv, NB, P, d, _ptr(sink),
                                        _stream_handle(stream), *ev), "simsd_stream_probe")


def read_probe(k_cache, v_cache, sink, start=None, stop=None, stream=None):
    """Plain vector-load read of the same two regions (no LDS), for
    comparison with stream_probe.  Events as for stream_probe."""
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(v_cache, "v_cache", torch.bfloat16, tuple(k_cache.shape), k_cache.device)
    _need(sink, "sink", torch.int32, None, k_cache.device)
    ev = [ctypes.c_void_p(0 if e is None else e.cuda_event) for e in (start, stop)]
    L.check(L.load().simsd_read_probe(_ptr(k_cache), _ptr(v_cache), k_cache.numel() * 2, _ptr(sink),
                                      _stream_handle(stream), *ev), "simsd_read_probe")


MFMA_PROBE_THREADS = 256
MFMA_PROBE_FLOPS_PER_ROUND = 4 * 2 * 32 * 32 * 16  # per wave: four 32x32x16 MFMAs


def mfma_probe(workgroups, iters, sink, start=None, stop=None, stream=None):
    """The bf16 matrix cores alone: `workgroups` x 4 waves of independent
    32x32x16 MFMAs on registers for `iters` rounds (MFMA_PROBE_FLOPS_PER_ROUND
    flops per wave and round).  `sink`: float32, at least workgroups * 256.
    Events as for stream_probe."""
    _need(sink, "sink", torch.float32)
    if sink.numel() < int(workgroups) * MFMA_PROBE_THREADS:
        raise ValueError("sink needs workgroups * 256 floats")
    ev = [ctypes.c_void_p(0 if e is None else e.cuda_event) for e in (start, stop)]
    L.check(L.load().simsd_mfma_probe(int(workgroups), int(iters), _ptr(sink), _stream_handle(stream), *ev),
            "simsd_mfma_probe")


def debug_mask(tau, mask_mode=L.MASK_TEMPORAL, stream=None):
    """Block visibility words [NB][2B][2] (int64 view of the uint64 bits)."""
    lib = L.load()
    NB, B = tau.shape
    _need(tau, "tau", torch.int32)
    bits = torch.zeros((NB, 2 * B, 2), dtype=torch.int64, device=tau.device)
    L.check(lib.simsd_debug_mask(_ptr(tau), NB, B, int(mask_mode), _ptr(bits), _stream_handle(stream)),
            "simsd_debug_mask")
    return bits


def debug_rope(q_blk, k_blk, prompt_len=None, pos_d=None, *, rope_base, p_max=0, rope_mode=L.ROPE_COPY,
               stream=None):
    """Rotated block rows (q_rot, k_rot) as the attention kernels use them."""
    lib = L.load()
    _need(q_blk, "q_blk", q_blk.dtype)
    _need(k_blk, "k_blk", q_blk.dtype)
    desc = make_desc(q_blk, k_blk, None, rope_base=rope_base, p_max=p_max, rope_mode=rope_mode)
    q_rot = torch.empty_like(q_blk)
    k_rot = torch.empty_like(k_blk)
    L.check(lib.simsd_debug_rope(ctypes.byref(desc), _ptr(q_blk), _ptr(k_blk), _ptr(prompt_len), _ptr(pos_d),
                                 _ptr(q_rot), _ptr(k_rot), _stream_handle(stream)), "simsd_debug_rope")
    return q_rot, k_rot
