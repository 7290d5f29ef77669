"""ctypes loader for libsimsd.so (the C ABI of include/simsd.h).

The library is built in-tree by ``diffusion_lm_speculative_amd.build``.  If it
is missing, every entry point raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_uint64 = ctypes.c_uint64
c_size_t = ctypes.c_size_t
c_void_p = ctypes.c_void_p
c_float = ctypes.c_float
c_double = ctypes.c_double

# Return codes and status flags (mirrors include/simsd.h).
OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_DTYPE = -3
ERR_WORKSPACE = -4
ERR_GAMMA = -5
ERR_ALIGN = -6
ERR_HIP = -7
ERR_KV_CHUNK = -8
ERR_SCRATCH = -9

ST_TAU_RANGE = 1
ST_TAU_NOT_PERM = 2
ST_PROMPT_LEN = 4
ST_TOKEN_RANGE = 8
ST_POS_NEG = 16

F32 = 0
BF16 = 1
MASK_TEMPORAL = 0
MASK_FULL = 1
IMPL_AUTO = 0
IMPL_VALU = 1
IMPL_MFMA = 2
ROPE_COPY = 0
ROPE_SEQUENTIAL = 1


class VerifyDesc(ctypes.Structure):
    _fields_ = [
        ("batch", c_int32),
        ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32),
        ("head_dim", c_int32),
        ("B", c_int32),
        ("p_max", c_int32),
        ("dtype", c_int32),
        ("mask_mode", c_int32),
        ("impl", c_int32),
        ("kv_chunk", c_int32),
        ("rope_base", c_double),
        ("softmax_scale", c_float),
        ("rope_mode", c_int32),
    ]


class VerifyPlan(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("impl", "threads", "rows_wg", "row_groups", "ksplit", "row_tiles", "nstage",
                                       "qsep", "blk_rows", "nsplit", "chunk", "lds_bytes", "kv_stream", "lpt")]


# name -> (restype, argtypes); every function declared in include/simsd.h.
SIGNATURES = {
    "simsd_verify_attn_workspace": (c_int32, [ctypes.POINTER(VerifyDesc), ctypes.POINTER(c_size_t)]),
    "simsd_verify_plan_info": (c_int32, [ctypes.POINTER(VerifyDesc), ctypes.POINTER(VerifyPlan)]),
    "simsd_verify_attn": (c_int32, [ctypes.POINTER(VerifyDesc)] + [c_void_p] * 12 + [c_size_t, c_void_p]),
    "simsd_verify_attn_timed": (c_int32, [ctypes.POINTER(VerifyDesc)] + [c_void_p] * 12 + [c_size_t, c_void_p,
                                                                                         c_void_p, c_void_p]),
    "simsd_accept_prefix_workspace": (c_int32, [c_int32, c_int32, c_int64, ctypes.POINTER(c_size_t)]),
    "simsd_accept_prefix": (c_int32, [c_void_p] * 4 + [c_int32, c_int32, c_int32, c_int64, c_uint64, c_uint64]
                            + [c_void_p] * 4 + [c_size_t, c_void_p]),
    "simsd_accept_prefix_noalloc": (c_int32, [c_void_p] * 4 + [c_int32, c_int32, c_int32, c_int64, c_uint64,
                                                          c_uint64] + [c_void_p] * 4),
    "simsd_accept_coupled_workspace": (c_int32, [c_int32, c_int32, c_int64, ctypes.POINTER(c_size_t)]),
    "simsd_accept_coupled": (c_int32, [c_void_p] * 4 + [c_int32, c_int32, c_int32, c_int64]
                             + [c_void_p] * 4 + [c_size_t, c_void_p]),
    "simsd_debug_mask": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "simsd_debug_rope": (c_int32, [ctypes.POINTER(VerifyDesc)] + [c_void_p] * 7),
    "simsd_stream_probe": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                     c_void_p, c_void_p]),
    "simsd_read_probe": (c_int32, [c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_void_p]),
    "simsd_mfma_probe": (c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "simsd_strerror": (ctypes.c_char_p, [c_int32]),
    "simsd_abi_version": (c_int32, []),
    "simsd_commit": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                               c_void_p]),
    "simsd_next_round": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                   c_void_p]),
    "simsd_append_kv": (c_int32, [ctypes.POINTER(VerifyDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_void_p]),
    "simsd_linear": (c_int32, [c_void_p, c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p]),
    "simsd_qkv_proj": (c_int32, [c_void_p, c_void_p, c_int64, c_int32, c_int32, c_int32, c_int32,
                                 c_void_p, c_void_p, c_void_p, c_void_p]),
}

_lib = None
_lock = threading.Lock()


class SimsdError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


def load(path: str = None):
    """Load libsimsd.so once and attach the C signatures.  The path defaults
    to the in-tree build, or SIMSD_LIBRARY when set (another build of the same
    sources, e.g. one with host sanitizers)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if path is None:
            path = os.environ.get("SIMSD_LIBRARY") or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built; run diffusion_lm_speculative_amd.build.build() "
                "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def strerror(code: int) -> str:
    return load().simsd_strerror(int(code)).decode()


def check(code: int, where: str) -> None:
    if code != OK:
        raise SimsdError(code, where)
