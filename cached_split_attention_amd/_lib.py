"""ctypes view of libba.so (the C-ABI declared in include/ba.h).

torch is imported first so that libba.so binds to the HIP runtime torch has
already loaded (both carry the soname libamdhip64.so.7): one runtime per
process, shared device memory and streams.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must load the HIP runtime before libba.so)

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libba.so")

BA_OK = 0
STATUS_NAMES = {0: "BA_OK", 1: "BA_ERR_NULL", 2: "BA_ERR_SHAPE", 3: "BA_ERR_DTYPE",
                4: "BA_ERR_UNSUPPORTED", 5: "BA_ERR_WORKSPACE", 6: "BA_ERR_HIP"}
BA_BF16, BA_F32 = 0, 1
BA_NOALLOC_SCRATCH_BYTES = 64 << 20   # as in ba.h
BA_GATE_COUNT, BA_GATE_COSINE, BA_GATE_COUNT_CUM, BA_GATE_ROWS = 0, 1, 2, 3

c_i64x3 = ctypes.c_int64 * 3
c_i64x2 = ctypes.c_int64 * 2


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("n_seq", ctypes.c_int32),
        ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("max_q", ctypes.c_int32), ("max_k", ctypes.c_int32), ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_stride", c_i64x3),
        ("k", ctypes.c_void_p), ("k_stride", c_i64x3),
        ("v", ctypes.c_void_p), ("v_stride", c_i64x3),
        ("cu_q", ctypes.c_void_p), ("cu_k", ctypes.c_void_p), ("decision", ctypes.c_void_p),
    ]


class GateDesc(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32), ("n_seq", ctypes.c_int32),
        ("n_blk", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("q_cur", ctypes.c_void_p), ("q_prev", ctypes.c_void_p), ("q_stride", c_i64x3),
        ("k_cur", ctypes.c_void_p), ("k_prev", ctypes.c_void_p),
        ("v_cur", ctypes.c_void_p), ("v_prev", ctypes.c_void_p), ("kv_stride", c_i64x3),
        ("upd_mask", ctypes.c_void_p), ("tau", ctypes.c_int32), ("gamma", ctypes.c_double),
        ("cache_valid", ctypes.c_int32), ("since_refresh", ctypes.c_void_p),
        ("wait_polls", ctypes.c_int32), ("gave_up", ctypes.c_void_p),
    ]


EXPORTS = {
    "ba_prefix_attn_workspace": (ctypes.c_size_t, [ctypes.POINTER(AttnDesc)]),
    "ba_prefix_attn": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "ba_prefix_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "ba_prefix_attn_rows": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]),
    "ba_sparse_prefix_attn_workspace": (ctypes.c_size_t, [ctypes.POINTER(AttnDesc), ctypes.c_int32]),
    "ba_sparse_prefix_attn": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p]),
    "ba_prefix_attn_merge": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "ba_split_attn": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnDesc), ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "ba_block_attn": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]),
    "ba_lse_merge": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]),
    "ba_reuse_gate_workspace": (ctypes.c_size_t, [ctypes.POINTER(GateDesc)]),
    "ba_reuse_gate": (ctypes.c_int, [ctypes.POINTER(GateDesc), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]),
    "ba_gated_split_attn_gate_workspace": (ctypes.c_size_t, [ctypes.POINTER(GateDesc)]),
    "ba_gated_split_attn": (ctypes.c_int, [ctypes.POINTER(GateDesc), ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnDesc),
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]),
    "ba_kl_lock": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "ba_varlen_pack": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                      ctypes.c_void_p, ctypes.c_void_p]),
    "ba_last_error": (ctypes.c_char_p, []),
    "ba_version": (ctypes.c_int32, []),
}

_lib = None


def lib():
    """The loaded library; raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class BaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status: int):
    if status != BA_OK:
        raise BaError(status, lib().ba_last_error().decode())
