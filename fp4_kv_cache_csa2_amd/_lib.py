"""ctypes loader for libcsa2.so (the HIP library built from csrc/).

There is no fallback: if the library is missing or fails to load, every call
raises.  Build it with ``python -m fp4_kv_cache_csa2_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")

P = ctypes.c_void_p
i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
f32 = ctypes.c_float
sz = ctypes.c_size_t

ABI_VERSION = 3
CSA2_OK, CSA2_EINVAL, CSA2_EUNSUPPORTED, CSA2_EWORKSPACE, CSA2_EMODE, CSA2_EHIP = range(6)
CSA2_F32, CSA2_BF16 = 0, 1
CSA2_FULL, CSA2_REINDEX, CSA2_REUSE = 0, 1, 2


class Fp4KV(ctypes.Structure):
    _fields_ = [("codes", P), ("scales", P), ("page_table", P), ("page_size", i32), ("max_pages", i32),
                ("seq_stride", i64), ("D", i32)]


class IdxK(ctypes.Structure):
    _fields_ = [("k", P), ("page_table", P), ("page_size", i32), ("max_pages", i32), ("seq_stride", i64),
                ("D_i", i32)]


class LayerArgs(ctypes.Structure):
    _fields_ = [("B", i32), ("Q", i32), ("H", i32), ("H_i", i32), ("K", i32), ("P", i32),
                ("q", P), ("qt", ctypes.c_int), ("q_idx", P), ("swa_kv", P), ("T", i32), ("q_pos", P),
                ("window", i32), ("sm_scale", f32), ("o", P), ("lse", P),
                ("kv", ctypes.POINTER(Fp4KV)), ("k", ctypes.POINTER(IdxK)), ("n_vis", P), ("n_max", i32),
                ("build_pool", i32), ("ws", P), ("ws_bytes", sz)]


class AppendArgs(ctypes.Structure):
    _fields_ = [("B", i32), ("x", P), ("xt", ctypes.c_int), ("pos", P), ("kv", ctypes.POINTER(Fp4KV)),
                ("k_new", P), ("k", ctypes.POINTER(IdxK)), ("n_layers", i32), ("swa_new", ctypes.POINTER(P)),
                ("swa_kv", ctypes.POINTER(P)), ("T", i32), ("tok", P)]


class ReplayArgs(ctypes.Structure):
    _fields_ = [("B", i32), ("n", i32), ("d_model", i32), ("D", i32), ("T", i32), ("t_end", P), ("n_layers", i32),
                ("h", ctypes.POINTER(P)), ("W", ctypes.POINTER(P)), ("swa_kv", ctypes.POINTER(P))]


class GroupState(ctypes.Structure):
    _fields_ = [("idx", P), ("pool", P), ("has_idx", i32), ("has_pool", i32), ("ws_clean", i32), ("clean_rows", i32),
                ("clean_ws", P), ("has_stage", i32), ("stage_n", i32)]


# name -> (restype, argtypes); every symbol declared in include/csa2.h
SIGNATURES = {
    "csa2_abi_version": (i32, []),
    "csa2_last_error": (ctypes.c_char_p, []),
    "csa2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "csa2_fp4_quantize": (ctypes.c_int, [P, ctypes.c_int, i64, i32, P, P, P]),
    "csa2_fp4_dequantize": (ctypes.c_int, [P, P, i64, i32, P, P]),
    "csa2_fp4_append": (ctypes.c_int, [P, ctypes.c_int, i32, P, ctypes.POINTER(Fp4KV), P]),
    "csa2_append_token": (ctypes.c_int, [ctypes.POINTER(AppendArgs), P]),
    "csa2_swa_replay": (ctypes.c_int, [ctypes.POINTER(ReplayArgs), P]),
    "csa2_index_full": (ctypes.c_int, [P, i32, i32, i32, ctypes.POINTER(IdxK), P, i32, P, P, P]),
    "csa2_index_reindex": (ctypes.c_int, [P, i32, i32, i32, ctypes.POINTER(IdxK), P, P, i32, P, P]),
    "csa2_topk_workspace_size": (sz, [i32, i32, i32]),
    "csa2_topk": (ctypes.c_int, [P, i32, i32, i32, P, P, P, sz, P]),
    "csa2_topk_noalloc": (ctypes.c_int, [P, i32, i32, i32, P, P, P]),
    "csa2_attn_workspace_size": (sz, [i32, i32, i32, i32]),
    "csa2_sparse_attn_fp4": (ctypes.c_int, [P, ctypes.c_int, i32, i32, i32, ctypes.POINTER(Fp4KV), P, i32, f32, P, P,
                                            P, sz, P]),
    "csa2_swa_attn": (ctypes.c_int, [P, ctypes.c_int, i32, i32, i32, i32, P, i32, P, i32, f32, i32, P, P, P, sz, P]),
    "csa2_layer_workspace_size": (sz, [i32, i32, i32, i32, i32, i32, i32]),
    "csa2_layer_forward": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(LayerArgs), ctypes.POINTER(GroupState), P]),
}

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"CSA2 HIP library not built: {LIB_PATH} is missing "
                               "(run python -m fp4_kv_cache_csa2_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        if lib.csa2_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH}: ABI version {lib.csa2_abi_version()}, binding expects {ABI_VERSION} "
                               "(rebuild with python -m fp4_kv_cache_csa2_amd.build)")
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != CSA2_OK:
        msg = load().csa2_last_error().decode(errors="replace")
        raise Csa2Error(status, msg)
