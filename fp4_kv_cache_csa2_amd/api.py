"""Thin Python binding of the CSA2 C ABI (include/csa2.h).

Each function has the name of the C entry point it calls and only marshals
arguments: PyTorch device tensors are passed as raw pointers, the stream is
PyTorch's current stream.  Every step of the computation runs in libcsa2.so;
a non-OK status raises Csa2Error with the library's message.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import CSA2_BF16, CSA2_F32, CSA2_FULL, CSA2_REINDEX, CSA2_REUSE, Csa2Error  # noqa: F401

MODES = {"F": CSA2_FULL, "R": CSA2_REINDEX, "U": CSA2_REUSE}


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA2_F32
    if t.dtype == torch.bfloat16:
        return CSA2_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass
class Fp4Cache:
    """FP4 main-KV cache planes: codes[rows][D/2] u8, scales[rows][D/16] u8.
    Contiguous (page_table None, seq_stride entries per sequence) or paged."""
    codes: torch.Tensor
    scales: torch.Tensor
    D: int
    seq_stride: int = 0
    page_table: torch.Tensor | None = None
    page_size: int = 0

    def view(self) -> _lib.Fp4KV:
        mp = 0 if self.page_table is None else self.page_table.shape[1]
        return _lib.Fp4KV(self.codes.data_ptr(), self.scales.data_ptr(), _ptr(self.page_table), self.page_size, mp,
                          self.seq_stride, self.D)


@dataclass
class IndexerK:
    """Indexer K plane k[rows][D_i] bf16, addressed like the FP4 cache."""
    k: torch.Tensor
    D_i: int
    seq_stride: int = 0
    page_table: torch.Tensor | None = None
    page_size: int = 0

    def view(self) -> _lib.IdxK:
        mp = 0 if self.page_table is None else self.page_table.shape[1]
        return _lib.IdxK(self.k.data_ptr(), _ptr(self.page_table), self.page_size, mp, self.seq_stride, self.D_i)


def _check_rows(view, B: int, what: str):
    """Contiguous views address B * seq_stride rows: they must exist in the
    tensors handed over (the library only sees pointers)."""
    if view is None or view.page_table is not None:
        return
    planes = [view.codes, view.scales] if isinstance(view, Fp4Cache) else [view.k]
    for t in planes:
        if B * view.seq_stride > t.shape[0]:
            raise ValueError(f"{what}: {B} sequences x seq_stride {view.seq_stride} rows exceed the "
                             f"{t.shape[0]} rows allocated")


def csa2_abi_version() -> int:
    return _lib.load().csa2_abi_version()


def csa2_fp4_quantize(x, codes, scales, stream=None):
    rows, D = x.shape
    _lib.check(_lib.load().csa2_fp4_quantize(_ptr(x), _dtype(x), rows, D, _ptr(codes), _ptr(scales), _stream(stream)))


def csa2_fp4_dequantize(codes, scales, y, stream=None):
    rows, D = y.shape
    _lib.check(_lib.load().csa2_fp4_dequantize(_ptr(codes), _ptr(scales), rows, D, _ptr(y), _stream(stream)))


def csa2_fp4_append(x, pos, cache: Fp4Cache, stream=None):
    _check_rows(cache, x.shape[0], "fp4_append")
    v = cache.view()
    _lib.check(_lib.load().csa2_fp4_append(_ptr(x), _dtype(x), x.shape[0], _ptr(pos), ctypes.byref(v),
                                           _stream(stream)))


def csa2_append_token(x, pos, cache: Fp4Cache, k_new=None, kview: IndexerK | None = None, swa_new=(), swa_kv=(),
                      tok=None, stream=None):
    """One launch per decode step: FP4 entry pos[b] from x[b], indexer-K entry
    pos[b] from k_new[b], and every window ring swa_kv[l] at row tok[b] mod T
    from swa_new[l][b] (tok: the new token's absolute position)."""
    _check_rows(cache, x.shape[0], "append_token")
    _check_rows(kview, x.shape[0], "append_token")
    v = cache.view()
    kv = kview.view() if kview is not None else None
    n = len(swa_new)
    if len(swa_kv) != n:
        raise ValueError("swa_new and swa_kv must have one tensor per layer each")
    new_arr = (_lib.P * max(n, 1))(*[t.data_ptr() for t in swa_new])
    kv_arr = (_lib.P * max(n, 1))(*[t.data_ptr() for t in swa_kv])
    T = swa_kv[0].shape[1] if n else 0
    a = _lib.AppendArgs(x.shape[0], x.data_ptr(), _dtype(x), pos.data_ptr(), ctypes.pointer(v),
                        None if k_new is None else k_new.data_ptr(), None if kv is None else ctypes.pointer(kv),
                        n, new_arr, kv_arr, T, None if tok is None else tok.data_ptr())
    _lib.check(_lib.load().csa2_append_token(ctypes.byref(a), _stream(stream)))


def csa2_swa_replay(h, W, swa_kv, t_end, stream=None):
    """Rebuild window rows: h[l] [B][n][d_model], W[l] [D][d_model] bf16,
    swa_kv[l] [B][T][D] bf16 (written), t_end [B] int32 on the device."""
    L = len(h)
    if len(W) != L or len(swa_kv) != L:
        raise ValueError("h, W and swa_kv must have one tensor per layer each")
    if L == 0:
        return
    B, n, dm = h[0].shape
    D = W[0].shape[0]
    T = swa_kv[0].shape[1]
    arr = lambda ts: (_lib.P * L)(*[t.data_ptr() for t in ts])
    a = _lib.ReplayArgs(B, n, dm, D, T, t_end.data_ptr(), L, arr(h), arr(W), arr(swa_kv))
    _lib.check(_lib.load().csa2_swa_replay(ctypes.byref(a), _stream(stream)))


def csa2_index_full(q_idx, kview: IndexerK, n_vis, n_max, scores, block_max=None, stream=None):
    B, Q, H_i, _ = q_idx.shape
    _check_rows(kview, B, "index_full")
    v = kview.view()
    _lib.check(_lib.load().csa2_index_full(_ptr(q_idx), B, Q, H_i, ctypes.byref(v), _ptr(n_vis), n_max, _ptr(scores),
                                           _ptr(block_max), _stream(stream)))


def csa2_index_reindex(q_idx, kview: IndexerK, n_vis, pool_blocks, pool_scores, stream=None):
    B, Q, H_i, _ = q_idx.shape
    _check_rows(kview, B, "index_reindex")
    v = kview.view()
    _lib.check(_lib.load().csa2_index_reindex(_ptr(q_idx), B, Q, H_i, ctypes.byref(v), _ptr(n_vis),
                                              _ptr(pool_blocks), pool_blocks.shape[-1], _ptr(pool_scores),
                                              _stream(stream)))


def csa2_topk_workspace_size(rows, n, k) -> int:
    return _lib.load().csa2_topk_workspace_size(rows, n, k)


def csa2_topk(scores, k, out_idx, pool_blocks=None, ws=None, stream=None):
    rows, n = scores.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _lib.check(_lib.load().csa2_topk(_ptr(scores), rows, n, k, _ptr(pool_blocks), _ptr(out_idx), _ptr(ws), nbytes,
                                     _stream(stream)))


def csa2_topk_noalloc(scores, k, out_idx, pool_blocks=None, stream=None):
    """Top-K without a workspace (the library's built-in scratch, <= 64 rows past 32768 positions)."""
    rows, n = scores.shape
    _lib.check(_lib.load().csa2_topk_noalloc(_ptr(scores), rows, n, k, _ptr(pool_blocks), _ptr(out_idx),
                                             _stream(stream)))


def csa2_attn_workspace_size(B, Q, H, D) -> int:
    return _lib.load().csa2_attn_workspace_size(B, Q, H, D)


def csa2_sparse_attn_fp4(q, cache: Fp4Cache, idx, sm_scale, o, lse, ws=None, stream=None):
    B, Q, H, _ = q.shape
    _check_rows(cache, B, "sparse_attn_fp4")
    v = cache.view()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _lib.check(_lib.load().csa2_sparse_attn_fp4(_ptr(q), _dtype(q), B, Q, H, ctypes.byref(v), _ptr(idx),
                                                idx.shape[-1], float(sm_scale), _ptr(o), _ptr(lse), _ptr(ws), nbytes,
                                                _stream(stream)))


def csa2_swa_attn(q, swa_kv, q_pos, window, sm_scale, merge, o, lse, ws=None, stream=None):
    """Window attention; swa_kv [B][T][D] is a ring (token t in row t mod T),
    q_pos [B][Q] the query tokens' absolute positions."""
    B, Q, H, D = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _lib.check(_lib.load().csa2_swa_attn(_ptr(q), _dtype(q), B, Q, H, D, _ptr(swa_kv), swa_kv.shape[1], _ptr(q_pos),
                                         window, float(sm_scale), int(merge), _ptr(o), _ptr(lse), _ptr(ws), nbytes,
                                         _stream(stream)))


def csa2_layer_workspace_size(B, Q, H, D, n_max, K, P) -> int:
    return _lib.load().csa2_layer_workspace_size(B, Q, H, D, n_max, K, P)


class GroupState:
    """Device buffers + host flags shared by the layers of one pattern."""

    def __init__(self, rows: int, K: int, P: int, device):
        self.idx = torch.empty(rows, K, dtype=torch.int32, device=device)
        self.pool = torch.empty(rows, max(P, 1), dtype=torch.int32, device=device)
        self.c = _lib.GroupState(self.idx.data_ptr(), self.pool.data_ptr(), 0, 0, 0, 0, None, 0, 0)


def csa2_layer_forward(mode: str, *, q, q_idx, swa_kv, q_pos, window, sm_scale, o, lse, cache: Fp4Cache,
                       kview: IndexerK, n_vis, n_max, K, P, build_pool, ws, state: GroupState, stream=None):
    B, Q, H, _ = q.shape
    _check_rows(cache, B, "layer_forward")
    _check_rows(kview, B, "layer_forward")
    H_i = 0 if q_idx is None else q_idx.shape[2]
    kv, kk = cache.view(), kview.view()
    a = _lib.LayerArgs(B, Q, H, H_i, K, P, q.data_ptr(), _dtype(q), _ptr(q_idx), swa_kv.data_ptr(), swa_kv.shape[1],
                       q_pos.data_ptr(), window, float(sm_scale), o.data_ptr(), lse.data_ptr(), ctypes.pointer(kv),
                       ctypes.pointer(kk), _ptr(n_vis), n_max, int(build_pool), ws.data_ptr(),
                       ws.numel() * ws.element_size())
    _lib.check(_lib.load().csa2_layer_forward(MODES[mode], ctypes.byref(a), ctypes.byref(state.c), _stream(stream)))
