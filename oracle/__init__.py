"""CSA2 reference oracle (Python side).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``fp4_kv_cache_csa2_amd``) never imports it, and this package never imports
the product package.  The arithmetic lives in ``csa2_oracle.c`` (plain C,
built with gcc); this module marshals numpy arrays into it and runs the static
layer-mode schedule.

Functions and the passages they follow (full citations in ``csa2_oracle.c``):
  fp4_encode / fp4_decode      aprilzz.com V4.1 Flash article, section
                               "FP4 KV 与部署层的几个改动" (E2M1, one E4M3 scale per
                               16 channels, no global scale); OCP MX v1.0 / OFP8.
  index_scores / reindex_scores / block_max
                               gkm0120.cn survey section 2.2.2-2.2.3; aprilzz.com
                               section "CSA2：在层的维度上共享缓存".
  topk                         same section (a new Top-512 per Full layer).
  attention                    aprilzz.com section "把 prefill 砍掉一半" (128-token SWA)
                               and the CSA2 section (own main Q and SWA KV per layer).
  run_stack                    gkm0120.cn section 2.2.2 mode table; aprilzz.com CSA2
                               section (group patterns, latest Top-K reused).
  bf16_round / swa_replay      aprilzz.com sections "把 prefill 砍掉一半" and
                               "FP4 KV 与部署层的几个改动" (a missing window is rebuilt
                               from the last 128 tokens); gkm0120.cn section 2.1
                               (SWA Bounded Replay); aimodeling.com "第三层".  The
                               projection itself is a reading: kv_p = bf16(h_p W^T),
                               one rounding.

Parity-unpinned readings (pinned only by the workload text or by the readings
themselves, never by the pages): the score has no ReLU / head weights / scale;
its fp32 evaluation order (head sum first, then one FMA chain over the channels:
equal to the per-head sums in exact arithmetic, but its rounding decides
near-ties of the Top-K); the pool ranks 8-entry blocks by their max score;
attention uses scale 1/sqrt(D), no RoPE, no sink and no de-duplication of tokens
present in both key sets; what the window projection of the replay contains
beyond one matrix product (norms, rotary parts).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 (no fast-math: IEEE semantics)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_e4m3fn_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3fn_decode.restype = ctypes.c_double
        lib.oracle_e4m3fn_round.argtypes = [ctypes.c_double]
        lib.oracle_e4m3fn_round.restype = ctypes.c_uint8
        lib.oracle_e2m1_magnitude.argtypes = [ctypes.c_int]
        lib.oracle_e2m1_magnitude.restype = ctypes.c_double
        lib.oracle_fp4_encode.argtypes = [P, i64, i32, P, P]
        lib.oracle_fp4_decode.argtypes = [P, P, i64, i32, P]
        lib.oracle_index_scores.argtypes = [P, i32, i32, P, i64, i64, P]
        lib.oracle_reindex_scores.argtypes = [P, i32, i32, P, i64, P, i32, P]
        lib.oracle_block_max.argtypes = [P, i64, P]
        lib.oracle_topk.argtypes = [P, i64, i32, P, P]
        lib.oracle_attention.argtypes = [P, i32, i32, P, P, P, i32, P, i32, i32, i32, ctypes.c_double, P, P]
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_swa_replay.argtypes = [P, P, i32, i32, i32, i64, i32, P]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------- formats
def e4m3fn_decode(code: int) -> float:
    return _load().oracle_e4m3fn_decode(int(code))


def e4m3fn_round(q: float) -> int:
    return int(_load().oracle_e4m3fn_round(float(q)))


def e2m1_magnitude(mag: int) -> float:
    return _load().oracle_e2m1_magnitude(int(mag))


def fp4_encode(x: np.ndarray):
    """x[rows][D] float32 -> (codes[rows][D/2] u8, scales[rows][D/16] u8)."""
    x = _c(x, np.float32)
    rows, D = x.shape
    assert D % 16 == 0
    codes = np.zeros((rows, D // 2), np.uint8)
    scales = np.zeros((rows, D // 16), np.uint8)
    _load().oracle_fp4_encode(_ptr(x), rows, D, _ptr(codes), _ptr(scales))
    return codes, scales


def fp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, half = codes.shape
    y = np.zeros((rows, 2 * half), np.float64)
    _load().oracle_fp4_decode(_ptr(codes), _ptr(scales), rows, 2 * half, _ptr(y))
    return y


# ----------------------------------------------------------------------------- indexer
def index_scores(q_idx: np.ndarray, K: np.ndarray, n_vis: int) -> np.ndarray:
    """q_idx[H_i][D_i] bf16 bits (uint16), K[n][D_i] bf16 bits -> scores[n] float32."""
    q_idx = _c(q_idx, np.uint16)
    K = _c(K, np.uint16)
    H_i, D_i = q_idx.shape
    n = K.shape[0]
    out = np.empty(n, np.float32)
    _load().oracle_index_scores(_ptr(q_idx), H_i, D_i, _ptr(K), n, int(n_vis), _ptr(out))
    return out


def reindex_scores(q_idx: np.ndarray, K: np.ndarray, n_vis: int, pool: np.ndarray) -> np.ndarray:
    q_idx = _c(q_idx, np.uint16)
    K = _c(K, np.uint16)
    pool = _c(pool, np.int32)
    H_i, D_i = q_idx.shape
    out = np.empty(8 * pool.shape[0], np.float32)
    _load().oracle_reindex_scores(_ptr(q_idx), H_i, D_i, _ptr(K), int(n_vis), _ptr(pool), pool.shape[0],
                                  _ptr(out))
    return out


def block_max(scores: np.ndarray) -> np.ndarray:
    scores = _c(scores, np.float32)
    out = np.empty((scores.shape[0] + 7) // 8, np.float32)
    _load().oracle_block_max(_ptr(scores), scores.shape[0], _ptr(out))
    return out


def topk(scores: np.ndarray, k: int, pool: np.ndarray | None = None) -> np.ndarray:
    scores = _c(scores, np.float32)
    pool = None if pool is None else _c(pool, np.int32)
    out = np.empty(k, np.int32)
    _load().oracle_topk(_ptr(scores), scores.shape[0], int(k), _ptr(pool), _ptr(out))
    return out


def build_pool(scores: np.ndarray, n_blocks: int) -> np.ndarray:
    """Pool = the best n_blocks aligned 8-entry blocks by block max, ascending."""
    return topk(block_max(scores), n_blocks)


def visible_entries(t: int, ratio: int) -> int:
    """Number of compressed entries the token at position t may attend when each
    entry compresses `ratio` consecutive tokens (entry j covers tokens
    ratio*j .. ratio*j + ratio - 1).  Reading of the encoder's causal mask
    (aprilzz.com CSA2 section: compression ratio 2 in the encoder): an entry is
    visible once every token it covers is at or before t, so the visible
    entries are j = 0 .. floor((t + 1) / ratio) - 1."""
    return (int(t) + 1) // int(ratio)


# ----------------------------------------------------------------------------- attention
def attention(q: np.ndarray, codes: np.ndarray | None, scales: np.ndarray | None, idx: np.ndarray | None,
              swa: np.ndarray | None, q_pos: int, window: int, sm_scale: float):
    """q[H][D] (any float dtype, used exactly as fp64); codes/scales the FP4 cache
    of one sequence in logical entry order; idx[K] (or None); swa[T][D] the
    layer's window ring (token t in row t mod T), or None; q_pos the query
    token's absolute position (window = tokens max(0, q_pos-window+1)..q_pos,
    window <= T).  Returns (o[H][D] fp64, lse[H] fp64)."""
    q = _c(q, np.float64)
    H, D = q.shape
    if idx is None:
        idx_a, K = None, 0
        codes = scales = None
    else:
        idx_a = _c(idx, np.int32)
        K = idx_a.shape[0]
        codes = _c(codes, np.uint8)
        scales = _c(scales, np.uint8)
    swa_a = None if swa is None else _c(swa, np.float64)
    T = 0 if swa_a is None else swa_a.shape[0]
    if swa_a is not None and window > T:
        raise ValueError(f"window {window} exceeds the ring's {T} rows")
    o = np.empty((H, D), np.float64)
    lse = np.empty(H, np.float64)
    _load().oracle_attention(_ptr(q), H, D, _ptr(codes), _ptr(scales), _ptr(idx_a), K, _ptr(swa_a), T, int(q_pos),
                             int(window), float(sm_scale), _ptr(o), _ptr(lse))
    return o, lse


# ----------------------------------------------------------------------------- window replay
def bf16_round(v: float) -> int:
    """fp64 -> bf16 bits, nearest / ties to even, in one rounding."""
    return int(_load().oracle_bf16_round(float(v)))


def swa_replay(h: np.ndarray, W: np.ndarray, t_end: int, T: int, ring: np.ndarray | None = None) -> np.ndarray:
    """h[n][d_model] and W[D][d_model] bf16 bits (uint16): the window rows of
    positions t_end-n+1 .. t_end, bf16(h_p W^T), written to rows p mod T of a
    copy of ring[T][D] (zeros when None), which is returned."""
    h = _c(h, np.uint16)
    W = _c(W, np.uint16)
    n, dm = h.shape
    D, dm2 = W.shape
    assert dm == dm2 and n <= T and t_end >= n - 1
    out = np.zeros((T, D), np.uint16) if ring is None else _c(ring, np.uint16).copy()
    _load().oracle_swa_replay(_ptr(h), _ptr(W), n, dm, D, int(t_end), T, _ptr(out))
    return out


# ----------------------------------------------------------------------------- layer schedule
def select_stack(pattern: str, K_idx: np.ndarray, n_vis: int, q_idx: list, K: int = 512, pool_blocks: int = 2048):
    """Selection half of the layer schedule for one query row: the Top-K index
    list each layer attends with (and the pool built by the Full layer).

    Full scores every visible entry and selects a new Top-K (plus the pool of
    the best ``pool_blocks`` 8-entry blocks when the pattern holds a Reindex
    layer); Reindex scores only the pool positions with its own indexer query
    and selects a new Top-K; Reuse takes the most recent selection."""
    need_pool = "R" in pattern
    idx, pool, out = None, None, []
    for mode, qi in zip(pattern, q_idx):
        if mode == "F":
            s = index_scores(qi, K_idx, n_vis)
            idx = topk(s, K)
            if need_pool:
                pool = build_pool(s, pool_blocks)
        elif mode == "R":
            if pool is None:
                raise ValueError("Reindex layer before any Full layer built a pool")
            idx = topk(reindex_scores(qi, K_idx, n_vis, pool), K, pool)
        elif mode == "U":
            if idx is None:
                raise ValueError("Reuse layer before any selection")
        else:
            raise ValueError(f"unknown mode {mode!r}")
        out.append(idx)
    return out, pool


def run_stack(pattern: str, seq: dict, layers: list[dict], K: int = 512, pool_blocks: int = 2048,
              window: int = 128, sm_scale: float | None = None, attn_heads: slice | None = None):
    """Run a static Full/Reindex/Reuse pattern (characters F, R, U) for ONE
    query row of one sequence.

    seq:    shared state of the sequence: K_idx[n][D_i] (bf16 bits), codes, scales
            (logical entry order), n_vis.
    layers: per-layer dict: q[H][D], q_idx[H_i][D_i] (F/R only), swa[T][D] (window
            ring, token t in row t mod T), q_pos (the query token's position).

    Follows the mode table: Full scores every visible entry and selects a new
    Top-K (and, when the pattern holds a Reindex layer, the pool of the best
    ``pool_blocks`` 8-entry blocks); Reindex scores only the pool positions with
    its own indexer query and selects a new Top-K; Reuse runs no indexer and
    takes the most recent selection.  Every layer attends with its own Q and SWA.
    Returns a list of per-layer dicts {idx, o, lse} (and pool for Full).
    """
    n_vis = int(seq["n_vis"])
    D = seq["codes"].shape[1] * 2
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    sel, pool = select_stack(pattern, seq["K_idx"], n_vis, [L.get("q_idx") for L in layers], K, pool_blocks)
    out = []
    for mode, L, idx in zip(pattern, layers, sel):
        q = L["q"] if attn_heads is None else L["q"][attn_heads]
        o, lse = attention(q, seq["codes"], seq["scales"], idx, L["swa"], L["q_pos"], window, sm_scale)
        rec = dict(idx=idx.copy(), o=o, lse=lse)
        if mode == "F" and pool is not None:
            rec["pool"] = pool
        out.append(rec)
    return out
