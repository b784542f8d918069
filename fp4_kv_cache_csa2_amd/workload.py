"""Device-resident instances of the CSA2 workloads and a runner for a static
layer pattern through the C ABI.

An instance holds, for B sequences: the FP4 main-KV cache (quantised on the GPU
by the library from an fp32 N(0,1) latent), the shared bf16 indexer K, and per
layer the main query, the indexer query and the window rows.  Ragged
workloads store both caches in 64-entry pages placed by a random page table.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import api, inputs
from .inputs import Workload


@dataclass
class Instance:
    w: Workload
    lengths: np.ndarray          # entries per sequence
    n_vis_host: np.ndarray       # [B][Q]
    n_vis: torch.Tensor          # [B][Q] int32, device
    n_max: int
    offsets: np.ndarray          # logical row offset of each sequence (flat latent / K)
    latent: torch.Tensor         # [sum lengths][D] fp32, logical order
    k_logical: torch.Tensor      # [sum lengths][D_i] bf16, logical order
    cache: api.Fp4Cache
    kview: api.IndexerK
    page_table_host: np.ndarray | None
    T: int                       # rows of each layer's window ring (token t in row t mod T)
    q_pos_host: np.ndarray       # [B][Q] absolute token position of each query row
    q_pos: torch.Tensor
    layers: list = field(default_factory=list)  # per layer: dict(q, q_idx, swa)

    @property
    def rows(self) -> int:
        return self.w.B * self.w.Q

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.w.D)

    def phys_rows(self, b: int, j: np.ndarray) -> np.ndarray:
        """Physical cache row of logical entries j of sequence b."""
        j = np.asarray(j, np.int64)
        if self.page_table_host is None:
            return b * self.cache.seq_stride + j
        ps = self.w.page_size
        return self.page_table_host[b, j // ps].astype(np.int64) * ps + j % ps


def _chunked_normal(rows: int, cols: int, tag: str, seed: int, device, dtype, chunk_rows: int = 1 << 20):
    out = torch.empty(rows, cols, dtype=dtype, device=device)
    for i, lo in enumerate(range(0, rows, chunk_rows)):
        hi = min(rows, lo + chunk_rows)
        out[lo:hi] = inputs.normal((hi - lo, cols), f"{tag}/{i}", seed, device, dtype)
    return out


def make_instance(w: Workload, seed: int = 0, device="cuda", lengths=None, Q: int | None = None) -> Instance:
    """Build a device instance of workload w (optionally with other lengths or
    fewer query rows, for reduced-size tests)."""
    if Q is not None and Q != w.Q:
        import dataclasses
        w = dataclasses.replace(w, Q=Q)
    B, D, D_i = w.B, w.D, w.D_i
    if lengths is None:
        lengths = (inputs.log_uniform_lengths(B, 4096, w.N, f"{w.name}/len", seed) if w.ragged
                   else np.full(B, w.N, np.int32))
    lengths = np.asarray(lengths, np.int32)
    offsets = np.concatenate([[0], np.cumsum(lengths.astype(np.int64))])
    total = int(offsets[-1])
    latent = _chunked_normal(total, D, f"{w.name}/latent", seed, device, torch.float32)
    k_log = _chunked_normal(total, D_i, f"{w.name}/kidx", seed, device, torch.bfloat16)

    # logical-order FP4 codes, then the physical layout
    codes_l = torch.empty(total, D // 2, dtype=torch.uint8, device=device)
    scales_l = torch.empty(total, D // 16, dtype=torch.uint8, device=device)
    api.csa2_fp4_quantize(latent, codes_l, scales_l)
    if w.ragged:
        table, n_pages = inputs.random_page_table(lengths, w.page_size, f"{w.name}/pages", seed)
        ps = w.page_size
        phys = np.concatenate([table[b, np.arange(lengths[b]) // ps].astype(np.int64) * ps + np.arange(lengths[b]) % ps
                               for b in range(B)])
        phys_t = torch.from_numpy(phys).to(device)
        codes = torch.zeros(n_pages * ps, D // 2, dtype=torch.uint8, device=device)
        scales = torch.zeros(n_pages * ps, D // 16, dtype=torch.uint8, device=device)
        kphys = torch.zeros(n_pages * ps, D_i, dtype=torch.bfloat16, device=device)
        codes[phys_t] = codes_l
        scales[phys_t] = scales_l
        kphys[phys_t] = k_log
        del codes_l, scales_l
        pt = torch.from_numpy(table).to(device)
        cache = api.Fp4Cache(codes, scales, D, 0, pt, ps)
        kview = api.IndexerK(kphys, D_i, 0, pt, ps)
        table_host = table
    else:
        cache = api.Fp4Cache(codes_l, scales_l, D, int(lengths.max()))
        kview = api.IndexerK(k_log, D_i, int(lengths.max()))
        table_host = None
        assert np.all(lengths == lengths.max())

    # query positions, visibility and the window ring.  An entry covers `ratio`
    # consecutive tokens and becomes visible to token t once complete: entry j
    # (tokens ratio*j .. ratio*j + ratio-1) is visible iff ratio*j + ratio-1 <= t,
    # so token t sees floor((t + 1) / ratio) entries.  The ring holds every
    # token any query row's window reaches: the last Q + window - 1 tokens.
    if w.Q == 1:  # decode: the query is each sequence's newest token and sees every entry
        q_pos_host = (lengths.astype(np.int64) * w.ratio - 1).reshape(B, 1)
        n_vis_host = lengths.reshape(B, 1).copy()
    else:
        tok = inputs.query_positions(w)
        q_pos_host = np.broadcast_to(tok, (B, w.Q)).copy()
        n_vis_host = (q_pos_host + 1) // w.ratio
    T = w.Q + w.window - 1
    q_pos_host = q_pos_host.astype(np.int32)
    n_vis_host = n_vis_host.astype(np.int32)
    layers = []
    for l, mode in enumerate(w.pattern):
        L = dict(q=inputs.normal((B, w.Q, w.H, D), f"{w.name}/L{l}/q", seed, device, w.q_dtype),
                 swa=inputs.normal((B, T, D), f"{w.name}/L{l}/swa", seed, device, torch.bfloat16),
                 q_idx=None)
        if mode in "FR":
            L["q_idx"] = inputs.normal((B, w.Q, w.H_i, D_i), f"{w.name}/L{l}/qidx", seed, device, torch.bfloat16)
        layers.append(L)
    return Instance(w=w, lengths=lengths, n_vis_host=n_vis_host, n_vis=torch.from_numpy(n_vis_host).to(device),
                    n_max=int(lengths.max()), offsets=offsets, latent=latent, k_logical=k_log, cache=cache,
                    kview=kview, page_table_host=table_host, T=T, q_pos_host=q_pos_host,
                    q_pos=torch.from_numpy(q_pos_host).to(device), layers=layers)


class StackRunner:
    """Runs the instance's static pattern with csa2_layer_forward, reusing
    preallocated outputs and workspace (nothing is allocated per step)."""

    def __init__(self, inst: Instance):
        self.inst = inst
        w = inst.w
        dev = inst.latent.device
        self.has_pool = "R" in w.pattern
        P = w.P if self.has_pool else 0
        self.ws_bytes = api.csa2_layer_workspace_size(w.B, w.Q, w.H, w.D, inst.n_max, w.K, P)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.state = api.GroupState(inst.rows, w.K, w.P, dev)
        self.o = [torch.empty(w.B, w.Q, w.H, w.D, dtype=torch.float32, device=dev) for _ in w.pattern]
        self.lse = [torch.empty(w.B, w.Q, w.H, dtype=torch.float32, device=dev) for _ in w.pattern]
        self.idx = [torch.empty(inst.rows, w.K, dtype=torch.int32, device=dev) for _ in w.pattern]
        self.pool = torch.empty(inst.rows, max(w.P, 1), dtype=torch.int32, device=dev)

    def step(self, keep_indices: bool = False):
        inst, w = self.inst, self.inst.w
        self.state.c.has_idx = 0
        self.state.c.has_pool = 0
        self.state.c.has_stage = 0
        for l, mode in enumerate(w.pattern):
            L = inst.layers[l]
            api.csa2_layer_forward(mode, q=L["q"], q_idx=L["q_idx"], swa_kv=L["swa"], q_pos=inst.q_pos,
                                   window=w.window, sm_scale=inst.sm_scale, o=self.o[l], lse=self.lse[l],
                                   cache=inst.cache, kview=inst.kview, n_vis=inst.n_vis, n_max=inst.n_max, K=w.K,
                                   P=w.P if self.has_pool else 0, build_pool=self.has_pool and mode == "F",
                                   ws=self.ws, state=self.state)
            if keep_indices:
                self.idx[l].copy_(self.state.idx)
                if mode == "F" and self.has_pool:
                    self.pool.copy_(self.state.pool)
