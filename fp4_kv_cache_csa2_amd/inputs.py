"""Seeded synthetic inputs for the CSA2 hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scoring, selection, quantisation or attention), so the
HIP path and the CPU oracle can both be fed from it.

Every tensor is drawn from its own PyTorch generator keyed by (seed, tag), so a
tensor does not depend on which other tensors were drawn before it.  On the CPU
the stream is PyTorch's CPU generator; ``device="cuda"`` uses the GPU's
generator (different numbers, same distribution) and is used only for inputs
too large to draw on the host.

Distributions follow the workloads: N(0,1) everywhere; bf16 tensors are the
round-to-nearest-even bf16 of an fp32 N(0,1) draw; the main-KV latent is an fp32
N(0,1) draw that the path quantises to FP4 itself.
"""
from __future__ import annotations

import dataclasses
import math
import zlib

import numpy as np
import torch


def _key(seed: int, tag: str) -> int:
    return (int(seed) * 0x9E3779B1 + zlib.crc32(tag.encode())) & 0x7FFF_FFFF_FFFF_FFFF


def generator(seed: int, tag: str, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_key(seed, tag))
    return g


def normal(shape, tag: str, seed: int = 0, device="cpu", dtype=torch.float32) -> torch.Tensor:
    """N(0,1) in fp32, then cast (RNE) to ``dtype``."""
    x = torch.randn(tuple(shape), generator=generator(seed, tag, device), device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def small_ints(shape, tag: str, lo: int, hi: int, seed: int = 0, device="cpu",
               dtype=torch.bfloat16) -> torch.Tensor:
    """Uniform integers in [lo, hi] stored as ``dtype`` (tie-heavy test inputs)."""
    x = torch.randint(lo, hi + 1, tuple(shape), generator=generator(seed, tag, device), device=device)
    return x.to(dtype)


def uniform(shape, tag: str, seed: int = 0, device="cpu") -> torch.Tensor:
    return torch.rand(tuple(shape), generator=generator(seed, tag, device), device=device, dtype=torch.float64)


def log_uniform_lengths(B: int, lo: int, hi: int, tag: str = "ctx_len", seed: int = 0) -> np.ndarray:
    """Context lengths floor(exp(U(ln lo, ln hi))), clipped to [lo, hi]."""
    u = uniform((B,), tag, seed).numpy()
    n = np.floor(np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))).astype(np.int64)
    return np.clip(n, lo, hi).astype(np.int32)


def random_page_table(lengths, page_size: int, tag: str = "page_perm", seed: int = 0):
    """Random physical placement of every sequence's pages.

    Returns (page_table[B][max_pages] int32, num_physical_pages).  Physical
    pages are a random permutation of 0..total-1; unused slots hold -1."""
    lengths = np.asarray(lengths, dtype=np.int64)
    pages = (lengths + page_size - 1) // page_size
    total = int(pages.sum())
    max_pages = int(pages.max()) if len(pages) else 0
    perm = torch.randperm(total, generator=generator(seed, tag)).numpy().astype(np.int32)
    table = np.full((len(lengths), max(max_pages, 1)), -1, np.int32)
    at = 0
    for b, p in enumerate(pages):
        table[b, :p] = perm[at:at + p]
        at += p
    return table, total


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a bf16 tensor (host numpy uint16)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one CSA2 workload (all sizes in compressed entries)."""
    name: str
    B: int                 # sequences
    Q: int                 # query tokens per sequence
    N: int                 # entries per sequence (max when ragged)
    D: int                 # main latent channels (FP4)
    H: int                 # main query heads
    H_i: int               # indexer heads
    D_i: int               # indexer head dim
    pattern: str           # static layer modes, F / R / U
    K: int = 512           # Top-K
    P: int = 2048          # pool blocks (x 8 positions)
    window: int = 128      # SWA tokens
    q_dtype: torch.dtype = torch.bfloat16
    ratio: int = 1         # tokens per compressed entry
    ragged: bool = False   # log-uniform lengths in [4096, N], paged cache
    page_size: int = 64

    @property
    def layers(self) -> int:
        return len(self.pattern)


WORKLOADS = {
    # Full-mode decode, one query token, 4096 entries, small dims.
    "full_decode_n4k": Workload("full_decode_n4k", B=1, Q=1, N=4096, D=128, H=16, H_i=4, D_i=64,
                                pattern="F", q_dtype=torch.float32),
    # Decoder group 1 (Full + 3 Reuse), batch 8, 64Ki entries each.
    "decoder_group_b8_n64k": Workload("decoder_group_b8_n64k", B=8, Q=1, N=65536, D=512, H=64, H_i=8, D_i=128,
                                      pattern="FUUU"),
    # Encoder prefill chunk: one 6-layer group (Full + 5 Reuse), ratio 2,
    # 2048 causal queries at the end of a 65,536-token context.
    "encoder_prefill_q2k_n32k": Workload("encoder_prefill_q2k_n32k", B=1, Q=2048, N=32768, D=512, H=64, H_i=8,
                                         D_i=128, pattern="FUUUUU", ratio=2),
    # Hierarchical decode at 1Mi entries: Full builds the pool, 3 Reindex layers.
    "hier_decode_b4_n1m": Workload("hier_decode_b4_n1m", B=4, Q=1, N=1 << 20, D=512, H=64, H_i=8, D_i=128,
                                   pattern="FRRR"),
    # Ragged paged batch: 64 sequences, lengths log-uniform in [4Ki, 1Mi],
    # 20-layer decoder pattern.
    "ragged_paged_b64": Workload("ragged_paged_b64", B=64, Q=1, N=1 << 20, D=512, H=64, H_i=8, D_i=128,
                                 pattern="FUUU" + "RUUU" * 4, ragged=True),
    # Multi-token decode (e.g. verifying 4 drafted tokens): the hierarchical
    # decode shape with 4 causal query tokens per sequence.
    "multi_decode_b4_q4_n1m": Workload("multi_decode_b4_q4_n1m", B=4, Q=4, N=1 << 20, D=512, H=64, H_i=8,
                                       D_i=128, pattern="FRRR"),
}


def query_positions(w: Workload) -> np.ndarray:
    """Absolute token positions of the Q query tokens of every sequence when
    all sequences hold N entries: the last Q tokens of an N*ratio-token
    context (layout only; which entries each may see is decided by the path)."""
    T_tok = w.N * w.ratio
    return np.arange(T_tok - w.Q, T_tok, dtype=np.int64)
