"""Shared helpers of the GPU parity tests (HIP path vs the CPU oracle)."""
import numpy as np
import pytest
import torch

ATTN_TOL = 2e-3      # row-wise max relative error of attention outputs
LSE_TOL = 1e-3       # absolute error of the natural-log LSE


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU (run with -m 'not gpu' on a CPU-only machine)")
    from fp4_kv_cache_csa2_amd import _lib
    _lib.load()  # raises if the HIP library is missing: no fallback


def case(msg: str):
    """Print the case name before a GPU step so a crash report names it."""
    print(f"[case] {msg}", flush=True)


def assert_attn_close(o, lse, o_ref, lse_ref, what=""):
    """o[..., H, D] vs o_ref (fp64): per (row, head), ||o-o_ref||_inf <= ATTN_TOL ||o_ref||_inf."""
    o = np.asarray(o, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    num = np.abs(o - o_ref).max(-1)
    den = np.abs(o_ref).max(-1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= ATTN_TOL, f"{what}: attention max row-relative error {worst:.3e} > {ATTN_TOL}"
    lse = np.asarray(lse, np.float64)
    lse_ref = np.asarray(lse_ref, np.float64)
    both_inf = np.isneginf(lse) & np.isneginf(lse_ref)
    d = np.where(both_inf, 0.0, np.abs(lse - lse_ref))
    assert np.all(d <= LSE_TOL), f"{what}: lse error {float(np.nanmax(d)):.3e}"
    return worst


def to_np(t):
    return t.detach().cpu().numpy()
