"""The allocation-free Top-K entry point (built-in scratch, no workspace)
against the workspace entry point, through the C ABI: identical indices on two
calls in a row (the second smaller, so stale scratch contents from the first
would show), with a pool map and with an overflowing threshold bin."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_csa2_amd import api, inputs
from gpu_common import case, require_gpu, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _scores(rows, n, kind, tag):
    if kind == "normal":
        s = inputs.normal((rows, n), tag).numpy() * 30
    else:  # ties: the threshold bin overflows the candidate lists (whole-row fallback)
        s = np.full((rows, n), 1.5, np.float32)
        s[:, ::7] = 2.5
    s[:, ::11] = -np.inf
    return s


def _both(s, k, pool=None):
    rows, n = s.shape
    sd = torch.from_numpy(s).to(DEV)
    pd = None if pool is None else torch.from_numpy(pool).to(DEV)
    ref = torch.empty(rows, k, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(api.csa2_topk_workspace_size(rows, n, k), 16), dtype=torch.uint8, device=DEV)
    api.csa2_topk(sd, k, ref, pool_blocks=pd, ws=ws)
    got = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    api.csa2_topk_noalloc(sd, k, got, pool_blocks=pd)
    torch.cuda.synchronize()
    return to_np(got), to_np(ref)


@pytest.mark.parametrize("calls", [
    [(64, 200000, 512, "normal"), (3, 70000, 2048, "normal")],
    [(16, 100000, 2048, "ties"), (2, 40000, 512, "ties")],
    [(8, 1 << 20, 512, "normal"), (4, 50000, 1, "normal"), (5, 16384, 512, "normal")]])
def test_topk_noalloc_matches_workspace_entry_point(calls):
    require_gpu()
    for rows, n, k, kind in calls:
        s = _scores(rows, n, kind, f"na{rows}_{n}_{k}")
        case(f"topk_noalloc rows={rows} n={n} k={k} {kind}")
        got, ref = _both(s, k)
        np.testing.assert_array_equal(got, ref)


def test_topk_noalloc_with_pool_map():
    require_gpu()
    rows, P, k = 4, 8192, 512
    s = inputs.normal((rows, 8 * P), "napool").numpy()
    pool = np.sort(np.random.default_rng(5).choice(1 << 20, (rows, P)), axis=1).astype(np.int32)
    case("topk_noalloc with a pool map")
    got, ref = _both(s, k, pool)
    np.testing.assert_array_equal(got, ref)


def test_topk_noalloc_rejects_rows_beyond_its_scratch():
    require_gpu()
    s = torch.zeros(65, 40000, device=DEV)
    out = torch.empty(65, 16, dtype=torch.int32, device=DEV)
    with pytest.raises(api.Csa2Error) as e:
        api.csa2_topk_noalloc(s, 16, out)
    assert e.value.status == api._lib.CSA2_EUNSUPPORTED
    # short rows need no scratch: any row count
    api.csa2_topk_noalloc(s[:, :30000].contiguous(), 16, out)
    torch.cuda.synchronize()
