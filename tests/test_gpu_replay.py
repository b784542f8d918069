"""GPU parity of the window replay (csa2_swa_replay) against the oracle.

The kernel accumulates in fp32 and rounds once to bf16; the oracle rounds the
exact sum.  The two agree bit for bit except where the exact value lies within
the fp32 accumulation error of a rounding boundary (a midpoint, or zero when
the sum cancels): there the kernel's value must still be the bf16 rounding of
a value within that error, |got - exact| <= delta + ulp(got)/2, with
delta = (d_model/32 + 32) * 2^-24 * sum_c |h_c W_dc| (at most d_model/32
accumulations of 32-term partial sums, each at most 32 fp32 roundings)."""
import numpy as np
import pytest
import torch

import oracle
from fp4_kv_cache_csa2_amd import api, inputs
from gpu_common import assert_attn_close, case, require_gpu, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL = 0x1234


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    oracle.build(force=False)


def _bits(t):
    return to_np(t.contiguous().view(torch.int16)).view(np.uint16)


def _f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def _assert_projection(got, ref, exact, absdot, dm, what):
    """got/ref bf16 bits of the same rows; exact/absdot fp64 of those rows."""
    mism = got != ref
    frac = float(mism.mean()) if mism.size else 0.0
    if mism.any():
        # the kernel's value must be the bf16 rounding of some fp32 sum within
        # the accumulation bound of the exact value: |got - exact| <= delta + ulp/2
        g = _f64(got[mism])
        mag = np.maximum(np.abs(g), 2.0 ** -126)
        half_ulp = 2.0 ** (np.floor(np.log2(mag)) - 8)
        delta = (dm / 32 + 32) * 2.0 ** -24 * absdot[mism]
        off = np.abs(g - exact[mism])
        assert np.all(off <= delta + half_ulp), f"{what}: {float((off - delta - half_ulp).max()):.3e} beyond the bound"
    if mism.size >= 4096:
        assert frac < 1e-3, f"{what}: {frac:.2e} of the rows' values differ"
    return frac


def _make(L, B, n, dm, D, T, tag):
    h = [inputs.normal((B, n, dm), f"{tag}/h{l}", dtype=torch.bfloat16) for l in range(L)]
    # projection scaled by 2^-k (exact) so that outputs are O(1)
    scale = 2.0 ** -round(np.log2(np.sqrt(dm)))
    W = [(inputs.normal((D, dm), f"{tag}/W{l}") * scale).to(torch.bfloat16) for l in range(L)]
    return h, W


def _run(h, W, t_end, T, D):
    B = h[0].shape[0]
    rings = [torch.full((B, T, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16) for _ in h]
    api.csa2_swa_replay([x.to(DEV) for x in h], [w.to(DEV) for w in W], rings,
                        torch.tensor(t_end, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    return [_bits(r) for r in rings]


@pytest.mark.parametrize("L,B,n,dm,D,T,t_end", [
    (3, 2, 37, 256, 192, 128, [36, 500]),       # ragged tokens and columns; start at 0 and wrapped
    (2, 3, 128, 128, 512, 128, [127, 1000, 4095]),  # a full window, every ring row rewritten
    (1, 5, 1, 128, 16, 4, [0, 1, 2, 3, 9]),      # one token (a decode step's projection), tiny ring
    (2, 1, 10, 64, 32, 16, [5]),                 # tokens before position 0 are skipped
])
def test_replay_matches_oracle(L, B, n, dm, D, T, t_end):
    tag = f"rp{L}{B}{n}{dm}{D}"
    h, W = _make(L, B, n, dm, D, T, tag)
    case(f"swa_replay L={L} B={B} n={n} d_model={dm} D={D} T={T}")
    got = _run(h, W, t_end, T, D)
    worst = 0.0
    for l in range(L):
        hb, Wb = _bits(h[l]), _bits(W[l])
        hf, Wf = _f64(hb), _f64(Wb)
        for b in range(B):
            first = max(0, n - 1 - t_end[b])  # tokens at positions < 0 are skipped
            init = np.full((T, D), SENTINEL, np.uint16)
            ref = oracle.swa_replay(hb[b, first:], Wb, t_end[b], T, ring=init) if first < n else init
            pos = np.arange(t_end[b] - n + 1 + first, t_end[b] + 1)
            rows = pos % T
            # rows no token maps to are untouched
            untouched = np.setdiff1d(np.arange(T), rows)
            assert (got[l][b][untouched] == SENTINEL).all()
            exact = hf[b, first:] @ Wf.T
            absdot = np.abs(hf[b, first:]) @ np.abs(Wf).T
            worst = max(worst, _assert_projection(got[l][b][rows], ref[rows], exact, absdot, dm, f"l={l} b={b}"))
    print(f"fraction of values one ulp off (near a midpoint): {worst:.2e}")


def test_replay_batch_equals_token_by_token():
    """Rebuilding 128 rows at once gives the bits that per-token projection
    (one token per call, as at each decode step) stored: a cache miss followed
    by a replay restores exactly the state that was lost."""
    L, B, n, dm, D, T = 2, 2, 128, 512, 256, 128
    h, W = _make(L, B, n, dm, D, T, "rpbatch")
    t_end = [300, 127]
    case("swa_replay batch vs token by token")
    full = _run(h, W, t_end, T, D)
    hd = [x.to(DEV) for x in h]
    Wd = [w.to(DEV) for w in W]
    rings = [torch.zeros(B, T, D, dtype=torch.bfloat16, device=DEV) for _ in range(L)]
    for i in range(n):
        te = torch.tensor([t - n + 1 + i for t in t_end], dtype=torch.int32, device=DEV)
        api.csa2_swa_replay([x[:, i:i + 1].contiguous() for x in hd], Wd, rings, te)
    torch.cuda.synchronize()
    for l in range(L):
        np.testing.assert_array_equal(_bits(rings[l]), full[l])


def test_replay_full_size_sampled():
    """20 layers x 4 sequences x 128 tokens, d_model 4096, D 512 (the replay
    workload); sampled tokens of sampled layers against the oracle."""
    L, B, n, dm, D, T = 20, 4, 128, 4096, 512, 128
    h, W = _make(L, B, n, dm, D, T, "rpfull")
    t_end = [1 << 20, 5000, 127, 77777]
    case("swa_replay full size")
    got = _run(h, W, t_end, T, D)
    rng = np.random.default_rng(7)
    for l in (0, 7, 19):
        hb, Wb = _bits(h[l]), _bits(W[l])
        Wf = _f64(Wb)
        for b in range(B):
            for i in list(rng.choice(n, 3, replace=False)) + [0, n - 1]:
                p = t_end[b] - n + 1 + int(i)
                ref = oracle.swa_replay(hb[b, i:i + 1], Wb, p, T)[p % T]
                hf = _f64(hb[b, i])
                _assert_projection(got[l][b][p % T][None], ref[None], (hf @ Wf.T)[None],
                                   (np.abs(hf) @ np.abs(Wf).T)[None], dm, f"l={l} b={b} i={i}")


@pytest.mark.parametrize("T,t_end", [(128, [1000, 4133]), (256, [1000, 300]), (131, [5000, 127])])
def test_replayed_ring_attended_at_its_position(T, t_end):
    """Rebuild a window ring by replay at positions whose ring row is not the
    last one (t_end mod T != T - 1), then attend from the token at t_end: the
    window must be exactly the replayed tokens t_end-127 .. t_end.  (The layer
    dispatcher reads rings by the same rule; the ragged workload's rings wrap
    at arbitrary rows.)"""
    B, n, dm, D, H, W = 2, 128, 256, 512, 64, 128
    h, Wp = _make(1, B, n, dm, D, T, f"rpatt{T}")
    rings = [torch.zeros(B, T, D, dtype=torch.bfloat16, device=DEV)]
    case(f"replay then window attention T={T} t_end={t_end}")
    api.csa2_swa_replay([h[0].to(DEV)], [Wp[0].to(DEV)], rings, torch.tensor(t_end, dtype=torch.int32, device=DEV))
    q = inputs.normal((B, 1, H, D), f"rpatt{T}/q", dtype=torch.bfloat16)
    qpos = torch.tensor(t_end, dtype=torch.int32).reshape(B, 1)
    sc = 1 / np.sqrt(D)
    o = torch.empty(B, 1, H, D, device=DEV)
    lse = torch.empty(B, 1, H, device=DEV)
    ws = torch.empty(max(api.csa2_attn_workspace_size(B, 1, H, D), 16), dtype=torch.uint8, device=DEV)
    api.csa2_swa_attn(q.to(DEV), rings[0], qpos.to(DEV), W, sc, 0, o, lse, ws=ws)
    torch.cuda.synchronize()
    hb, Wb = _bits(h[0]), _bits(Wp[0])
    for b in range(B):
        ring_ref = oracle.swa_replay(hb[b], Wb, t_end[b], T)
        ref, lref = oracle.attention(q[b, 0].double().numpy(), None, None, None, _f64(ring_ref), t_end[b], W, sc)
        assert_attn_close(to_np(o)[b, 0], to_np(lse)[b, 0], ref, lref, f"replayed ring b={b}")
