"""Pins of the oracle's window replay: the bf16 rounding against an exact
rational search over the bf16 grid and named IEEE cases, and the replay
against closed forms (one-hot inputs pick one column of the projection),
its ring-slot rule and exact rational sums on tiny inputs."""
from fractions import Fraction

import numpy as np
import pytest
import torch


def _bf16_values():
    """Every finite non-negative bf16 value, ascending, with its code."""
    codes = np.arange(0, 0x7F80, dtype=np.uint16)  # +0 .. largest finite
    vals = torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return codes, vals


_CODES, _VALS = _bf16_values()


def _exact_rne(x: Fraction) -> int:
    """bf16 code nearest to x (ties to the even code) by searching the grid."""
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    top = Fraction(2) ** 127 * (2 - Fraction(1, 2 ** 8))  # halfway to the next binade past the largest
    if a >= top:  # past the largest finite value, or tied with it (odd code): infinity
        return sign | 0x7F80
    i = int(np.searchsorted(_VALS, float(a)))
    best = None
    for j in range(max(0, i - 2), min(len(_VALS), i + 3)):
        d = abs(Fraction(_VALS[j]) - a)
        key = (d, int(_CODES[j]) & 1)
        if best is None or key < best[0]:
            best = (key, int(_CODES[j]))
    return sign | best[1]


@pytest.mark.parametrize("v,code", [
    (1.0, 0x3F80), (-1.5, 0xBFC0), (0.0, 0x0000), (-0.0, 0x8000),
    (1 + 2 ** -8, 0x3F80),                # tie -> even (down)
    (1 + 3 * 2 ** -8, 0x3F82),            # tie -> even (up)
    (1 + 2 ** -8 + 2 ** -30, 0x3F81),     # just past the tie: one rounding, not two
    (2.0 ** -133, 0x0001),                # smallest subnormal
    (2.0 ** -134, 0x0000),                # tie with zero -> even
    (1.5 * 2.0 ** -133, 0x0002),          # tie between 1 and 2 quanta -> even
    (3.3895313892515355e38, 0x7F7F),      # largest finite
    (2.0 ** 127 * (2 - 2 ** -8), 0x7F80), # tie at the top -> infinity (even)
    (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
])
def test_bf16_round_named(orc, v, code):
    assert orc.bf16_round(v) == code


def test_bf16_round_vs_exact_grid_search(orc):
    rng = np.random.default_rng(11)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-40, 38, 3000),
                         rng.standard_normal(500) * 2.0 ** -128])
    # and midpoints of neighbouring bf16 values, the hard cases
    k = rng.integers(1, len(_VALS) - 1, 500)
    mids = (_VALS[k] + _VALS[k + 1]) / 2
    for x in np.concatenate([xs, mids, -mids]):
        assert orc.bf16_round(float(x)) == _exact_rne(Fraction(float(x))), x


def _bf16_bits(shape, rng, scale=1.0):
    x = torch.from_numpy(rng.standard_normal(shape) * scale).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def _to_f64(bits):
    return torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_replay_one_hot_picks_projection_column(orc):
    rng = np.random.default_rng(3)
    n, dm, D, T = 6, 48, 16, 8  # d_model != D: a transposed W cannot pass
    W = _bf16_bits((D, dm), rng)
    cols = np.array([0, 5, 47, 13, 13, 30])
    h = np.zeros((n, dm), np.uint16)
    h[np.arange(n), cols] = 0x3F80  # 1.0
    ring = orc.swa_replay(h, W, t_end=n - 1, T=T)
    for i in range(n):
        np.testing.assert_array_equal(ring[i], W[:, cols[i]])
    assert not ring[n:].any()


def test_replay_ring_slots(orc):
    rng = np.random.default_rng(4)
    n, dm, D, T = 5, 32, 16, 128
    W = _bf16_bits((D, dm), rng)
    h = np.zeros((n, dm), np.uint16)
    h[np.arange(n), np.arange(n)] = 0x4000  # 2.0 on channel i
    old = np.full((T, D), 0x1234, np.uint16)
    ring = orc.swa_replay(h, W, t_end=300, T=T, ring=old)
    # positions 296..300 -> slots 40..44
    for i, p in enumerate(range(296, 301)):
        np.testing.assert_array_equal(_to_f64(ring[p % T]), 2 * _to_f64(W[:, i]))
    keep = np.setdiff1d(np.arange(T), np.arange(296, 301) % T)
    assert (ring[keep] == 0x1234).all()
    # a full window wraps: every slot written exactly once
    h2 = _bf16_bits((T, dm), rng)
    full = orc.swa_replay(h2, W, t_end=1000, T=T, ring=old)
    assert not (full == 0x1234).all(axis=1).any()
    np.testing.assert_array_equal(full[1000 % T], orc.swa_replay(h2[-1:], W, 1000, T)[1000 % T])


def test_replay_exact_rational_sums(orc):
    rng = np.random.default_rng(5)
    n, dm, D, T = 3, 40, 12, 4
    h = _bf16_bits((n, dm), rng)
    W = _bf16_bits((D, dm), rng, scale=0.125)
    ring = orc.swa_replay(h, W, t_end=n - 1, T=T)
    hf, Wf = _to_f64(h), _to_f64(W)
    for i in range(n):
        for d in range(D):
            exact = sum(Fraction(hf[i, c]) * Fraction(Wf[d, c]) for c in range(dm))
            assert ring[i, d] == _exact_rne(exact), (i, d)


def test_replay_power_of_two_scaling_is_exact(orc):
    rng = np.random.default_rng(6)
    h = _bf16_bits((4, 64), rng)
    W = _bf16_bits((16, 64), rng)
    a = _to_f64(orc.swa_replay(h, W, 3, 4))
    h2 = (torch.from_numpy(_to_f64(h)) * 4).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    b = _to_f64(orc.swa_replay(h2, W, 3, 4))
    np.testing.assert_array_equal(b, 4 * a)


@pytest.mark.parametrize("T,t_end", [(128, 1000), (256, 1000), (128, 127), (131, 5000)])
def test_replay_then_attention_sees_the_logical_window(orc, T, t_end):
    # A window rebuilt by replaying the last 128 tokens (t_end mod T need not be
    # T - 1) and attended by the token at t_end covers exactly the replayed
    # tokens t_end-127..t_end.  Expected: fp64 softmax attention over the same
    # projected rows in token order, from a replay into a 128-row ring that
    # ends at position 127 (token i on row i).
    rng = np.random.default_rng(T + t_end)
    n, dm, D, H, sc = 128, 64, 128, 16, 0.08
    W = _bf16_bits((D, dm), rng, scale=0.125)
    h = _bf16_bits((n, dm), rng)
    ring = orc.swa_replay(h, W, t_end, T)
    in_order = _to_f64(orc.swa_replay(h, W, n - 1, n))
    q = rng.standard_normal((H, D))
    o, lse = orc.attention(q, None, None, None, _to_f64(ring), t_end, 128, sc)
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(in_order)[None, None].expand(1, H, -1, -1)
    o_ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=sc)[0, :, 0].numpy()
    lse_ref = torch.logsumexp((qt @ kt.transpose(-1, -2)) * sc, -1)[0, :, 0].numpy()
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)
