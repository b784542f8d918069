"""Pins of the oracle's FP4 / E4M3 codec against the format specifications,
a library routine (PyTorch's float8_e4m3fn cast) and closed-form cases."""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden


def test_e2m1_grid_matches_ocp_table(orc):
    for code, value in read_golden("e2m1_grid.txt"):
        assert orc.e2m1_magnitude(int(code)) == float(value)


def test_e4m3fn_named_points(orc):
    for code, value in read_golden("e4m3fn_points.txt"):
        got = orc.e4m3fn_decode(int(code, 16))
        if value == "nan":
            assert math.isnan(got)
        else:
            assert got == float(value)


def test_e4m3fn_decode_all_codes_vs_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = orc.e4m3fn_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], c


def _torch_e4m3_code(q: float) -> int:
    # PyTorch casts through fp32, so callers pass values whose fp32 rounding
    # cannot move them across an E4M3 rounding boundary (see the two users).
    return int(torch.tensor([q], dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8)[0])


def test_e4m3fn_round_vs_torch_cast(orc):
    # Every representable value, every midpoint between neighbours (exact
    # ties), and the fp32 neighbours either side of each midpoint; all are
    # fp32 values, so the library's cast rounds them once.
    vals = sorted({orc.e4m3fn_decode(c) for c in range(0x7F)})
    pts = list(vals)
    for a, b in zip(vals[:-1], vals[1:]):
        m = np.float32((a + b) / 2)
        assert float(m) == (a + b) / 2
        pts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(np.inf))]
    rng = np.random.default_rng(0)
    pts += list(np.exp(rng.uniform(math.log(1e-4), math.log(460.0), 4000)).astype(np.float32))
    pts = [float(p) for p in pts]
    for q in pts:
        if q >= 464.0:  # torch returns NaN past the rounding range; the scale saturates instead
            continue
        assert orc.e4m3fn_round(q) == _torch_e4m3_code(q), q


def test_e4m3fn_round_saturates(orc):
    for q in [448.0, 463.99, 464.0, 480.0, 1e6]:
        assert orc.e4m3fn_round(q) == 0x7E


def test_fp4_byte_layout_and_sign(orc):
    # Channel 0 -> low nibble of byte 0, channel 1 -> high nibble; sign bit 3.
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 6.0, -3.0, -0.0
    codes, scales = orc.fp4_encode(x)
    assert scales[0, 0] == 0x38  # amax/6 = 1.0
    assert codes[0, 0] == (0x7 | (0xD << 4))  # +6 (mag 7), -3 (sign 8 | mag 5)
    assert codes[0, 1] == 0x08  # -0.0 keeps its sign bit, channel 3 is +0
    y = orc.fp4_decode(codes, scales)
    assert y[0, 0] == 6.0 and y[0, 1] == -3.0 and y[0, 2] == 0.0


def test_fp4_ties_go_to_even_code(orc):
    # scale 1.0 (amax = 6); midpoints between E2M1 neighbours.
    mids = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for m, expect in mids.items():
        x = np.zeros((1, 16), np.float32)
        x[0, 0] = 6.0
        x[0, 1] = m
        x[0, 2] = -m
        codes, scales = orc.fp4_encode(x)
        y = orc.fp4_decode(codes, scales)
        assert y[0, 1] == expect and y[0, 2] == -expect, m
        # one ulp either side leaves the tie
        for side, tgt in [(np.nextafter(np.float32(m), np.float32(0)), None),
                          (np.nextafter(np.float32(m), np.float32(10)), None)]:
            x[0, 1] = side
            codes, scales = orc.fp4_encode(x)
            yy = orc.fp4_decode(codes, scales)[0, 1]
            grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
            assert yy == grid[np.argmin(np.abs(grid - side))]


def test_fp4_round_trip_on_grid(orc):
    rng = np.random.default_rng(1)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    scales = [orc.e4m3fn_decode(c) for c in range(1, 0x7F)]
    for s in scales:
        mags = grid[rng.integers(0, 8, 16)]
        mags[rng.integers(0, 16)] = 6.0  # amax = 6 s  ->  scale exactly s
        sign = rng.choice([-1.0, 1.0], 16)
        x = (sign * mags * s).astype(np.float32)[None, :]
        assert np.all(x.astype(np.float64) == sign * mags * s)  # representable in fp32
        codes, sc = orc.fp4_encode(x)
        assert orc.e4m3fn_decode(int(sc[0, 0])) == s
        np.testing.assert_array_equal(orc.fp4_decode(codes, sc), x.astype(np.float64))


def test_fp4_error_bound_and_scale_rule(orc):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((300, 64)).astype(np.float32) * np.exp(rng.uniform(-6, 6, (300, 1))).astype(np.float32)
    codes, sc = orc.fp4_encode(x)
    y = orc.fp4_decode(codes, sc)
    g = x.reshape(300, 4, 16).astype(np.float64)
    amax = np.abs(g).max(-1)
    for r in range(300):
        for j in range(4):
            # scale = the library's RNE E4M3 of amax/6 (in range here).  Its
            # rounding through fp32 is harmless: fl32(amax/6) lands on an E4M3
            # midpoint only when amax/6 itself does (6*midpoint fits in fp32).
            assert sc[r, j] == _torch_e4m3_code(amax[r, j] / 6.0)
    s = np.vectorize(orc.e4m3fn_decode)(sc).astype(np.float64)
    # Error never exceeds half the local grid step (largest step 2 between 4 and 6),
    # up to the saturation at 6*s.
    err = np.abs(y.reshape(300, 4, 16) - g)
    within = np.abs(g) <= 6 * s[..., None]
    # Half-step bound per region: |x| < 2s -> 0.25 s; 2s..4s -> 0.5 s; 4s..6s -> 1.0 s
    a = np.abs(g)
    sr = s[..., None].repeat(16, -1)
    step = np.where(a < 2 * sr, 0.25, np.where(a < 4 * sr, 0.5, 1.0)) * sr
    assert np.all(err[within] <= step[within])


def test_fp4_saturation_far_out_of_range(orc):
    # amax/6 ~ 1e29: the scale saturates at 448 and every element at 6 * 448
    x = np.zeros((1, 32), np.float32)
    x[0, :16] = 1e30
    x[0, 3] = -1e30
    x[0, 16:] = np.linspace(-3e38, 3e38, 16, dtype=np.float32)
    codes, sc = orc.fp4_encode(x)
    assert sc[0, 0] == 0x7E and sc[0, 1] == 0x7E
    y = orc.fp4_decode(codes, sc)
    assert y[0, 0] == 2688 and y[0, 3] == -2688 and y[0, 16] == -2688 and y[0, 31] == 2688
    for q in [448.0, 455.0, 463.999, 3e38, 1e300]:
        assert orc.e4m3fn_round(q) == 0x7E


def test_fp4_saturation_and_zero_group(orc):
    x = np.zeros((2, 16), np.float32)
    x[0, :] = 1e5                      # amax/6 far above 448
    x[0, 1] = -1e5
    codes, sc = orc.fp4_encode(x)
    assert sc[0, 0] == 0x7E
    y = orc.fp4_decode(codes, sc)
    assert y[0, 0] == 6 * 448 and y[0, 1] == -6 * 448
    assert sc[1, 0] == 0 and np.all(codes[1] == 0) and np.all(y[1] == 0)
    # amax so small that amax/6 rounds to scale 0 -> every magnitude 0
    x = np.full((1, 16), 6 * 2.0 ** -10 * 0.99, np.float32)
    codes, sc = orc.fp4_encode(x)
    assert sc[0, 0] == 0 and np.all(orc.fp4_decode(codes, sc) == 0)


def test_fp4_bytes_per_entry(orc):
    # 512 channels -> 256 code bytes + 32 scale bytes = 288 B per entry.
    x = np.random.default_rng(3).standard_normal((3, 512)).astype(np.float32)
    codes, sc = orc.fp4_encode(x)
    group = int(dict(read_golden("pages_constants.txt"))["scale_group"])
    assert codes.shape[1] + sc.shape[1] == 512 // 2 + 512 // group == 288
    # 2.5 main-KV entries per token (3 encoder Full layers at ratio 2 plus one
    # decoder KV at ratio 1) fit in the stated 890 B/token global budget.
    budget = int(dict(read_golden("pages_constants.txt"))["global_kv_bytes_per_token"])
    assert 2.5 * 288 <= budget
