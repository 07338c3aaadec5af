"""Pins for the MXFP8 oracle: hand-derived bit patterns and scales, agreement
with torch's float8 conversions on in-range values, round-trip exactness,
the error bound, the quantisation axis, and an MXFP8 layer on exactly
representable operands reducing to the exact layer."""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            out.append(line.split())
    return out


@pytest.mark.parametrize("row", _rows("e4m3_codes.txt"))
def test_e4m3_hand_patterns(row):
    v, code, r = float(row[0]), int(row[1], 16), float(row[2])
    got = mx.e4m3_round(np.array([v]))
    assert got[0] == r
    assert int(mx.e4m3_encode(got)[0]) == code
    assert mx.e4m3_decode(np.array([code]))[0] == r


@pytest.mark.parametrize("row", _rows("mx_scales.txt"))
def test_scale_hand_values(row):
    amax, stored = float(row[0]), int(row[1])
    block = np.zeros(32)
    block[5] = -amax
    block[9] = amax / 3
    _, s = mx.mx_quantize(block[None, :], axis=1)
    assert int(s[0, 0]) == stored


def test_all_codes_decode_and_reencode():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = mx.e4m3_decode(codes)
    # -0 (0x80) re-encodes to 0x80 because the sign bit is kept
    assert np.array_equal(mx.e4m3_encode(vals), codes.astype(np.uint8))
    assert np.array_equal(mx.e4m3_round(vals), vals)


def test_matches_torch_float8_on_in_range_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1.0, 30.0, 150.0)])
    v = v[np.abs(v) <= 448].astype(np.float32)
    ours = mx.e4m3_encode(mx.e4m3_round(v.astype(np.float64)))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_scales_match_torch_e8m0_of_power_of_two():
    rng = np.random.default_rng(1)
    blocks = rng.standard_normal((200, 32)) * np.exp2(rng.integers(-30, 30, (200, 1)))
    _, s = mx.mx_quantize(blocks, axis=1)
    amax = np.abs(blocks).max(1)
    expect = np.exp2(np.floor(np.log2(amax)) - 8).astype(np.float32)
    ref = torch.from_numpy(expect).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    assert np.array_equal(s[:, 0], ref)


def test_roundtrip_exact_on_representable_blocks():
    rng = np.random.default_rng(2)
    grid = mx.e4m3_decode(np.array([c for c in range(0x7F)]))
    vals = rng.choice(grid, size=(50, 64)) * rng.choice([-1, 1], size=(50, 64))
    vals[:, 0] = 448.0                     # pins the scale of block 0 to 2^0
    vals[:, 32] = -256.0                   # and of block 1
    scale = np.exp2(rng.integers(-20, 20, (50, 1)))
    v = vals * scale
    np.testing.assert_array_equal(mx.mx_roundtrip(v, axis=1), v)


def test_relative_error_bound():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((300, 128)) * np.exp2(rng.integers(-10, 10, (300, 1)))
    q = mx.mx_roundtrip(v, axis=1)
    c, s = mx.mx_quantize(v, axis=1)
    X = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    r = np.abs(v) / X                       # in [0, 512): the block maximum lands in [256, 512)
    assert np.all(r.max(axis=1) >= 256) and np.all(r < 512)
    sat = r > 448
    assert np.all(q[sat] == np.sign(v[sat]) * 448 * X[sat])   # saturated elements
    # normal E4M3 range: half a unit in the last place, 2^-4 relative
    normal = (r >= 2.0 ** -6) & ~sat
    assert np.all(np.abs(q - v)[normal] <= np.abs(v)[normal] * 2.0 ** -4)
    sub = r < 2.0 ** -6
    assert np.all(np.abs(q - v)[sub] <= X[sub] * 2.0 ** -10)


def test_axis_and_ragged_tail():
    # rows at very different scales: exact along the row (axis 1), lossy along axis 0
    rng = np.random.default_rng(4)
    grid = np.array([1.0, 1.25, 1.5, 1.75, -1.0, -1.5, 0.0])
    v = rng.choice(grid, size=(40, 40)) * np.exp2(-3.0 * np.arange(40))[:, None]
    np.testing.assert_array_equal(mx.mx_roundtrip(v, axis=1), v)
    assert not np.array_equal(mx.mx_roundtrip(v, axis=0), v)
    c, s = mx.mx_quantize(v, axis=1)
    assert c.shape == (40, 40) and s.shape == (40, 2)             # 40 = 32 + ragged 8
    c0, s0 = mx.mx_quantize(v, axis=0)
    assert c0.shape == (40, 40) and s0.shape == (2, 40)
    # the ragged tail block is quantised as if zero-padded
    pad = np.concatenate([v, np.zeros((40, 24))], axis=1)
    np.testing.assert_array_equal(mx.mx_roundtrip(pad, axis=1)[:, :40], mx.mx_roundtrip(v, axis=1))


def _mx_exact_layer(seed, T=32, H=64, I=32, E=2):
    """Operands that MXFP8 represents exactly along every axis, and g >= 40 so
    that sigma(g) == 1 in float64 and h, dg, du stay exactly representable."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-1, 2, (T, H)).astype(np.float64)
    x[:, 0] = 1.0
    wg = np.zeros((E, I, H))
    wg[:, :, 0] = rng.choice([40.0, 48.0, 56.0, 64.0], size=(E, I))
    wu = np.zeros((E, I, H))
    for e in range(E):
        for i in range(I):
            cols = rng.choice(np.arange(1, H), size=2, replace=False)
            wu[e, i, cols] = rng.choice([-1.0, 1.0], size=2)
    wd = np.zeros((E, H, I))
    for e in range(E):
        for i in range(I):
            rows = rng.choice(np.arange(H), size=2, replace=False)
            wd[e, rows, i] = rng.choice([-1.0, 1.0], size=2)
    L = rng.standard_normal((T, E)).astype(np.float32)
    dy = rng.integers(-1, 2, (T, H)).astype(np.float64)
    return x, wg, wu, wd, L, dy


def test_mx_layer_reduces_to_exact_layer_on_representable_operands():
    x, wg, wu, wd, L, dy = _mx_exact_layer(5)
    idx, w = oracle.route(L, 1)                    # k = 1: every weight is exactly 1
    sched = oracle.schedule(idx, 2)
    fe = oracle.forward(x, wg, wu, wd, idx, w)
    fm = oracle.forward(x, wg, wu, wd, idx, w, mx=True)
    np.testing.assert_array_equal(fm["y"], fe["y"])
    be = oracle.backward(x, wg, wu, wd, idx, w, dy)
    bm = oracle.backward(x, wg, wu, wd, idx, w, dy, mx=True, sched=sched)
    np.testing.assert_array_equal(bm["dx"], be["dx"])
    np.testing.assert_array_equal(bm["dw"], be["dw"])
    for e in be["dWg"]:
        np.testing.assert_array_equal(bm["dWg"][e], be["dWg"][e])
        np.testing.assert_array_equal(bm["dWu"][e], be["dWu"][e])
        np.testing.assert_array_equal(bm["dWd"][e], be["dWd"][e])


def test_mx_layer_is_close_but_not_equal_on_gaussian_operands():
    rng = np.random.default_rng(6)
    T, H, I, E, k = 40, 64, 32, 4, 2
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((E, I, H)) / 8
    wu = rng.standard_normal((E, I, H)) / 8
    wd = rng.standard_normal((E, H, I)) / 6
    idx, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    fe = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    fm = oracle.forward(x, wg, wu, wd, idx, w, mx=True)["y"]
    # three mantissa bits: each quantised operand carries ~3% rms relative error,
    # and the output compounds five of them
    rel_rms = np.sqrt(np.mean((fm - fe) ** 2) / np.mean(fe ** 2))
    assert 0.02 < rel_rms < 0.12
