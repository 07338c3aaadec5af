"""Pins for the MXFP8 oracle: hand-derived bit patterns and scales, agreement
with torch's float8 conversions on in-range values, round-trip exactness,
the error bound, the quantisation axis, and an MXFP8 layer on exactly
representable operands reducing to the exact layer."""
import math
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


# ------------------------------------------------------------------ quantisation axes
# Each MXFP8 operand is quantised along its GEMM's reduction axis (oracle.ffn.mm).
# The pins below use operands that E4M3 blocks represent exactly along the
# intended axis and lossily along the other (values 2^20 apart inside a block
# of the wrong axis), so the MXFP8 layer equals the exact layer only if every
# operand is quantised along the intended axis.  Each pin is run once more
# with a planted mistake (an mm quantising an operand along the wrong axis)
# to show that it would catch it.
S20 = 2.0 ** 20


def _mm_wrong_a(A, B, mx=False):
    """planted mistake: the left operand quantised along its first axis"""
    A, B = np.asarray(A, np.float64), np.asarray(B, np.float64)
    if mx:
        A, B = oracle.mx_roundtrip(A, 0), oracle.mx_roundtrip(B, 0)
    return A @ B


def _mm_wrong_b(A, B, mx=False):
    """planted mistake: the right operand quantised along its last axis"""
    A, B = np.asarray(A, np.float64), np.asarray(B, np.float64)
    if mx:
        A, B = oracle.mx_roundtrip(A, -1), oracle.mx_roundtrip(B, -1)
    return A @ B


def test_mm_quantises_both_operands_along_the_contraction_axis():
    rng = np.random.default_rng(8)
    grid = np.array([1.0, 1.25, 1.5, 1.75, -1.0, -1.5, 0.0])
    A = rng.choice(grid, size=(8, 64)) * np.where(np.arange(8) % 2, S20, 1.0)[:, None]
    B = rng.choice(grid, size=(64, 6)) * np.where(np.arange(6) % 2, S20, 1.0)[None, :]
    np.testing.assert_array_equal(oracle.ffn.mm(A, B, mx=True), A @ B)     # exact along K
    Ak = rng.choice(grid, size=(8, 64)) * np.where(np.arange(64) % 2, S20, 1.0)[None, :]
    Bk = rng.choice(grid, size=(64, 6)) * np.where(np.arange(64) % 2, S20, 1.0)[:, None]
    assert not np.array_equal(oracle.ffn.mm(Ak, B, mx=True), Ak @ B)      # lossy along K
    assert not np.array_equal(oracle.ffn.mm(A, Bk, mx=True), A @ Bk)
    # ragged K (40 = 32 + 8): brute force, block by block, element by element
    A = rng.standard_normal((3, 40))
    B = rng.standard_normal((40, 2))

    def q_block(vals):
        amax = max(abs(v) for v in vals)
        s = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
        return [float(mx.e4m3_round(v / 2.0 ** s)) * 2.0 ** s for v in vals]

    Aq = np.array([sum((q_block(list(A[r, b:b + 32])) for b in (0, 32)), []) for r in range(3)])
    Bq = np.array([sum((q_block(list(B[b:b + 32, c])) for b in (0, 32)), []) for c in range(2)]).T
    got = oracle.ffn.mm(A, B, mx=True)
    for r in range(3):
        for c in range(2):
            want = sum(Aq[r, q] * Bq[q, c] for q in range(40))
            assert abs(got[r, c] - want) <= 1e-12 * max(1.0, abs(want))


def _axis_case(kind, seed=5):
    """The exactly representable layer of _mx_exact_layer with one operand
    made exact along its intended axis only."""
    x, wg, wu, wd, L, dy = _mx_exact_layer(seed)
    H = x.shape[1]
    rng = np.random.default_rng(9)
    alt = lambda n: np.where(np.arange(n) % 2, S20, 1.0)
    if kind == "x_rows":           # token rows 2^20 apart: x along H, and h along I
        x = x * alt(x.shape[0])[:, None]
    elif kind == "wgu_rows":       # W_gate rows 2^20 apart (W_up rows the inverse): along H
        f = alt(wg.shape[1])[None, :, None]
        wg, wu = wg * f, wu / f
    elif kind == "wd_rows":        # W_down rows 2^20 apart: the forward's W_down along I
        wd = wd * alt(wd.shape[1])[None, :, None]
    elif kind == "dy_rows":        # dy rows 2^20 apart: dy along H, then dg, du along I
        dy = dy * alt(dy.shape[0])[:, None]
    elif kind == "wd_cols":        # W_down columns 2^20 apart: the dgrad's W_down along H
        wd = wd * alt(wd.shape[2])[None, None, :]
    elif kind == "wgu_tail":       # tiny W_gate / W_up entries beside 40..64 in one H block,
        x[:, 1:32] = 0             # where x is zero: the input gradient's weights along I
        wg[:, :, 1:32] = rng.choice([-1.0, 0.0, 1.0], size=wg[:, :, 1:32].shape) / S20
        wu[:, :, 1:32] = rng.choice([-1.0, 0.0, 1.0], size=wu[:, :, 1:32].shape) / S20
    elif kind == "dy_cols":        # dy columns 2^20 apart: w * dy along the rows (dW_down)
        dy = dy * alt(H)[None, :]
    elif kind == "x_cols_tail":    # x columns 2^20 apart where the weights are zero: x along rows
        wg[:, :, H // 2:] = 0
        wu[:, :, H // 2:] = 0
        x[:, H // 2:] = rng.choice([-1.0, 0.0, 1.0], size=x[:, H // 2:].shape) * alt(H // 2)
    elif kind == "wu_rows":        # W_up rows 2^20 apart: dg and h along the rows
        wu = wu * alt(wu.shape[1])[None, :, None]
    return x, wg, wu, wd, L, dy


def _axis_outputs(kind):
    x, wg, wu, wd, L, dy = _axis_case(kind)
    idx, w = oracle.route(L, 1)
    sched = oracle.schedule(idx, 2)
    out = {}
    for mode in (False, True):
        f = oracle.forward(x, wg, wu, wd, idx, w, mx=mode)
        b = oracle.backward(x, wg, wu, wd, idx, w, dy, mx=mode, sched=sched)
        out[mode] = {"y": f["y"], "dx": b["dx"], "dw": b["dw"],
                     "dWg": np.stack([b["dWg"][e] for e in sorted(b["dWg"])]),
                     "dWu": np.stack([b["dWu"][e] for e in sorted(b["dWu"])]),
                     "dWd": np.stack([b["dWd"][e] for e in sorted(b["dWd"])])}
    return out


# kind: (outputs that the MXFP8 layer must give exactly, the planted mistake
# that breaks them, and which of them it breaks)
AXIS_PINS = {
    "x_rows": (("y", "dx", "dw"), _mm_wrong_a, ("y",)),
    "wgu_rows": (("y",), _mm_wrong_b, ("y",)),
    "wd_rows": (("y",), _mm_wrong_b, ("y",)),
    "dy_rows": (("dx", "dw"), _mm_wrong_a, ("dx", "dw")),
    "wd_cols": (("dw",), _mm_wrong_b, ("dw",)),
    "wgu_tail": (("y", "dx"), _mm_wrong_b, ("dx",)),
    "dy_cols": (("dWd",), _mm_wrong_a, ("dWd",)),
    "x_cols_tail": (("y", "dx", "dWg", "dWu"), _mm_wrong_b, ("dWg", "dWu")),
    "wu_rows": (("dw", "dWg", "dWu", "dWd"), _mm_wrong_a, ("dWg",)),
}


@pytest.mark.parametrize("kind", list(AXIS_PINS))
def test_mx_layer_quantises_each_operand_along_its_reduction_axis(kind, monkeypatch):
    exact_outputs, planted, broken = AXIS_PINS[kind]
    out = _axis_outputs(kind)
    for name in exact_outputs:
        np.testing.assert_array_equal(out[True][name], out[False][name], err_msg=f"{kind}: {name}")
    monkeypatch.setattr(oracle.ffn, "mm", planted)
    bad = _axis_outputs(kind)
    for name in broken:
        assert not np.array_equal(bad[True][name], bad[False][name]), f"{kind}: {name} misses the mistake"


def _straddle_case(seed=7, T=96, M=48, H=64, I=32):
    """One routed expert (k = 1) and a shared expert over two macrobatches of
    48 tokens.  Tokens 32..47 are 2^20 times larger than the rest, so the
    weight-gradient operands (rows of x, dg, du, h) are exact in 32-row blocks
    of each macrobatch's group ([0, 32), [32, 48) | [48, 80), [80, 96)) and
    lossy in blocks that cross the boundary ([32, 64))."""
    rng = np.random.default_rng(seed)

    def weights():
        wg = np.zeros((I, H))
        wg[:, 0] = rng.choice([40.0, 48.0, 56.0, 64.0], size=I)
        wu = np.zeros((I, H))
        wd = np.zeros((H, I))
        for i in range(I):
            wu[i, rng.choice(np.arange(1, H), size=2, replace=False)] = rng.choice([-1.0, 1.0], size=2)
            wd[rng.choice(np.arange(H), size=2, replace=False), i] = rng.choice([-1.0, 1.0], size=2)
        return wg, wu, wd

    x = rng.integers(-1, 2, (T, H)).astype(np.float64)
    x[:, 0] = 1.0
    scale = np.ones(T)
    scale[32:48] = S20
    x = x * scale[:, None]
    wg, wu, wd = weights()
    shared = weights()
    dy = rng.integers(-1, 2, (T, H)).astype(np.float64)
    L = np.zeros((T, 1), np.float32)
    return x, wg[None], wu[None], wd[None], shared, L, dy, M


def test_mx_weight_gradients_block_rows_per_macrobatch_group():
    x, wg, wu, wd, sh, L, dy, M = _straddle_case()
    idx, w = oracle.route(L, 1)
    ex = oracle.backward(x, wg, wu, wd, idx, w, dy, shared=sh)
    fe = oracle.forward(x, wg, wu, wd, idx, w, shared=sh)["y"]
    fm = oracle.forward(x, wg, wu, wd, idx, w, shared=sh, mx=True)["y"]
    np.testing.assert_array_equal(fm, fe)
    two = oracle.schedule(idx, 1, macrobatch=M)
    bm = oracle.backward(x, wg, wu, wd, idx, w, dy, shared=sh, mx=True, sched=two)
    for n in ("dx", "dw"):
        np.testing.assert_array_equal(bm[n], ex[n], err_msg=n)
    for n in ("dWg", "dWu", "dWd"):
        np.testing.assert_array_equal(bm[n][0], ex[n][0], err_msg=n)
    for n in ("dW_sg", "dW_su", "dW_sd"):
        np.testing.assert_array_equal(bm[n], ex[n], err_msg=n)
    # planted mistake: the same stream blocked as if it were one macrobatch
    one = oracle.schedule(idx, 1)
    bw = oracle.backward(x, wg, wu, wd, idx, w, dy, shared=sh, mx=True, sched=one)
    for n in ("dWg", "dWu", "dWd"):
        assert not np.array_equal(bw[n][0], ex[n][0]), n
    for n in ("dW_sg", "dW_su", "dW_sd"):
        assert not np.array_equal(bw[n], ex[n]), n


# ------------------------------------------------------------------ MXFP4 (the weight variant)
def _golden_rows(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_e2m1_codes_match_the_hand_derived_table():
    rows = _golden_rows("e2m1_codes.txt")
    v = np.array([float(r[0]) for r in rows])
    r = mx.e2m1_round(v)
    np.testing.assert_array_equal(r, [float(x[2]) for x in rows])
    np.testing.assert_array_equal(mx.e2m1_encode(r), [int(x[1], 16) for x in rows])
    np.testing.assert_array_equal(mx.e2m1_decode(mx.e2m1_encode(r)), r)


def test_mxfp4_scales_match_the_hand_derived_table():
    for row in _golden_rows("mx4_scales.txt"):
        amax, want = float(row[0]), int(row[1])
        block = np.zeros(32)
        block[5] = amax
        block[9] = -amax / 3
        _, s = mx.mxfp4_quantize(block)
        assert int(s[0]) == want, (amax, int(s[0]), want)


def test_mxfp4_roundtrip_and_error_bound():
    rng = np.random.default_rng(12)
    # blocks of grid values times a power of two are exact
    v = rng.choice(np.concatenate([mx.E2M1_GRID, -mx.E2M1_GRID]), size=(16, 64))
    v[:, ::32] = 6.0                       # every block holds its maximum
    v = v * np.exp2(rng.integers(-20, 20, size=(16, 1)))
    np.testing.assert_array_equal(mx.mxfp4_roundtrip(v, axis=1), v)
    # Gaussian blocks: every element within half a quantum of its block
    g = rng.standard_normal((64, 96))
    q = mx.mxfp4_roundtrip(g, axis=1)
    c, s = mx.mxfp4_quantize(g, axis=1)
    X = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    a = np.abs(g) / X
    quantum = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0)) * X
    inside = a <= 6.0
    assert np.all((np.abs(q - g) <= quantum / 2)[inside])
    # the scale rule leaves a block's largest magnitudes in [4, 8) quanta; those
    # above 6 saturate to 6
    np.testing.assert_array_equal(np.abs(q)[~inside], 6.0 * X[~inside])
    # the quantiser is along the given axis only
    np.testing.assert_array_equal(mx.mxfp4_roundtrip(g.T, axis=0), q.T)


def _w4_exact_layer(seed, T=32, H=64, I=32, E=2):
    """Operands exact in MXFP4 (weights) and MXFP8 (activations) along K:
    W_gate's one nonzero per row from {48, 64, 96, 128} (g >= 48, so
    sigma(g) == 1 in float64), the other entries and x in {-1, 0, 1}."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-1, 2, (T, H)).astype(np.float64)
    x[:, 0] = 1.0
    wg = np.zeros((E, I, H))
    wg[:, :, 0] = rng.choice([48.0, 64.0, 96.0, 128.0], size=(E, I))
    wu = np.zeros((E, I, H))
    wd = np.zeros((E, H, I))
    for e in range(E):
        for i in range(I):
            wu[e, i, rng.choice(np.arange(1, H), size=2, replace=False)] = rng.choice([-1.0, 1.0], size=2)
            wd[e, rng.choice(np.arange(H), size=2, replace=False), i] = rng.choice([-1.0, 1.0], size=2)
    L = rng.standard_normal((T, E)).astype(np.float32)
    return x, wg, wu, wd, L


def test_w4_layer_equals_the_exact_layer_on_representable_operands(monkeypatch):
    x, wg, wu, wd, L = _w4_exact_layer(7)
    idx, w = oracle.route(L, 1)
    ex = oracle.forward(x, wg, wu, wd, idx, w)["y"]
    np.testing.assert_array_equal(oracle.forward(x, wg, wu, wd, idx, w, mx="w4")["y"], ex)
    # weight rows 2^20 apart: exact along K (H) only; a weight quantised along
    # the wrong axis breaks it
    f = np.where(np.arange(wg.shape[1]) % 2, 2.0 ** 20, 1.0)[None, :, None]
    wg2, wu2 = wg * f, wu / f
    np.testing.assert_array_equal(oracle.forward(x, wg2, wu2, wd, idx, w, mx="w4")["y"], ex)

    def wrong_axis(A, B, mx=False):
        return oracle.mx_roundtrip(np.asarray(A, np.float64), -1) @ oracle.mxfp4_roundtrip(
            np.asarray(B, np.float64), -1)

    monkeypatch.setattr(oracle.ffn, "mm", wrong_axis)
    assert not np.array_equal(oracle.forward(x, wg2, wu2, wd, idx, w, mx="w4")["y"], ex)


def test_w4_layer_rounds_the_weights_to_e2m1_not_e4m3(monkeypatch):
    """W_up entries of 1.25 are exact in E4M3 but not in E2M1: a block holding
    +-1.25 as its largest values gets scale 2^-2, 1.25 / 0.25 = 5 rounds to 4
    (ties to even), so the MXFP4 layer equals the exact layer with 1.0."""
    x, wg, wu, wd, L = _w4_exact_layer(8)
    idx, w = oracle.route(L, 1)
    wu5 = wu * 1.25
    got = oracle.forward(x, wg, wu5, wd, idx, w, mx="w4")["y"]
    np.testing.assert_array_equal(got, oracle.forward(x, wg, wu, wd, idx, w)["y"])
    assert not np.array_equal(got, oracle.forward(x, wg, wu5, wd, idx, w)["y"])
    # planted mistake: the weights in MXFP8 instead
    monkeypatch.setattr(oracle.ffn, "mm", lambda A, B, mx=False: oracle.mx_roundtrip(
        np.asarray(A, np.float64), -1) @ oracle.mx_roundtrip(np.asarray(B, np.float64), 0))
    assert not np.array_equal(oracle.forward(x, wg, wu5, wd, idx, w, mx="w4")["y"], got)


def test_w4_backward_is_refused():
    x, wg, wu, wd, L = _w4_exact_layer(9)
    idx, w = oracle.route(L, 1)
    with pytest.raises(ValueError):
        oracle.backward(x, wg, wu, wd, idx, w, x, mx="w4")


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("axis", [0, 1])
def test_roundtrip_equals_dequantised_codes(fmt, axis):
    """mx_roundtrip / mxfp4_roundtrip return grid value x block scale without
    forming the bit patterns; they must equal decoding the quantiser's codes,
    bit for bit, on Gaussian data, all-zero blocks, saturating blocks (one
    large element beside small ones), values far below a block's scale
    (E4M3 subnormals, flushes to zero), signed zeros and a ragged tail."""
    rng = np.random.default_rng(41)
    v = rng.standard_normal((70, 97)) * np.exp(rng.uniform(-30, 30, (70, 1)))
    v[3, :] = 0.0
    v[5, :] = -0.0
    v[7, 10] = 1e6
    v[9, :32] = np.ldexp(1.0, -140) * rng.standard_normal(32)
    v[11, 40] = 1e-30
    v[:, 64] *= 1e-12
    v = v if axis == 1 else v.T.copy()
    if fmt == "e4m3":
        want = mx.mx_dequantize(*mx.mx_quantize(v, axis=axis), axis=axis)
        got = mx.mx_roundtrip(v, axis=axis)
    else:
        want = mx.mxfp4_dequantize(*mx.mxfp4_quantize(v, axis=axis), axis=axis)
        got = mx.mxfp4_roundtrip(v, axis=axis)
    assert got.shape == v.shape
    np.testing.assert_array_equal(got.view(np.uint64), want.view(np.uint64))
