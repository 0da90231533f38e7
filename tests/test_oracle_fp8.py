"""Pins of the oracle's FP8 activation quantiser (CPU only).

The quantiser writes E4M3 codes with one UE8M0 scale per block ([D] "Three
bugs", item 2: DeepSeek's activation quantiser, ue8m0 scales, FP8 out;
[OCP-MX] MXFP8 for blocks of 32). It is pinned by things other than itself:

* every finite E4M3 value, placed in a block whose shared exponent is 0,
  comes back as its own code (exact values round to themselves);
* the codes of random blocks equal torch's float8_e4m3fn conversion (a library
  routine) of v / 2^X clamped to +-448, with X derived here from math.frexp;
* hand-worked cases of both scale rules, of round-half-to-even on the E4M3
  grid (normal and subnormal) and of saturation.
"""
import math

import numpy as np
import pytest
import torch


def _x_floor(amax):
    m, e = math.frexp(amax)  # amax = m * 2^e, m in [0.5, 1)
    return (e - 1) - 8


def _x_ceil(amax):
    return math.ceil(math.log2(amax / 448.0)) if amax > 0 else 0


def test_every_e4m3_value_roundtrips(orc):
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = torch.tensor(finite, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    # a block whose max is 256 (= 2^8) has shared exponent 0 under the floor rule
    for i in range(0, len(finite), 31):
        chunk = list(vals[i:i + 31]) + [256.0]
        codes, sb = orc.fp8_quant(chunk, orc.SCALE_FLOOR)
        assert sb == 127
        for c, v in zip(codes[:-1], finite[i:i + 31]):
            assert c == v or (v == 0x80 and c == 0x80), (hex(c), hex(v))


@pytest.mark.parametrize("rule", ["floor", "ceil"])
@pytest.mark.parametrize("block", [32, 128])
def test_blocks_match_torch_float8(orc, rule, block):
    rng = np.random.default_rng(7 + block)
    for trial in range(200):
        scale = 2.0 ** rng.integers(-30, 30)
        v = rng.standard_normal(block) * scale
        if trial % 5 == 0:
            v[rng.integers(0, block, 3)] = 0.0
        if trial % 7 == 0:
            v *= 1e-3 ** rng.integers(1, 4)
        amax = float(np.abs(v).max())
        X = _x_floor(amax) if rule == "floor" else _x_ceil(amax)
        X = max(-127, min(127, X))
        t = torch.tensor(np.ldexp(v, -X)).clamp(-448.0, 448.0).to(torch.float32)
        ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        codes, sb = orc.fp8_quant(v, orc.SCALE_FLOOR if rule == "floor" else orc.SCALE_CEIL)
        assert sb == X + 127
        assert (codes == ref).all(), (trial, np.nonzero(codes != ref))


def test_scale_rules_hand_cases(orc):
    # amax 1.0: floor(log2 1) - 8 = -8; ceil(log2(1/448)) = -8
    assert orc.fp8_quant([1.0, 0.5], orc.SCALE_FLOOR)[1] == 119
    assert orc.fp8_quant([1.0, 0.5], orc.SCALE_CEIL)[1] == 119
    # amax 1.8: floor rule X = -8 and 1.8 * 256 = 460.8 saturates to 448 (0x7E);
    # ceil rule X = -7 and 1.8 * 128 = 230.4 rounds to 224 = 1.75 * 2^7 (0x76)
    c, sb = orc.fp8_quant([1.8, -1.0], orc.SCALE_FLOOR)
    assert sb == 119 and c[0] == 0x7E and c[1] == 0xF8
    c, sb = orc.fp8_quant([1.8, -1.0], orc.SCALE_CEIL)
    assert sb == 120 and c[0] == 0x76 and c[1] == 0xF0
    # amax 448 exactly: both rules give X = 0 and the code of 448
    for rule in (orc.SCALE_FLOOR, orc.SCALE_CEIL):
        c, sb = orc.fp8_quant([448.0, 1.0], rule)
        assert sb == 127 and c[0] == 0x7E and c[1] == 0x38
    # all-zero block: scale byte 0, codes keep the sign of zero
    c, sb = orc.fp8_quant([0.0, -0.0, 0.0], orc.SCALE_FLOOR)
    assert sb == 0 and list(c) == [0, 0x80, 0]


def test_round_half_even_on_the_e4m3_grid(orc):
    # shared exponent 0 (max 256); midpoints between neighbouring E4M3 values
    cases = [
        (1.0625, 0x38),        # between 1.0 (0x38) and 1.125 (0x39): even -> 1.0
        (1.1875, 0x3A),        # between 1.125 (0x39) and 1.25 (0x3A): even -> 1.25
        (2.0 ** -10, 0x00),    # half of the smallest subnormal 2^-9: even -> 0
        (3 * 2.0 ** -10, 0x02),  # between 2^-9 (0x01) and 2^-8 (0x02): even -> 0x02
        (-(2.0 ** -12), 0x80),  # rounds to zero, keeps its sign
        (304.0, 0x7A),         # between 288 (0x79) and 320 (0x7A): even -> 320
        (300.0, 0x79),         # nearer to 288
    ]
    for v, code in cases:
        c, sb = orc.fp8_quant([v, 256.0], orc.SCALE_FLOOR)
        assert sb == 127 and c[0] == code, (v, hex(c[0]), hex(code))


def test_rows_layout(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 96)).astype(np.float32)
    codes, sc = orc.quant_fp8_rows(x, block=32)
    assert codes.shape == (3, 96) and sc.shape == (3, 3)
    for t in range(3):
        for b in range(3):
            c, sb = orc.fp8_quant(x[t, 32 * b:32 * b + 32].astype(np.float64))
            assert (codes[t, 32 * b:32 * b + 32] == c).all() and sc[t, b] == sb
    with pytest.raises(ValueError):
        orc.quant_fp8_rows(x, block=64)


# ---------------------------------------------------------------------------
# row-scaled FP8 GEMV


def test_gemv_fp8_integer_exact(orc):
    """Codes of small integers, integer x and unit scales: every partial sum
    is an exact integer, so the result equals numpy's integer product."""
    rng = np.random.default_rng(11)
    ints = np.array([0, 1, 2, 3, 4, -1, -2, -3, -4, 6, -6, 8], np.float32)
    codes = torch.tensor(ints).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sel = rng.integers(0, len(ints), (7, 96))
    W = codes[sel]
    x = rng.integers(-5, 6, 96).astype(np.float32)
    y = orc.gemv_fp8(W, np.ones(7, np.float32), x)
    ref = ints[sel].astype(np.int64) @ x.astype(np.int64)
    assert (y == ref).all()


def test_gemv_fp8_matches_torch_decode_and_numpy(orc):
    """Against torch's float8_e4m3fn decoder and a float64 numpy product."""
    import synthgen as sg
    W = sg.fp8_matrix(33, 512, 1).numpy()
    s = sg.fp8_row_scales(33, 1).numpy()
    x = sg.fp8_vector(512, 1).numpy()
    Wf = torch.from_numpy(W).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = s.astype(np.float64) * (Wf @ x.astype(np.float64))
    y = orc.gemv_fp8(W, s, x)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
    # the row scale belongs to its own row: a shift by one row is far off
    assert np.abs(np.roll(s, 1) * (Wf @ x) - y).max() > 0.1 * np.abs(y).max()


def test_fp8_matrix_generator_skips_nan_codes():
    import synthgen as sg
    W = sg.fp8_matrix(64, 1024, 3).numpy()
    assert not np.isin(W, [0x7F, 0xFF]).any()
    assert len(np.unique(W)) == 254
