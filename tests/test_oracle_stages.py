"""Pins of the oracle's stage-wise prefill entry points (CPU only): the row
rounding, the gate/up stage on a list of assignments (with the absolute-value
sums that bound any finite-precision evaluation of its dot products) and the
down projection + combine on a caller-given h~.

Each is compared with something other than itself: numpy fp64 on
independently dequantised weights (the dequantisation is pinned exhaustively
in test_oracle_formats.py), an independent bit-level bf16 rounding, the
scalar quantisers (pinned against torch and hand cases), the rounding-error
bound of recursive summation (Higham, "Accuracy and Stability of Numerical
Algorithms", 2nd ed., section 4.2: |fl(sum) - sum| <= gamma_(n-1) sum |p_i|
with gamma_m = m u / (1 - m u)), integer-exact cases and planted mistakes.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

from test_oracle_math import rnd_block


def bf16_rne_bits(v):
    """Round fp64 values to bfloat16, to nearest, ties to even, by integer
    operations on the fp64 bit pattern (an implementation independent of the
    oracle's frexp/nearbyint one). Normal fp32 range only. Returns the value."""
    v = np.asarray(v, np.float64)
    b = v.view(np.uint64).copy()
    shift = np.uint64(52 - 7)                 # keep 7 explicit mantissa bits
    lsb = (b >> shift) & np.uint64(1)
    b = b + (np.uint64(1) << (shift - np.uint64(1))) - np.uint64(1) + lsb
    b &= ~((np.uint64(1) << shift) - np.uint64(1))
    return b.view(np.float64)


def near_bf16_midpoint(v, rel):
    """|v| within rel * |v| of a point halfway between two bf16 neighbours."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    step = 2.0 ** (e - 7)
    frac = a / step - np.floor(a / step)
    return np.abs(frac - 0.5) * step <= rel * a


def _layer(fmt, H, I, E, rng):
    return np.stack([rnd_block(fmt, H, I, rng) for _ in range(E)])


# ------------------------------------------------------------ row rounding ---

def test_round_rows_bf16_matches_scalar_and_bit_rule(orc):
    rng = np.random.default_rng(101)
    v = rng.normal(size=(7, 96)) * np.exp2(rng.integers(-20, 20, size=(7, 96)))
    v[0, :4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # two exact ties
    got = orc.round_rows(orc.ACT_BF16, v)
    scal = orc.bf16_value(orc.bf16_rne(v))
    assert np.array_equal(got, scal)
    assert np.array_equal(got, bf16_rne_bits(v))
    assert got[0, 2] == 1.0 and got[0, 3] == 1.0 + 4 * 2 ** -8        # ties to even
    assert np.signbit(got[0, 1])


def test_round_rows_mxfp4_matches_block_quantiser(orc):
    rng = np.random.default_rng(102)
    v = rng.normal(size=(3, 128)) * 3.0
    v[1, 32:64] = 0.0
    v[2, 64:96] = np.linspace(-6, 6, 32)
    got = orc.round_rows(orc.ACT_MXFP4, v)
    for r in range(3):
        for b0 in range(0, 128, 32):
            codes, sb = orc.mxfp4_quant(v[r, b0:b0 + 32])
            ref = np.array([orc.e2m1(int(c)) for c in codes]) * orc.ue8m0(sb)
            assert np.array_equal(got[r, b0:b0 + 32], ref), (r, b0)
    assert np.array_equal(orc.round_rows(orc.ACT_NONE, v), v)
    with pytest.raises(ValueError):
        orc.round_rows(orc.ACT_MXFP4, v[:, :40])


# -------------------------------------------------------------- gate/up stage ---

@pytest.mark.parametrize("fmt,act", [("nvfp4", 1), ("mxfp4", 2), ("nvfp4", 0)])
def test_stage_hidden_vs_numpy(orc, fmt, act):
    rng = np.random.default_rng(103)
    H, I, E, k, T = 128, 64, 5, 2, 6
    blocks = _layer(fmt, H, I, E, rng)
    x = rng.normal(size=(T, H)).astype(np.float32)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32)
    ids = np.array([11, 0, 3, 7, 3], np.int32)             # any order, a repeat
    hp, hq, gu, agu = orc.prefill_stage_hidden(fmt, H, I, E, x, blocks, idx, act, ids)
    for row, a in enumerate(ids):
        t, j = divmod(int(a), k)
        g, u, _ = (m.astype(np.float64) for m in orc.dequant_block(fmt, H, I, blocks[idx[t, j]]))
        xq = orc.round_rows(act, x[t].astype(np.float64)) if act else x[t].astype(np.float64)
        ga, ua = g @ xq, u @ xq
        h = ga * expit(ga) * ua
        assert np.abs(hp[row] - h).max() <= 1e-13 * np.abs(h).max()
        assert np.abs(gu[row, 0] - ga).max() <= 1e-13 * np.abs(ga).max()
        assert np.abs(gu[row, 1] - ua).max() <= 1e-13 * np.abs(ua).max()
        assert np.abs(agu[row, 0] - np.abs(g * xq).sum(1)).max() <= 1e-13 * agu[row, 0].max()
        assert np.abs(agu[row, 1] - np.abs(u * xq).sum(1)).max() <= 1e-13 * agu[row, 1].max()
        assert np.array_equal(hq[row], orc.round_rows(act, hp[row]) if act else hp[row])
    assert np.array_equal(hp[2], hp[4])


def test_stage_hidden_abs_sums_bound_an_fp32_evaluation(orc):
    """The products of x~ (bf16) and NVFP4 weights (at most 6 significant
    bits) are exact in fp32, so a sequential fp32 sum of them differs from
    the exact dot product by at most gamma_(H-1) * sum |p| (Higham 4.2);
    agu is that sum. With all weights and inputs non-negative it equals the
    dot product itself."""
    rng = np.random.default_rng(104)
    H, I, E, k, T = 1024, 16, 2, 1, 3
    blocks = _layer("nvfp4", H, I, E, rng)
    x = (rng.normal(size=(T, H)) * 50).astype(np.float32)
    idx = np.array([[0], [1], [0]], np.int32)
    ids = np.arange(T, dtype=np.int32)
    hp, hq, gu, agu = orc.prefill_stage_hidden("nvfp4", H, I, E, x, blocks, idx, 1, ids)
    u = 2.0 ** -24
    gamma = (H - 1) * u / (1 - (H - 1) * u)
    for t in range(T):
        g, up, _ = orc.dequant_block("nvfp4", H, I, blocks[idx[t, 0]])
        xq = orc.round_rows(1, x[t].astype(np.float64)).astype(np.float32)
        for m, W in enumerate((g, up)):
            p = (W * xq[None, :]).astype(np.float32)              # exact products
            assert np.array_equal(p.astype(np.float64), W.astype(np.float64) * xq.astype(np.float64))
            s32 = np.add.accumulate(p, axis=1, dtype=np.float32)[:, -1].astype(np.float64)
            assert (np.abs(s32 - gu[t, m]) <= gamma * agu[t, m]).all()
            assert (agu[t, m] >= np.abs(gu[t, m])).all()
    # non-negative weights (codes 0..7, positive scales) and inputs: no cancellation
    nb = blocks.copy()
    n = 3 * H * I // 2
    nb[:, :n] &= 0x77
    xp = np.abs(x)
    _, _, gu2, agu2 = orc.prefill_stage_hidden("nvfp4", H, I, E, xp, nb, idx, 1, ids)
    assert np.array_equal(agu2, gu2)


def test_stage_hidden_equals_full_prefill_bitwise(orc):
    """The stage entry point runs the same fp64 arithmetic as orc_moe_prefill."""
    rng = np.random.default_rng(105)
    for fmt, act, H, I in (("nvfp4", 1, 256, 64), ("mxfp4", 2, 256, 96)):
        E, k, T = 6, 3, 5
        blocks = _layer(fmt, H, I, E, rng)
        x = rng.normal(size=(T, H)).astype(np.float32)
        idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32)
        w = rng.random((T, k)).astype(np.float32)
        out, hp, hq = orc.moe_prefill(fmt, H, I, E, x, blocks, idx, w, act=act, want_h=True)
        ids = np.arange(T * k, dtype=np.int32)[::-1].copy()
        sp, sq, _, _ = orc.prefill_stage_hidden(fmt, H, I, E, x, blocks, idx, act, ids, nthreads=3)
        assert np.array_equal(sp[::-1].reshape(T, k, I), hp)
        assert np.array_equal(sq[::-1].reshape(T, k, I), hq)
        # and the down stage on the oracle's own h~ gives its output bit for bit
        assert np.array_equal(orc.prefill_down_combine(fmt, H, I, E, blocks, idx, w, hq, nthreads=4), out)


# -------------------------------------------------------------- down + combine ---

@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_down_combine_vs_numpy(orc, fmt):
    rng = np.random.default_rng(106)
    H, I, E, k, T = 96, 64, 4, 3, 5
    blocks = _layer(fmt, H, I, E, rng)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32)
    w = rng.normal(size=(T, k)).astype(np.float32)
    hq = rng.normal(size=(T, k, I))
    out = orc.prefill_down_combine(fmt, H, I, E, blocks, idx, w, hq)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            d = orc.dequant_block(fmt, H, I, blocks[idx[t, j]])[2].astype(np.float64)
            acc += float(w[t, j]) * (d @ hq[t, j])
        assert np.abs(out[t] - acc).max() <= 1e-13 * np.abs(acc).max()


def test_down_combine_integer_exact(orc):
    """All scales 1.0 (E4M3 0x38), codes e2m1, h~ and w small integers:
    every product and partial sum is exact in fp64, in any order."""
    rng = np.random.default_rng(107)
    H, I, E, k, T = 64, 32, 3, 2, 4
    n = 3 * H * I // 2
    blocks = np.empty((E, n + 3 * H * I // 16), np.uint8)
    blocks[:, :n] = rng.integers(0, 256, (E, n))
    blocks[:, n:] = 0x38
    idx = np.array([[0, 1], [2, 0], [1, 2], [0, 2]], np.int32)
    w = rng.integers(-3, 4, (T, k)).astype(np.float32)
    hq = rng.integers(-4, 5, (T, k, I)).astype(np.float64)
    out = orc.prefill_down_combine("nvfp4", H, I, E, blocks, idx, w, hq)
    lut = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            byt = blocks[idx[t, j], 2 * H * I // 2: 3 * H * I // 2].reshape(H, I // 2)
            d = np.stack([lut[byt & 15], lut[byt >> 4]], axis=2).reshape(H, I)   # low nibble first
            acc += float(w[t, j]) * (d @ hq[t, j])
        assert np.array_equal(out[t], acc)


def test_down_combine_bf16_output_bit_exact(orc):
    """bf16 output: the round-to-nearest-even of the fp64 combine, bit for bit
    (checked with an independent bit-level rounding), except where the fp64
    value lies within 1e-12 relative of a bf16 midpoint (there a different
    summation order may legitimately round the other way)."""
    rng = np.random.default_rng(108)
    H, I, E, k, T = 512, 64, 4, 2, 20
    blocks = _layer("mxfp4", H, I, E, rng)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32)
    w = rng.random((T, k)).astype(np.float32)
    hq = orc.round_rows(2, rng.normal(size=(T, k, I)))
    out = orc.prefill_down_combine("mxfp4", H, I, E, blocks, idx, w, hq, out_bf16=True)
    f64 = orc.prefill_down_combine("mxfp4", H, I, E, blocks, idx, w, hq, out_bf16=False)
    ok = ~near_bf16_midpoint(f64, 1e-12)
    assert ok.mean() > 0.999
    assert np.array_equal(out[ok], bf16_rne_bits(f64[ok]))
    # truncation instead of rounding would be caught: many elements round up
    trunc = np.trunc(f64 / 2.0 ** (np.floor(np.log2(np.abs(f64))) - 7)) * 2.0 ** (np.floor(np.log2(np.abs(f64))) - 7)
    assert (out[ok] != trunc[ok]).mean() > 0.3


def test_down_combine_must_break(orc):
    """Planted mistakes in the down matrix (swapped nibbles, scales shifted by
    one byte) or a shifted expert index move the output by more than 10%."""
    rng = np.random.default_rng(109)
    H, I, E, k, T = 128, 64, 4, 2, 3
    blocks = _layer("nvfp4", H, I, E, rng)
    idx = np.array([[0, 1], [1, 2], [2, 3]], np.int32)
    w = np.full((T, k), 0.5, np.float32)
    hq = rng.normal(size=(T, k, I))
    ref = orc.prefill_down_combine("nvfp4", H, I, E, blocks, idx, w, hq)
    lay = orc.layout("nvfp4", H, I)
    sw = blocks.copy()
    seg = sw[:, lay[2]:lay[3]]
    sw[:, lay[2]:lay[3]] = (seg >> 4) | (seg << 4)
    sc = blocks.copy()
    sc[:, lay[5]:lay[6]] = np.roll(blocks[:, lay[5]:lay[6]], 1, axis=1)
    for bad_blocks, bad_idx in ((sw, idx), (sc, idx), (blocks, (idx + 1) % E)):
        got = orc.prefill_down_combine("nvfp4", H, I, E, bad_blocks, bad_idx, w, hq)
        assert np.abs(got - ref).max() / np.abs(ref).max() > 0.1
