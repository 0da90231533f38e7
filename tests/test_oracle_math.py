"""Pins of the oracle's router, expert SwiGLU, combine, quantisers, grouping
and prefill (CPU only).

Each check compares the oracle with something other than itself: closed
forms, brute force over all subsets, numpy/scipy/torch library routines on
independently dequantised weights, integer-exact special cases, or hand cases.
"""
import itertools

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax


def rnd_block(fmt, H, I, rng, scale_range=None):
    G = 16 if fmt == "nvfp4" else 32
    n = 3 * H * I
    b = np.empty(n // 2 + n // G, np.uint8)
    b[: n // 2] = rng.integers(0, 256, n // 2)
    lo, hi = scale_range or ((0x18, 0x48) if fmt == "nvfp4" else (121, 129))
    b[n // 2:] = rng.integers(lo, hi + 1, n // G)
    return b


def np_expert(orc, fmt, H, I, block, x):
    """Independent reference: dequantise (pinned separately) then numpy fp64."""
    g, u, d = orc.dequant_block(fmt, H, I, block)
    g, u, d = g.astype(np.float64), u.astype(np.float64), d.astype(np.float64)
    a = g @ x
    h = a * expit(a) * (u @ x)
    return h, d @ h


# ---------------------------------------------------------------- router ---

def test_topk_brute_matches_sort_random_and_ties(orc):
    rng = np.random.default_rng(0)
    for E in range(1, 11):
        for k in range(1, E + 1):
            for trial in range(3):
                if trial == 0:
                    l = rng.normal(size=E)
                else:  # heavy ties
                    l = rng.integers(0, 3, size=E).astype(np.float64)
                b, n = orc.topk_brute(l, k)
                assert n == 1
                assert (b == orc.topk_sort(l, k)).all(), (E, k, l)


def test_topk_tie_rule_lower_index_first(orc):
    l = np.array([1.0, 5.0, 5.0, 2.0, 5.0, 0.0])
    assert list(orc.topk_sort(l, 4)) == [1, 2, 4, 3]
    assert list(orc.topk_brute(l, 4)[0]) == [1, 2, 4, 3]


def test_topk_vs_torch_on_distinct_logits(orc):
    rng = np.random.default_rng(3)
    l = rng.normal(size=512)
    ref = torch.topk(torch.tensor(l), 10).indices.numpy()
    assert (orc.topk_sort(l, 10) == ref).all()


def test_route_two_experts_closed_form(orc):
    """E = 2, k = 2: the top expert's weight is sigmoid(l_top - l_other)."""
    rng = np.random.default_rng(5)
    H = 8
    x = rng.normal(size=(4, H)).astype(np.float32)
    Wr = rng.normal(size=(2, H)).astype(np.float32)
    lg, idx, w = orc.route(x, Wr, 2)
    for t in range(4):
        a, b = idx[t]
        assert lg[t, a] >= lg[t, b]
        assert abs(w[t, 0] - expit(lg[t, a] - lg[t, b])) < 1e-15
        assert abs(w[t].sum() - 1.0) < 1e-15


def test_route_vs_numpy_scipy(orc):
    rng = np.random.default_rng(7)
    T, H, E, k = 5, 96, 24, 6
    x = rng.normal(size=(T, H)).astype(np.float32)
    Wr = (0.02 * rng.normal(size=(E, H))).astype(np.float32)
    lg, idx, w = orc.route(x, Wr, k)
    ref_l = x.astype(np.float64) @ Wr.astype(np.float64).T
    assert np.abs(lg - ref_l).max() <= 1e-12 * np.abs(ref_l).max()
    p = softmax(lg, axis=1)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        assert list(idx[t]) == order
        ref_w = p[t, order] / p[t, order].sum()
        assert np.abs(w[t] - ref_w).max() < 1e-14
    # softmax invariance: a constant added to every logit changes nothing
    p2 = softmax(lg + 3.0, axis=1)
    assert np.abs(p2 - p).max() < 1e-12


# ---------------------------------------------------------------- expert ---

def test_matvec_hand_case_272(orc):
    """A 1x16 NVFP4 row of codes 0x2 (1.0) with scale 0x40 (2.0) dotted with
    x = 1..16 gives 2 * 136 = 272. Built as row 0 of the gate matrix with
    every other row zero and up = 1.0 everywhere, so h[0] = silu(272) * sum(x)."""
    H, I = 16, 16
    q = orc.layout("nvfp4", H, I)
    b = np.zeros(q[6], np.uint8)
    b[q[3]:q[4]] = 0x40
    b[q[4]:q[5]] = 0x38
    b[q[5]:] = 0x38
    b[q[0]:q[0] + 8] = 0x22                  # gate row 0: 16 codes of 1.0
    b[q[1]:q[2]] = 0x22                      # up: all 1.0
    x = np.arange(1, 17, dtype=np.float64)
    h, y = orc.expert("nvfp4", H, I, b, x)
    g0 = 272.0
    assert h[0] == pytest.approx(g0 * expit(g0) * 136.0, rel=1e-15)
    assert (h[1:] == 0.0).all()              # silu(0) = 0


def test_swiglu_one_hot_closed_form(orc):
    """One-hot gate/up rows (code 2 = 1.0, scale 1.0): h_i = silu(x_a) * x_b;
    one-hot down rows pick h."""
    H, I = 32, 16
    q = orc.layout("nvfp4", H, I)
    b = np.zeros(q[6], np.uint8)
    b[q[3]:] = 0x38
    rng = np.random.default_rng(11)
    a_idx = rng.integers(0, H, I)
    b_idx = rng.integers(0, H, I)
    for i in range(I):
        for base, col in ((q[0], a_idx[i]), (q[1], b_idx[i])):
            byte = base + i * (H // 2) + col // 2
            b[byte] |= (2 << 4) if col % 2 else 2
    for r in range(H):                       # down[r][r % I] = 1
        col = r % I
        byte = q[2] + r * (I // 2) + col // 2
        b[byte] |= (2 << 4) if col % 2 else 2
    x = rng.normal(size=H)
    h, y = orc.expert("nvfp4", H, I, b, x)
    ref_h = x[a_idx] * expit(x[a_idx]) * x[b_idx]
    assert np.abs(h - ref_h).max() < 1e-15
    assert np.abs(y - ref_h[np.arange(H) % I]).max() < 1e-15


@pytest.mark.parametrize("fmt,H,I", [("nvfp4", 64, 48), ("mxfp4", 64, 96)])
def test_expert_vs_numpy(orc, fmt, H, I):
    rng = np.random.default_rng(13)
    b = rnd_block(fmt, H, I, rng)
    x = rng.normal(size=H)
    h, y = orc.expert(fmt, H, I, b, x)
    rh, ry = np_expert(orc, fmt, H, I, b, x)
    assert np.abs(h - rh).max() <= 1e-13 * np.abs(rh).max()
    assert np.abs(y - ry).max() <= 1e-13 * np.abs(ry).max()


def test_integer_exact_matvec(orc):
    """All scales 1.0 and small-integer x: every partial sum is an exact
    binary fraction, so the oracle's gate products equal numpy's exactly."""
    H, I = 128, 32
    q = orc.layout("nvfp4", H, I)
    rng = np.random.default_rng(17)
    b = np.empty(q[6], np.uint8)
    b[:q[3]] = rng.integers(0, 256, q[3])
    b[q[3]:] = 0x38
    x = rng.integers(-8, 9, H).astype(np.float64)
    g, u, d = orc.dequant_block("nvfp4", H, I, b)
    # gate with up = 1 is not separable from the oracle's SwiGLU, so compare
    # h against the closed form with exact g, u
    gg = g.astype(np.float64) @ x
    uu = u.astype(np.float64) @ x
    assert (gg == np.round(gg * 2) / 2).all()
    h, _ = orc.expert("nvfp4", H, I, b, x)
    assert np.abs(h - gg * expit(gg) * uu).max() <= 1e-13 * np.abs(h).max()


@pytest.mark.parametrize("fmt,H,I,k", [("nvfp4", 64, 32, 3), ("mxfp4", 64, 64, 2)])
def test_moe_decode_vs_numpy(orc, fmt, H, I, k):
    rng = np.random.default_rng(19)
    blocks = [rnd_block(fmt, H, I, rng) for _ in range(k)]
    x = rng.normal(size=H).astype(np.float32)
    w = rng.random(k)
    w /= w.sum()
    y, h = orc.moe_decode(fmt, H, I, x, blocks, w)
    ref = np.zeros(H)
    for j in range(k):
        rh, ry = np_expert(orc, fmt, H, I, blocks[j], x.astype(np.float64))
        ref += w[j] * ry
        assert np.abs(h[j] - rh).max() <= 1e-13 * np.abs(rh).max()
    assert np.abs(y - ref).max() <= 1e-13 * np.abs(ref).max()
    # threads do not change the result
    y4, _ = orc.moe_decode(fmt, H, I, x, blocks, w, nthreads=4)
    assert (y4 == y).all()


def test_moe_decode_shared_expert_vs_numpy(orc):
    rng = np.random.default_rng(23)
    H, I, k = 64, 32, 2
    blocks = [rnd_block("nvfp4", H, I, rng) for _ in range(k)]
    x = rng.normal(size=H).astype(np.float32)
    w = np.array([0.7, 0.3])
    mats = [torch.tensor(0.02 * rng.normal(size=s), dtype=torch.float32).to(torch.bfloat16)
            for s in ((I, H), (I, H), (H, I))]
    bits = [m.view(torch.int16).numpy().view(np.uint16) for m in mats]
    y, _ = orc.moe_decode("nvfp4", H, I, x, blocks, w, shared=bits)
    sg, su, sd = (m.to(torch.float64).numpy() for m in mats)
    xd = x.astype(np.float64)
    a = sg @ xd
    ref = sd @ (a * expit(a) * (su @ xd))
    for j in range(k):
        ref = ref + w[j] * np_expert(orc, "nvfp4", H, I, blocks[j], xd)[1]
    assert np.abs(y - ref).max() <= 1e-13 * np.abs(ref).max()


def test_must_break_controls(orc):
    """Nibble swap, shifted expert index and a scale off by one byte each
    move the output by more than 10% of its max."""
    rng = np.random.default_rng(29)
    H, I, k = 64, 32, 3
    E = 6
    blocks = [rnd_block("nvfp4", H, I, rng) for _ in range(E)]
    x = rng.normal(size=H).astype(np.float32)
    w = np.array([0.5, 0.3, 0.2])
    sel = [1, 3, 4]
    y, _ = orc.moe_decode("nvfp4", H, I, x, [blocks[e] for e in sel], w)
    m = np.abs(y).max()
    nc = 3 * H * I // 2
    sw = [b.copy() for b in blocks]
    for b in sw:
        b[:nc] = (b[:nc] >> 4) | (b[:nc] << 4)
    y1, _ = orc.moe_decode("nvfp4", H, I, x, [sw[e] for e in sel], w)
    y2, _ = orc.moe_decode("nvfp4", H, I, x, [blocks[e + 1] for e in sel], w)
    sh = [b.copy() for b in blocks]
    for b in sh:
        b[nc:] = np.roll(b[nc:], 1)
    y3, _ = orc.moe_decode("nvfp4", H, I, x, [sh[e] for e in sel], w)
    for yy in (y1, y2, y3):
        assert np.abs(yy - y).max() / m > 0.1


# ---------------------------------------------------------- quantisers ---

def test_bf16_rne_vs_torch(orc):
    rng = np.random.default_rng(31)
    v = np.concatenate([
        rng.normal(size=2000).astype(np.float32),
        (rng.normal(size=200) * 1e-39).astype(np.float32),          # subnormals
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.3895e38, 0.0, -0.0], np.float32),
    ])
    ref = torch.tensor(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_rne(v.astype(np.float64))
    assert (got == ref).all()
    rows = orc.quant_bf16_rows(v.reshape(1, -1))
    assert (rows.reshape(-1) == ref).all()


def test_bf16_rne_ties_hand(orc):
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0 (0x3F80)
    assert orc.bf16_rne([1.0 + 2 ** -8])[0] == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even -> 0x3F82
    assert orc.bf16_rne([1.0 + 3 * 2 ** -8])[0] == 0x3F82
    # just above the midpoint rounds up (fp64 input keeps the extra bit)
    assert orc.bf16_rne([1.0 + 2 ** -8 + 2 ** -40])[0] == 0x3F81


def test_mxfp4_hand_cases(orc):
    # amax = 6: X = 0, grid values unchanged
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    v = np.array(grid * 4)
    c, s = orc.mxfp4_quant(v)
    assert s == 127 and list(c[:8]) == list(range(8))
    # amax = 7: X = 0 and 7 saturates to 6
    c, s = orc.mxfp4_quant([7.0] + [1.0] * 31)
    assert s == 127 and c[0] == 7 and c[1] == 2
    # ties to even mantissa (X = 0 via a 6.0 anchor)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, code in ties.items():
        c, s = orc.mxfp4_quant([6.0, t, -t] + [0.0] * 29)
        assert s == 127 and c[1] == code and c[2] == code | 8, t
    # amax = 0.3: floor(log2 0.3) = -2 -> X = -4, 0.3 / 2^-4 = 4.8 -> 4 (code 6)
    c, s = orc.mxfp4_quant([0.3] + [0.0] * 31)
    assert s == 127 - 4 and c[0] == 6
    # all zero
    c, s = orc.mxfp4_quant([0.0] * 32)
    assert s == 0 and not c.any()
    # negative values rounding to zero keep the sign
    c, s = orc.mxfp4_quant([6.0, -0.1] + [0.0] * 30)
    assert c[1] == 8


def test_mxfp4_exact_on_representable_blocks(orc):
    """A block of grid values times 2^X with a code of exponent 2 (magnitude
    4 or 6) present converts to exactly those codes and X."""
    rng = np.random.default_rng(37)
    for _ in range(200):
        X = int(rng.integers(-20, 20))
        codes = rng.integers(0, 16, 32)
        codes[rng.integers(0, 32)] = rng.choice([6, 7, 14, 15])
        v = np.array([orc.e2m1(int(c)) for c in codes]) * 2.0 ** X
        c, s = orc.mxfp4_quant(v)
        assert s == X + 127
        assert ((c & 7) == (codes & 7)).all()
        nz = (codes & 7) != 0
        assert (c[nz] == codes[nz]).all()


def test_quant_mxfp4_rows_packing(orc):
    x = np.zeros((2, 64), np.float32)
    x[0, 0], x[0, 1] = 0.5 * 4, 1.0 * 4          # X = 0 anchor below
    x[0, 2] = 6.0 * 4
    x[1, 32] = -6.0
    p, s = orc.quant_mxfp4_rows(x)
    assert s[0, 0] == 129 and s[1, 1] == 127
    assert p[0, 0] == (1 | (2 << 4)) and p[0, 1] == 7
    assert p[1, 16] == 15


# ------------------------------------------------------------- grouping ---

def test_group_vs_numpy_stable_argsort(orc):
    rng = np.random.default_rng(41)
    for T, k, E in ((1, 1, 1), (7, 3, 5), (100, 10, 64), (33, 6, 384)):
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        count, off, perm = orc.group(idx, E)
        flat = idx.reshape(-1)
        assert (count == np.bincount(flat, minlength=E)).all()
        assert (off == np.concatenate([[0], np.cumsum(count)])).all()
        assert (perm == np.argsort(flat, kind="stable")).all()
        assert sorted(perm) == list(range(T * k))


# -------------------------------------------------------------- prefill ---

@pytest.mark.parametrize("fmt,H,I", [("nvfp4", 64, 32), ("mxfp4", 64, 64)])
def test_prefill_without_rounding_equals_decode(orc, fmt, H, I):
    rng = np.random.default_rng(43)
    E, k, T = 5, 2, 3
    blocks = np.stack([rnd_block(fmt, H, I, rng) for _ in range(E)])
    x = rng.normal(size=(T, H)).astype(np.float32)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    out = orc.moe_prefill(fmt, H, I, E, x, blocks, idx, w, act=0)
    for t in range(T):
        y, _ = orc.moe_decode(fmt, H, I, x[t], [blocks[e] for e in idx[t]], w[t].astype(np.float64))
        assert (out[t] == y).all()


def test_prefill_bf16_rounding_points_vs_numpy(orc):
    rng = np.random.default_rng(47)
    fmt, H, I, E, k, T = "nvfp4", 64, 32, 4, 2, 3
    blocks = np.stack([rnd_block(fmt, H, I, rng) for _ in range(E)])
    x = rng.normal(size=(T, H)).astype(np.float32)
    idx = np.array([[0, 1], [2, 0], [3, 2]], np.int32)
    w = np.array([[0.6, 0.4], [0.5, 0.5], [0.9, 0.1]], np.float32)
    out, hp, hq = orc.moe_prefill(fmt, H, I, E, x, blocks, idx, w, act=1, want_h=True)
    bf = lambda a: torch.tensor(a).to(torch.bfloat16).to(torch.float64).numpy()
    for t in range(T):
        xq = bf(x[t])                          # fp32 -> bf16 is exact-input rounding
        acc = np.zeros(H)
        for j in range(k):
            g, u, d = (m.astype(np.float64) for m in orc.dequant_block(fmt, H, I, blocks[idx[t, j]]))
            a = g @ xq
            h = a * expit(a) * (u @ xq)
            assert np.abs(hp[t, j] - h).max() <= 1e-13 * np.abs(h).max()
            hr = orc.bf16_value(orc.bf16_rne(hp[t, j]))
            assert (hq[t, j] == hr).all()
            acc += float(w[t, j]) * (d @ hq[t, j])
        assert np.abs(out[t] - acc).max() <= 1e-13 * np.abs(acc).max()


def test_prefill_mxfp4_rounding_points(orc):
    rng = np.random.default_rng(53)
    fmt, H, I, E, k, T = "mxfp4", 64, 64, 3, 2, 2
    blocks = np.stack([rnd_block(fmt, H, I, rng) for _ in range(E)])
    x = rng.normal(size=(T, H)).astype(np.float32)
    idx = np.array([[0, 2], [1, 0]], np.int32)
    w = np.array([[0.7, 0.3], [0.2, 0.8]], np.float32)
    out, hp, hq = orc.moe_prefill(fmt, H, I, E, x, blocks, idx, w, act=2, out_bf16=True, want_h=True)
    for t in range(T):
        p, s = orc.quant_mxfp4_rows(x[t:t + 1])
        codes = np.stack([p[0] & 15, p[0] >> 4], axis=1).reshape(-1)
        xq = np.array([orc.e2m1(int(c)) for c in codes]) * np.repeat([orc.ue8m0(int(b)) for b in s[0]], 32)
        acc = np.zeros(H)
        for j in range(k):
            g, u, d = (m.astype(np.float64) for m in orc.dequant_block(fmt, H, I, blocks[idx[t, j]]))
            a = g @ xq
            h = a * expit(a) * (u @ xq)
            assert np.abs(hp[t, j] - h).max() <= 1e-13 * np.abs(h).max()
            acc += float(w[t, j]) * (d @ hq[t, j])
            # h~ is on the MX grid of its blocks
            for b0 in range(0, I, 32):
                c2, s2 = orc.mxfp4_quant(hp[t, j, b0:b0 + 32])
                ref = np.array([orc.e2m1(int(c)) for c in c2]) * orc.ue8m0(s2)
                assert (hq[t, j, b0:b0 + 32] == ref).all()
        # bf16 out: round-to-nearest-even of the fp64 combine, bit for bit
        # (independent bit-level rounding), except within 1e-12 relative of a
        # bf16 midpoint, where numpy's summation order may round the other way
        from test_oracle_stages import bf16_rne_bits, near_bf16_midpoint
        ok = ~near_bf16_midpoint(acc, 1e-12)
        assert np.array_equal(out[t][ok], bf16_rne_bits(acc[ok]))
