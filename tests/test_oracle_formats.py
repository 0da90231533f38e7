"""Pins of the oracle's format decoders and block layout (CPU only).

The oracle's closed-form decoders are checked against things other than
themselves: the OCP MX table of E2M1 values (golden fixture), torch's own
float8_e4m3fn / float8_e8m0fnu decoders (library routines, exhaustive over
all 256 bytes), and the byte counts the pages print.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e2m1():
    vals = {}
    for line in open(os.path.join(GOLD, "e2m1_values.txt")):
        if line.startswith("#") or not line.strip():
            continue
        c, v = line.split()
        vals[int(c)] = float(v)
    return vals


def test_e2m1_matches_ocp_table(orc):
    g = _golden_e2m1()
    assert len(g) == 16
    for c in range(16):
        v = orc.e2m1(c)
        assert v == g[c], c
        assert math.copysign(1.0, v) == math.copysign(1.0, g[c]), c  # -0 for code 8


def test_e4m3_exhaustive_vs_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = orc.e4m3(b)
        if math.isnan(ref[b]):
            assert math.isnan(v), hex(b)
        else:
            assert v == ref[b], hex(b)
    # the worked values
    assert orc.e4m3(0x38) == 1.0 and orc.e4m3(0x18) == 2.0 ** -4
    assert orc.e4m3(0x48) == 4.0 and orc.e4m3(0x7E) == 448.0 and orc.e4m3(0x01) == 2.0 ** -9


def test_ue8m0_exhaustive_vs_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for b in range(256):
        v = orc.ue8m0(b)
        if math.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b], b
    assert orc.ue8m0(121) == 2.0 ** -6 and orc.ue8m0(129) == 4.0 and orc.ue8m0(127) == 1.0


def test_scaled_products_exact_in_fp32_and_bf16(orc):
    """Every e2m1 x E4M3 product (16 x 256) and every e2m1 x UE8M0 product
    with a scale up to 2^125 is representable in fp32 (and in bf16 in its
    normal range), so dequantised weights have one exact value. Scales of
    2^126 and 2^127 can overflow fp32 (6 x 2^127 > FLT_MAX)."""
    for c in range(16):
        for s in range(256):
            for scale in (orc.e4m3(s), orc.ue8m0(s) if s <= 252 else float("nan")):
                if math.isnan(scale):
                    continue
                p = orc.e2m1(c) * scale
                f32 = float(np.float32(p))
                assert f32 == p
                bf = torch.tensor([p], dtype=torch.float32).to(torch.bfloat16).to(torch.float64).item()
                if abs(p) >= 2.0 ** -126:  # bf16 normal range (all NVFP4 products are)
                    assert bf == p


def _page_counts():
    d = {}
    for line in open(os.path.join(GOLD, "page_byte_counts.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, val = [s.strip() for s in line.split("|")[:2]]
        d[name] = val
    return d


def test_layout_matches_page_byte_counts(orc):
    pc = _page_counts()
    q = orc.layout("nvfp4", 2560, 640)
    assert q[6] == int(pc["qwen_block_bytes"]) == 675 * 4096 == int(pc["qwen_block_pages"]) * 4096
    # order gate | up | down | gate_scale | up_scale | down_scale, increasing offsets
    assert q == sorted(q) and q[0] == 0
    assert q[1] - q[0] == q[2] - q[1] == q[3] - q[2] == 2560 * 640 // 2
    assert q[4] - q[3] == q[5] - q[4] == q[6] - q[5] == 2560 * 640 // 16
    L, E, k = (int(v) for v in pc["qwen_layers_experts_topk"].split("/"))
    assert round(L * k * q[6] / 1e9, 2) == float(pc["qwen_bytes_per_token_over_pcie"])
    d = orc.layout("mxfp4", 4096, 2880)
    assert round(d[6] / 2 ** 20, 2) == float(pc["deepseek_expert_mib"])
    assert round(d[3] / 1e6, 1) == float(pc["deepseek_codes_mb"])
    assert round((d[6] - d[3]) / 1e6, 1) == float(pc["deepseek_scales_mb"])
    L, E, k = (int(v) for v in pc["deepseek_layers_experts_topk"].split("/"))
    assert round(L * k * d[6] / 2 ** 30, 1) == float(pc["deepseek_gib_per_token"])


def test_layout_rejects_bad_shapes(orc):
    with pytest.raises(ValueError):
        orc.layout("nvfp4", 2560 + 8, 640)
    with pytest.raises(ValueError):
        orc.layout("mxfp4", 4096, 2880 + 16)


def _tiny_block(fmt, H, I, rng):
    G = 16 if fmt == "nvfp4" else 32
    n = 3 * H * I
    b = np.empty(n // 2 + n // G, np.uint8)
    b[: n // 2] = rng.integers(0, 256, n // 2)
    b[n // 2:] = rng.integers(0x18, 0x49, n // G) if fmt == "nvfp4" else rng.integers(121, 130, n // G)
    return b


def test_dequant_hand_case_nibble_order(orc):
    """Byte 0x21 holds element 0 = code 1 (0.5) in the low nibble and element 1
    = code 2 (1.0) in the high nibble; scale 0x38 = 1.0."""
    H, I = 32, 16
    q = orc.layout("nvfp4", H, I)
    b = np.zeros(q[6], np.uint8)
    b[q[3]:] = 0x38
    b[0] = 0x21
    g, u, d = orc.dequant_block("nvfp4", H, I, b)
    assert g[0, 0] == 0.5 and g[0, 1] == 1.0 and np.count_nonzero(g) == 2
    assert not u.any() and not d.any()
    # a scale byte on row 0, group 1 (columns 16..31) only touches that group
    b[q[0] + 8] = 0x77          # elements 16, 17 = codes 7, 7 = 6.0
    b[q[3] + 1] = 0x40          # scale 2.0
    g, _, _ = orc.dequant_block("nvfp4", H, I, b)
    assert g[0, 16] == 12.0 and g[0, 17] == 12.0 and g[0, 0] == 0.5


def test_dequant_mx_scale_groups(orc):
    H, I = 64, 64                              # down rows: 2 groups of 32
    q = orc.layout("mxfp4", H, I)
    b = np.zeros(q[6], np.uint8)
    b[q[0]:q[3]] = 0x22                       # every element code 2 = 1.0
    b[q[3]:] = 127
    b[q[5] + 3] = 129                         # down row 1, group 1 -> x4
    g, u, d = orc.dequant_block("mxfp4", H, I, b)
    assert (g == 1.0).all() and (u == 1.0).all()
    assert (d[1, :32] == 1.0).all() and (d[1, 32:] == 4.0).all() and (d[0] == 1.0).all()
    assert np.count_nonzero(d != 1.0) == 32


def test_dequant_must_break_on_nibble_swap(orc):
    rng = np.random.default_rng(1)
    b = _tiny_block("nvfp4", 64, 32, rng)
    g, _, _ = orc.dequant_block("nvfp4", 64, 32, b)
    sw = b.copy()
    n = 3 * 64 * 32 // 2
    sw[:n] = ((b[:n] >> 4) | (b[:n] << 4)).astype(np.uint8)
    g2, _, _ = orc.dequant_block("nvfp4", 64, 32, sw)
    assert np.abs(g2 - g).max() / np.abs(g).max() > 0.1
