"""Controls on the GPU path that must break ([Q] "How we know it's right":
swapped nibbles and removed experts are checks that have to fail), and the
scale codes at the ends of the UE8M0 range.

Must-break: the GPU kernels run on deliberately corrupted device copies of the
expert blocks (nibbles of every code byte swapped; the expert pointer table
shifted by one expert; every block's scale bytes rolled by one position)
while the oracle runs on the intact blocks. The comparison that passes on
intact blocks (max|d|/max|ref| <= 1e-4) must then fail by a wide margin
(> 0.1), for decode (the one-shot and the streaming kernels) and for prefill
(both formats).

Scale bytes: UE8M0 byte 0 is 2^-127 and byte 0xFF is NaN ([OCP-MX] E8M0).
The decode kernels must give what the oracle gives: rows whose only scales
are 2^-127 keep their (tiny, normal-range) values; a NaN scale in a down row
makes exactly that output row NaN.
"""
import numpy as np
import pytest
import torch

import synthgen as sg
from gpu_helpers import NTHREADS, host_blocks, layer_blocks, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-4
BREAK = 0.1


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_scaled_fp4_route_amd as m
    return m


def swap_nibbles(blocks, H, I):
    b = blocks.clone()
    n = 3 * H * I // 2
    c = b[:, :n].to(torch.int32)
    b[:, :n] = (((c >> 4) | (c << 4)) & 0xFF).to(torch.uint8)
    return b


def roll_scales(blocks, H, I):
    b = blocks.clone()
    n = 3 * H * I // 2
    b[:, n:] = torch.roll(blocks[:, n:], 1, dims=1)
    return b


def shifted_table(m, blocks):
    E = blocks.shape[0]
    return m.expert_ptr_table([blocks[(e + 1) % E] for e in range(E)])


def corruptions(m, blocks, H, I):
    yield "nibble swap", swap_nibbles(blocks, H, I), None
    yield "scales rolled one byte", roll_scales(blocks, H, I), None
    yield "index shifted by one", blocks, shifted_table(m, blocks)


@pytest.mark.parametrize("name,E", [("qwen_layer_decode", 16), ("deepseek_decode", 12)])
def test_decode_must_break(m, orc, name, E):
    wl = sg.get(name)
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    blocks = layer_blocks(wl, 0, E=E)
    x = sg.activations(wl, 0, 0, T=1, device="cuda").view(-1)
    idx, w = sg.decode_routing(sg.Workload(**{**wl.__dict__, "E": E}), 0, 0)
    idx_d = idx.to(torch.int32).cuda()
    w_d = w.float().cuda()
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    hb = host_blocks(blocks, idx.numpy())
    ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x.cpu().numpy(), [hb[int(e)] for e in idx.numpy()],
                            w.numpy().astype(np.float64), nthreads=NTHREADS)
    y = torch.empty(wl.H, device="cuda")

    def run(bl, table):
        m.moe_expert_decode(d, x, table if table is not None else m.expert_ptr_table(bl), idx_d, w_d, None, y, ws)
        torch.cuda.synchronize()
        return y.cpu().numpy()

    assert rel_err(run(blocks, None), ref) <= TOL
    for what, bl, table in corruptions(m, blocks, wl.H, wl.I):
        err = rel_err(run(bl, table), ref)
        print(f"{name} decode, {what}: max|d|/max|ref| = {err:.3f}")
        assert err > BREAK, what


@pytest.mark.parametrize("fmt,H,I,E,k,T", [("nvfp4", 512, 128, 8, 2, 40), ("mxfp4", 512, 64, 8, 2, 40)])
def test_prefill_must_break(m, orc, fmt, H, I, E, k, T):
    lo, hi = (0x18, 0x48) if fmt == "nvfp4" else (121, 129)
    wl = sg.Workload("mb_pf", 97, H, I, E, k, fmt, 1, T, False, "zipf", 1.1, lo, hi, False)
    d = m.desc(H, I, E, k, fmt)
    blocks = layer_blocks(wl, 0)
    x = sg.activations(wl, 0, 0, T=T, device="cuda")
    idx, w = sg.routing(wl, T=T)
    ws = m.alloc_workspace(d, T, m.MOE_MODE_PREFILL)
    out = torch.empty((T, H), device="cuda")
    act = 1 if fmt == "nvfp4" else 2
    ref = orc.moe_prefill(fmt, H, I, E, x.cpu().numpy(), host_blocks(blocks, idx.numpy().ravel()), idx.numpy(),
                          w.numpy(), act=act, nthreads=NTHREADS)

    def run(bl, table):
        m.moe_expert_prefill(d, x, T, table if table is not None else m.expert_ptr_table(bl), idx.cuda(), w.cuda(),
                             out, m.MOE_OUT_F32, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    assert rel_err(run(blocks, None), ref) <= 2e-3  # end to end, h~ rounding flips included
    for what, bl, table in corruptions(m, blocks, H, I):
        err = rel_err(run(bl, table), ref)
        print(f"prefill {fmt}, {what}: max|d|/max|ref| = {err:.3f}")
        assert err > BREAK, what


@pytest.mark.parametrize("H,I,E,k", [
    (4096, 2880, 12, 6),   # the DeepSeek shape: streaming kernels
    (1024, 96, 6, 2),      # a small layer: one-shot kernels
])
def test_decode_ue8m0_scale_bytes_0_and_ff(m, orc, H, I, E, k):
    wl = sg.Workload("ue8m0_ends", 98, H, I, E, k, "mxfp4", 1, 1, False, "router", 0.0, 121, 129, False)
    d = m.desc(H, I, E, k, "mxfp4")
    blocks = layer_blocks(wl, 0)
    lay = orc.layout("mxfp4", H, I)
    hb = blocks.cpu().numpy()
    rng = np.random.default_rng(99)
    KS_gu, KS_d = H // 32, I // 32
    for e in range(E):
        b = hb[e]
        # gate/up: a few scattered groups at 2^-127
        gs = b[lay[3]:lay[5]]
        gs[rng.integers(0, gs.size, 40)] = 0
        ds = b[lay[5]:lay[6]].reshape(H, KS_d)
        ds[rng.integers(0, H, 30), rng.integers(0, KS_d, 30)] = 0
        ds[7, :] = 0                # down row 7: every scale 2^-127, in every expert
        ds[100 + 3 * e, 1] = 0xFF   # a NaN scale: that output row is NaN
    blocks.copy_(torch.from_numpy(hb))
    x = sg.activations(wl, 0, 0, T=1, device="cuda").view(-1)
    idx = torch.arange(k, dtype=torch.int32, device="cuda") * 2 % E
    w = torch.softmax(torch.linspace(-1, 1, k, device="cuda"), 0)
    y = torch.empty(H, device="cuda")
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    m.moe_expert_decode(d, x, m.expert_ptr_table(blocks), idx, w, None, y, ws)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    ref, _ = orc.moe_decode("mxfp4", H, I, x.cpu().numpy(), [hb[int(e)] for e in gi],
                            w.cpu().numpy().astype(np.float64), nthreads=NTHREADS)
    got = y.cpu().numpy()
    nan_ref = np.isnan(ref)
    assert nan_ref.sum() == k
    assert np.array_equal(np.isnan(got), nan_ref)
    fin = ~nan_ref
    assert rel_err(got[fin], ref[fin]) <= TOL
    # the row whose down scales are all 2^-127: tiny but not flushed, to 1e-4 of itself
    assert 0 < abs(ref[7]) < 1e-30
    assert abs(got[7] - ref[7]) <= TOL * abs(ref[7]), (got[7], ref[7])
