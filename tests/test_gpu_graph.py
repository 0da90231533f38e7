"""The launch configuration bench.py times: calls captured in a HIP graph.

Each graph is replayed several times with the program's own eager work and
synchronisations between the replays, and every replay must equal the eager
result bit for bit (the kernels have no float atomics, and the library
records no memset into a graph). One decode layer of the captured graph is
also checked against the oracle.
"""
import hashlib

import numpy as np
import pytest
import torch

import synthgen as sg
from gpu_helpers import NTHREADS, bf16_bits, host_blocks, layer_blocks, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_scaled_fp4_route_amd as m
    return m


def capture(fn):
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            fn()
    torch.cuda.current_stream().wait_stream(cs)
    torch.cuda.synchronize()
    return g


def eager_noise():
    """Unrelated eager work between replays (allocations, kernels, a sync)."""
    a = torch.randn(1 << 20, device="cuda")
    (a * 2.0 + 1.0).sum().item()


def test_decode_layers_in_a_graph(m, orc):
    """Three full Qwen-shaped layers (512 NVFP4 experts + bf16 shared expert
    each) through moe_layer_decode, one workspace, as the bench's graph."""
    wl = sg.get("qwen_decode")
    L = 3
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    blocks = [layer_blocks(wl, l) for l in range(L)]
    ptrs = [m.expert_ptr_table(b) for b in blocks]
    Wr = [sg.router_weights(wl, l, device="cuda") for l in range(L)]
    shared = [[t.contiguous() for t in sg.shared_expert(wl, l, device="cuda")] for l in range(L)]
    xs = [sg.activations(wl, 9, l, T=1, device="cuda").view(-1) for l in range(L)]
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    ys = [torch.empty(wl.H, device="cuda") for _ in range(L)]
    idx = [torch.empty(wl.k, dtype=torch.int32, device="cuda") for _ in range(L)]
    w = [torch.empty(wl.k, device="cuda") for _ in range(L)]

    def run():
        for l in range(L):
            m.moe_layer_decode(d, xs[l], Wr[l], ptrs[l], shared[l], ys[l], idx[l], w[l], ws)

    run()
    torch.cuda.synchronize()
    ref_y = [y.clone() for y in ys]
    ref_i = [i.clone() for i in idx]
    ref_w = [v.clone() for v in w]
    g = capture(run)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        for i in idx:
            i.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(ys[l].view(torch.int32), ref_y[l].view(torch.int32)), (rep, l)
            assert torch.equal(idx[l], ref_i[l]) and torch.equal(w[l].view(torch.int32), ref_w[l].view(torch.int32))
        eager_noise()
    # the last layer of the replayed graph against the oracle
    l = L - 1
    _, oi, ow = orc.route(xs[l].cpu().numpy(), Wr[l].cpu().numpy(), wl.k)
    gi = idx[l].cpu().numpy()
    assert (gi == oi[0]).all()
    hb = host_blocks(blocks[l], gi)
    ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, xs[l].cpu().numpy(), [hb[int(e)] for e in gi], ow[0],
                            shared=[bf16_bits(s) for s in shared[l]], nthreads=NTHREADS)
    assert rel_err(ys[l].cpu().numpy(), ref) <= 1e-4


def test_48_layer_decode_graph_replays_identical(m, orc):
    """The benchmark's configuration: all 48 Qwen-shaped layers (512 NVFP4
    experts each, 63.3 GiB resident) + the bf16 shared experts through
    moe_layer_decode on one workspace, captured in one HIP graph. Five
    replays, with unrelated eager work between them, give identical outputs,
    routing and weights in every layer (a hash of all 48 layers' results per
    replay), equal to the eager run; the last layer matches the oracle.
    A race between layers that share the workspace would show up as a
    changed hash."""
    wl = sg.get("qwen_decode")
    L = wl.layers
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    blocks = torch.empty((L * wl.E, wl.block_bytes), dtype=torch.uint8, device="cuda")
    for l in range(L):
        sg.fill_layer_blocks(wl, l, blocks[l * wl.E:(l + 1) * wl.E])
    ptrs = [m.expert_ptr_table(blocks[l * wl.E:(l + 1) * wl.E]) for l in range(L)]
    Wr = [sg.router_weights(wl, l, device="cuda") for l in range(L)]
    shared = [[t.contiguous() for t in sg.shared_expert(wl, l, device="cuda")] for l in range(L)]
    xs = [sg.activations(wl, 21, l, T=1, device="cuda").view(-1) for l in range(L)]
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    ys = torch.empty((L, wl.H), device="cuda")
    idx = torch.empty((L, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, wl.k), device="cuda")

    def run():
        for l in range(L):
            m.moe_layer_decode(d, xs[l], Wr[l], ptrs[l], shared[l], ys[l], idx[l], w[l], ws)

    def digest():
        h = hashlib.sha256()
        for t in (ys, idx, w):
            h.update(t.cpu().numpy().tobytes())
        return h.hexdigest()

    try:
        run()
        torch.cuda.synchronize()
        eager = digest()
        g = capture(run)
        seen = []
        for rep in range(5):
            ys.fill_(float("nan"))
            idx.fill_(-1)
            w.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            seen.append(digest())
            eager_noise()
        print(f"48-layer graph: eager {eager[:16]}, replays {[s[:16] for s in seen]}")
        assert all(s == eager for s in seen), seen
        l = L - 1
        _, oi, ow = orc.route(xs[l].cpu().numpy(), Wr[l].cpu().numpy(), wl.k)
        gi = idx[l].cpu().numpy()
        assert (gi == oi[0]).all()
        hb = host_blocks(blocks[l * wl.E:(l + 1) * wl.E], gi)
        ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, xs[l].cpu().numpy(), [hb[int(e)] for e in gi], ow[0],
                                shared=[bf16_bits(s) for s in shared[l]], nthreads=NTHREADS)
        assert rel_err(ys[l].cpu().numpy(), ref) <= 1e-4
    finally:
        del blocks
        torch.cuda.empty_cache()


def test_fp8_kernels_in_a_graph(m, orc):
    rows, cols = 300, 4096
    x = sg.fp8_activations(rows, cols, 11, device="cuda")
    codes = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    W = sg.fp8_matrix(2560, 8192, 2, device="cuda")
    s = sg.fp8_row_scales(2560, 2, device="cuda")
    v = sg.fp8_vector(8192, 2, device="cuda")
    y = torch.empty(2560, device="cuda")

    def run():
        m.moe_act_quant_fp8(x, rows, cols, 32, m.MOE_SCALE_FLOOR, codes, scales)
        m.moe_gemv_fp8(W, s, v, 2560, 8192, y)

    run()
    torch.cuda.synchronize()
    rc, rs, ry = codes.clone(), scales.clone(), y.clone()
    g = capture(run)
    for rep in range(3):
        codes.fill_(0x7F)
        scales.fill_(0xFF)
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, rc) and torch.equal(scales, rs), rep
        assert torch.equal(y.view(torch.int32), ry.view(torch.int32)), rep
        eager_noise()
    oc, osc = orc.quant_fp8_rows(x.cpu().numpy(), block=32, rule=0)
    assert (codes.cpu().numpy() == oc).all() and (scales.cpu().numpy() == osc).all()
    assert rel_err(y.cpu().numpy(), orc.gemv_fp8(W.cpu().numpy(), s.cpu().numpy(), v.cpu().numpy())) <= 1e-4


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_prefill_in_a_graph(m, fmt):
    """moe_expert_prefill captured in a graph: the call's tile counters and
    tile list are rebuilt by its own first launch on every replay, so each
    replay equals the eager result bit for bit."""
    if fmt == "nvfp4":
        wl = sg.Workload("pf_graph", 95, 2560, 640, 64, 10, "nvfp4", 1, 300, False, "zipf", 1.1, 0x18, 0x48, False)
    else:
        wl = sg.Workload("pf_graph_mx", 96, 4096, 2880, 48, 6, "mxfp4", 1, 60, False, "zipf", 1.1, 121, 129, True)
    T = wl.T
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    blocks = layer_blocks(wl, 0)
    ptrs = m.expert_ptr_table(blocks)
    x = sg.activations(wl, 0, 0, T=T, device="cuda")
    idx, w = sg.routing(wl, T=T)
    idx, w = idx.cuda(), w.cuda()
    ws = m.alloc_workspace(d, T, m.MOE_MODE_PREFILL)
    od = m.MOE_OUT_BF16 if wl.out_bf16 else m.MOE_OUT_F32
    out = torch.empty((T, wl.H), dtype=torch.bfloat16 if wl.out_bf16 else torch.float32, device="cuda")
    view = torch.int16 if wl.out_bf16 else torch.int32

    def run():
        m.moe_expert_prefill(d, x, T, ptrs, idx, w, out, od, ws)

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    assert torch.isfinite(ref.float()).all()
    g = capture(run)
    for rep in range(3):
        out.fill_(float("nan"))
        ws.fill_(0xA5)  # the workspace carries nothing from one call to the next
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(view), ref.view(view)), rep
        eager_noise()
