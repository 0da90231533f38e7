"""GPU parity of the decode path (router, FP4 GEMVs, combine) against the CPU
oracle, through the C ABI. Inputs come from the seeded generator; the oracle
gets host copies of the same inputs and never sees a GPU output.

Bars: dequantised weights bit-exact; top-k indices bit-exact where the
logits are exact (integer case) and otherwise equal up to oracle near-ties;
outputs max|d|/max|ref| <= 1e-4 (fp32 activations, fp32 accumulation against
fp64); reruns bit-identical.
"""
import numpy as np
import pytest
import torch

import synthgen as sg
from gpu_helpers import NTHREADS, bf16_bits, cosine, host_blocks, layer_blocks, rel_err, same_f32_bits

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_scaled_fp4_route_amd as m
    return m


def _dequant_gpu(m, d, block):
    H, I = d.H, d.I
    g = torch.empty((I, H), dtype=torch.float32, device="cuda")
    u = torch.empty((I, H), dtype=torch.float32, device="cuda")
    dn = torch.empty((H, I), dtype=torch.float32, device="cuda")
    m.moe_dequant_block(d, block, g, u, dn)
    torch.cuda.synchronize()
    return g.cpu().numpy(), u.cpu().numpy(), dn.cpu().numpy()


@pytest.mark.parametrize("name", ["qwen_layer_decode", "deepseek_decode"])
def test_dequant_bitexact_full_shape(m, orc, name):
    wl = sg.get(name)
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    blocks = layer_blocks(wl, 0, E=2)
    for e in range(2):
        got = _dequant_gpu(m, d, blocks[e])
        ref = orc.dequant_block(wl.fmt, wl.H, wl.I, blocks[e].cpu().numpy())
        for a, b in zip(got, ref):
            assert same_f32_bits(a, b)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_dequant_bitexact_every_code_scale_pair(m, orc, fmt):
    """Every group holds all 16 codes and the scale bytes cycle through all
    256 values (NaN scales, subnormal and overflowing products included)."""
    H = I = 256
    G = 16 if fmt == "nvfp4" else 32
    d = m.desc(H, I, 4, 1, fmt)
    nb = 3 * H * I // 2
    pattern = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8)
    codes = np.tile(pattern, nb // 8)
    scales = (np.arange(3 * H * I // G) % 256).astype(np.uint8)
    blk = np.concatenate([codes, scales])
    got = _dequant_gpu(m, d, torch.tensor(blk, device="cuda"))
    ref = orc.dequant_block(fmt, H, I, blk)
    for a, b in zip(got, ref):
        assert same_f32_bits(a, b)


def _decode_case(m, orc, wl, E, idx, w, x, blocks, shared=None):
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    ptrs = m.expert_ptr_table(blocks)
    y = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    idx_d = torch.tensor(idx, dtype=torch.int32, device="cuda")
    w_d = torch.tensor(w, dtype=torch.float32, device="cuda")
    m.moe_expert_decode(d, x, ptrs, idx_d, w_d, shared, y, ws)
    torch.cuda.synchronize()
    hb = host_blocks(blocks, idx)
    sh = None if shared is None else [bf16_bits(s) for s in shared]
    ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x.cpu().numpy(), [hb[int(e)] for e in idx],
                            np.asarray(w, np.float32).astype(np.float64), shared=sh, nthreads=NTHREADS)
    return y.cpu().numpy(), ref, (d, ws, ptrs, idx_d, w_d, y)


@pytest.mark.parametrize("name,E", [("qwen_layer_decode", 64), ("deepseek_decode", 24)])
def test_decode_parity_given_routing(m, orc, name, E):
    wl = sg.get(name)
    blocks = layer_blocks(wl, 0, E=E)
    for step in range(2):
        x = sg.activations(wl, step, 0, T=1, device="cuda").view(-1)
        idx, w = sg.decode_routing(sg.Workload(**{**wl.__dict__, "E": E}), 0, step)
        got, ref, _ = _decode_case(m, orc, wl, E, idx.numpy(), w.numpy(), x, blocks)
        err = rel_err(got, ref)
        print(f"{name} step {step}: max|d|/max|ref| = {err:.3e} cosine {cosine(got, ref):.9f}")
        assert err <= TOL


def test_decode_parity_shared_expert_full_layer(m, orc):
    """Qwen decode layer at full size: 512 resident experts, the bf16 shared
    expert, routing by moe_route on the device (no host sync between)."""
    wl = sg.get("qwen_decode")
    blocks = layer_blocks(wl, 0)
    Wr = sg.router_weights(wl, 0, device="cuda")
    shared = [t.to("cuda") for t in sg.shared_expert(wl, 0, device="cuda")]
    x = sg.activations(wl, 0, 0, T=1, device="cuda").view(-1)
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    wsr = m.alloc_workspace(d, 1, m.MOE_MODE_ROUTE)
    wsd = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    idx = torch.empty(wl.k, dtype=torch.int32, device="cuda")
    w = torch.empty(wl.k, dtype=torch.float32, device="cuda")
    y = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    ptrs = m.expert_ptr_table(blocks)
    m.moe_route(d, x, 1, Wr, idx, w, None, wsr)
    m.moe_expert_decode(d, x, ptrs, idx, w, shared, y, wsd)
    torch.cuda.synchronize()
    lg, oidx, ow = orc.route(x.cpu().numpy(), Wr.cpu().numpy(), wl.k)
    gi = idx.cpu().numpy()
    assert (gi == oidx[0]).all(), (gi, oidx[0])
    assert rel_err(w.cpu().numpy(), ow[0]) <= TOL
    hb = host_blocks(blocks, gi)
    ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x.cpu().numpy(), [hb[int(e)] for e in gi], ow[0],
                            shared=[bf16_bits(s) for s in shared], nthreads=NTHREADS)
    err = rel_err(y.cpu().numpy(), ref)
    print(f"qwen full layer + shared: max|d|/max|ref| = {err:.3e}")
    assert err <= TOL


def test_decode_deterministic_reruns(m, orc):
    wl = sg.get("qwen_layer_decode")
    blocks = layer_blocks(wl, 0, E=16)
    x = sg.activations(wl, 5, 0, T=1, device="cuda").view(-1)
    idx, w = sg.decode_routing(sg.Workload(**{**wl.__dict__, "E": 16}), 0, 5)
    _, _, (d, ws, ptrs, idx_d, w_d, y) = _decode_case(m, orc, wl, 16, idx.numpy(), w.numpy(), x, blocks)
    first = y.clone()
    for _ in range(5):
        m.moe_expert_decode(d, x, ptrs, idx_d, w_d, None, y, ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), first.view(torch.int32))


@pytest.mark.parametrize("fmt,H,I,E,k", [
    ("nvfp4", 512, 16, 3, 1),      # smallest shapes, one expert
    ("nvfp4", 512, 48, 4, 4),      # k = E
    ("mxfp4", 1024, 96, 5, 2),
    ("nvfp4", 4096, 4096, 2, 2),   # largest supported H and I
    ("mxfp4", 4096, 4096, 2, 1),
    ("nvfp4", 3072, 1040, 6, 3),   # down rows of 130 dwords: ragged lane coverage
    ("nvfp4", 512, 256, 40, 32),   # k = 32: sixteen routed pairs fill the down workgroup
    ("mxfp4", 512, 320, 9, 7),     # odd k: the last down pair holds one item
    # layers of >= 32 MB of gate/up codes without a shared expert take the
    # streaming kernels: one 1 KB chunk per lane and row, 1.5 chunks, 2 chunks
    ("mxfp4", 2048, 2048, 10, 8),
    ("nvfp4", 3072, 1536, 9, 8),
    # 65-96 chunks per down row: two rows share the load of their tails
    # (2 tail chunks, 26 as at I = 2880, a full 32)
    ("mxfp4", 2560, 2112, 8, 7),
    ("mxfp4", 2048, 2880, 9, 6),
    ("nvfp4", 2048, 3072, 8, 6),
])
def test_decode_edge_shapes(m, orc, fmt, H, I, E, k):
    wl = sg.Workload("edge", 90, H, I, E, k, fmt, 1, 1, False, "router", 0.0,
                     0x18 if fmt == "nvfp4" else 121, 0x48 if fmt == "nvfp4" else 129, False)
    blocks = layer_blocks(wl, 0)
    x = sg.activations(wl, 0, 0, T=1, device="cuda").view(-1)
    idx, w = sg.decode_routing(wl, 0, 0)
    got, ref, _ = _decode_case(m, orc, wl, E, idx.numpy(), w.numpy(), x, blocks)
    assert rel_err(got, ref) <= TOL


# ------------------------------------------------------------------ router ---

def _route_gpu(m, d, x, Wr, T, want_logits=True):
    idx = torch.empty((T, d.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, d.k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, d.E), dtype=torch.float32, device="cuda") if want_logits else None
    ws = m.alloc_workspace(d, T, m.MOE_MODE_ROUTE)
    m.moe_route(d, x, T, Wr, idx, w, lg, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), (lg.cpu().numpy() if want_logits else None)


@pytest.mark.parametrize("T", [1, 3, 16, 17, 40])
@pytest.mark.parametrize("name", ["qwen_layer_decode", "qwen_decode", "deepseek_decode"])
def test_route_parity(m, orc, name, T):
    wl = sg.get(name)
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    Wr = sg.router_weights(wl, 0, device="cuda")
    x = sg.activations(wl, 11, 0, T=T, device="cuda")
    gi, gw, gl = _route_gpu(m, d, x, Wr, T)
    ol, oi, ow = orc.route(x.cpu().numpy(), Wr.cpu().numpy(), wl.k)
    assert rel_err(gl, ol) <= TOL
    for t in range(T):
        if not (gi[t] == oi[t]).all():
            # only a near-tie in the oracle's own logits may reorder the choice
            diff = set(gi[t]) ^ set(oi[t])
            vals = ol[t, list(diff)] if diff else ol[t, gi[t]]
            assert np.ptp(vals) <= 1e-5 * np.abs(ol[t]).max(), (t, gi[t], oi[t])
        else:
            assert rel_err(gw[t], ow[t]) <= TOL


@pytest.mark.parametrize("T", [1, 5, 33])
def test_route_exact_logits_with_ties(m, orc, T):
    """Small-integer router weights and activations make every logit exact in
    fp32 in any summation order, and planted duplicates create ties, so the
    GPU's chosen indices must equal the oracle's sort-based top-k bit for bit
    (tie rule: lower expert index first)."""
    H, E, k = 512, 64, 10
    d = m.desc(H, 64, E, k, "nvfp4")
    g = torch.Generator().manual_seed(123)
    Wr = torch.randint(-3, 4, (E, H), generator=g).float()
    Wr[7] = Wr[3]
    Wr[40] = Wr[3]
    Wr[12] = Wr[50]
    x = torch.randint(-2, 3, (T, H), generator=g).float()
    gi, gw, gl = _route_gpu(m, d, x.cuda(), Wr.cuda(), T)
    ol, oi, ow = orc.route(x.numpy(), Wr.numpy(), k)
    assert (gl == ol).all()
    assert (gi == oi).all()
    assert rel_err(gw, ow) <= TOL


@pytest.mark.parametrize("T", [1, 17, 40])
@pytest.mark.parametrize("E,k", [(128, 10), (256, 8), (384, 6), (512, 10), (1024, 32)])
def test_topk_bitexact_from_gpu_logits(m, orc, E, k, T):
    """Given the GPU's own fp32 logits, the GPU's chosen experts equal the
    oracle's sort-based top-k bit for bit (lane counts of 2, 4, 6, 8 and 16
    logits per lane), and its weights match the softmax over those logits
    renormalised over the chosen k."""
    from scipy.special import softmax
    H = 2560 if E != 384 else 4096
    wl = sg.Workload("topk", 93, H, 640, E, k, "nvfp4", 1, 1, False, "router", 0.0, 0x18, 0x48, False)
    d = m.desc(H, 640, E, k, "nvfp4")
    Wr = sg.router_weights(wl, 0, device="cuda")
    x = sg.activations(wl, 3, 0, T=T, device="cuda")
    gi, gw, gl = _route_gpu(m, d, x, Wr, T)
    for t in range(T):
        l = gl[t].astype(np.float64)
        oi = orc.topk_sort(l, k)
        assert (gi[t] == oi).all(), (t, gi[t], oi)
        p = softmax(l)
        assert rel_err(gw[t], p[oi] / p[oi].sum()) <= TOL


@pytest.mark.parametrize("path", ["route", "layer"])
def test_exact_logits_with_ties_at_512_experts(m, orc, path):
    """512 experts (eight logits per lane, sort network + lane shifts) with
    integer router weights and activations: exact logits, planted duplicate
    rows across lanes and within one lane; moe_route and moe_layer_decode
    must both pick the oracle's experts bit for bit."""
    H, I, E, k = 2560, 640, 512, 10
    d = m.desc(H, I, E, k, "nvfp4")
    g = torch.Generator().manual_seed(512)
    Wr = torch.randint(-3, 4, (E, H), generator=g).float()
    x = torch.randint(-2, 3, (H,), generator=g).float()
    lg = (Wr @ x).numpy()
    top = int(np.argsort(-lg, kind="stable")[0])
    dups = [v for v in (3, 4, 5, 200, 201, 511) if v != top][:5]
    for dup in dups:                            # ties with the best row: same lane and other lanes
        Wr[dup] = Wr[top]
    Wr[100] = Wr[17]
    lx = (Wr @ x).numpy()
    if path == "route":
        gi, gw, gl = _route_gpu(m, d, x[None].cuda(), Wr.cuda(), 1)
        assert (gl[0] == orc.logits(x.numpy(), Wr.numpy())[0]).all()
        gi = gi[0]
    else:
        wl = sg.Workload("ties512", 94, H, I, E, k, "nvfp4", 1, 1, False, "router", 0.0, 0x18, 0x48, False)
        blocks = layer_blocks(wl, 0)
        ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
        y = torch.empty(H, dtype=torch.float32, device="cuda")
        idx = torch.empty(k, dtype=torch.int32, device="cuda")
        w = torch.empty(k, dtype=torch.float32, device="cuda")
        m.moe_layer_decode(d, x.cuda(), Wr.cuda(), m.expert_ptr_table(blocks), None, y, idx, w, ws)
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()
    _, oi, _ = orc.route(x.numpy()[None], Wr.numpy(), k)
    assert (gi == oi[0]).all(), (gi, oi[0])
    assert (lx[gi[:6]] == lx[top]).all()        # the planted ties are among the chosen


def test_one_workspace_across_layers_and_calls(m, orc):
    """Route and decode of several layers share one workspace (its reserved
    first 4096 bytes are never written); each layer matches the oracle."""
    wl = sg.get("qwen_decode")
    E = 48
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    n = max(m.moe_workspace_bytes(d, 1, m.MOE_MODE_ROUTE), m.moe_workspace_bytes(d, 1, m.MOE_MODE_DECODE))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for layer in range(3):
        blocks = layer_blocks(wl, layer, E=E)
        Wr = sg.router_weights(wl, layer, device="cuda")[:E].contiguous()
        shared = [t.contiguous() for t in sg.shared_expert(wl, layer, device="cuda")]
        x = sg.activations(wl, 2, layer, T=1, device="cuda").view(-1)
        idx = torch.empty(wl.k, dtype=torch.int32, device="cuda")
        w = torch.empty(wl.k, dtype=torch.float32, device="cuda")
        y = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        for _ in range(2):
            m.moe_route(d, x, 1, Wr, idx, w, None, ws)
            m.moe_expert_decode(d, x, m.expert_ptr_table(blocks), idx, w, shared, y, ws)
        torch.cuda.synchronize()
        assert not ws[:4096].any(), "reserved workspace bytes written"
        _, oi, ow = orc.route(x.cpu().numpy(), Wr.cpu().numpy(), wl.k)
        assert (idx.cpu().numpy() == oi[0]).all()
        hb = host_blocks(blocks, oi[0])
        ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x.cpu().numpy(), [hb[int(e)] for e in oi[0]], ow[0],
                                shared=[bf16_bits(s) for s in shared], nthreads=NTHREADS)
        assert rel_err(y.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("name", ["qwen_layer_decode", "deepseek_decode"])
def test_expert_index_out_of_range_poisons_output(m, name):
    """An expert index outside [0, E) is not dereferenced: the output turns
    NaN instead (the host cannot check device-resident indices). The
    DeepSeek shape runs the streaming kernels."""
    wl = sg.get(name)
    E = 12
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    blocks = layer_blocks(wl, 0, E=E)
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    x = sg.activations(wl, 0, 0, T=1, device="cuda").view(-1)
    idx = torch.tensor(list(range(wl.k - 1)) + [15], dtype=torch.int32, device="cuda")
    w = torch.full((wl.k,), 0.1, dtype=torch.float32, device="cuda")
    y = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    m.moe_expert_decode(d, x, m.expert_ptr_table(blocks), idx, w, None, y, ws)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()
    assert not ws[:4096].any()


# ----------------------------------------------------------- fused layer ---

def _layer_inputs(wl, E, layer, step, with_shared):
    blocks = layer_blocks(wl, layer, E=E)
    Wr = sg.router_weights(wl, layer, device="cuda")[:E].contiguous()
    shared = [t.contiguous() for t in sg.shared_expert(wl, layer, device="cuda")] if with_shared else None
    x = sg.activations(wl, step, layer, T=1, device="cuda").view(-1)
    return blocks, Wr, shared, x


@pytest.mark.parametrize("name,E,with_shared", [
    ("qwen_decode", 512, True),        # the full Qwen layer: 512 experts + shared expert
    ("qwen_layer_decode", 64, False),
    ("deepseek_decode", 384, False),   # the full DeepSeek layer
    ("deepseek_decode", 40, True),     # MXFP4 with a (synthetic) shared expert
])
def test_layer_decode_parity_and_equal_to_two_calls(m, orc, name, E, with_shared):
    """moe_layer_decode against the oracle (route, then the experts it chose),
    and bit for bit against moe_route followed by moe_expert_decode."""
    wl = sg.get(name)
    blocks, Wr, shared, x = _layer_inputs(wl, E, 0, 3, with_shared)
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    ptrs = m.expert_ptr_table(blocks)
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    y = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    idx = torch.full((wl.k,), -7, dtype=torch.int32, device="cuda")
    w = torch.full((wl.k,), -1.0, dtype=torch.float32, device="cuda")
    m.moe_layer_decode(d, x, Wr, ptrs, shared, y, idx, w, ws)
    # the two-call path on the same inputs
    wsr = m.alloc_workspace(d, 1, m.MOE_MODE_ROUTE)
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    y2 = torch.empty_like(y)
    m.moe_route(d, x, 1, Wr, idx2, w2, None, wsr)
    m.moe_expert_decode(d, x, ptrs, idx2, w2, shared, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    assert not ws[:4096].any(), "reserved workspace bytes written"

    _, oi, ow = orc.route(x.cpu().numpy(), Wr.cpu().numpy(), wl.k)
    gi = idx.cpu().numpy()
    assert (gi == oi[0]).all(), (gi, oi[0])
    assert rel_err(w.cpu().numpy(), ow[0]) <= TOL
    hb = host_blocks(blocks, gi)
    sh = None if shared is None else [bf16_bits(s) for s in shared]
    ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x.cpu().numpy(), [hb[int(e)] for e in gi], ow[0],
                            shared=sh, nthreads=NTHREADS)
    err = rel_err(y.cpu().numpy(), ref)
    print(f"{name} E={E} shared={with_shared}: max|d|/max|ref| = {err:.3e}")
    assert err <= TOL


def test_layer_decode_many_layers_one_workspace(m, orc):
    """Several layers enqueued back to back on one workspace with no host
    synchronisation between them (each with its own seeded input); every
    layer then matches the oracle and the reserved bytes stay untouched."""
    wl = sg.get("qwen_decode")
    E = 96
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    layers = [_layer_inputs(wl, E, layer, 4, True) for layer in range(4)]
    outs = []
    for blocks, Wr, shared, x in layers:
        y = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        idx = torch.empty(wl.k, dtype=torch.int32, device="cuda")
        w = torch.empty(wl.k, dtype=torch.float32, device="cuda")
        m.moe_layer_decode(d, x, Wr, m.expert_ptr_table(blocks), shared, y, idx, w, ws)
        outs.append((y, idx))
    torch.cuda.synchronize()
    assert not ws[:4096].any()
    for (blocks, Wr, shared, x), (y, idx) in zip(layers, outs):
        xin = x.cpu().numpy()
        _, oi, ow = orc.route(xin, Wr.cpu().numpy(), wl.k)
        gi = idx.cpu().numpy()
        assert (gi == oi[0]).all(), (gi, oi[0])
        hb = host_blocks(blocks, gi)
        ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, xin, [hb[int(e)] for e in gi], ow[0],
                                shared=[bf16_bits(s) for s in shared], nthreads=NTHREADS)
        assert rel_err(y.cpu().numpy(), ref) <= TOL


def test_layer_decode_exact_router_ties(m, orc):
    """Integer router weights with planted duplicate rows make the logits
    exact and tied; the fused top-k must pick the oracle's experts (lower
    index first among equals)."""
    H, I, E, k = 512, 64, 48, 6
    d = m.desc(H, I, E, k, "nvfp4")
    wl = sg.Workload("ties", 91, H, I, E, k, "nvfp4", 1, 1, False, "router", 0.0, 0x18, 0x48, False)
    blocks = layer_blocks(wl, 0)
    g = torch.Generator().manual_seed(7)
    Wr = torch.randint(-3, 4, (E, H), generator=g).float()
    Wr[9] = Wr[2]
    Wr[30] = Wr[2]
    Wr[17] = Wr[44]
    x = torch.randint(-2, 3, (H,), generator=g).float()
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    y = torch.empty(H, dtype=torch.float32, device="cuda")
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    w = torch.empty(k, dtype=torch.float32, device="cuda")
    m.moe_layer_decode(d, x.cuda(), Wr.cuda(), m.expert_ptr_table(blocks), None, y, idx, w, ws)
    torch.cuda.synchronize()
    _, oi, ow = orc.route(x.numpy()[None], Wr.numpy(), k)
    assert (idx.cpu().numpy() == oi[0]).all()
    hb = host_blocks(blocks, oi[0])
    ref, _ = orc.moe_decode("nvfp4", H, I, x.numpy(), [hb[int(e)] for e in oi[0]], ow[0], nthreads=NTHREADS)
    assert rel_err(y.cpu().numpy(), ref) <= TOL


def test_workspace_contents_do_not_matter(m):
    """The workspace needs no initialisation: a workspace full of junk gives
    bit-identical results to a zero-filled one (both entry points)."""
    wl = sg.get("qwen_decode")
    E = 64
    blocks, Wr, shared, x = _layer_inputs(wl, E, 1, 6, True)
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    ptrs = m.expert_ptr_table(blocks)
    outs = []
    for fill in (0x00, 0xFF, 0x7F):
        ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
        ws.fill_(fill)
        y = torch.empty(wl.H, dtype=torch.float32, device="cuda")
        y2 = torch.empty_like(y)
        idx = torch.empty(wl.k, dtype=torch.int32, device="cuda")
        w = torch.empty(wl.k, dtype=torch.float32, device="cuda")
        m.moe_layer_decode(d, x, Wr, ptrs, shared, y, idx, w, ws)
        ws.fill_(fill)
        m.moe_expert_decode(d, x, ptrs, idx, w, shared, y2, ws)
        torch.cuda.synchronize()
        outs.append((y.view(torch.int32).clone(), y2.view(torch.int32).clone(), idx.clone()))
    for o in outs[1:]:
        assert all(torch.equal(p, q) for p, q in zip(o, outs[0]))
    assert torch.equal(outs[0][0], outs[0][1])


@pytest.mark.parametrize("k", [31, 32])
def test_layer_decode_large_k_with_shared(m, orc, k):
    """k routed experts plus the shared expert: more down units than one
    workgroup's waves, so the down launch loops waves over single items."""
    wl = sg.Workload("largek", 92, 1024, 256, 48, k, "nvfp4", 1, 1, True, "router", 0.0, 0x18, 0x48, False)
    blocks, Wr, shared, x = _layer_inputs(wl, wl.E, 0, 0, True)
    d = m.desc(wl.H, wl.I, wl.E, k, wl.fmt)
    ptrs = m.expert_ptr_table(blocks)
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    y = torch.empty(wl.H, dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y)
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    w = torch.empty(k, dtype=torch.float32, device="cuda")
    m.moe_layer_decode(d, x, Wr, ptrs, shared, y, idx, w, ws)
    m.moe_expert_decode(d, x, ptrs, idx, w, shared, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    _, oi, ow = orc.route(x.cpu().numpy(), Wr.cpu().numpy(), k)
    gi = idx.cpu().numpy()
    assert (gi == oi[0]).all()
    hb = host_blocks(blocks, gi)
    ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x.cpu().numpy(), [hb[int(e)] for e in gi], ow[0],
                            shared=[bf16_bits(s) for s in shared], nthreads=NTHREADS)
    assert rel_err(y.cpu().numpy(), ref) <= TOL
