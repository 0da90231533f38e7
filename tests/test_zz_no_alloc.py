"""moe_layer_decode_noalloc (the decode layer with the library's static
scratch as its workspace) against moe_layer_decode with a caller workspace,
through the C ABI: two calls in a row, the second on a smaller layer, each
bit-identical to the workspace entry point (itself checked against the
oracle), and the first also against the oracle."""
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


def _layer(m, wl, E, with_shared, step):
    blocks = layer_blocks(wl, 0, E=E)
    Wr = sg.router_weights(wl, 0, device="cuda")[:E].contiguous()
    shared = [t.contiguous() for t in sg.shared_expert(wl, 0, device="cuda")] if with_shared else None
    x = sg.activations(wl, step, 0, T=1, device="cuda").view(-1)
    return blocks, Wr, shared, x


def _both(m, wl, E, blocks, Wr, shared, x):
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    ptrs = m.expert_ptr_table(blocks)
    outs = []
    for noalloc in (True, False):
        y = torch.full((wl.H,), float("nan"), device="cuda")
        idx = torch.full((wl.k,), -1, dtype=torch.int32, device="cuda")
        w = torch.full((wl.k,), float("nan"), device="cuda")
        if noalloc:
            m.moe_layer_decode_noalloc(d, x, Wr, ptrs, shared, y, idx, w)
        else:
            m.moe_layer_decode(d, x, Wr, ptrs, shared, y, idx, w, m.alloc_workspace(d, 1, m.MOE_MODE_DECODE))
        torch.cuda.synchronize()
        outs.append((y, idx, w))
    (y0, i0, w0), (y1, i1, w1) = outs
    assert torch.equal(i0, i1)
    assert torch.equal(w0.view(torch.int32), w1.view(torch.int32))
    assert torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    return y0, i0, w0


def test_noalloc_decode_two_calls_second_smaller(m, orc):
    # call 1: the full Qwen-shaped layer (512 NVFP4 experts + bf16 shared expert)
    wl = sg.get("qwen_decode")
    blocks, Wr, shared, x = _layer(m, wl, wl.E, True, 3)
    y, idx, w = _both(m, wl, wl.E, blocks, Wr, shared, x)
    _, oi, ow = orc.route(x.cpu().numpy(), Wr.cpu().numpy(), wl.k)
    gi = idx.cpu().numpy()
    assert (gi == oi[0]).all()
    hb = host_blocks(blocks, gi)
    ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x.cpu().numpy(), [hb[int(e)] for e in gi], ow[0],
                            shared=[bf16_bits(s) for s in shared], nthreads=NTHREADS)
    assert rel_err(y.cpu().numpy(), ref) <= 1e-4
    # call 2, right after: a smaller layer (64 experts, k = 6, no shared expert)
    wl2 = sg.Workload("noalloc_small", 99, 1024, 256, 64, 6, "nvfp4", 1, 1, False, "router", 0.0, 0x18, 0x48, False)
    blocks2, Wr2, _, x2 = _layer(m, wl2, wl2.E, False, 4)
    _both(m, wl2, wl2.E, blocks2, Wr2, None, x2)
