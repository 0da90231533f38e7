"""Speculative expert prefetch through the C ABI: the kernel's only output is
an XOR checksum of every 64 KiB chunk of each guessed expert's block, which
must equal numpy's XOR of the same words (so every byte was read); skipped
indices give zeros. A decode layer running next to a prefetch on a second
stream is bit-identical to one running alone, and both match the oracle."""
import numpy as np
import pytest
import torch

import synthgen as sg
from gpu_helpers import NTHREADS, host_blocks, layer_blocks, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_scaled_fp4_route_amd as m
    return m


def chunk_xor(block: np.ndarray) -> np.ndarray:
    w = block.view(np.uint32)
    n = -(-w.size // 16384)
    pad = np.zeros(n * 16384, np.uint32)
    pad[:w.size] = w
    return np.bitwise_xor.reduce(pad.reshape(n, 16384), axis=1)


@pytest.mark.parametrize("name,E", [("qwen_layer_decode", 24), ("deepseek_decode", 6)])
def test_prefetch_checksums(m, name, E):
    wl = sg.get(name)
    blocks = layer_blocks(wl, 0, E=E)
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    ptrs = m.expert_ptr_table(blocks)
    idx_h = np.array([3, E - 1, -1, 0, E, 2][:min(6, wl.k + 2)], np.int32)
    idx = torch.from_numpy(idx_h).cuda()
    n = len(idx_h)
    sink = torch.full((m.moe_prefetch_sink_bytes(d, n) // 4,), 0xABCD, dtype=torch.int32, device="cuda")
    m.moe_expert_prefetch(d, ptrs, idx, n, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(n, -1)
    hb = blocks.cpu().numpy()
    for j, e in enumerate(idx_h):
        want = chunk_xor(hb[e]) if 0 <= e < E else np.zeros(got.shape[1], np.uint32)
        assert (got[j] == want).all(), (j, e)


def test_prefetch_beside_decode_changes_nothing(m, orc):
    wl = sg.get("qwen_layer_decode")
    E = 64
    blocks = layer_blocks(wl, 0, E=E)
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    ptrs = m.expert_ptr_table(blocks)
    Wr = sg.router_weights(wl, 0, device="cuda")[:E].contiguous()
    x = sg.activations(wl, 5, 0, T=1, device="cuda").view(-1)
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    y0, y1 = torch.empty(wl.H, device="cuda"), torch.empty(wl.H, device="cuda")
    i0, i1 = torch.empty(wl.k, dtype=torch.int32, device="cuda"), torch.empty(wl.k, dtype=torch.int32, device="cuda")
    w0, w1 = torch.empty(wl.k, device="cuda"), torch.empty(wl.k, device="cuda")
    m.moe_layer_decode(d, x, Wr, ptrs, None, y0, i0, w0, ws)
    torch.cuda.synchronize()
    guess = torch.arange(wl.k, dtype=torch.int32, device="cuda")
    sink = torch.empty(m.moe_prefetch_sink_bytes(d, wl.k) // 4, dtype=torch.int32, device="cuda")
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    m.moe_expert_prefetch(d, ptrs, guess, wl.k, sink, stream=s2)
    m.moe_layer_decode(d, x, Wr, ptrs, None, y1, i1, w1, ws)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(y0.view(torch.int32), y1.view(torch.int32))
    # the decode that ran beside the prefetch against the oracle
    _, oi, ow = orc.route(x.cpu().numpy(), Wr.cpu().numpy(), wl.k)
    gi = i1.cpu().numpy()
    assert (gi == oi[0]).all()
    hb = host_blocks(blocks, gi)
    ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x.cpu().numpy(), [hb[int(e)] for e in gi], ow[0], nthreads=NTHREADS)
    assert rel_err(y1.cpu().numpy(), ref) <= 1e-4
