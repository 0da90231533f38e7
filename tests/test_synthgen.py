"""The seeded generator: tensor path equals the scalar SplitMix64 definition,
draws are deterministic, and distributions/shapes are the workloads'."""
import numpy as np
import torch

import synthgen as sg


def test_words_match_scalar_splitmix64():
    key = 1234567
    st, ref = key, []
    for _ in range(64):
        st = (st + sg.GAMMA) & ((1 << 64) - 1)
        ref.append(sg.mix64_int(st))
    got = [int(v) & ((1 << 64) - 1) for v in sg.words(key, 64)]
    assert got == ref


def test_block_bytes_and_scale_ranges():
    for name in ("qwen_layer_decode", "deepseek_decode"):
        wl = sg.get(name)
        b = sg.expert_blocks(wl, 0, [0, 5])
        cb, sb = sg.block_region_sizes(wl)
        assert b.shape == (2, wl.block_bytes) and cb + sb == wl.block_bytes
        sc = b[:, cb:]
        assert int(sc.min()) == wl.scale_lo and int(sc.max()) == wl.scale_hi
        # all 16 nibble values appear, roughly uniformly
        nib = torch.cat([b[:, :cb] & 15, b[:, :cb] >> 4]).flatten().long()
        cnt = torch.bincount(nib, minlength=16).double()
        assert (cnt / cnt.mean() - 1).abs().max() < 0.02
        assert torch.equal(b, sg.expert_blocks(wl, 0, [0, 5]))  # deterministic


def test_routing_draws():
    wl = sg.get("qwen_prefill")
    idx, w = sg.routing(wl, T=300)
    assert idx.shape == (300, 10) and w.shape == (300, 10)
    for t in range(300):
        assert len(set(idx[t].tolist())) == 10
    assert torch.allclose(w.sum(1), torch.ones(300), atol=1e-6)
    cnt = torch.bincount(idx.view(-1).long(), minlength=512)
    assert cnt.max() > 10 * cnt.float().median()   # Zipf skew
    wl5 = sg.get("deepseek_prefill")
    i5, _ = sg.routing(wl5)
    assert i5.shape == (311, 6) and int(i5.max()) < 384


def test_normals():
    z = sg.normal(sg.stream_key(9), 100000).numpy().astype(np.float64)
    assert abs(z.mean()) < 0.02 and abs(z.std() - 1) < 0.02
