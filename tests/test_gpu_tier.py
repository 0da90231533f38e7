"""The expert tier ([Q] "The engine", items 2-3): pinned host blocks, an HBM
slot cache, and the per-layer pointer tables the decode kernels read.

* Decode with every expert read in place from pinned host memory equals the
  decode of HBM-resident blocks bit for bit (same kernels, same data).
* Over several decode steps with promotions and evictions (fewer slots than
  experts per step), every step's output stays bit-identical to the
  HBM-resident decode; afterwards every table entry points at its slot or at
  its host block, and every slot holds its expert's block.
* A hand-worked routing sequence checks the LRU choice of victims.
* Several decode steps and tier updates enqueued back to back with no host
  synchronisation between them (so slots are overwritten while kernels that
  read the old entries may still be queued) stay bit-identical to the
  HBM-resident decode, step by step; tier decode matches the oracle.
"""
import numpy as np
import pytest
import torch

import synthgen as sg
from gpu_helpers import NTHREADS, bf16_bits, host_blocks, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_scaled_fp4_route_amd as m
    return m


def make_tier(m, wl, E, L, n_slots, with_shared):
    d = m.desc(wl.H, wl.I, E, wl.k, wl.fmt)
    bb = wl.block_bytes
    dev = torch.empty((L * E, bb), dtype=torch.uint8, device="cuda")
    for l in range(L):
        sg.fill_layer_blocks(wl, l, dev[l * E:(l + 1) * E])
    host = torch.empty((L * E, bb), dtype=torch.uint8, pin_memory=True)
    host.copy_(dev)
    slots = torch.empty((max(n_slots, 1), bb), dtype=torch.uint8, device="cuda") if n_slots else None
    table = torch.empty(L * E, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    tier = m.ExpertTier(d, L, host, slots, n_slots, table)
    Wr = [sg.router_weights(wl, l, device="cuda")[:E].contiguous() for l in range(L)]
    shared = ([[t.contiguous() for t in sg.shared_expert(wl, l, device="cuda")] for l in range(L)]
              if with_shared else [None] * L)
    ref_ptrs = [m.expert_ptr_table(dev[l * E:(l + 1) * E]) for l in range(L)]
    return d, tier, dev, host, slots, table, Wr, shared, ref_ptrs


def decode_both(m, wl, d, tier, Wr, shared, ref_ptrs, L, step):
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    ws2 = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    ys, refs, idxs = [], [], []
    for l in range(L):
        x = sg.activations(wl, step, l, T=1, device="cuda").view(-1)
        y = torch.empty(wl.H, device="cuda")
        idx = torch.empty(wl.k, dtype=torch.int32, device="cuda")
        w = torch.empty(wl.k, device="cuda")
        m.moe_layer_decode(d, x, Wr[l], tier.table(l), shared[l], y, idx, w, ws)
        y2 = torch.empty(wl.H, device="cuda")
        idx2 = torch.empty_like(idx)
        w2 = torch.empty_like(w)
        m.moe_layer_decode(d, x, Wr[l], ref_ptrs[l], shared[l], y2, idx2, w2, ws2)
        ys.append(y), refs.append(y2), idxs.append((idx, idx2))
    torch.cuda.synchronize()
    for l in range(L):
        assert torch.equal(idxs[l][0], idxs[l][1])
        assert torch.equal(ys[l].view(torch.int32), refs[l].view(torch.int32)), (step, l)
    return np.stack([i[0].cpu().numpy() for i in idxs])


def test_zero_copy_decode_from_pinned_host(m):
    wl = sg.get("qwen_layer_decode")
    L, E = 2, 64
    d, tier, dev, host, slots, table, Wr, shared, ref_ptrs = make_tier(m, wl, E, L, 0, True)
    try:
        tab = table.cpu().numpy()
        assert (tab == host.data_ptr() + np.arange(L * E) * wl.block_bytes).all()
        decode_both(m, wl, d, tier, Wr, shared, ref_ptrs, L, 0)
    finally:
        tier.close()


def test_promotions_evictions_stay_bit_exact(m):
    wl = sg.get("qwen_layer_decode")
    L, E, n_slots = 2, 64, 12
    d, tier, dev, host, slots, table, Wr, shared, ref_ptrs = make_tier(m, wl, E, L, n_slots, False)
    try:
        steps = 6
        for step in range(steps):
            idx = decode_both(m, wl, d, tier, Wr, shared, ref_ptrs, L, step)
            tier.update(idx, 8)
        tier.update(np.full((L, wl.k), -1, np.int32), 0)  # commits the last newcomers
        torch.cuda.synchronize()
        decode_both(m, wl, d, tier, Wr, shared, ref_ptrs, L, steps)
        st = tier.stats()
        assert st["hits"] + st["misses"] == steps * L * wl.k
        assert st["pending"] == 0 and 0 < st["resident"] <= n_slots
        assert st["promotions"] - st["evictions"] == st["resident"]
        tab = table.cpu().numpy()
        sl = slots.cpu().numpy()
        hb = host.numpy()
        seen = 0
        for l in range(L):
            for e in range(E):
                key = l * E + e
                s = tier.slot_of(l, e)
                if s >= 0:
                    seen += 1
                    assert tab[key] == slots.data_ptr() + s * wl.block_bytes
                    assert (sl[s] == hb[key]).all()
                else:
                    assert tab[key] == host.data_ptr() + key * wl.block_bytes
        assert seen == st["resident"]
    finally:
        tier.close()


def test_lru_victims_hand_worked(m):
    """One layer, k = 2, three slots. Step 1 routes {0, 1}: both take free
    slots (0 and 1) and start copying. Step 2 routes {2, 3}: 0 and 1 become
    resident, 2 takes the free slot 2, 3 evicts the least recently used of
    {0, 1} (equally old: the lower slot, expert 0). Step 3 routes {1, 4}: 2
    and 3 become resident, 1 is a hit, 4 evicts the least recently used
    expert this step does not use: 2 and 3 are equally old, so the lower slot
    (expert 3, in slot 0)."""
    wl = sg.get("qwen_layer_decode")
    d, tier, dev, host, slots, table, Wr, shared, ref_ptrs = make_tier(
        m, sg.Workload(**{**wl.__dict__, "k": 2, "E": 8}), 8, 1, 3, False)
    try:
        tier.update(np.array([[0, 1]], np.int32), 8)
        st = tier.stats()
        assert st["pending"] == 2 and st["resident"] == 0 and tier.slot_of(0, 0) == -1
        tier.update(np.array([[2, 3]], np.int32), 8)
        st = tier.stats()
        assert tier.slot_of(0, 0) == -1 and tier.slot_of(0, 1) == 1  # 0 evicted, 1 resident
        assert st["evictions"] == 1 and st["pending"] == 2 and st["promotions"] == 4
        tier.update(np.array([[1, 4]], np.int32), 8)
        st = tier.stats()
        assert st["hits"] == 1 and st["misses"] == 5 and st["promotions"] == 5 and st["evictions"] == 2
        assert tier.slot_of(0, 1) == 1 and tier.slot_of(0, 2) == 2 and tier.slot_of(0, 3) == -1
        assert tier.slot_of(0, 4) == -1 and st["pending"] == 1
        tier.update(np.full((1, 2), -1, np.int32), 8)  # commits 4
        assert tier.slot_of(0, 4) == 0
        torch.cuda.synchronize()
        tab = table.cpu().numpy()
        sl = slots.cpu().numpy()
        for e in range(8):
            s = tier.slot_of(0, e)
            want = slots.data_ptr() + s * wl.block_bytes if s >= 0 else host.data_ptr() + e * wl.block_bytes
            assert tab[e] == want, e
            if s >= 0:
                assert (sl[s] == host.numpy()[e]).all(), e
    finally:
        tier.close()


def test_tier_steps_without_host_sync(m, orc):
    """Eight steps of two layers, each followed by a tier update, all
    enqueued on one stream with no host synchronisation between them: the
    routing each update receives was computed beforehand by a resident
    decode of the same inputs (the tier never changes results, so it is the
    routing the step itself produces). Every step's output is then compared
    bit for bit with the resident decode, and one tier step with the oracle."""
    wl = sg.get("qwen_layer_decode")
    L, E, n_slots, S = 2, 64, 12, 8
    d, tier, dev, host, slots, table, Wr, shared, ref_ptrs = make_tier(m, wl, E, L, n_slots, True)
    try:
        ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
        xs = [[sg.activations(wl, 40 + s, l, T=1, device="cuda").view(-1) for l in range(L)] for s in range(S)]

        def outputs():
            return (torch.empty((S, L, wl.H), device="cuda"), torch.empty((S, L, wl.k), dtype=torch.int32, device="cuda"),
                    torch.empty((S, L, wl.k), device="cuda"))

        ry, ri, rw = outputs()
        for s in range(S):
            for l in range(L):
                m.moe_layer_decode(d, xs[s][l], Wr[l], ref_ptrs[l], shared[l], ry[s, l], ri[s, l], rw[s, l], ws)
        torch.cuda.synchronize()
        routing = ri.cpu().numpy()
        ty, ti, tw = outputs()
        for s in range(S):
            for l in range(L):
                m.moe_layer_decode(d, xs[s][l], Wr[l], tier.table(l), shared[l], ty[s, l], ti[s, l], tw[s, l], ws)
            tier.update(routing[s], 8)   # no synchronisation: copies overlap the next step's kernels
        torch.cuda.synchronize()
        st = tier.stats()
        assert st["promotions"] > 0 and st["evictions"] > 0, st
        assert torch.equal(ti, ri)
        assert torch.equal(ty.view(torch.int32), ry.view(torch.int32))
        # one tier step against the oracle
        s, l = S - 1, 1
        x = xs[s][l].cpu().numpy()
        _, oi, ow = orc.route(x, Wr[l].cpu().numpy(), wl.k)
        gi = ti[s, l].cpu().numpy()
        assert (gi == oi[0]).all()
        hb = host_blocks(dev[l * E:(l + 1) * E], gi)
        ref, _ = orc.moe_decode(wl.fmt, wl.H, wl.I, x, [hb[int(e)] for e in gi], ow[0],
                                shared=[bf16_bits(t) for t in shared[l]], nthreads=NTHREADS)
        assert rel_err(ty[s, l].cpu().numpy(), ref) <= 1e-4
    finally:
        tier.close()
