"""GPU parity of the prefill path (grouping, activation rounding, ragged
grouped GEMMs, combine) against the CPU oracle, through the C ABI, stage by
stage.

Bars (every checked token, no allowance unless stated):
  * perm/off bit-exact against the oracle's stable counting sort;
  * x~ bit-exact (bf16 RNE; MXFP4 codes compared modulo +-0);
  * gate/up stage: the GPU's h before rounding (debug output) against the
    oracle's fp64 h, max|d|/max|ref| <= 1e-4 per token;
  * the GPU's rounding step: its h~ equals the oracle's rounding (bf16 RNE
    or MXFP4 per 32) of the GPU's own h, bit for bit;
  * down + combine: the oracle replays the down projection and the combine
    on the GPU's h~; the GPU's output matches it to max|d|/max|ref| <= 1e-4
    per token;
  * element by element, the GPU's h before rounding lies within 2^-20 of the
    oracle's, measured relative to the element's accumulation magnitude
    (|silu'(g) u| sum_c |Wg x~| + |silu(g)| sum_c |Wu x~|: the quantity that
    bounds the rounding error of any fp32 evaluation; it is at least |h| and
    equals it where nothing cancels);
  * end to end: where the oracle's own h~ differs from the GPU's (a "flip"),
    the oracle's pre-rounding value must lie within 2^-18 of a rounding
    boundary, relative to the same magnitude, and at most a quarter of those
    near-tie elements may flip (aside from the fp32 range class: below
    g = -ln(FLT_MAX) e^-g overflows and an fp32 SiLU is 0, while the exact
    |h| < 3e-37 may still round to a nonzero bf16);
    the oracle's fully independent output then matches the GPU's per token to
    1e-4 of max|ref| plus the exact effect of the flipped elements
    (sum_j |w| |Wd| |h~_gpu - h~_oracle| over flips only).
The flip and near-tie counts of every check are printed and, when the
environment names a directory in MOE_PARITY_SUMMARY_DIR, written there as JSON.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import synthgen as sg
from gpu_helpers import NTHREADS, host_blocks, layer_blocks, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-4
# Near-tie window, relative to an element's accumulation magnitude.
TIE = 2.0 ** -18
# Largest deviation of the GPU's pre-rounding h from the oracle's, relative to
# each element's accumulation magnitude (an fp32-class bound: 16 units of
# fp32 roundoff).
DEV = 2.0 ** -20
# Largest fraction of the near-tie elements that may round the other way. A
# flip needs the deviation to exceed the distance to the boundary; with every
# deviation under DEV = TIE / 4, about DEV / TIE of the near-ties can flip
# when distances are spread evenly over the window.
FLIP_CAP = 0.25
MX_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
EXP_OVERFLOW = float(np.log(np.finfo(np.float32).max))  # 88.72


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import block_scaled_fp4_route_amd as m
    return m


def wl_small(fmt, H, I, E, k, T, s=1.1):
    if fmt == "nvfp4":
        return sg.Workload("pf_small", 95, H, I, E, k, fmt, 1, T, False, "zipf", s, 0x18, 0x48, False)
    return sg.Workload("pf_small_mx", 96, H, I, E, k, fmt, 1, T, False, "zipf", s, 121, 129, True)


def run_gpu(m, wl, blocks, x, idx, w, out_bf16, dbg=True):
    T, k = idx.shape
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    ws = m.alloc_workspace(d, T, m.MOE_MODE_PREFILL)
    n = T * k
    out = torch.empty((T, wl.H), dtype=torch.bfloat16 if out_bf16 else torch.float32, device="cuda")
    dd = None
    if dbg:
        dd = dict(h_pre=torch.empty((n, wl.I), dtype=torch.float32, device="cuda"),
                  h_q=torch.empty((n, wl.I), dtype=torch.float32, device="cuda"),
                  perm=torch.empty(n, dtype=torch.int32, device="cuda"),
                  off=torch.empty(wl.E + 1, dtype=torch.int32, device="cuda"))
        if wl.fmt == "nvfp4":
            dd["x_bf16"] = torch.empty((T, wl.H), dtype=torch.bfloat16, device="cuda")
        else:
            dd["x_codes"] = torch.empty((T, wl.H // 2), dtype=torch.uint8, device="cuda")
            dd["x_scales"] = torch.empty((T, wl.H // 32), dtype=torch.uint8, device="cuda")
    m.moe_expert_prefill(d, x, T, m.expert_ptr_table(blocks), idx, w, out,
                         m.MOE_OUT_BF16 if out_bf16 else m.MOE_OUT_F32, ws, dbg=dd)
    torch.cuda.synchronize()
    res = {"out": out.float().cpu().numpy(), "out_raw": out}
    if dbg:
        res.update({kk: v.cpu() for kk, v in dd.items()})
    return res


def to_token_order(a, perm, k):
    """[T*k, I] in grouped order -> [T, k, I]."""
    a = np.asarray(a)
    res = np.empty_like(a)
    res[np.asarray(perm)] = a
    return res.reshape(-1, k, a.shape[1])


def accumulation_magnitude(gu, agu):
    """Per element of h = silu(g) u: |silu'(g) u| sum|Wg x~| + |silu(g)| sum|Wu x~|,
    the first-order magnitude of the rounding error of an evaluation of h."""
    g, u = gu[..., 0, :], gu[..., 1, :]
    sg_ = expit(g)
    dsilu = sg_ * (1.0 + g * (1.0 - sg_))
    return np.abs(dsilu * u) * agu[..., 0, :] + np.abs(g * sg_) * agu[..., 1, :]


def near_tie_bf16(h, mag):
    """|h| within TIE * mag of a point halfway between two bf16 neighbours."""
    a = np.abs(h)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    step = 2.0 ** (e - 7)
    frac = a / step - np.floor(a / step)
    return np.abs(frac - 0.5) * step <= TIE * mag


def near_tie_mx(h, mag):
    """Per element of MXFP4 blocks of 32 along the row: the block's largest
    magnitude within TIE * (its magnitude) of a power of two (the shared
    exponent may differ), or the element within TIE * mag of an e2m1
    rounding boundary at the block's scale."""
    n, I = h.shape
    hb = np.abs(h).reshape(n, I // 32, 32)
    mb = mag.reshape(n, I // 32, 32)
    am = hb.argmax(axis=-1)
    amax = np.take_along_axis(hb, am[..., None], -1)[..., 0]
    amag = np.take_along_axis(mb, am[..., None], -1)[..., 0]
    safe = np.maximum(amax, 2.0 ** -140)
    pow2 = 2.0 ** np.round(np.log2(safe))
    blk = (np.abs(amax - pow2) <= TIE * amag) & (amax > 0)
    scale = 2.0 ** (np.floor(np.log2(safe)) - 2)
    t = hb / scale[..., None]
    d = np.min(np.abs(t[..., None] - MX_MIDS), axis=-1) * scale[..., None]
    el = d <= TIE * mb
    return (el | blk[..., None]).reshape(n, I)


def summary(name, rec):
    print(f"[parity] {name}: " + ", ".join(f"{k} {v}" for k, v in rec.items()), flush=True)
    out = os.environ.get("MOE_PARITY_SUMMARY_DIR")
    if out:
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, f"{name}.json"), "w") as f:
            json.dump(rec, f, indent=1)


def full_check(m, orc, wl, T, seed_layer=0, sample=None, tag=None, routing=None, x=None):
    blocks = layer_blocks(wl, seed_layer)
    if x is None:
        x = sg.activations(wl, 0, seed_layer, T=T, device="cuda")
    idx, w = sg.routing(wl, T=T, layer=seed_layer) if routing is None else routing
    g = run_gpu(m, wl, blocks, x, idx.cuda(), w.cuda(), False)
    k, I, H = wl.k, wl.I, wl.H
    # grouping: bit-exact
    cnt, off, perm = orc.group(idx.numpy(), wl.E)
    assert (g["perm"].numpy() == perm).all()
    assert (g["off"].numpy() == off).all()
    # x~ bit-exact
    xh = x.cpu().numpy()
    if wl.fmt == "nvfp4":
        ref = orc.quant_bf16_rows(xh)
        assert (g["x_bf16"].view(torch.int16).numpy().view(np.uint16) == ref).all()
        act = 1
    else:
        rc, rs = orc.quant_mxfp4_rows(xh)
        gc = g["x_codes"].numpy()
        lo_eq = ((gc & 15) == (rc & 15)) | (((gc & 7) == 0) & ((rc & 7) == 0))
        hi_eq = ((gc >> 4) == (rc >> 4)) | ((((gc >> 4) & 7) == 0) & (((rc >> 4) & 7) == 0))
        assert lo_eq.all() and hi_eq.all()
        assert (g["x_scales"].numpy() == rs).all()
        act = 2
    # the bf16 output is the round-to-nearest-even of the same fp32 sums
    if wl.out_bf16:
        gb = run_gpu(m, wl, blocks, x, idx.cuda(), w.cuda(), True, dbg=False)["out_raw"]
        assert torch.equal(gb.cpu(), torch.tensor(g["out"]).to(torch.bfloat16))
    toks = np.arange(T) if sample is None else np.asarray(sorted(set(int(t) for t in sample)))
    nt = len(toks)
    ih, wh = idx.numpy()[toks], w.numpy()[toks]
    hb = host_blocks(blocks, ih.reshape(-1))
    ids = (toks[:, None] * k + np.arange(k)[None, :]).reshape(-1).astype(np.int32)
    hp, hq, gu, agu = orc.prefill_stage_hidden(wl.fmt, H, I, wl.E, xh, hb, idx.numpy(), act, ids,
                                               nthreads=NTHREADS)
    gp = to_token_order(g["h_pre"].numpy(), perm, k)[toks].reshape(-1, I).astype(np.float64)
    gq = to_token_order(g["h_q"].numpy(), perm, k)[toks].reshape(-1, I).astype(np.float64)
    # gate/up stage, per token
    e_h = 0.0
    for i in range(nt):
        r = slice(i * k, (i + 1) * k)
        e = rel_err(gp[r], hp[r])
        assert e <= TOL, (int(toks[i]), e)
        e_h = max(e_h, e)
    # the GPU's rounding is the oracle's rounding of the GPU's own h
    assert np.array_equal(gq, orc.round_rows(act, gp)), "GPU h~ is not the rounding of its own h"
    # down + combine replayed on the GPU's h~, per token, no allowance
    rep = orc.prefill_down_combine(wl.fmt, H, I, wl.E, hb, ih, wh, gq.reshape(nt, k, I), nthreads=NTHREADS)
    gout = g["out"][toks]
    e_rep = 0.0
    for i in range(nt):
        e = rel_err(gout[i], rep[i])
        assert e <= TOL, (int(toks[i]), e)
        e_rep = max(e_rep, e)
    # flips of h~ against the oracle's own, each a near-tie
    flip = gq != hq
    mag = accumulation_magnitude(gu, agu)
    tie = near_tie_bf16(hp, mag) if act == 1 else near_tie_mx(hp, mag)
    # beyond fp32's range of e^-g (g < -ln(FLT_MAX)) an fp32 SiLU is +-0 while
    # the exact |h| < 89 e^-88.7 (< 3e-37) may still round to a nonzero bf16
    tail = (gu[:, 0, :] < -EXP_OVERFLOW) & (gp == 0)
    n_flip, n_el = int(flip.sum()), flip.size
    bad = flip & ~tie & ~tail
    n_range = int((flip & tail & ~tie).sum())
    # end to end against the oracle's own h~: 1e-4 plus the flips' exact effect
    e2e = orc.prefill_down_combine(wl.fmt, H, I, wl.E, hb, ih, wh, hq.reshape(nt, k, I), nthreads=NTHREADS)
    rows = np.nonzero(flip.any(axis=1))[0]
    allow = np.zeros((nt, H))
    row_e = ih.reshape(-1)[rows]
    for e in np.unique(row_e):
        ad = np.abs(orc.dequant_block(wl.fmt, H, I, hb[int(e)])[2]).astype(np.float64)
        for r in rows[row_e == e]:
            t_i, j = divmod(int(r), k)
            fm = flip[r]
            allow[t_i] += abs(float(wh[t_i, j])) * (ad[:, fm] @ np.abs(gq[r, fm] - hq[r, fm]))
    e2e_ok = np.ones(nt, bool)
    e_e2e = 0.0
    for i in range(nt):
        lim = TOL * np.abs(e2e[i]).max() + allow[i]
        e2e_ok[i] = (np.abs(gout[i] - e2e[i]) <= lim).all()
        e_e2e = max(e_e2e, rel_err(gout[i], e2e[i]))
    live = ~(gu[:, 0, :] < -EXP_OVERFLOW)
    dev = (np.abs(gp - hp) / np.maximum(mag, 1e-300))[live]
    summary(tag or f"{wl.name}_{wl.fmt}_H{H}_I{I}_E{wl.E}_k{k}_T{T}", {
        "tokens_checked": nt, "tokens": T, "h_elements": n_el, "gateup_max_rel_err": float(f"{e_h:.3e}"),
        "replay_max_rel_err": float(f"{e_rep:.3e}"), "e2e_max_rel_err": float(f"{e_e2e:.3e}"),
        "flips": n_flip, "flips_fp32_exp_range": n_range, "flips_off_tie": int(bad.sum()),
        "flip_rows": int(len(rows)), "near_tie_elements": int(tie.sum()),
        "h_dev_over_magnitude_max": float(f"{float(dev.max(initial=0.0)):.3e}"),
        "h_dev_over_magnitude_p999": float(f"{float(np.quantile(dev, 0.999)) if dev.size else 0.0:.3e}"),
        "flip_cap": int(FLIP_CAP * int(tie.sum()))})
    assert dev.max(initial=0.0) <= DEV, float(dev.max())
    assert not bad.any(), f"{int(bad.sum())} h~ elements differ from the oracle away from a near-tie"
    assert n_flip - n_range <= FLIP_CAP * int(tie.sum()), (n_flip, n_range, int(tie.sum()))
    assert e2e_ok.all(), [int(t) for t in toks[~e2e_ok][:8]]
    return g


@pytest.mark.parametrize("T", [1, 2, 17, 63, 64, 65, 300, 1024])
def test_prefill_nvfp4_T_sweep(m, orc, T):
    full_check(m, orc, wl_small("nvfp4", 512, 128, 8, 2, T), T)


@pytest.mark.parametrize("T", [1, 2, 17, 63, 64, 65, 300, 1024])
def test_prefill_mxfp4_T_sweep(m, orc, T):
    full_check(m, orc, wl_small("mxfp4", 512, 64, 8, 2, T), T)


def test_prefill_grouping_many_assignments(m, orc):
    """28,000 assignments: the grouping kernel's waves take their slices in
    more than one round of loads; perm/off stay bit-exact."""
    full_check(m, orc, wl_small("nvfp4", 512, 128, 9, 4, 7000), 7000, sample=[0, 1, 3500, 6999])


def test_prefill_nvfp4_qwen_shape_small_E(m, orc):
    """Qwen expert shape (H 2560, I 640, top-10) with 24 experts, 40 tokens,
    some experts unused, Zipf skew."""
    wl = wl_small("nvfp4", 2560, 640, 24, 10, 40)
    full_check(m, orc, wl, 40)


@pytest.mark.parametrize("H,I,E,k,T", [(768, 1024, 6, 3, 70), (512, 1152, 5, 2, 40)])
def test_prefill_nvfp4_down_scale_staging(m, orc, H, I, E, k, T):
    """The NVFP4 down GEMM stages its weight rows' scales in LDS up to
    I = 1024 (256 rows x 64 scale bytes) and loads them per chunk above it:
    both forms, with tiles of more than one row block."""
    full_check(m, orc, wl_small("nvfp4", H, I, E, k, T), T)


def counts_routing(counts, T):
    """Routing with exactly counts[e] assignments to expert e over T tokens of
    k = 2 (two distinct experts per token: slot 0 takes the first T expert
    ids in expert order, slot 1 the rest; no count exceeds T), weights from a
    seeded generator."""
    ids = np.repeat(np.arange(len(counts)), counts)
    assert ids.size == 2 * T and max(counts) <= T
    idx = np.stack([ids[:T], ids[T:]], axis=1).astype(np.int32)
    assert (idx[:, 0] != idx[:, 1]).all()
    z = np.random.default_rng(7).standard_normal((T, 2))
    w = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    return torch.from_numpy(idx), torch.from_numpy(w.astype(np.float32))


@pytest.mark.parametrize("H,I,E,k,T", [(8192, 256, 4, 2, 9), (16384, 128, 3, 2, 5)])
def test_prefill_nvfp4_wide_rows(m, orc, H, I, E, k, T):
    """Rows of 8192 and 16384 values: the activation conversion takes its
    rows in several blocks per lane, and the gate/up K loop runs 32 and 64
    chunks."""
    full_check(m, orc, wl_small("nvfp4", H, I, E, k, T), T)


def test_prefill_nvfp4_activation_ranges(m, orc):
    """The NVFP4 gate/up GEMM takes x~ = bf16(x) as fp16 times a power of two
    per token. Rows far above and below 1, a row spanning 2^40 from its largest
    to its smallest element, an all-zero row, a row with one nonzero element
    and a row of largest-magnitude ties stay at the stage-wise bar."""
    wl = wl_small("nvfp4", 512, 128, 8, 2, 40)
    T, H = 40, wl.H
    x = sg.activations(wl, 0, 0, T=T, device="cuda").clone()
    x[0] *= 2.0 ** 24
    x[1] *= 2.0 ** -40
    x[2] *= torch.exp2(-40.0 * torch.arange(H, device="cuda", dtype=torch.float32) / H)
    x[3] = 0.0
    x[4] = 0.0
    x[4, 7] = -3.0
    x[5] = torch.where(torch.arange(H, device="cuda") % 2 == 0, 1.0, -1.0) * 65504.0
    x[6, ::3] *= 2.0 ** -30
    full_check(m, orc, wl, T, x=x, tag="pf_nvfp4_activation_ranges")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_prefill_tile_row_counts(m, orc, fmt):
    """Experts with exactly 1, 16, 17, 32, 33, 64, 65, 127, 128 and 129 rows
    (plus one of 148): every row-block specialisation of the grouped GEMMs,
    both NVFP4 tile heights (64 rows up to 64, 128 rows above) and the ragged
    last tile of a multi-tile expert."""
    counts = [1, 16, 17, 32, 33, 64, 65, 127, 128, 129, 148]
    T = sum(counts) // 2
    wl = wl_small(fmt, 512, 128 if fmt == "nvfp4" else 64, len(counts), 2, T)
    full_check(m, orc, wl, T, routing=counts_routing(counts, T), tag=f"tile_row_counts_{fmt}")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("case,counts", [
    ("all_multi_tile", [129, 200, 257, 300, 140, 130]),
    ("two_heavy_tiles", [200, 1, 5, 16, 33, 64, 100, 3, 7, 9]),
    ("few_single_tiles", [130, 140, 150, 160, 170, 1, 2, 3]),
])
def test_prefill_tile_order_edges(m, orc, fmt, case, counts):
    """The tile slots' order (each XCD: a run of the multi-tile experts'
    tiles spread among single tiles) where it has edges: no single tiles at
    all (NVFP4), fewer multi-tile tiles than XCDs, and as many whole rounds of
    8 tiles as of multi-tile tiles (few single tiles left over). Every tile
    must be run exactly once."""
    T = sum(counts) // 2
    wl = wl_small(fmt, 512, 128 if fmt == "nvfp4" else 64, len(counts), 2, T)
    full_check(m, orc, wl, T, routing=counts_routing(counts, T), tag=f"tile_order_{case}_{fmt}")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_prefill_largest_expert_count_and_top_k(m, orc, fmt):
    """E = 1024 experts (the tile list's scans at their full 1024 threads)
    and top-32 routing (the combine's widest groups), uniform routing so
    that most experts hold a few rows."""
    wl = wl_small(fmt, 512, 128 if fmt == "nvfp4" else 64, 1024, 32, 80, s=0.0)
    full_check(m, orc, wl, 80, tag=f"largest_E_k_{fmt}")


def test_prefill_mxfp4_deepseek_shape_small_E(m, orc):
    wl = wl_small("mxfp4", 4096, 2880, 12, 6, 20, s=0.0)
    full_check(m, orc, wl, 20)


@pytest.mark.parametrize("H,I,E,k,T", [(4608, 320, 6, 3, 40), (1536, 4160, 4, 2, 33)])
def test_prefill_mxfp4_odd_shapes(m, orc, H, I, E, k, T):
    """Hidden sizes whose weight rows end inside a streamed chunk (4608) or
    whose scale rows are 3 pieces of 16 bytes (1536), and scale areas past
    8 KB per 64 weight rows (H 4608 for gate/up, I 4160 for down)."""
    full_check(m, orc, wl_small("mxfp4", H, I, E, k, T), T)


def test_prefill_qwen_full_size(m, orc):
    """Qwen-shaped prefill at full size (512 experts, 2451 tokens, 24,510
    assignments, Zipf 1.1): every token, in the launch configuration the
    benchmark times."""
    wl = sg.get("qwen_prefill")
    full_check(m, orc, wl, wl.T, tag="qwen_prefill_full")


def test_prefill_deepseek_full_size(m, orc):
    """DeepSeek-shaped prefill at full size (384 experts, 311 tokens, uniform
    routing, bf16 out): every token."""
    wl = sg.get("deepseek_prefill")
    full_check(m, orc, wl, wl.T, tag="deepseek_prefill_full")


def test_prefill_deterministic(m):
    wl = wl_small("nvfp4", 512, 128, 8, 2, 300)
    blocks = layer_blocks(wl, 0)
    x = sg.activations(wl, 0, 0, T=300, device="cuda")
    idx, w = sg.routing(wl, T=300)
    first = run_gpu(m, wl, blocks, x, idx.cuda(), w.cuda(), False, dbg=False)["out_raw"].clone()
    for _ in range(4):
        again = run_gpu(m, wl, blocks, x, idx.cuda(), w.cuda(), False, dbg=False)["out_raw"]
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))


def test_prefill_workspace_reused_across_routings(m):
    """Two calls with different routings on one workspace (and a third
    repeating the first): each equals the same call on a fresh workspace bit
    for bit, so no counter, tile list or cached activation carries over."""
    wl = wl_small("nvfp4", 2560, 640, 48, 10, 200)
    blocks = layer_blocks(wl, 0)
    x = sg.activations(wl, 0, 0, T=200, device="cuda")
    routes = [sg.routing(wl, T=200, layer=0), sg.routing(wl, T=200, layer=1, zipf_s=0.0)]
    fresh = [run_gpu(m, wl, blocks, x, i.cuda(), w.cuda(), False, dbg=False)["out_raw"].clone() for i, w in routes]
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    ws = m.alloc_workspace(d, 200, m.MOE_MODE_PREFILL)
    ptrs = m.expert_ptr_table(blocks)
    out = torch.empty((200, wl.H), dtype=torch.float32, device="cuda")
    for r in (0, 1, 0):
        i, w = routes[r]
        m.moe_expert_prefill(d, x, 200, ptrs, i.cuda(), w.cuda(), out, m.MOE_OUT_F32, ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), fresh[r].view(torch.int32)), r


def test_prefill_unmet_tile_wait_poisons_outputs(m):
    """The NVFP4 GEMM launch's down tiles wait (bounded) for their gate/up
    tiles; a wait that ends unmet writes NaN over the tile's outputs instead
    of using an incomplete h~. Forced from the host: every wait asks for one
    more publication than exists, with a short poll limit. The call ends,
    every output is NaN, and the next ordinary call on the same workspace is
    bit-identical to a fresh one."""
    wl = wl_small("nvfp4", 512, 128, 8, 2, 40)
    blocks = layer_blocks(wl, 0)
    x = sg.activations(wl, 0, 0, T=40, device="cuda")
    idx, w = sg.routing(wl, T=40)
    idx, w = idx.cuda(), w.cuda()
    ref = run_gpu(m, wl, blocks, x, idx, w, False, dbg=False)["out_raw"].clone()
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    ws = m.alloc_workspace(d, 40, m.MOE_MODE_PREFILL)
    ptrs = m.expert_ptr_table(blocks)
    out = torch.empty((40, wl.H), dtype=torch.float32, device="cuda")
    m.moe_expert_prefill(d, x, 40, ptrs, idx, w, out, m.MOE_OUT_F32, ws,
                         dbg={"tile_wait_polls": 16, "tile_wait_unmet": 1})
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    m.moe_expert_prefill(d, x, 40, ptrs, idx, w, out, m.MOE_OUT_F32, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


def test_prefill_invalid_expert_index_gives_nan_row(m):
    wl = wl_small("nvfp4", 512, 128, 8, 2, 5)
    blocks = layer_blocks(wl, 0)
    x = sg.activations(wl, 0, 0, T=5, device="cuda")
    idx, w = sg.routing(wl, T=5)
    idx[2, 1] = 99
    idx[4, 0] = wl.E  # just past the last expert
    g = run_gpu(m, wl, blocks, x, idx.cuda(), w.cuda(), False, dbg=False)
    assert np.isnan(g["out"][[2, 4]]).all()
    assert np.isfinite(np.delete(g["out"], [2, 4], axis=0)).all()
