"""Seeded, counter-based synthetic inputs for the routed FP4 mixture-of-experts FFN.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
callers. It holds no arithmetic of the method itself (no dequantisation, no
routing, no SwiGLU, no rounding rule of the method): it only draws random
bytes, scale codes, normals and routing assignments, with the shapes and
distributions of the workloads described on the pages:

  [Q] "Running a 133 GB MoE model on an 8 GB GPU at 11 tokens/s by streaming
      experts from NVMe" (aiwithghost.com), section "Why this model, of all
      models" (48 layers, 512 experts, top-10, three 2560x640 matrices per
      expert in NVFP4) and section "The engine", item 1 (one 2,764,800-byte
      block per expert).
  [D] "Running the 510 GB DeepSeek-V4.1-Flash on an 8 GB GPU, and three bugs
      that never raise an error" (dev.to), section "Bytes per token decide
      everything" (384 experts, 6 chosen per token, FP4 with ue8m0 scales).

Generator: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), used counter-based: word i of a
stream with key K is mix64(K + (i + 1) * GAMMA), which is exactly the i-th
output of a SplitMix64 generator seeded with K. Integer ops run on int64 torch
tensors (two's-complement wraparound), so the same bytes come out on the CPU
and on the GPU. Normals use the Box-Muller transform in float64.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence

import torch

SEED = 20261202

_M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_MUL1 = 0xBF58476D1CE4E5B9
_MUL2 = 0x94D049BB133111EB


def _signed(v: int) -> int:
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


_GAMMA_S = _signed(GAMMA)
_MUL1_S = _signed(_MUL1)
_MUL2_S = _signed(_MUL2)


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2^64)."""
    z &= _M64
    z = ((z ^ (z >> 30)) * _MUL1) & _M64
    z = ((z ^ (z >> 27)) * _MUL2) & _M64
    return z ^ (z >> 31)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 lanes viewed as uint64."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output function on int64 tensors (uint64 bit patterns)."""
    z = z ^ _lsr(z, 30)
    z = z * _MUL1_S
    z = z ^ _lsr(z, 27)
    z = z * _MUL2_S
    return z ^ _lsr(z, 31)


def stream_key(*ids: int, seed: int = SEED) -> int:
    """Key of the stream named by a tuple of small non-negative integers."""
    k = mix64_int(seed + GAMMA)
    for i in ids:
        k = mix64_int(k ^ mix64_int((int(i) + 1) * GAMMA))
    return k


def words(keys: Sequence[int] | int, count: int, device="cpu", start: int = 0) -> torch.Tensor:
    """int64 tensor [len(keys), count] (or [count]) of stream words start..start+count-1."""
    single = isinstance(keys, int)
    kl = [keys] if single else list(keys)
    kt = torch.tensor([_signed(k) for k in kl], dtype=torch.int64, device=device).view(-1, 1)
    ctr = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device).view(1, -1)
    w = mix64(kt + ctr * _GAMMA_S)
    return w[0] if single else w


def uniform_bytes(keys, nbytes: int, device="cpu") -> torch.Tensor:
    """Uniform random bytes (8 per word, little-endian); [len(keys), nbytes] or [nbytes]."""
    nw = (nbytes + 7) // 8
    w = words(keys, nw, device)
    b = w.contiguous().view(torch.uint8)
    return b[..., :nbytes]


def uniform_codes(keys, n: int, lo: int, hi: int, device="cpu") -> torch.Tensor:
    """Byte codes uniform over the integers lo..hi (one word per code, top 32 bits)."""
    w = words(keys, n, device)
    u32 = _lsr(w, 32)
    return (lo + ((u32 * (hi - lo + 1)) >> 32)).to(torch.uint8)


def uniform01(keys, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """float64 uniforms in [0, 1) from the top 53 bits of each word."""
    w = words(keys, n, device, start=start)
    return _lsr(w, 11).to(torch.float64) * (2.0 ** -53)


def normal(keys, n: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """float32 N(0, std^2) by Box-Muller; element i uses words 2i and 2i+1."""
    w = words(keys, 2 * n, device)
    w = w.view(*w.shape[:-1], n, 2)
    u1 = (_lsr(w[..., 0], 11).to(torch.float64) + 1.0) * (2.0 ** -53)  # (0, 1]
    u2 = _lsr(w[..., 1], 11).to(torch.float64) * (2.0 ** -53)          # [0, 1)
    z = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)
    return (z * std).to(torch.float32)


# ---------------------------------------------------------------------------
# Stream identifiers (fields of a workload)
F_CODES, F_SCALES, F_ROUTER, F_X, F_SHARED, F_ROUTE_PERM, F_ROUTE_KEYS, F_ROUTE_W = range(8)


from .configs import WORKLOADS, Workload, get  # noqa: E402


def block_region_sizes(wl: Workload) -> tuple[int, int]:
    """(code bytes, scale bytes) of one expert block: three matrices of H*I
    4-bit codes, then one scale byte per group of G codes."""
    n = 3 * wl.H * wl.I
    return n // 2, n // wl.group


def expert_blocks(wl: Workload, layer: int, experts: Iterable[int], device="cpu",
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """uint8 [n, block_bytes]: codes uniform over all 16 nibble values, scale
    bytes uniform over the workload's scale-code range."""
    ex = list(experts)
    cb, sb = block_region_sizes(wl)
    if out is None:
        out = torch.empty((len(ex), cb + sb), dtype=torch.uint8, device=device)
    kc = [stream_key(wl.cfg_id, layer, e, F_CODES) for e in ex]
    ks = [stream_key(wl.cfg_id, layer, e, F_SCALES) for e in ex]
    out[:, :cb] = uniform_bytes(kc, cb, device)
    out[:, cb:] = uniform_codes(ks, sb, wl.scale_lo, wl.scale_hi, device)
    return out


def fill_layer_blocks(wl: Workload, layer: int, dst: torch.Tensor, batch: int = 32) -> None:
    """Fill dst ([E, block_bytes] uint8, any device) with all experts of a layer."""
    for e0 in range(0, wl.E, batch):
        e1 = min(wl.E, e0 + batch)
        expert_blocks(wl, layer, range(e0, e1), device=dst.device, out=dst[e0:e1])


def router_weights(wl: Workload, layer: int, device="cpu") -> torch.Tensor:
    """fp32 [E, H], N(0, 0.02^2)."""
    return normal(stream_key(wl.cfg_id, layer, 0, F_ROUTER), wl.E * wl.H, 0.02, device).view(wl.E, wl.H)


def shared_expert(wl: Workload, layer: int, device="cpu") -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """bf16 gate [I, H], up [I, H], down [H, I], entries N(0, 0.02^2) rounded to bf16."""
    def mat(i, r, c):
        return normal(stream_key(wl.cfg_id, layer, i, F_SHARED), r * c, 0.02, device).view(r, c).to(torch.bfloat16)
    return mat(0, wl.I, wl.H), mat(1, wl.I, wl.H), mat(2, wl.H, wl.I)


def activations(wl: Workload, step: int, layer: int, T: int | None = None, device="cpu") -> torch.Tensor:
    """fp32 [T, H], N(0, 1); a fresh draw per (step, layer)."""
    T = wl.T if T is None else T
    return normal(stream_key(wl.cfg_id, layer, step, F_X), T * wl.H, 1.0, device).view(T, wl.H)


def routing(wl: Workload, T: int | None = None, layer: int = 0, device="cpu",
            zipf_s: float | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Directly drawn routing for prefill: (idx int32 [T, k], w fp32 [T, k]).

    Each token draws k distinct experts without replacement with
    p(rank r) proportional to r^-s over a seeded permutation of expert ids
    (Gumbel-top-k on log p; s = 0 gives uniform routing). The weights are
    exp(z_j) / sum_j exp(z_j) of k standard normal draws z.
    """
    T = wl.T if T is None else T
    s = wl.zipf_s if zipf_s is None else zipf_s
    E, k = wl.E, wl.k
    kp = stream_key(wl.cfg_id, layer, 0, F_ROUTE_PERM)
    perm = torch.argsort(words(kp, E, device))  # seeded permutation of expert ids
    ranks = torch.arange(1, E + 1, dtype=torch.float64, device=device)
    logp = -s * torch.log(ranks)
    kk = stream_key(wl.cfg_id, layer, T, F_ROUTE_KEYS)
    u = uniform01(kk, T * E, device).view(T, E)
    u = torch.clamp(u, min=2.0 ** -60)
    gumbel = -torch.log(-torch.log(u))
    top = torch.topk(logp.view(1, E) + gumbel, k, dim=1).indices
    idx = perm[top].to(torch.int32)
    z = normal(stream_key(wl.cfg_id, layer, T, F_ROUTE_W), T * k, 1.0, device).view(T, k).to(torch.float64)
    ez = torch.exp(z - z.max(dim=1, keepdim=True).values)
    w = (ez / ez.sum(dim=1, keepdim=True)).to(torch.float32)
    return idx.contiguous(), w.contiguous()


def decode_routing(wl: Workload, layer: int, step: int = 0, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """Routing for one decode token given directly (uniform k-subset, random
    weights), for tests that check the expert path separately from the router."""
    idx, w = routing(wl, T=1, layer=1000 + layer + 7919 * step, device=device, zipf_s=0.0)
    return idx.view(wl.k), w.view(wl.k)


# ---------------------------------------------------------------------------
# FP8 inputs (stream namespace 90: the activation quantiser, 91: the
# row-scaled GEMV)
F8_ACT, F8_CODES, F8_SCALES, F8_X = 90, 91, 92, 93


def fp8_activations(rows: int, cols: int, seed_id: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [rows, cols] N(0, 1) rows for the FP8 activation quantiser."""
    return normal(stream_key(F8_ACT, seed_id, rows, cols), rows * cols, 1.0, device).view(rows, cols)


def fp8_matrix(rows: int, cols: int, seed_id: int = 0, device="cpu") -> torch.Tensor:
    """uint8 [rows, cols] codes uniform over the 254 finite E4M3 bytes
    (0x7F and 0xFF, the two NaN codes, are skipped)."""
    u = uniform_codes(stream_key(F8_CODES, seed_id, rows, cols), rows * cols, 0, 253, device).to(torch.int32)
    return (u + (u >= 127).to(torch.int32)).to(torch.uint8).view(rows, cols)


def fp8_row_scales(rows: int, seed_id: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [rows] positive row scales 2^-8 * (1 + u), u uniform in [0, 1)."""
    u = uniform01(stream_key(F8_SCALES, seed_id, rows), rows, device)
    return ((1.0 + u) * 2.0 ** -8).to(torch.float32)


def fp8_vector(cols: int, seed_id: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [cols] N(0, 1) input vector of the GEMV."""
    return normal(stream_key(F8_X, seed_id, cols), cols, 1.0, device)


__all__ = [
    "SEED", "GAMMA", "mix64", "mix64_int", "stream_key", "words", "uniform_bytes",
    "uniform_codes", "uniform01", "normal", "WORKLOADS", "Workload", "get",
    "block_region_sizes", "expert_blocks", "fill_layer_blocks", "router_weights",
    "shared_expert", "activations", "routing", "decode_routing", "fp8_activations", "fp8_matrix",
    "fp8_row_scales", "fp8_vector",
]
