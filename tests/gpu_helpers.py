"""Helpers shared by the GPU parity tests: device inputs from the seeded
generator, host copies for the oracle, and the comparison metrics."""
from __future__ import annotations

import os

import numpy as np
import torch

import synthgen as sg

NTHREADS = min(16, os.cpu_count() or 1)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (the parity metric)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def cosine(got, ref) -> float:
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    return float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref) + 1e-300))


def layer_blocks(wl: sg.Workload, layer: int = 0, E: int | None = None, device="cuda") -> torch.Tensor:
    E = wl.E if E is None else E
    out = torch.empty((E, wl.block_bytes), dtype=torch.uint8, device=device)
    for e0 in range(0, E, 16):
        e1 = min(E, e0 + 16)
        sg.expert_blocks(wl, layer, range(e0, e1), device=device, out=out[e0:e1])
    return out


def host_blocks(blocks: torch.Tensor, experts) -> dict[int, np.ndarray]:
    return {int(e): blocks[int(e)].cpu().numpy() for e in sorted(set(int(v) for v in experts))}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def same_f32_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit equality of fp32 arrays, NaNs compared as a class."""
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    if not (na == nb).all():
        return False
    return bool((a[~na].view(np.uint32) == b[~nb].view(np.uint32)).all())
