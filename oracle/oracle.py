"""ctypes wrapper of the C oracle (libmoe_oracle.so).

TEST INFRASTRUCTURE ONLY: loaded by tests/, by the smoke check and by the
benchmark's CPU-baseline leg. The GPU library never imports it, and it imports
nothing of the GPU library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

NVFP4, MXFP4 = 1, 2
ACT_NONE, ACT_BF16, ACT_MXFP4 = 0, 1, 2
FMT = {"nvfp4": NVFP4, "mxfp4": MXFP4}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-o", tmp, SRC, "-lm", "-lpthread"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        P, I32, I64, D = C.c_void_p, C.c_int, C.c_int64, C.c_double
        L.orc_e2m1.restype = D; L.orc_e2m1.argtypes = [I32]
        L.orc_e4m3.restype = D; L.orc_e4m3.argtypes = [I32]
        L.orc_ue8m0.restype = D; L.orc_ue8m0.argtypes = [I32]
        L.orc_layout.restype = I32; L.orc_layout.argtypes = [I32, I32, I32, P]
        L.orc_dequant_block.restype = I32; L.orc_dequant_block.argtypes = [I32, I32, I32, P, P, P, P]
        L.orc_logits.restype = None; L.orc_logits.argtypes = [I32, I32, I32, P, P, P]
        L.orc_topk_sort.restype = None; L.orc_topk_sort.argtypes = [I32, I32, P, P]
        L.orc_topk_brute.restype = I32; L.orc_topk_brute.argtypes = [I32, I32, P, P]
        L.orc_route.restype = None; L.orc_route.argtypes = [I32, I32, I32, I32, P, P, P, P, P]
        L.orc_expert.restype = I32; L.orc_expert.argtypes = [I32, I32, I32, P, P, P, P]
        L.orc_moe_decode.restype = I32
        L.orc_moe_decode.argtypes = [I32, I32, I32, I32, P, P, P, P, P, P, P, P, I32]
        L.orc_bf16_rne.restype = C.c_uint16; L.orc_bf16_rne.argtypes = [D]
        L.orc_bf16_value.restype = D; L.orc_bf16_value.argtypes = [C.c_uint16]
        L.orc_mxfp4_quant.restype = None; L.orc_mxfp4_quant.argtypes = [P, I32, P, P]
        L.orc_quant_bf16_rows.restype = None; L.orc_quant_bf16_rows.argtypes = [I32, I32, P, P]
        L.orc_quant_mxfp4_rows.restype = I32; L.orc_quant_mxfp4_rows.argtypes = [I32, I32, P, P, P]
        L.orc_group.restype = I32; L.orc_group.argtypes = [I32, I32, I32, P, P, P, P]
        L.orc_fp8_quant.restype = None; L.orc_fp8_quant.argtypes = [P, I32, I32, P, P]
        L.orc_quant_fp8_rows.restype = I32; L.orc_quant_fp8_rows.argtypes = [I32, I32, I32, I32, P, P, P]
        L.orc_gemv_fp8.restype = None; L.orc_gemv_fp8.argtypes = [I32, I32, P, P, P, P]
        L.orc_moe_prefill.restype = I32
        L.orc_moe_prefill.argtypes = [I32, I32, I32, I32, I32, I32, P, P, P, P, I32, I32, P, P, P, I32]
        L.orc_round_rows.restype = I32; L.orc_round_rows.argtypes = [I32, I32, I32, P, P]
        L.orc_prefill_stage_hidden.restype = I32
        L.orc_prefill_stage_hidden.argtypes = [I32, I32, I32, I32, I32, I32, P, P, P, I32, I32, P, P, P, P, P, I32]
        L.orc_prefill_down_combine.restype = I32
        L.orc_prefill_down_combine.argtypes = [I32, I32, I32, I32, I32, I32, P, P, P, P, I32, P, I32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def fmt_id(fmt) -> int:
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def e2m1(code: int) -> float:
    return lib().orc_e2m1(code)


def e4m3(b: int) -> float:
    return lib().orc_e4m3(b)


def ue8m0(b: int) -> float:
    return lib().orc_ue8m0(b)


def layout(fmt, H: int, I: int) -> list[int]:
    off = np.zeros(7, np.int64)
    if lib().orc_layout(fmt_id(fmt), H, I, _p(off)):
        raise ValueError("bad shape for format")
    return [int(v) for v in off]


def dequant_block(fmt, H, I, block) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    b = _c(block, np.uint8)
    g = np.empty((I, H), np.float32); u = np.empty((I, H), np.float32); d = np.empty((H, I), np.float32)
    if lib().orc_dequant_block(fmt_id(fmt), H, I, _p(b), _p(g), _p(u), _p(d)):
        raise ValueError("bad shape")
    return g, u, d


def logits(x, Wr) -> np.ndarray:
    x = _c(x, np.float32); Wr = _c(Wr, np.float32)
    T, H = x.reshape(-1, Wr.shape[1]).shape
    out = np.empty((T, Wr.shape[0]), np.float64)
    lib().orc_logits(T, H, Wr.shape[0], _p(x), _p(Wr), _p(out))
    return out


def topk_sort(l, k) -> np.ndarray:
    l = _c(l, np.float64); idx = np.empty(k, np.int32)
    lib().orc_topk_sort(l.size, k, _p(l), _p(idx))
    return idx


def topk_brute(l, k) -> tuple[np.ndarray, int]:
    l = _c(l, np.float64); idx = np.full(k, -1, np.int32)
    n = lib().orc_topk_brute(l.size, k, _p(l), _p(idx))
    return idx, n


def route(x, Wr, k):
    """-> (logits f64 [T,E], idx i32 [T,k], w f64 [T,k])"""
    x = _c(x, np.float32); Wr = _c(Wr, np.float32)
    E, H = Wr.shape
    x = x.reshape(-1, H); T = x.shape[0]
    lg = np.empty((T, E), np.float64); idx = np.empty((T, k), np.int32); w = np.empty((T, k), np.float64)
    lib().orc_route(T, H, E, k, _p(x), _p(Wr), _p(lg), _p(idx), _p(w))
    return lg, idx, w


def expert(fmt, H, I, block, x):
    """One expert, fp64 input, no rounding -> (h [I], y [H])."""
    b = _c(block, np.uint8); xd = _c(x, np.float64)
    h = np.empty(I, np.float64); y = np.empty(H, np.float64)
    if lib().orc_expert(fmt_id(fmt), H, I, _p(b), _p(xd), _p(h), _p(y)):
        raise ValueError("bad shape")
    return h, y


def moe_decode(fmt, H, I, x, blocks, w, shared=None, nthreads=1):
    """y = sum_j w_j expert_j(x) (+ shared). blocks: list of k uint8 arrays.
    shared: None or (gate [I,H], up [I,H], down [H,I]) as uint16 bf16 bit patterns."""
    k = len(blocks)
    bl = [_c(b, np.uint8) for b in blocks]
    ptrs = (C.c_void_p * k)(*[b.ctypes.data for b in bl])
    xf = _c(x, np.float32).reshape(-1); wd = _c(w, np.float64).reshape(-1)
    y = np.empty(H, np.float64); h = np.empty((k, I), np.float64)
    if shared is not None:
        sg, su, sd = (_c(s, np.uint16) for s in shared)
        sp = (_p(sg), _p(su), _p(sd))
    else:
        sp = (None, None, None)
    r = lib().orc_moe_decode(fmt_id(fmt), H, I, k, _p(xf), C.cast(ptrs, C.c_void_p), _p(wd), *sp, _p(y), _p(h), nthreads)
    if r:
        raise ValueError("bad arguments")
    return y, h


def bf16_rne(v) -> np.ndarray:
    v = np.asarray(v, np.float64)
    f = lib().orc_bf16_rne
    return np.array([f(float(a)) for a in v.reshape(-1)], np.uint16).reshape(v.shape)


def bf16_value(b) -> np.ndarray:
    b = np.asarray(b, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def mxfp4_quant(v):
    v = _c(v, np.float64).reshape(-1)
    assert v.size <= 32
    codes = np.empty(v.size, np.uint8); sb = np.empty(1, np.uint8)
    lib().orc_mxfp4_quant(_p(v), v.size, _p(codes), _p(sb))
    return codes, int(sb[0])


def quant_bf16_rows(x) -> np.ndarray:
    x = _c(x, np.float32); x2 = x.reshape(x.shape[0], -1) if x.ndim > 1 else x.reshape(1, -1)
    out = np.empty(x2.shape, np.uint16)
    lib().orc_quant_bf16_rows(x2.shape[0], x2.shape[1], _p(x2), _p(out))
    return out


def quant_mxfp4_rows(x):
    x = _c(x, np.float32); x2 = x.reshape(x.shape[0], -1) if x.ndim > 1 else x.reshape(1, -1)
    T, n = x2.shape
    packed = np.empty((T, n // 2), np.uint8); sc = np.empty((T, n // 32), np.uint8)
    if lib().orc_quant_mxfp4_rows(T, n, _p(x2), _p(packed), _p(sc)):
        raise ValueError("row length must be a multiple of 32")
    return packed, sc


SCALE_FLOOR, SCALE_CEIL = 0, 1


def fp8_quant(v, rule=SCALE_FLOOR):
    """One block to E4M3 codes and its UE8M0 scale byte."""
    v = _c(v, np.float64)
    codes = np.empty(v.size, np.uint8); sb = np.zeros(1, np.uint8)
    lib().orc_fp8_quant(_p(v), v.size, int(rule), _p(codes), _p(sb))
    return codes, int(sb[0])


def quant_fp8_rows(x, block=32, rule=SCALE_FLOOR):
    """Rows of fp32 values to E4M3 codes [T][n] and UE8M0 scales [T][n/block]."""
    x = _c(x, np.float32); x2 = x.reshape(x.shape[0], -1) if x.ndim > 1 else x.reshape(1, -1)
    T, n = x2.shape
    codes = np.empty((T, n), np.uint8); sc = np.empty((T, n // block), np.uint8)
    if lib().orc_quant_fp8_rows(T, n, int(block), int(rule), _p(x2), _p(codes), _p(sc)):
        raise ValueError("row length must be a multiple of the block")
    return codes, sc


def gemv_fp8(W, s, x):
    """y = s * (e4m3(W) x) in fp64; W uint8 [rows, cols], s fp32 [rows], x fp32 [cols]."""
    W = _c(W, np.uint8); s = _c(s, np.float32); x = _c(x, np.float32)
    rows, cols = W.shape
    y = np.empty(rows, np.float64)
    lib().orc_gemv_fp8(rows, cols, _p(W), _p(s), _p(x), _p(y))
    return y


def group(idx, E):
    idx = _c(idx, np.int32); T, k = idx.reshape(idx.shape[0], -1).shape
    count = np.empty(E, np.int32); off = np.empty(E + 1, np.int32); perm = np.empty(T * k, np.int32)
    if lib().orc_group(T, k, E, _p(idx), _p(count), _p(off), _p(perm)):
        raise ValueError("expert index out of range")
    return count, off, perm


def _block_table(blocks, E, idx):
    """Pointer table of E expert blocks (dict {expert: array} or [E, bytes])."""
    keep = []
    ptrs = (C.c_void_p * E)()
    if isinstance(blocks, dict):
        for e, b in blocks.items():
            bb = _c(b, np.uint8); keep.append(bb); ptrs[e] = bb.ctypes.data
    else:
        bb = _c(blocks, np.uint8); keep.append(bb)
        for e in range(E):
            ptrs[e] = bb.ctypes.data + e * bb.shape[1]
    for e in np.unique(idx):
        if not ptrs[int(e)]:
            raise ValueError(f"expert {e} is routed to but its block is missing")
    return ptrs, keep


def round_rows(act, v):
    """Rows through the activation rounding (ACT_BF16 / ACT_MXFP4 / ACT_NONE), as fp64 values."""
    v = _c(v, np.float64)
    v2 = v.reshape(-1, v.shape[-1])
    out = np.empty_like(v2)
    if lib().orc_round_rows(int(act), v2.shape[0], v2.shape[1], _p(v2), _p(out)):
        raise ValueError("row length must be a multiple of 32 for MXFP4")
    return out.reshape(v.shape)


def prefill_stage_hidden(fmt, H, I, E, x, blocks, idx, act, ids, nthreads=1):
    """Gate/up stage of prefill for assignments ids (a = t*k + j).
    -> h_pre [n,I], h_q [n,I], gu [n,2,I] (g, u), agu [n,2,I] (sum |W x~| of g and u)."""
    x = _c(x, np.float32); idx = _c(idx, np.int32); ids = _c(ids, np.int32).reshape(-1)
    T, k = idx.shape
    ptrs, keep = _block_table(blocks, E, idx.reshape(-1)[ids] if ids.size else [])
    n = ids.size
    hp = np.empty((n, I)); hq = np.empty((n, I)); gu = np.empty((n, 2, I)); agu = np.empty((n, 2, I))
    r = lib().orc_prefill_stage_hidden(fmt_id(fmt), H, I, E, k, T, _p(x), C.cast(ptrs, C.c_void_p), _p(idx),
                                       int(act), n, _p(ids), _p(hp), _p(hq), _p(gu), _p(agu), nthreads)
    if r:
        raise ValueError("bad arguments")
    return hp, hq, gu, agu


def prefill_down_combine(fmt, H, I, E, blocks, idx, w, h_q, out_bf16=False, nthreads=1):
    """Down projection + combine on a given h~ [T,k,I] (token order) -> out f64 [T,H]."""
    idx = _c(idx, np.int32); w = _c(w, np.float32); hq = _c(h_q, np.float64)
    T, k = idx.shape
    assert hq.shape == (T, k, I), hq.shape
    ptrs, keep = _block_table(blocks, E, idx)
    out = np.empty((T, H), np.float64)
    r = lib().orc_prefill_down_combine(fmt_id(fmt), H, I, E, k, T, C.cast(ptrs, C.c_void_p), _p(idx), _p(w),
                                       _p(hq), int(out_bf16), _p(out), nthreads)
    if r:
        raise ValueError("bad arguments")
    return out


def moe_prefill(fmt, H, I, E, x, blocks, idx, w, act, out_bf16=False, want_h=False, nthreads=1):
    """blocks: dict {expert: uint8 array} or a [E, block_bytes] array.
    -> out f64 [T,H] (and h_pre, h_q f64 [T,k,I] if want_h)."""
    x = _c(x, np.float32); idx = _c(idx, np.int32); w = _c(w, np.float32)
    T, k = idx.shape
    keep = []
    ptrs = (C.c_void_p * E)()
    if isinstance(blocks, dict):
        for e, b in blocks.items():
            bb = _c(b, np.uint8); keep.append(bb); ptrs[e] = bb.ctypes.data
    else:
        bb = _c(blocks, np.uint8); keep.append(bb)
        for e in range(E):
            ptrs[e] = bb.ctypes.data + e * bb.shape[1]
    used = np.unique(idx)
    for e in used:
        if not ptrs[int(e)]:
            raise ValueError(f"expert {e} is routed to but its block is missing")
    out = np.empty((T, H), np.float64)
    hp = np.empty((T, k, I), np.float64) if want_h else None
    hq = np.empty((T, k, I), np.float64) if want_h else None
    r = lib().orc_moe_prefill(fmt_id(fmt), H, I, E, k, T, _p(x), C.cast(ptrs, C.c_void_p), _p(idx), _p(w),
                              act, int(out_bf16), _p(out), _p(hp) if want_h else None,
                              _p(hq) if want_h else None, nthreads)
    if r:
        raise ValueError("bad arguments")
    return (out, hp, hq) if want_h else out
