"""Thin ctypes binding of libmoe_fp4.so (argument marshalling only).

Every function has the name and the argument order of the C entry point in
include/moe_fp4.h; tensors are torch tensors on the GPU (their data_ptr() is
passed), the stream defaults to torch's current stream. A non-zero status
raises MoeError with the library's own message. All arithmetic happens in the
HIP kernels; nothing here computes on the data.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_fp4.so")

MOE_FMT_NVFP4, MOE_FMT_MXFP4 = 1, 2
MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_WORKSPACE = 0, -1, -2, -3, -4
MOE_MODE_ROUTE, MOE_MODE_DECODE, MOE_MODE_PREFILL = 0, 1, 2
MOE_OUT_F32, MOE_OUT_BF16 = 0, 1
MOE_NOALLOC_SCRATCH_BYTES = 1 << 20
FORMATS = {"nvfp4": MOE_FMT_NVFP4, "mxfp4": MOE_FMT_MXFP4}

# every symbol declared in include/moe_fp4.h
EXPORTS = ("moe_block_bytes", "moe_block_layout", "moe_workspace_bytes", "moe_route", "moe_expert_decode",
           "moe_layer_decode", "moe_layer_decode_noalloc", "moe_expert_prefill", "moe_dequant_block", "moe_act_quant_fp8", "moe_gemv_fp8",
           "moe_prefetch_sink_bytes", "moe_expert_prefetch", "moe_tier_create", "moe_tier_destroy", "moe_tier_update", "moe_tier_get_stats", "moe_tier_slot_of",
           "moe_status_string", "moe_last_error")


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class moe_desc(C.Structure):
    _fields_ = [("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("k", C.c_int32), ("format", C.c_int32)]


class moe_shared(C.Structure):
    _fields_ = [("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p)]


class moe_prefill_debug(C.Structure):
    _fields_ = [("x_bf16", C.c_void_p), ("x_codes", C.c_void_p), ("x_scales", C.c_void_p), ("h_pre", C.c_void_p),
                ("h_q", C.c_void_p), ("perm", C.c_void_p), ("off", C.c_void_p),
                ("tile_wait_polls", C.c_int32), ("tile_wait_unmet", C.c_int32)]


class moe_tier_stats(C.Structure):
    _fields_ = [("resident", C.c_int64), ("pending", C.c_int64), ("hits", C.c_int64), ("misses", C.c_int64),
                ("promotions", C.c_int64), ("evictions", C.c_int64)]


def _load():
    # torch ships its own HIP runtime (same soname as the system one). Loading
    # torch first makes the library bind to that one, so the process holds a
    # single runtime; loaded the other way round, the library's launches
    # found no device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python block_scaled_fp4_route_amd/build.py")
    L = C.CDLL(LIB_PATH)
    P, I32, SZ = C.c_void_p, C.c_int32, C.c_size_t
    D = C.POINTER(moe_desc)
    L.moe_block_bytes.restype = SZ; L.moe_block_bytes.argtypes = [D]
    L.moe_block_layout.restype = C.c_int; L.moe_block_layout.argtypes = [D, P]
    L.moe_workspace_bytes.restype = SZ; L.moe_workspace_bytes.argtypes = [D, I32, I32]
    L.moe_route.restype = C.c_int; L.moe_route.argtypes = [D, P, I32, P, P, P, P, P, SZ, P]
    L.moe_expert_decode.restype = C.c_int
    L.moe_expert_decode.argtypes = [D, P, P, P, P, C.POINTER(moe_shared), P, P, SZ, P]
    L.moe_layer_decode.restype = C.c_int
    L.moe_layer_decode.argtypes = [D, P, P, P, C.POINTER(moe_shared), P, P, P, P, SZ, P]
    L.moe_layer_decode_noalloc.restype = C.c_int
    L.moe_layer_decode_noalloc.argtypes = [D, P, P, P, C.POINTER(moe_shared), P, P, P, P]
    L.moe_expert_prefill.restype = C.c_int
    L.moe_expert_prefill.argtypes = [D, P, I32, P, P, P, P, I32, P, SZ, C.POINTER(moe_prefill_debug), P]
    L.moe_dequant_block.restype = C.c_int; L.moe_dequant_block.argtypes = [D, P, P, P, P, P]
    L.moe_act_quant_fp8.restype = C.c_int; L.moe_act_quant_fp8.argtypes = [P, I32, I32, I32, I32, P, P, P]
    L.moe_gemv_fp8.restype = C.c_int; L.moe_gemv_fp8.argtypes = [P, P, P, I32, I32, P, P]
    L.moe_prefetch_sink_bytes.restype = SZ; L.moe_prefetch_sink_bytes.argtypes = [D, I32]
    L.moe_expert_prefetch.restype = C.c_int; L.moe_expert_prefetch.argtypes = [D, P, P, I32, P, SZ, P]
    L.moe_tier_create.restype = C.c_int
    L.moe_tier_create.argtypes = [D, I32, P, P, I32, P, C.POINTER(P)]
    L.moe_tier_destroy.restype = C.c_int; L.moe_tier_destroy.argtypes = [P]
    L.moe_tier_update.restype = C.c_int; L.moe_tier_update.argtypes = [P, P, I32, P]
    L.moe_tier_get_stats.restype = C.c_int; L.moe_tier_get_stats.argtypes = [P, C.POINTER(moe_tier_stats)]
    L.moe_tier_slot_of.restype = I32; L.moe_tier_slot_of.argtypes = [P, I32, I32]
    L.moe_status_string.restype = C.c_char_p; L.moe_status_string.argtypes = [C.c_int]
    L.moe_last_error.restype = C.c_char_p; L.moe_last_error.argtypes = []
    return L


lib = _load()


def desc(H: int, I: int, E: int, k: int, fmt) -> moe_desc:
    return moe_desc(H, I, E, k, FORMATS[fmt] if isinstance(fmt, str) else int(fmt))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib.moe_last_error().decode() or lib.moe_status_string(status).decode())


def moe_block_bytes(d: moe_desc) -> int:
    return int(lib.moe_block_bytes(C.byref(d)))


def moe_block_layout(d: moe_desc) -> list[int]:
    off = (C.c_int64 * 7)()
    _check(lib.moe_block_layout(C.byref(d), off))
    return list(off)


def moe_workspace_bytes(d: moe_desc, T: int, mode: int) -> int:
    return int(lib.moe_workspace_bytes(C.byref(d), T, mode))


def moe_route(d, x, T, Wr, idx, w, logits_out, ws, ws_bytes=None, stream=None):
    wsb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib.moe_route(C.byref(d), _ptr(x), T, _ptr(Wr), _ptr(idx), _ptr(w), _ptr(logits_out), _ptr(ws), wsb,
                         _stream(stream)))


def moe_expert_decode(d, x, expert_ptrs, idx, w, shared, y, ws, ws_bytes=None, stream=None):
    """shared: None or (gate, up, down) bf16 tensors."""
    sh = None
    if shared is not None:
        sh = C.byref(moe_shared(_ptr(shared[0]), _ptr(shared[1]), _ptr(shared[2])))
    wsb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib.moe_expert_decode(C.byref(d), _ptr(x), _ptr(expert_ptrs), _ptr(idx), _ptr(w), sh, _ptr(y), _ptr(ws),
                                 wsb, _stream(stream)))


def moe_layer_decode(d, x, Wr, expert_ptrs, shared, y, idx_out, w_out, ws, ws_bytes=None, stream=None):
    """shared: None or (gate, up, down) bf16 tensors."""
    sh = None
    if shared is not None:
        sh = C.byref(moe_shared(_ptr(shared[0]), _ptr(shared[1]), _ptr(shared[2])))
    wsb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib.moe_layer_decode(C.byref(d), _ptr(x), _ptr(Wr), _ptr(expert_ptrs), sh, _ptr(y), _ptr(idx_out),
                                _ptr(w_out), _ptr(ws), wsb, _stream(stream)))


def moe_layer_decode_noalloc(d, x, Wr, expert_ptrs, shared, y, idx_out, w_out, stream=None):
    """moe_layer_decode with the library's static scratch as its workspace."""
    sh = None
    if shared is not None:
        sh = C.byref(moe_shared(_ptr(shared[0]), _ptr(shared[1]), _ptr(shared[2])))
    _check(lib.moe_layer_decode_noalloc(C.byref(d), _ptr(x), _ptr(Wr), _ptr(expert_ptrs), sh, _ptr(y), _ptr(idx_out),
                                        _ptr(w_out), _stream(stream)))


def moe_expert_prefill(d, x, T, expert_ptrs, idx, w, out, out_dtype, ws, ws_bytes=None, dbg=None, stream=None):
    """dbg: None or a dict with any of the moe_prefill_debug member names -> tensors
    (the two wait controls take ints)."""
    db = None
    if dbg is not None:
        db = C.byref(moe_prefill_debug(**{k: (v if isinstance(v, int) else _ptr(v)) for k, v in dbg.items()}))
    wsb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(lib.moe_expert_prefill(C.byref(d), _ptr(x), T, _ptr(expert_ptrs), _ptr(idx), _ptr(w), _ptr(out),
                                  out_dtype, _ptr(ws), wsb, db, _stream(stream)))


def moe_dequant_block(d, block, gate, up, down, stream=None):
    _check(lib.moe_dequant_block(C.byref(d), _ptr(block), _ptr(gate), _ptr(up), _ptr(down), _stream(stream)))


# --- allocation helpers for callers (torch owns the memory) ----------------

def alloc_workspace(d: moe_desc, T: int, mode: int, device="cuda"):
    """A workspace of the size the library asks for (zero-filled; any contents would do)."""
    import torch
    n = moe_workspace_bytes(d, T, mode)
    if n == 0:
        raise MoeError(MOE_ERR_ARG, "invalid descriptor for workspace sizing")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def expert_ptr_table(blocks, block_bytes: int | None = None):
    """Device int64 table of E block addresses for a resident [E, block_bytes]
    uint8 tensor (or a list of per-expert uint8 tensors)."""
    import torch
    if isinstance(blocks, (list, tuple)):
        ptrs = [b.data_ptr() for b in blocks]
        dev = blocks[0].device
    else:
        bb = block_bytes or blocks.shape[1]
        base = blocks.data_ptr()
        ptrs = [base + e * bb for e in range(blocks.shape[0])]
        dev = blocks.device
    return torch.tensor(ptrs, dtype=torch.int64, device=dev)


MOE_SCALE_FLOOR, MOE_SCALE_CEIL = 0, 1


def moe_act_quant_fp8(x, rows, cols, block, rule, codes, scales, stream=None):
    _check(lib.moe_act_quant_fp8(_ptr(x), rows, cols, block, rule, _ptr(codes), _ptr(scales), _stream(stream)))


def moe_gemv_fp8(W, row_scale, x, rows, cols, y, stream=None):
    _check(lib.moe_gemv_fp8(_ptr(W), _ptr(row_scale), _ptr(x), rows, cols, _ptr(y), _stream(stream)))


class ExpertTier:
    """Owner of a moe_tier (pinned host blocks + HBM slots + the per-layer
    pointer tables); table(layer) is the expert_ptrs argument of the decode
    entry points."""

    def __init__(self, d, layers, host_blocks, slots, n_slots, table):
        self.d, self.E = d, d.E
        self._keep = (host_blocks, slots, table)
        h = C.c_void_p()
        _check(lib.moe_tier_create(C.byref(d), layers, _ptr(host_blocks), _ptr(slots), n_slots, _ptr(table),
                                   C.byref(h)))
        self.h = h
        self.table_tensor = table

    def table(self, layer):
        return self.table_tensor[layer * self.E:(layer + 1) * self.E]

    def update(self, idx_host, max_promote, stream=None):
        import numpy as np
        a = np.ascontiguousarray(idx_host, dtype=np.int32)
        _check(lib.moe_tier_update(self.h, a.ctypes.data_as(C.c_void_p), max_promote, _stream(stream)))

    def stats(self) -> dict:
        st = moe_tier_stats()
        _check(lib.moe_tier_get_stats(self.h, C.byref(st)))
        return {f: getattr(st, f) for f, _ in moe_tier_stats._fields_}

    def slot_of(self, layer, expert) -> int:
        return int(lib.moe_tier_slot_of(self.h, layer, expert))

    def close(self):
        if self.h:
            lib.moe_tier_destroy(self.h)
            self.h = None


def moe_prefetch_sink_bytes(d: moe_desc, n: int) -> int:
    return int(lib.moe_prefetch_sink_bytes(C.byref(d), n))


def moe_expert_prefetch(d, expert_ptrs, idx, n, sink, stream=None):
    _check(lib.moe_expert_prefetch(C.byref(d), _ptr(expert_ptrs), _ptr(idx), n, _ptr(sink),
                                   sink.numel() * sink.element_size(), _stream(stream)))
