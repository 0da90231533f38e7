"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, computes layouts and workspace sizes, and rejects bad arguments
with documented status codes before launching anything (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

import block_scaled_fp4_route_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    src = open(os.path.join(ROOT, "include", "moe_fp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    syms = header_symbols()
    assert set(syms) == set(m.EXPORTS)
    raw = C.CDLL(m.LIB_PATH)
    for s in syms:
        assert hasattr(raw, s), s


def test_layout_matches_oracle(orc):
    for fmt, H, I in (("nvfp4", 2560, 640), ("mxfp4", 4096, 2880), ("nvfp4", 512, 16), ("mxfp4", 1024, 96)):
        d = m.desc(H, I, 8, 2, fmt)
        assert m.moe_block_layout(d) == orc.layout(fmt, H, I)
        assert m.moe_block_bytes(d) == orc.layout(fmt, H, I)[6]


def test_workspace_sizes_positive_and_monotone():
    d = m.desc(2560, 640, 512, 10, "nvfp4")
    for mode in (m.MOE_MODE_ROUTE, m.MOE_MODE_DECODE):
        assert m.moe_workspace_bytes(d, 1, mode) >= 4096
    assert m.moe_workspace_bytes(d, 64, m.MOE_MODE_ROUTE) > m.moe_workspace_bytes(d, 1, m.MOE_MODE_ROUTE)
    assert m.moe_workspace_bytes(m.desc(2560, 640, 512, 10, 7), 1, m.MOE_MODE_DECODE) == 0


def _err(fn, *a):
    with pytest.raises(m.MoeError) as ei:
        fn(*a)
    return ei.value.status


FAKE = 1 << 20          # a 16-byte-aligned, never dereferenced address
ODD = FAKE + 4          # misaligned for 16-byte arguments


def test_descriptor_errors():
    for bad in (m.desc(0, 640, 8, 2, "nvfp4"), m.desc(2560, 640, 8, 9, "nvfp4"),
                m.desc(2560, 640 + 8, 8, 2, "nvfp4"), m.desc(2560, 640, 8, 2, 5)):
        assert _err(m.moe_route, bad, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, 0) == m.MOE_ERR_ARG


def test_route_argument_errors():
    d = m.desc(2560, 640, 64, 10, "nvfp4")
    assert _err(m.moe_route, d, None, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, 0) == m.MOE_ERR_ARG
    assert _err(m.moe_route, d, ODD, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, 0) == m.MOE_ERR_ARG
    assert _err(m.moe_route, d, FAKE, 0, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, 0) == m.MOE_ERR_ARG
    assert _err(m.moe_route, d, FAKE, 1, FAKE, FAKE, FAKE, None, None, 0, 0) == m.MOE_ERR_WORKSPACE
    assert _err(m.moe_route, d, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 16, 0) == m.MOE_ERR_WORKSPACE
    assert _err(m.moe_route, d, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE + 16, 1 << 20, 0) == m.MOE_ERR_WORKSPACE
    big = m.desc(2560, 640, 2048, 10, "nvfp4")
    assert _err(m.moe_route, big, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 24, 0) == m.MOE_ERR_UNSUPPORTED


def test_decode_argument_errors():
    d = m.desc(2560, 640, 64, 10, "nvfp4")
    assert _err(m.moe_expert_decode, d, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 20, 0) == m.MOE_ERR_ARG
    assert _err(m.moe_expert_decode, d, FAKE, FAKE + 4, FAKE, FAKE, None, FAKE, FAKE, 1 << 20, 0) == m.MOE_ERR_ARG
    assert _err(m.moe_expert_decode, d, FAKE, FAKE, FAKE, FAKE, (FAKE, None, FAKE), FAKE, FAKE, 1 << 20, 0) \
        == m.MOE_ERR_ARG
    assert _err(m.moe_expert_decode, d, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1024, 0) == m.MOE_ERR_WORKSPACE
    odd_h = m.desc(2560 + 16, 640, 64, 10, "nvfp4")       # H not a multiple of 512
    assert _err(m.moe_expert_decode, odd_h, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 24, 0) \
        == m.MOE_ERR_UNSUPPORTED
    big_k = m.desc(2560, 640, 64, 40, "nvfp4")
    assert _err(m.moe_expert_decode, big_k, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 24, 0) \
        == m.MOE_ERR_UNSUPPORTED


def test_prefill_argument_errors():
    d = m.desc(2560, 640, 512, 10, "nvfp4")
    need = m.moe_workspace_bytes(d, 100, m.MOE_MODE_PREFILL)
    f32 = m.MOE_OUT_F32

    def call(d=d, x=FAKE, T=100, ptrs=FAKE, idx=FAKE, w=FAKE, out=FAKE, od=f32, ws=FAKE, wsb=need):
        return _err(m.moe_expert_prefill, d, x, T, ptrs, idx, w, out, od, ws, wsb, None, 0)

    assert call(T=0) == m.MOE_ERR_ARG
    assert call(T=-3) == m.MOE_ERR_ARG
    assert call(x=None) == m.MOE_ERR_ARG
    assert call(x=ODD) == m.MOE_ERR_ARG          # x: 16-byte alignment
    assert call(ptrs=None) == m.MOE_ERR_ARG
    assert call(idx=None) == m.MOE_ERR_ARG
    assert call(w=None) == m.MOE_ERR_ARG
    assert call(out=ODD) == m.MOE_ERR_ARG
    assert call(od=7) == m.MOE_ERR_ARG            # unknown output type
    assert call(ws=None, wsb=0) == m.MOE_ERR_WORKSPACE
    assert call(wsb=need - 256) == m.MOE_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == m.MOE_ERR_WORKSPACE   # 256-byte alignment
    # no kernel for H % 256 != 0 (NVFP4) or H % 512 != 0 (MXFP4), nor for a
    # token count whose rounded activations exceed 2 GiB
    assert call(d=m.desc(2560 + 128, 640, 512, 10, "nvfp4"), wsb=1 << 40) == m.MOE_ERR_UNSUPPORTED
    assert call(d=m.desc(2560 + 256, 640, 384, 6, "mxfp4"), wsb=1 << 40) == m.MOE_ERR_UNSUPPORTED
    assert call(T=1 << 20, wsb=1 << 40) == m.MOE_ERR_UNSUPPORTED


def test_layer_decode_argument_errors():
    d = m.desc(2560, 640, 512, 10, "nvfp4")
    need = m.moe_workspace_bytes(d, 1, m.MOE_MODE_DECODE)
    args = [d, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, need, 0]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return _err(m.moe_layer_decode, *a)

    assert call(a1=None) == m.MOE_ERR_ARG           # x
    assert call(a2=FAKE + 4) == m.MOE_ERR_ARG       # Wr misaligned
    assert call(a3=None) == m.MOE_ERR_ARG           # expert_ptrs
    assert call(a4=(FAKE, FAKE, None)) == m.MOE_ERR_ARG
    assert call(a6=None) == m.MOE_ERR_ARG           # idx_out
    assert call(a7=FAKE + 2) == m.MOE_ERR_ARG       # w_out misaligned
    assert call(a9=need - 1) == m.MOE_ERR_WORKSPACE
    assert call(a8=None, a9=0) == m.MOE_ERR_WORKSPACE
    assert call(a0=m.desc(2560, 640, 2048, 10, "nvfp4"), a9=1 << 24) == m.MOE_ERR_UNSUPPORTED  # E > 1024
    assert call(a0=m.desc(2560 + 256, 640, 512, 10, "nvfp4"), a9=1 << 24) == m.MOE_ERR_UNSUPPORTED  # H % 512
    assert call(a0=m.desc(2560, 640, 512, 0, "nvfp4")) == m.MOE_ERR_ARG


def test_layer_decode_noalloc_argument_errors():
    """Argument errors come before the scratch lookup (no device needed), and
    the largest supported layer fits the static scratch."""
    d = m.desc(2560, 640, 512, 10, "nvfp4")
    args = [d, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return _err(m.moe_layer_decode_noalloc, *a)

    assert call(a1=None) == m.MOE_ERR_ARG
    assert call(a2=FAKE + 4) == m.MOE_ERR_ARG
    assert call(a3=None) == m.MOE_ERR_ARG
    assert call(a4=(FAKE, None, FAKE)) == m.MOE_ERR_ARG
    assert call(a7=FAKE + 2) == m.MOE_ERR_ARG
    assert call(a0=m.desc(2560, 640, 2048, 10, "nvfp4")) == m.MOE_ERR_UNSUPPORTED
    assert call(a0=m.desc(2560, 8192, 512, 10, "nvfp4")) == m.MOE_ERR_UNSUPPORTED
    big = m.desc(4096, 4096, 1024, 32, "nvfp4")
    assert m.moe_workspace_bytes(big, 1, m.MOE_MODE_DECODE) <= m.MOE_NOALLOC_SCRATCH_BYTES


def test_fp8_argument_errors():
    q = m.moe_act_quant_fp8
    q(FAKE, 0, 4096, 32, 0, FAKE, FAKE, 0)  # empty: nothing enqueued, MOE_OK
    assert _err(q, FAKE, -1, 4096, 32, 0, FAKE, FAKE, 0) == m.MOE_ERR_ARG
    assert _err(q, FAKE, 4, 4096, 64, 0, FAKE, FAKE, 0) == m.MOE_ERR_ARG       # block
    assert _err(q, FAKE, 4, 4000, 128, 0, FAKE, FAKE, 0) == m.MOE_ERR_ARG      # cols % block
    assert _err(q, FAKE, 4, 4096, 32, 2, FAKE, FAKE, 0) == m.MOE_ERR_ARG       # rule
    assert _err(q, None, 4, 4096, 32, 0, FAKE, FAKE, 0) == m.MOE_ERR_ARG
    assert _err(q, ODD, 4, 4096, 32, 0, FAKE, FAKE, 0) == m.MOE_ERR_ARG
    assert _err(q, FAKE, 4, 4096, 32, 0, FAKE + 2, FAKE, 0) == m.MOE_ERR_ARG   # codes alignment
    g = m.moe_gemv_fp8
    g(FAKE, FAKE, FAKE, 0, 2560, FAKE, 0)
    assert _err(g, FAKE, FAKE, FAKE, 8, 2560 + 64, FAKE, 0) == m.MOE_ERR_UNSUPPORTED
    assert _err(g, FAKE, FAKE, FAKE, 8, 9 * 512, FAKE, 0) == m.MOE_ERR_UNSUPPORTED
    assert _err(g, FAKE, FAKE, FAKE, 8, 20 * 512, FAKE, 0) == m.MOE_ERR_UNSUPPORTED
    assert _err(g, FAKE, FAKE, FAKE, -1, 2560, FAKE, 0) == m.MOE_ERR_ARG
    assert _err(g, FAKE + 8, FAKE, FAKE, 8, 2560, FAKE, 0) == m.MOE_ERR_ARG   # W alignment
    assert _err(g, FAKE, FAKE, None, 8, 2560, FAKE, 0) == m.MOE_ERR_ARG


def test_tier_argument_errors():
    import ctypes
    d = m.desc(2560, 640, 64, 10, "nvfp4")
    out = ctypes.c_void_p()
    L = m.lib
    assert L.moe_tier_create(ctypes.byref(d), 2, FAKE, FAKE, 4, FAKE, None) == m.MOE_ERR_ARG       # out NULL
    assert L.moe_tier_create(ctypes.byref(d), 0, FAKE, FAKE, 4, FAKE, ctypes.byref(out)) == m.MOE_ERR_ARG
    assert L.moe_tier_create(ctypes.byref(d), 2, FAKE, FAKE, -1, FAKE, ctypes.byref(out)) == m.MOE_ERR_ARG
    assert L.moe_tier_create(ctypes.byref(d), 2, None, FAKE, 4, FAKE, ctypes.byref(out)) == m.MOE_ERR_ARG
    assert L.moe_tier_create(ctypes.byref(d), 2, FAKE, None, 4, FAKE, ctypes.byref(out)) == m.MOE_ERR_ARG
    assert L.moe_tier_create(ctypes.byref(d), 2, FAKE + 16, FAKE, 4, FAKE, ctypes.byref(out)) == m.MOE_ERR_ARG
    bad = m.desc(2560, 640, 64, 11, 7)
    assert L.moe_tier_create(ctypes.byref(bad), 2, FAKE, FAKE, 4, FAKE, ctypes.byref(out)) == m.MOE_ERR_ARG
    assert out.value is None
    assert L.moe_tier_update(None, FAKE, 1, None) == m.MOE_ERR_ARG
    assert L.moe_tier_destroy(None) == m.MOE_OK
    assert L.moe_tier_slot_of(None, 0, 0) == -1


def test_prefetch_argument_errors():
    d = m.desc(2560, 640, 64, 10, "nvfp4")
    nch = -(-m.moe_block_bytes(d) // 65536)
    assert m.moe_prefetch_sink_bytes(d, 10) == 10 * nch * 4
    assert m.moe_prefetch_sink_bytes(d, 0) == 0
    L = m.lib
    import ctypes
    assert L.moe_expert_prefetch(ctypes.byref(d), FAKE, FAKE, 0, FAKE, 1 << 20, None) == m.MOE_ERR_ARG
    assert L.moe_expert_prefetch(ctypes.byref(d), FAKE + 4, FAKE, 10, FAKE, 1 << 20, None) == m.MOE_ERR_ARG
    assert L.moe_expert_prefetch(ctypes.byref(d), FAKE, FAKE, 10, FAKE, 16, None) == m.MOE_ERR_ARG
    assert L.moe_expert_prefetch(ctypes.byref(d), FAKE, None, 10, FAKE, 1 << 20, None) == m.MOE_ERR_ARG


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert m.lib.moe_status_string(s)
    assert m.lib.moe_status_string(-99) == b"unknown status"


def test_oracle_and_library_share_nothing():
    """The oracle and the GPU library import, include and link nothing of
    each other."""
    pkg = os.path.join(ROOT, "block_scaled_fp4_route_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.lower().replace("oracle-free", ""), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            txt = open(os.path.join(ROOT, "oracle", f)).read()
            assert "block_scaled_fp4_route_amd" not in txt and "moe_fp4.h" not in txt, f
