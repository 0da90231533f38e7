// C ABI of the library (declared in include/moe_fp4.h): argument checks,
// workspace sizing and kernel launches on the caller's stream. No
// allocation, no synchronisation, no device reads on the host.
#include "../../include/moe_fp4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "moe_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = 0;
    return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int group_size(int fmt) { return fmt == MOE_FMT_NVFP4 ? 16 : (fmt == MOE_FMT_MXFP4 ? 32 : 0); }

int check_desc(const moe_desc* d) {
    if (!d) return fail(MOE_ERR_ARG, "desc is NULL");
    const int G = group_size(d->format);
    if (!G) return fail(MOE_ERR_ARG, "unknown format %d", d->format);
    if (d->H <= 0 || d->I <= 0 || d->E <= 0 || d->k <= 0)
        return fail(MOE_ERR_ARG, "H, I, E, k must be positive (H=%d I=%d E=%d k=%d)", d->H, d->I, d->E, d->k);
    if (d->k > d->E) return fail(MOE_ERR_ARG, "k=%d exceeds E=%d", d->k, d->E);
    if (d->H % G || d->I % G) return fail(MOE_ERR_ARG, "H=%d and I=%d must be multiples of the group size %d", d->H, d->I, G);
    return MOE_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
    if (!p) return fail(MOE_ERR_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(MOE_ERR_ARG, "%s is not %zu-byte aligned", name, align);
    return MOE_OK;
}

int check_ws(const void* ws, size_t have, size_t need) {
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (!aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (have < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

size_t moe_block_bytes(const moe_desc* d) {
    if (check_desc(d) != MOE_OK) return 0;
    const size_t n = (size_t)3 * d->H * d->I;
    return n / 2 + n / group_size(d->format);
}

int moe_block_layout(const moe_desc* d, int64_t off[7]) {
    int r = check_desc(d);
    if (r) return r;
    if (!off) return fail(MOE_ERR_ARG, "off is NULL");
    const int64_t codes = (int64_t)d->H * d->I / 2, scales = (int64_t)d->H * d->I / group_size(d->format);
    off[0] = 0;
    off[1] = codes;
    off[2] = 2 * codes;
    off[3] = 3 * codes;
    off[4] = 3 * codes + scales;
    off[5] = 3 * codes + 2 * scales;
    off[6] = 3 * codes + 3 * scales;
    return ok();
}

size_t moe_workspace_bytes(const moe_desc* d, int32_t T, int32_t mode) {
    if (check_desc(d) != MOE_OK || T < 0) return 0;
    switch (mode) {
        case MOE_MODE_ROUTE: return moe::route_ws_bytes(T, d->E);
        case MOE_MODE_DECODE: return moe::decode_ws_bytes(d->H, d->I, d->k, d->E);
        case MOE_MODE_PREFILL: return moe::prefill_ws_bytes(d->format, d->H, d->I, d->E, d->k, T);
        default: return 0;
    }
}

int moe_route(const moe_desc* d, const float* x, int32_t T, const float* Wr, int32_t* idx, float* w,
              float* logits_out, void* ws, size_t ws_bytes, void* stream) {
    int r;
    if ((r = check_desc(d))) return r;
    if (T < 1) return fail(MOE_ERR_ARG, "T=%d must be >= 1", T);
    if ((r = check_ptr(x, 16, "x")) || (r = check_ptr(Wr, 16, "Wr")) || (r = check_ptr(idx, 4, "idx")) ||
        (r = check_ptr(w, 4, "w")))
        return r;
    if (logits_out && !aligned(logits_out, 4)) return fail(MOE_ERR_ARG, "logits_out is not 4-byte aligned");
    if (!moe::route_supported(d->H, d->E, d->k))
        return fail(MOE_ERR_UNSUPPORTED, "router needs H %% 256 == 0, H <= 8192, E <= %d, k <= %d (H=%d E=%d k=%d)",
                    moe::kMaxE, moe::kMaxK, d->H, d->E, d->k);
    if ((r = check_ws(ws, ws_bytes, moe::route_ws_bytes(T, d->E)))) return r;
    return hip_status(moe::launch_route(d->H, d->E, d->k, T, x, Wr, idx, w, logits_out, ws,
                                        reinterpret_cast<hipStream_t>(stream)),
                      "router launch");
}

int moe_expert_decode(const moe_desc* d, const float* x, const void* const* expert_ptrs, const int32_t* idx,
                      const float* w, const moe_shared* shared, float* y, void* ws, size_t ws_bytes, void* stream) {
    int r;
    if ((r = check_desc(d))) return r;
    if ((r = check_ptr(x, 16, "x")) || (r = check_ptr(expert_ptrs, 8, "expert_ptrs")) ||
        (r = check_ptr(idx, 4, "idx")) || (r = check_ptr(w, 4, "w")) || (r = check_ptr(y, 4, "y")))
        return r;
    if (shared) {
        if ((r = check_ptr(shared->gate, 16, "shared->gate")) || (r = check_ptr(shared->up, 16, "shared->up")) ||
            (r = check_ptr(shared->down, 16, "shared->down")))
            return r;
    }
    if (d->k > moe::kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k=%d exceeds %d", d->k, moe::kMaxK);
    if (d->E > moe::kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E=%d exceeds %d", d->E, moe::kMaxE);
    moe::DecodePlan plan;
    if (!moe::plan_decode(d->format, d->H, d->I, &plan))
        return fail(MOE_ERR_UNSUPPORTED, "no decode kernel for H=%d I=%d (needs H %% 512 == 0, H <= 4096, I <= 4096)",
                    d->H, d->I);
    if ((r = check_ws(ws, ws_bytes, moe::decode_ws_bytes(d->H, d->I, d->k, d->E)))) return r;
    return hip_status(moe::launch_decode(d->format, plan, d->E, d->H, d->I, d->k, x, expert_ptrs, idx, w,
                                         shared ? shared->gate : nullptr, shared ? shared->up : nullptr,
                                         shared ? shared->down : nullptr, y, ws,
                                         reinterpret_cast<hipStream_t>(stream)),
                      "decode launch");
}

}  // extern "C"

namespace {

// Every argument check of moe_layer_decode except the workspace.
int layer_decode_checks(const moe_desc* d, const float* x, const float* Wr, const void* const* expert_ptrs,
                        const moe_shared* shared, float* y, int32_t* idx_out, float* w_out, moe::DecodePlan* plan) {
    int r;
    if ((r = check_desc(d))) return r;
    if ((r = check_ptr(x, 16, "x")) || (r = check_ptr(Wr, 16, "Wr")) || (r = check_ptr(expert_ptrs, 8, "expert_ptrs")) ||
        (r = check_ptr(y, 4, "y")) || (r = check_ptr(idx_out, 4, "idx_out")) || (r = check_ptr(w_out, 4, "w_out")))
        return r;
    if (shared) {
        if ((r = check_ptr(shared->gate, 16, "shared->gate")) || (r = check_ptr(shared->up, 16, "shared->up")) ||
            (r = check_ptr(shared->down, 16, "shared->down")))
            return r;
    }
    if (!moe::route_supported(d->H, d->E, d->k))
        return fail(MOE_ERR_UNSUPPORTED, "router needs H %% 256 == 0, H <= 8192, E <= %d, k <= %d (H=%d E=%d k=%d)",
                    moe::kMaxE, moe::kMaxK, d->H, d->E, d->k);
    if (!moe::plan_decode(d->format, d->H, d->I, plan))
        return fail(MOE_ERR_UNSUPPORTED, "no decode kernel for H=%d I=%d (needs H %% 512 == 0, H <= 4096, I <= 4096)",
                    d->H, d->I);
    return MOE_OK;
}

int layer_decode_launch(const moe_desc* d, const moe::DecodePlan& plan, const float* x, const float* Wr,
                        const void* const* expert_ptrs, const moe_shared* shared, float* y, int32_t* idx_out,
                        float* w_out, void* ws, void* stream) {
    return hip_status(moe::launch_layer_decode(d->format, plan, d->E, d->H, d->I, d->k, x, Wr, expert_ptrs,
                                               shared ? shared->gate : nullptr, shared ? shared->up : nullptr,
                                               shared ? shared->down : nullptr, y, idx_out, w_out, ws,
                                               reinterpret_cast<hipStream_t>(stream)),
                      "layer decode launch");
}

// ---- the allocation-free decode ----
// Its workspace: one copy of this array on every GPU the library runs on,
// loaded with the library's code object (zero-filled) and held until the
// process ends. In host code the name stands for a host-side shadow, not a
// device address: only the address hipGetSymbolAddress returns for the
// current device may reach a kernel.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch_addr[kMaxDevices];  // device address of scratch, per device, once looked up

// Device address of the current device's scratch (looked up on the first
// call on that device; a lookup by two threads at once stores the same value).
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_decode(const moe_desc* d, const float* x, const float* Wr, const void* const* expert_ptrs,
                     const moe_shared* shared, float* y, int32_t* idx_out, float* w_out, void* ws, size_t ws_bytes,
                     void* stream) {
    int r;
    moe::DecodePlan plan;
    if ((r = layer_decode_checks(d, x, Wr, expert_ptrs, shared, y, idx_out, w_out, &plan))) return r;
    if ((r = check_ws(ws, ws_bytes, moe::decode_ws_bytes(d->H, d->I, d->k, d->E)))) return r;
    return layer_decode_launch(d, plan, x, Wr, expert_ptrs, shared, y, idx_out, w_out, ws, stream);
}

int moe_layer_decode_noalloc(const moe_desc* d, const float* x, const float* Wr, const void* const* expert_ptrs,
                             const moe_shared* shared, float* y, int32_t* idx_out, float* w_out, void* stream) {
    int r;
    moe::DecodePlan plan;
    if ((r = layer_decode_checks(d, x, Wr, expert_ptrs, shared, y, idx_out, w_out, &plan))) return r;
    const size_t need = moe::decode_ws_bytes(d->H, d->I, d->k, d->E);
    if (need > kScratchBytes)
        return fail(MOE_ERR_WORKSPACE, "this layer needs %zu bytes of scratch; the static scratch holds %zu", need,
                    kScratchBytes);
    void* ws = nullptr;
    if ((r = scratch_address(&ws))) return r;
    return layer_decode_launch(d, plan, x, Wr, expert_ptrs, shared, y, idx_out, w_out, ws, stream);
}

int moe_expert_prefill(const moe_desc* d, const float* x, int32_t T, const void* const* expert_ptrs,
                       const int32_t* idx, const float* w, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                       const moe_prefill_debug* dbg, void* stream) {
    int r;
    if ((r = check_desc(d))) return r;
    if (T < 1) return fail(MOE_ERR_ARG, "T=%d must be >= 1", T);
    if ((r = check_ptr(x, 16, "x")) || (r = check_ptr(expert_ptrs, 8, "expert_ptrs")) ||
        (r = check_ptr(idx, 4, "idx")) || (r = check_ptr(w, 4, "w")) || (r = check_ptr(out, 16, "out")))
        return r;
    if (out_dtype != MOE_OUT_F32 && out_dtype != MOE_OUT_BF16) return fail(MOE_ERR_ARG, "unknown out_dtype %d", out_dtype);
    if (!moe::prefill_supported(d->format, d->H, d->I, d->E, d->k))
        return fail(MOE_ERR_UNSUPPORTED, "no prefill kernel for format=%d H=%d I=%d E=%d k=%d", d->format, d->H, d->I,
                    d->E, d->k);
    if (!moe::prefill_tokens_supported(d->H, d->I, d->k, T))
        return fail(MOE_ERR_UNSUPPORTED, "T=%d: the rounded activations would exceed 2 GiB (H=%d I=%d k=%d)", T, d->H,
                    d->I, d->k);
    if ((r = check_ws(ws, ws_bytes, moe::prefill_ws_bytes(d->format, d->H, d->I, d->E, d->k, T)))) return r;
    moe::PrefillDebug pd = {};
    if (dbg) {
        pd.x_bf16 = dbg->x_bf16;
        pd.x_codes = dbg->x_codes;
        pd.x_scales = dbg->x_scales;
        pd.h_pre = dbg->h_pre;
        pd.h_q = dbg->h_q;
        pd.perm = dbg->perm;
        pd.off = dbg->off;
        pd.tile_wait_polls = dbg->tile_wait_polls;
        pd.tile_wait_unmet = dbg->tile_wait_unmet;
    }
    return hip_status(moe::launch_prefill(d->format, d->H, d->I, d->E, d->k, T, x, expert_ptrs, idx, w, out,
                                          out_dtype == MOE_OUT_BF16, ws, dbg ? &pd : nullptr,
                                          reinterpret_cast<hipStream_t>(stream)),
                      "prefill launch");
}

int moe_dequant_block(const moe_desc* d, const void* block, float* gate, float* up, float* down, void* stream) {
    int r;
    if ((r = check_desc(d))) return r;
    if ((r = check_ptr(block, 16, "block")) || (r = check_ptr(gate, 4, "gate")) || (r = check_ptr(up, 4, "up")) ||
        (r = check_ptr(down, 4, "down")))
        return r;
    return hip_status(moe::launch_dequant(d->format, d->H, d->I, block, gate, up, down,
                                          reinterpret_cast<hipStream_t>(stream)),
                      "dequant launch");
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape (no tuned kernel)";
        case MOE_ERR_HIP: return "HIP launch error";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

int moe_act_quant_fp8(const float* x, int32_t rows, int32_t cols, int32_t block, int32_t rule, uint8_t* codes,
                      uint8_t* scales, void* stream) {
    if (rows < 0) return fail(MOE_ERR_ARG, "rows=%d is negative", rows);
    if (block != 32 && block != 128) return fail(MOE_ERR_ARG, "block=%d (32 or 128)", block);
    if (cols <= 0 || cols % block) return fail(MOE_ERR_ARG, "cols=%d must be a positive multiple of block=%d", cols, block);
    if (rule != MOE_SCALE_FLOOR && rule != MOE_SCALE_CEIL) return fail(MOE_ERR_ARG, "unknown scale rule %d", rule);
    if ((size_t)rows * cols > ((size_t)1 << 34)) return fail(MOE_ERR_ARG, "rows*cols too large");
    if (rows == 0) return ok();
    int r;
    if ((r = check_ptr(x, 16, "x")) || (r = check_ptr(codes, 4, "codes")) || (r = check_ptr(scales, 1, "scales")))
        return r;
    return hip_status(moe::launch_act_quant_fp8(x, rows, cols, block, rule, codes, scales, (hipStream_t)stream),
                      "act_quant_fp8 launch");
}

int moe_gemv_fp8(const uint8_t* W, const float* row_scale, const float* x, int32_t rows, int32_t cols, float* y,
                 void* stream) {
    if (rows < 0) return fail(MOE_ERR_ARG, "rows=%d is negative", rows);
    if (cols <= 0) return fail(MOE_ERR_ARG, "cols=%d must be positive", cols);
    if (!moe::gemv_fp8_supported(cols))
        return fail(MOE_ERR_UNSUPPORTED, "cols=%d: no kernel (512*d, d in 1..8, 10, 12, 16)", cols);
    if ((size_t)rows * cols >= ((size_t)1 << 31)) return fail(MOE_ERR_UNSUPPORTED, "rows*cols too large");
    if (rows == 0) return ok();
    int r;
    if ((r = check_ptr(W, 16, "W")) || (r = check_ptr(row_scale, 4, "row_scale")) || (r = check_ptr(x, 16, "x")) ||
        (r = check_ptr(y, 4, "y")))
        return r;
    return hip_status(moe::launch_gemv_fp8(W, row_scale, x, y, rows, cols, (hipStream_t)stream), "gemv_fp8 launch");
}

size_t moe_prefetch_sink_bytes(const moe_desc* d, int32_t n) {
    const size_t bb = moe_block_bytes(d);
    if (!bb || n < 1 || n > 1024) return 0;
    return (size_t)n * moe::prefetch_chunks(bb) * sizeof(uint32_t);
}

int moe_expert_prefetch(const moe_desc* d, const void* const* expert_ptrs, const int32_t* idx, int32_t n,
                        uint32_t* sink, size_t sink_bytes, void* stream) {
    int r;
    if ((r = check_desc(d))) return r;
    if (n < 1 || n > 1024) return fail(MOE_ERR_ARG, "n=%d (1..1024)", n);
    if ((r = check_ptr(expert_ptrs, 8, "expert_ptrs")) || (r = check_ptr(idx, 4, "idx")) ||
        (r = check_ptr(sink, 4, "sink")))
        return r;
    const size_t need = moe_prefetch_sink_bytes(d, n);
    if (sink_bytes < need) return fail(MOE_ERR_ARG, "sink has %zu bytes, needs %zu", sink_bytes, need);
    return hip_status(moe::launch_prefetch(expert_ptrs, idx, n, d->E, moe_block_bytes(d), sink,
                                           reinterpret_cast<hipStream_t>(stream)),
                      "prefetch launch");
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"
