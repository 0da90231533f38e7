// Host-side launch entry points of the kernels (internal to the library).
// Each returns hipSuccess or the launch error; shapes were validated by the
// C-ABI layer (moe_api.cpp) before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Workspace: [0, kCounterBytes) is reserved (no kernel writes it, so it
// stays as the caller zero-filled it), then the data regions of each mode.
constexpr size_t kCounterBytes = 4096;
constexpr int kMaxK = 32;
constexpr int kMaxE = 1024;
constexpr int kRouteSplitMaxT = 16;  // tokens routed by the row-split kernels

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// ---- decode ----
struct DecodePlan {
    int gate_D;        // dwords of codes per lane per gate/up row (H / 512)
    int gate_P;        // row pairs per wave
    int gate_wg_per_slot;
    int down_L;        // lanes per down row (16 or 64)
    int down_D;        // dwords per lane per down row
    int down_RB;       // rows per workgroup
    int down_nrb;      // row blocks (H / RB)
};
bool plan_decode(int fmt, int H, int I, DecodePlan* p);
size_t decode_ws_bytes(int H, int I, int k, int E);

hipError_t launch_decode(int fmt, const DecodePlan& p, int E, int H, int I, int k, const float* x,
                         const void* const* expert_ptrs, const int32_t* idx, const float* w,
                         const uint16_t* sh_gate, const uint16_t* sh_up, const uint16_t* sh_down, float* y,
                         void* ws, hipStream_t s);

hipError_t launch_layer_decode(int fmt, const DecodePlan& p, int E, int H, int I, int k, const float* x,
                               const float* Wr, const void* const* expert_ptrs, const uint16_t* sh_gate,
                               const uint16_t* sh_up, const uint16_t* sh_down, float* y, int32_t* idx_out,
                               float* w_out, void* ws, hipStream_t s);

// ---- router ----
size_t route_ws_bytes(int T, int E);
bool route_supported(int H, int E, int k);
hipError_t launch_route(int H, int E, int k, int T, const float* x, const float* Wr, int32_t* idx, float* w,
                        float* logits_out, void* ws, hipStream_t s);

// ---- dequant (test support) ----
hipError_t launch_dequant(int fmt, int H, int I, const void* block, float* gate, float* up, float* down,
                          hipStream_t s);

// ---- prefill ----
bool prefill_supported(int fmt, int H, int I, int E, int k);
bool prefill_tokens_supported(int H, int I, int k, int T);
size_t prefill_ws_bytes(int fmt, int H, int I, int E, int k, int T);
struct PrefillDebug {
    uint16_t* x_bf16;
    uint8_t* x_codes;
    uint8_t* x_scales;
    float* h_pre;
    float* h_q;
    int32_t* perm;
    int32_t* off;
    int tile_wait_polls;  // > 0: poll limit of the GEMM launch's waits
    int tile_wait_unmet;  // nonzero: those waits ask for one more publication than exists
};
hipError_t launch_prefill(int fmt, int H, int I, int E, int k, int T, const float* x,
                          const void* const* expert_ptrs, const int32_t* idx, const float* w, void* out,
                          int out_bf16, void* ws, const PrefillDebug* dbg, hipStream_t s);

// ---- FP8 activation quantiser and row-scaled GEMV ----
constexpr int kScaleFloor = 0;  // OCP MX shared exponent floor(log2 amax) - 8
constexpr int kScaleCeil = 1;   // smallest exponent with amax <= 448 * 2^X
hipError_t launch_act_quant_fp8(const float* x, int rows, int cols, int block, int rule, uint8_t* codes,
                                uint8_t* scales, hipStream_t s);
bool gemv_fp8_supported(int cols);
hipError_t launch_gemv_fp8(const uint8_t* W, const float* rs, const float* x, float* y, int rows, int cols,
                           hipStream_t s);

// ---- speculative expert prefetch ----
int prefetch_chunks(size_t block_bytes);
hipError_t launch_prefetch(const void* const* ptrs, const int32_t* idx, int n, int E, size_t block_bytes,
                           uint32_t* sink, hipStream_t s);

}  // namespace moe
