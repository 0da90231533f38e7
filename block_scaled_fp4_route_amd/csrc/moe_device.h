// Device helpers shared by the gfx950 kernels: scale and e2m1 decode, wave
// reductions. CDNA4 only (wave64, v_cvt_scalef32_pk_f32_fp4, DPP).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f2v __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kFmtNvfp4 = 1;
constexpr int kFmtMxfp4 = 2;

template <int FMT>
struct Fmt;
template <>
struct Fmt<kFmtNvfp4> {
    static constexpr int G = 16;  // codes per scale
};
template <>
struct Fmt<kFmtMxfp4> {
    static constexpr int G = 32;
};

// E4M3 (OCP FP8 E4M3FN) byte (low byte of b) -> fp32: exponent bias 7,
// subnormal M/8 * 2^-6, S.1111.111 is NaN. gfx950's v_cvt_f32_fp8 decodes
// exactly this encoding (checked over all 256 bytes).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// UE8M0 byte -> fp32: 2^(u - 127); 255 is NaN; 0 is the fp32 subnormal 2^-127.
__device__ __forceinline__ float ue8m0_to_f32(uint32_t u) {
    u &= 0xFFu;
    if (u == 0xFFu) return __uint_as_float(0x7FC00000u);
    return u ? __uint_as_float(u << 23) : __uint_as_float(0x00400000u);
}

template <int FMT>
__device__ __forceinline__ float scale_to_f32(uint32_t b) {
    if constexpr (FMT == kFmtNvfp4)
        return e4m3_to_f32(b);
    else
        return ue8m0_to_f32(b);
}

// Two e2m1 codes of byte SEL of w -> fp32 (.x = low nibble). The hardware
// conversion takes an E8M0-style scale from the exponent of its second
// operand; 1.0 leaves the values unscaled.
template <int SEL>
__device__ __forceinline__ f2v fp4x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// sum_{i<8} e2m1(nibble i of w) * x[i], nibble 0 = low nibble of byte 0.
__device__ __forceinline__ float dot8_fp4(uint32_t w, const float* x) {
    f2v p0 = fp4x2<0>(w), p1 = fp4x2<1>(w), p2 = fp4x2<2>(w), p3 = fp4x2<3>(w);
    float a = p0.x * x[0];
    a = fmaf(p0.y, x[1], a);
    a = fmaf(p1.x, x[2], a);
    a = fmaf(p1.y, x[3], a);
    a = fmaf(p2.x, x[4], a);
    a = fmaf(p2.y, x[5], a);
    a = fmaf(p3.x, x[6], a);
    a = fmaf(p3.y, x[7], a);
    return a;
}

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each row of 16 lanes; every lane of the row receives the sum.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float v) {
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    v += dppf<0x141>(v);
    v += dppf<0x140>(v);
    return v;
}

// Sum over all 64 lanes of the wave (result uniform, in every lane).
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (a + b) + (c + d);
}

// Max over all 64 lanes (uniform result).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dppf<0xB1>(v));
    v = fmaxf(v, dppf<0x4E>(v));
    v = fmaxf(v, dppf<0x141>(v));
    v = fmaxf(v, dppf<0x140>(v));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// ---------------------------------------------------------------------------
// Cross-workgroup hand-off inside one kernel.
// Data that one workgroup produces for another is written and read with
// agent-scope atomic accesses, which the memory system keeps coherent across
// the chip's XCDs (their L2s are not coherent with each other), and a
// producer waits for its own stores to complete (s_waitcnt) before it bumps
// a completion counter. This avoids agent-scope fences, whose L2 write-back
// costs far more than the few kilobytes handed over here.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
    return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_agent(int* p, int v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory access this wave issued has completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Spin (bounded) until *cnt >= target. Returns false on timeout. The bound
// (about 2^21 polls with a short sleep, tenths of a second) is far beyond
// any legitimate wait and only ends a wait that could otherwise never end.
__device__ __forceinline__ bool wait_count(const int* cnt, int target) {
    for (int it = 0; it < (1 << 21); it++) {
        if (ld_agent(cnt) >= target) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

}  // namespace moe
