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
// (selects, no branches: a divergent branch makes LLVM wait for every
// outstanding load at its join)
__device__ __forceinline__ float ue8m0_to_f32(uint32_t u) {
    u &= 0xFFu;
    uint32_t b = u << 23;
    b = u == 0u ? 0x00400000u : b;
    b = u == 0xFFu ? 0x7FC00000u : b;
    return __uint_as_float(b);
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

// sum_{i<16} e2m1(code i) * x[i] over the 16 codes of (w0, w1) (w0 first,
// low nibble first), one fma chain.
__device__ __forceinline__ float dot16_fp4(uint32_t w0, uint32_t w1, const float* x) {
    f2v p0 = fp4x2<0>(w0), p1 = fp4x2<1>(w0), p2 = fp4x2<2>(w0), p3 = fp4x2<3>(w0);
    f2v p4 = fp4x2<0>(w1), p5 = fp4x2<1>(w1), p6 = fp4x2<2>(w1), p7 = fp4x2<3>(w1);
    float a = p0.x * x[0];
    a = fmaf(p0.y, x[1], a);
    a = fmaf(p1.x, x[2], a);
    a = fmaf(p1.y, x[3], a);
    a = fmaf(p2.x, x[4], a);
    a = fmaf(p2.y, x[5], a);
    a = fmaf(p3.x, x[6], a);
    a = fmaf(p3.y, x[7], a);
    a = fmaf(p4.x, x[8], a);
    a = fmaf(p4.y, x[9], a);
    a = fmaf(p5.x, x[10], a);
    a = fmaf(p5.y, x[11], a);
    a = fmaf(p6.x, x[12], a);
    a = fmaf(p6.y, x[13], a);
    a = fmaf(p7.x, x[14], a);
    a = fmaf(p7.y, x[15], a);
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

// Unsigned max over all 64 lanes (uniform result).
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dppu<0xB1>(v));
    v = max(v, dppu<0x4E>(v));
    v = max(v, dppu<0x141>(v));
    v = max(v, dppu<0x140>(v));
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key; +0
// and -0 must be folded before): negative values have all bits flipped,
// others get the sign bit set. A NaN with the sign bit clear maps above
// +inf.
__device__ __forceinline__ uint32_t f32_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// silu(g) * u = g / (1 + e^-g) * u. expf, not __expf: the fast form rounds
// -g * log2(e) to fp32 before the hardware exp2, a relative error of about
// |g| * 2^-24 in e^-g (1e-6 at g = -20); expf keeps it to a few ulp. For
// g < -ln(FLT_MAX) e^-g overflows and the result is +-0.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

constexpr int kTopkMaxE = 1024;

// Top-k of E <= 64 * NI logits by one full wave: afterwards lane j < kk
// holds the j-th chosen expert (larger logit first, lower expert index first
// among equal logits) in my_e and its weight, the softmax renormalised over
// the first kk chosen, in my_w. f[i] is logit lane * NI + i of this lane
// (any value past E - 1); kk <= E.
// The logits are compared as order-preserving integer keys (-0 folded onto
// +0; a NaN ranks above +inf, so every chosen index is in [0, E)).
// Lane l holds experts l*NI .. l*NI + NI - 1 and first sorts them (key
// descending, then index ascending; Batcher's odd-even merge network over
// registers). A round then only compares the lanes' heads: the largest head
// wins, and among equal heads the lowest lane, which holds the lowest expert
// indices; the winning lane shifts its sorted list by one.
template <int NI>
__device__ __forceinline__ void topk_select_vals(const float (&f)[NI], int E, int kk, int& my_e, float& my_w) {
    const int lane = threadIdx.x & 63;
    uint32_t v[NI];
    int ix[NI];
    {
#pragma unroll
        for (int i = 0; i < NI; i++) {
            v[i] = lane * NI + i < E ? f32_key(f[i] + 0.0f) : 0u;  // + 0 folds -0 onto +0; 0 = padding
            ix[i] = i;
        }
    }
    // local sort: position a before b iff v[a] > v[b], or equal and ix[a] < ix[b]
#pragma unroll
    for (int p = 1; p < NI; p <<= 1) {
#pragma unroll
        for (int q = p; q >= 1; q >>= 1) {
#pragma unroll
            for (int j = q % p; j + q < NI; j += 2 * q) {
#pragma unroll
                for (int i = 0; i < q && i + j + q < NI; i++) {
                    const int lo = i + j, hi = i + j + q;
                    if (lo / (2 * p) == hi / (2 * p)) {
                        const bool keep = v[lo] > v[hi] || (v[lo] == v[hi] && ix[lo] < ix[hi]);
                        const uint32_t va = v[lo], vb = v[hi];
                        const int ia = ix[lo], ib = ix[hi];
                        v[lo] = keep ? va : vb;
                        v[hi] = keep ? vb : va;
                        ix[lo] = keep ? ia : ib;
                        ix[hi] = keep ? ib : ia;
                    }
                }
            }
        }
    }
    my_e = -1;
    uint32_t my_k = 0;
    for (int j = 0; j < kk; j++) {
        const uint32_t m = wave_max_u32(v[0]);
        const unsigned long long b = __ballot(v[0] == m);  // never empty: m is some lane's head
        const int L = __ffsll((long long)b) - 1;
        const int e = L * NI + __builtin_amdgcn_readlane(ix[0], L);
        if (lane == L) {
#pragma unroll
            for (int i = 0; i + 1 < NI; i++) {
                v[i] = v[i + 1];
                ix[i] = ix[i + 1];
            }
            v[NI - 1] = 0u;
        }
        if (lane == j) {
            my_e = e;
            my_k = m;
        }
    }
    const float my_l = key_f32(my_k);
    const float lmax = __shfl(my_l, 0, 64);
    const float ex = lane < kk ? expf(my_l - lmax) : 0.f;
    const float z = wave_sum(ex);
    my_w = ex / z;
}

// As topk_select_vals, the logits read by LOAD(e) (0 <= e < E); all loads
// are issued before the first use.
template <int NI, class LOAD>
__device__ __forceinline__ void topk_select_n(LOAD load, int E, int kk, int& my_e, float& my_w) {
    const int lane = threadIdx.x & 63;
    float f[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) f[i] = load(min(lane * NI + i, E - 1));
    topk_select_vals<NI>(f, E, kk, my_e, my_w);
}

// topk_select_n with the smallest register count that holds E logits.
template <class LOAD>
__device__ __forceinline__ void topk_select(LOAD load, int E, int k, int& my_e, float& my_w) {
    if (E <= 64)
        topk_select_n<1>(load, E, k, my_e, my_w);
    else if (E <= 128)
        topk_select_n<2>(load, E, k, my_e, my_w);
    else if (E <= 256)
        topk_select_n<4>(load, E, k, my_e, my_w);
    else if (E <= 512)
        topk_select_n<8>(load, E, k, my_e, my_w);
    else
        topk_select_n<16>(load, E, k, my_e, my_w);
}

// As topk_select, writing idx[0..k) and w[0..k).
template <class LOAD>
__device__ __forceinline__ void topk_wave(LOAD load, int E, int k, int32_t* idx, float* w) {
    int e;
    float wt;
    topk_select(load, E, k, e, wt);
    const int lane = threadIdx.x & 63;
    if (lane < k) {
        idx[lane] = e;
        w[lane] = wt;
    }
}

// ---------------------------------------------------------------------------
// Buffer-resource loads over one expert block. The base address is made
// wave-uniform (it lives in SGPRs), offsets are 32-bit byte offsets, and the
// hardware returns 0 for any offset at or beyond `bytes` instead of reading
// past the block. Word 3 (0x00020000) is the raw-buffer format of the gfx9
// family.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
// p and bytes must be wave-uniform; they are read from the first active lane.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(p)), (short)0,
                                             (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
// Workgroup barrier that orders LDS only: every LDS access before it is done
// and visible after it, while global loads stay in flight across it (a plain
// __syncthreads also waits for every outstanding global load, which would
// drain any prefetch).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Buffer offset beyond every buffer the kernels address: loads from it
// return 0 without touching memory (used for loads that must be issued but
// have nothing to read, so that every path issues the same loads).
constexpr uint32_t kOOB = 0x7FFFFFF0u;

// The wave's index in its workgroup, as a value the compiler knows is uniform.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ uint32_t ld_b32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint2 ld_b64(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t ld_b8(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

}  // namespace moe
