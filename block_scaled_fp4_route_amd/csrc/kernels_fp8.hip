// FP8 kernels for gfx950 beside the MoE path:
//
//  1. k_act_quant_fp8: activations to E4M3 codes with one UE8M0 (power of
//     two) scale per block of 32 or 128 values along the row ([D] "Three
//     bugs", item 2: DeepSeek's activation quantiser writes FP8 with ue8m0
//     scales; OCP MX: MXFP8 = E4M3 elements, E8M0 scale, blocks of 32).
//  2. k_gemv_fp8: y = s * (W x) for a matrix of E4M3 codes with one fp32
//     scale per row ([Q] "The engine", item 4: the FP8 row-scaled
//     matrix-vector kernel; [Q] "Why this model, of all models": the large
//     dense matrices stored in FP8 with one scale per row).
//
// Both are HBM streams: every byte is read once with 16- or 8-byte loads per
// lane, whole waves on contiguous memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// 1. activation quantiser
//
// Workgroup b covers 256 * kQuantPer float4 pieces; thread t takes
// pieces 256 kQuantPer b + t + 256 j (j < kQuantPer), so for every j
// the LPB = block/4 lanes of a block are consecutive and aligned and the
// block maximum is a butterfly over LPB lanes. Shared exponent X from the
// exponent field of the block maximum a = m * 2^(e - 127) (m in [1, 2),
// e = biased exponent):
//   floor rule (OCP MX):  X = floor(log2 a) - 8 = e - 135 (8 = largest
//                         exponent of E4M3; quotients up to 511 saturate);
//   ceil rule:            the smallest X with a <= 448 * 2^X: e - 135, plus
//                         one when m > 1.75 (448 = 1.75 * 2^8).
// A subnormal or zero maximum gives X = -127. X is clamped to [-127, 127]
// and stored as the byte X + 127 (0 for an all-zero block). The quotients
// v * 2^-X are exact (2^-X is a normal fp32 power of two), clamped to +-448
// and rounded to nearest even by v_cvt_pk_fp8_f32 (OCP E4M3FN on gfx950).
constexpr int kQuantPer = 2;  // float4 pieces per thread (1 and 4 measured slower)

template <int LPB>
__device__ __forceinline__ void quant_piece(const float4 v, size_t i, int rule, uint32_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales) {
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int o = 1; o < LPB; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    const uint32_t ab = __float_as_uint(a);
    const int e = (int)(ab >> 23);
    int X = e - 135 + ((rule == kScaleCeil && (ab & 0x7FFFFFu) > 0x600000u) ? 1 : 0);
    X = e == 0 ? -127 : min(127, max(-127, X));
    const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X
    auto q = [inv](float t) { return fminf(fmaxf(t * inv, -448.0f), 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q(v.x), q(v.y), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q(v.z), q(v.w), w, true);
    codes[i] = (uint32_t)w;
    if ((threadIdx.x & (LPB - 1)) == 0) scales[i / LPB] = a == 0.0f ? 0 : (uint8_t)(X + 127);
}

template <int LPB>
__global__ __launch_bounds__(256) void k_act_quant_fp8(const float4* __restrict__ x, size_t n4, int rule,
                                                       uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const size_t base = (size_t)blockIdx.x * 256 * kQuantPer + threadIdx.x;
    float4 v[kQuantPer];
#pragma unroll
    for (int j = 0; j < kQuantPer; j++)
        if (base + 256 * j < n4) v[j] = x[base + 256 * j];
#pragma unroll
    for (int j = 0; j < kQuantPer; j++)
        // n4 is a multiple of LPB and 256 of LPB: whole blocks are in or out
        if (base + 256 * j < n4) quant_piece<LPB>(v[j], base + 256 * j, rule, codes, scales);
}

hipError_t launch_act_quant_fp8(const float* x, int rows, int cols, int block, int rule, uint8_t* codes,
                                uint8_t* scales, hipStream_t s) {
    const size_t n4 = (size_t)rows * cols / 4;
    const dim3 grid((unsigned)((n4 + 256 * kQuantPer - 1) / (256 * kQuantPer)));
    const float4* x4 = reinterpret_cast<const float4*>(x);
    uint32_t* c4 = reinterpret_cast<uint32_t*>(codes);
    if (block == 32)
        hipLaunchKernelGGL(k_act_quant_fp8<8>, grid, dim3(256), 0, s, x4, n4, rule, c4, scales);
    else
        hipLaunchKernelGGL(k_act_quant_fp8<32>, grid, dim3(256), 0, s, x4, n4, rule, c4, scales);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 2. row-scaled FP8 GEMV
//
// A wave owns R consecutive rows. Lane l owns the 8-byte code pieces
// p = l + 64*i (i < D) of every row, i.e. columns 8p .. 8p+7 (cols = 512*D),
// and keeps those x values in registers for all its rows. The R*D loads of
// a wave's rows are issued together (rows past the end read the zero-length
// out-of-range offset), then each row is reduced over the wave with DPP and
// multiplied by its scale. E4M3 codes are decoded two at a time by
// v_cvt_pk_f32_fp8 (exact); products and sums in fp32.
template <int D, int R>
__global__ __launch_bounds__(256) void k_gemv_fp8(const uint8_t* __restrict__ W, const float* __restrict__ rs,
                                                  const float* __restrict__ x, float* __restrict__ y, int rows) {
    constexpr int cols = 512 * D;
    const int lane = threadIdx.x & 63;
    const int r0 = (blockIdx.x * 4 + wave_id()) * R;
    if (r0 >= rows) return;  // wave-uniform
    float xr[D][8];
#pragma unroll
    for (int i = 0; i < D; i++) {
        const float4 a = reinterpret_cast<const float4*>(x)[2 * (lane + 64 * i)];
        const float4 b = reinterpret_cast<const float4*>(x)[2 * (lane + 64 * i) + 1];
        xr[i][0] = a.x; xr[i][1] = a.y; xr[i][2] = a.z; xr[i][3] = a.w;
        xr[i][4] = b.x; xr[i][5] = b.y; xr[i][6] = b.z; xr[i][7] = b.w;
    }
    const int nr = min(R, rows - r0);
    const rsrc_t rw = make_rsrc(W + (size_t)r0 * cols, (uint32_t)(nr * cols));
    uint2 c[R][D];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int i = 0; i < D; i++) c[r][i] = ld_b64(rw, (uint32_t)(r * cols + 8 * (lane + 64 * i)));
#pragma unroll
    for (int r = 0; r < R; r++) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < D; i++) {
            const f2v p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[r][i].x, false);
            const f2v p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[r][i].x, true);
            const f2v p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[r][i].y, false);
            const f2v p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[r][i].y, true);
            acc = fmaf(p0.x, xr[i][0], acc);
            acc = fmaf(p0.y, xr[i][1], acc);
            acc = fmaf(p1.x, xr[i][2], acc);
            acc = fmaf(p1.y, xr[i][3], acc);
            acc = fmaf(p2.x, xr[i][4], acc);
            acc = fmaf(p2.y, xr[i][5], acc);
            acc = fmaf(p3.x, xr[i][6], acc);
            acc = fmaf(p3.y, xr[i][7], acc);
        }
        acc = wave_sum(acc);
        if (lane == 0 && r < nr) y[r0 + r] = rs[r0 + r] * acc;
    }
}

bool gemv_fp8_supported(int cols) {
    if (cols < 512 || cols % 512) return false;
    const int d = cols / 512;
    return d <= 8 || d == 10 || d == 12 || d == 16;
}

template <int D>
static hipError_t launch_gemv_d(const uint8_t* W, const float* rs, const float* x, float* y, int rows, hipStream_t s) {
    constexpr int R = D <= 8 ? 4 : 2;
    const unsigned waves = (unsigned)((rows + R - 1) / R);
    hipLaunchKernelGGL((k_gemv_fp8<D, R>), dim3((waves + 3) / 4), dim3(256), 0, s, W, rs, x, y, rows);
    return hipGetLastError();
}

hipError_t launch_gemv_fp8(const uint8_t* W, const float* rs, const float* x, float* y, int rows, int cols,
                           hipStream_t s) {
    switch (cols / 512) {
        case 1: return launch_gemv_d<1>(W, rs, x, y, rows, s);
        case 2: return launch_gemv_d<2>(W, rs, x, y, rows, s);
        case 3: return launch_gemv_d<3>(W, rs, x, y, rows, s);
        case 4: return launch_gemv_d<4>(W, rs, x, y, rows, s);
        case 5: return launch_gemv_d<5>(W, rs, x, y, rows, s);
        case 6: return launch_gemv_d<6>(W, rs, x, y, rows, s);
        case 7: return launch_gemv_d<7>(W, rs, x, y, rows, s);
        case 8: return launch_gemv_d<8>(W, rs, x, y, rows, s);
        case 10: return launch_gemv_d<10>(W, rs, x, y, rows, s);
        case 12: return launch_gemv_d<12>(W, rs, x, y, rows, s);
        case 16: return launch_gemv_d<16>(W, rs, x, y, rows, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
