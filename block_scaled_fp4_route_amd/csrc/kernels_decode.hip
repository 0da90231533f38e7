// Single-token decode kernels for gfx950: the FP4-weight GEMVs of one MoE
// layer ([Q] "The engine", item 4: a single-token SwiGLU expert kernel over
// NVFP4 weights), re-designed for CDNA4:
//  * k_gateup: gate and up rows of every chosen expert (plus the bf16 shared
//    expert) against the LDS-staged activation vector, SiLU*mul epilogue.
//  * k_down:   down rows of every chosen expert against its hidden vector;
//    per-(expert, row block) partial sums, then the last workgroup of each row
//    block (completion ticket) forms the weighted combine in fixed order.
// Both are HBM-bound GEMVs: every code byte is read once with coalesced
// dword loads (64 lanes x 4 B contiguous), e2m1 pairs are converted by
// v_cvt_scalef32_pk_f32_fp4, the group scale is applied once per 8 codes in
// registers, and rows are reduced with DPP.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kMaxI = 4096;

size_t decode_ws_bytes(int H, int I, int k) {
    return kCounterBytes + align256((size_t)(k + 1) * I * sizeof(float)) +
           align256((size_t)(k + 1) * H * sizeof(float));
}

bool plan_decode(int fmt, int H, int I, DecodePlan* p) {
    const int G = fmt == kFmtNvfp4 ? 16 : 32;
    if (H % 512 || H / 512 < 1 || H / 512 > 8) return false;
    if (I % G || I < 16 || I > kMaxI) return false;
    p->gate_D = H / 512;
    p->gate_P = p->gate_D <= 5 ? 4 : 2;
    p->gate_wg_per_slot = (I + 4 * p->gate_P - 1) / (4 * p->gate_P);
    const int KD = I / 8;
    if (KD <= 16 * 8) {
        p->down_L = 16;
        p->down_D = (KD + 15) / 16;
        p->down_RB = 4 * 4 * 4;  // 4 waves x 4 rows per pass x 4 passes
    } else {
        p->down_L = 64;
        p->down_D = (KD + 63) / 64;
        p->down_RB = 4 * 1 * 8;  // 4 waves x 1 row per pass x 8 passes
    }
    if (p->down_D > 8 || H % p->down_RB) return false;
    p->down_nrb = H / p->down_RB;
    if (p->down_nrb > kMaxCounters) return false;
    return true;
}

// ----------------------------------------------------------------------------
// gate/up GEMV + SiLU*mul.
// Grid: (k + shared) * wg_per_slot workgroups of 256 threads. Workgroup
// (slot, tile): wave v handles row pairs pair0 .. pair0+P-1 with
// pair0 = (tile*4 + v)*P; each pair is gate row i and up row i. Lane l reads
// code dwords l + 64m (m < D) of every row: 8 codes at columns 8(l+64m)..+7,
// whose 8 activations it keeps in registers. Gate codes [I][H/2] and up
// codes [I][H/2] are adjacent in the block, as are their scales.
template <int FMT, int D, int P>
__global__ __launch_bounds__(256) void k_gateup(const float* __restrict__ x, const void* const* __restrict__ expert_ptrs,
                                                const int32_t* __restrict__ idx, int E, int k, int I, int wg_per_slot,
                                                const uint16_t* __restrict__ sh_gate, const uint16_t* __restrict__ sh_up,
                                                float* __restrict__ h) {
    constexpr int K = 512 * D;     // H
    constexpr int KD = K / 8;      // code dwords per row (= 16-byte bf16 chunks per shared row)
    constexpr int G = Fmt<FMT>::G;
    constexpr int KS = K / G;      // scale bytes per row
    __shared__ f4v xs[K / 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = blockIdx.x / wg_per_slot;
    const int pair0 = ((blockIdx.x % wg_per_slot) * 4 + wave) * P;

    for (int i = tid; i < K / 4; i += 256) xs[i] = reinterpret_cast<const f4v*>(x)[i];
    __syncthreads();
    float xr[8 * D];
#pragma unroll
    for (int m = 0; m < D; m++) {
        const f4v a = xs[2 * (lane + 64 * m)], b = xs[2 * (lane + 64 * m) + 1];
        xr[8 * m + 0] = a.x; xr[8 * m + 1] = a.y; xr[8 * m + 2] = a.z; xr[8 * m + 3] = a.w;
        xr[8 * m + 4] = b.x; xr[8 * m + 5] = b.y; xr[8 * m + 6] = b.z; xr[8 * m + 7] = b.w;
    }
    const int np = min(P, I - pair0);  // wave-uniform
    if (np <= 0) return;

    float acc[2 * P];
    const int e = slot < k ? idx[slot] : 0;
    if (slot < k && (unsigned)e >= (unsigned)E) {
        // an expert index outside [0, E) poisons this slot's output instead of
        // dereferencing a pointer beyond the table
#pragma unroll
        for (int r = 0; r < 2 * P; r++) acc[r] = __uint_as_float(0x7FC00000u);
    } else if (slot < k) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(expert_ptrs[e]);
        const uint32_t* codes = reinterpret_cast<const uint32_t*>(blk);
        const uint8_t* scl = blk + (size_t)3 * I * (K / 2);
        uint32_t wv[2 * P][D], sv[2 * P][D];
#pragma unroll
        for (int r = 0; r < 2 * P; r++) {
            const int p = r % P;
            const size_t row = (size_t)(r / P) * I + pair0 + p;
            if (p < np) {
#pragma unroll
                for (int m = 0; m < D; m++) {
                    const int c = lane + 64 * m;
                    wv[r][m] = codes[row * KD + c];
                    sv[r][m] = scl[row * KS + c * 8 / G];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 2 * P; r++) {
            float a = 0.f;
            if (r % P < np) {
#pragma unroll
                for (int m = 0; m < D; m++) a = fmaf(scale_to_f32<FMT>(sv[r][m]), dot8_fp4(wv[r][m], &xr[8 * m]), a);
            }
            acc[r] = a;
        }
    } else {
        // dense bf16 shared expert: 16-byte chunk c of a row holds columns 8c..8c+7
        const uint4* gq = reinterpret_cast<const uint4*>(sh_gate);
        const uint4* uq = reinterpret_cast<const uint4*>(sh_up);
        uint4 v[2 * P][D];
#pragma unroll
        for (int r = 0; r < 2 * P; r++) {
            const int p = r % P;
            const size_t row = (size_t)pair0 + p;
            if (p < np) {
#pragma unroll
                for (int m = 0; m < D; m++) v[r][m] = (r < P ? gq : uq)[row * KD + lane + 64 * m];
            }
        }
#pragma unroll
        for (int r = 0; r < 2 * P; r++) {
            float a = 0.f;
            if (r % P < np) {
#pragma unroll
                for (int m = 0; m < D; m++) {
                    const float* xx = &xr[8 * m];
                    a = fmaf(bf16_lo(v[r][m].x), xx[0], a); a = fmaf(bf16_hi(v[r][m].x), xx[1], a);
                    a = fmaf(bf16_lo(v[r][m].y), xx[2], a); a = fmaf(bf16_hi(v[r][m].y), xx[3], a);
                    a = fmaf(bf16_lo(v[r][m].z), xx[4], a); a = fmaf(bf16_hi(v[r][m].z), xx[5], a);
                    a = fmaf(bf16_lo(v[r][m].w), xx[6], a); a = fmaf(bf16_hi(v[r][m].w), xx[7], a);
                }
            }
            acc[r] = a;
        }
    }
#pragma unroll
    for (int r = 0; r < 2 * P; r++) acc[r] = wave_sum(acc[r]);
    if (lane == 0) {
#pragma unroll
        for (int p = 0; p < P; p++)
            if (p < np) h[(size_t)slot * I + pair0 + p] = silu_mul(acc[p], acc[P + p]);
    }
}

// ----------------------------------------------------------------------------
// down GEMV + weighted combine.
// Grid: nslots * nrb workgroups of 256 threads; workgroup (slot, rb) computes
// rows rb*RB .. +RB of slot's down matrix against h[slot] (staged in LDS).
// A row is covered by L lanes (64/L rows per wave pass); lane s of a row
// reads code dwords s + L*m (m < D, while < I/8). Partial rows go to
// Yp[slot][row]; the workgroup that completes row block rb last (ticket
// cnt[rb]) writes y[row] = sum_j w[j] * Yp[j][row] (+ Yp[k][row]) in
// increasing j, and resets cnt[rb] to zero.
template <int FMT, int L, int D, int PASSES>
__global__ __launch_bounds__(256) void k_down(const float* __restrict__ h, const void* const* __restrict__ expert_ptrs,
                                              const int32_t* __restrict__ idx, const float* __restrict__ w, int E,
                                              int k, int nslots, int H, int I, const uint16_t* __restrict__ sh_down,
                                              float* __restrict__ Yp, int* __restrict__ cnt, float* __restrict__ y) {
    constexpr int G = Fmt<FMT>::G;
    constexpr int RPW = 64 / L;                // rows per wave pass
    constexpr int RB = 4 * RPW * PASSES;       // rows per workgroup
    __shared__ f4v hs[kMaxI / 4];
    __shared__ int is_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nrb = H / RB;
    const int slot = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int KD = I / 8, KS = I / G;

    for (int i = tid; i < I / 4; i += 256) hs[i] = reinterpret_cast<const f4v*>(h + (size_t)slot * I)[i];
    __syncthreads();
    const int grp = lane / L, s = lane % L;
    float hr[8 * D];
#pragma unroll
    for (int m = 0; m < D; m++) {
        const int c = s + L * m;
        f4v a = {0.f, 0.f, 0.f, 0.f}, b = a;
        if (c < KD) { a = hs[2 * c]; b = hs[2 * c + 1]; }
        hr[8 * m + 0] = a.x; hr[8 * m + 1] = a.y; hr[8 * m + 2] = a.z; hr[8 * m + 3] = a.w;
        hr[8 * m + 4] = b.x; hr[8 * m + 5] = b.y; hr[8 * m + 6] = b.z; hr[8 * m + 7] = b.w;
    }
    const int row0 = rb * RB + wave * (RPW * PASSES) + grp;  // row of pass q: row0 + q * RPW

    float part[PASSES];
    const int e = slot < k ? idx[slot] : 0;
    if (slot < k && (unsigned)e >= (unsigned)E) {
#pragma unroll
        for (int q = 0; q < PASSES; q++) part[q] = __uint_as_float(0x7FC00000u);
    } else if (slot < k) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(expert_ptrs[e]);
        const uint32_t* codes = reinterpret_cast<const uint32_t*>(blk + (size_t)I * H);  // after gate, up
        const uint8_t* scl = blk + (size_t)3 * I * H / 2 + (size_t)2 * I * H / G;
        uint32_t wv[PASSES][D], sv[PASSES][D];
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const size_t row = (size_t)row0 + q * RPW;
#pragma unroll
            for (int m = 0; m < D; m++) {
                const int c = s + L * m;
                if (c < KD) {
                    wv[q][m] = codes[row * KD + c];
                    sv[q][m] = scl[row * KS + c * 8 / G];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            float a = 0.f;
#pragma unroll
            for (int m = 0; m < D; m++)
                if (s + L * m < KD) a = fmaf(scale_to_f32<FMT>(sv[q][m]), dot8_fp4(wv[q][m], &hr[8 * m]), a);
            part[q] = a;
        }
    } else {
        const uint4* dq = reinterpret_cast<const uint4*>(sh_down);
        uint4 v[PASSES][D];
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const size_t row = (size_t)row0 + q * RPW;
#pragma unroll
            for (int m = 0; m < D; m++)
                if (s + L * m < KD) v[q][m] = dq[row * KD + s + L * m];
        }
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            float a = 0.f;
#pragma unroll
            for (int m = 0; m < D; m++) {
                if (s + L * m < KD) {
                    const float* xx = &hr[8 * m];
                    a = fmaf(bf16_lo(v[q][m].x), xx[0], a); a = fmaf(bf16_hi(v[q][m].x), xx[1], a);
                    a = fmaf(bf16_lo(v[q][m].y), xx[2], a); a = fmaf(bf16_hi(v[q][m].y), xx[3], a);
                    a = fmaf(bf16_lo(v[q][m].z), xx[4], a); a = fmaf(bf16_hi(v[q][m].z), xx[5], a);
                    a = fmaf(bf16_lo(v[q][m].w), xx[6], a); a = fmaf(bf16_hi(v[q][m].w), xx[7], a);
                }
            }
            part[q] = a;
        }
    }
#pragma unroll
    for (int q = 0; q < PASSES; q++) {
        const float r = (L == 16) ? row16_sum(part[q]) : wave_sum(part[q]);
        if (s == 0) Yp[(size_t)slot * H + row0 + q * RPW] = r;
    }

    // completion ticket for row block rb
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = atomicAdd(&cnt[rb], 1) == nslots - 1;
    __syncthreads();
    if (is_last) {
        __threadfence();
        for (int r = tid; r < RB; r += 256) {
            const int row = rb * RB + r;
            float acc = 0.f;
            for (int j = 0; j < k; j++) acc = fmaf(w[j], Yp[(size_t)j * H + row], acc);
            if (nslots > k) acc += Yp[(size_t)k * H + row];
            y[row] = acc;
        }
        if (tid == 0) cnt[rb] = 0;
    }
}

// ----------------------------------------------------------------------------
template <int FMT>
static hipError_t launch_gateup(const DecodePlan& p, int E, int I, int nslots, int k, const float* x,
                                const void* const* ep, const int32_t* idx, const uint16_t* sg, const uint16_t* su,
                                float* h, hipStream_t s) {
    dim3 grid(nslots * p.gate_wg_per_slot), block(256);
#define GU(DD, PP) \
    case DD: hipLaunchKernelGGL((k_gateup<FMT, DD, PP>), grid, block, 0, s, x, ep, idx, E, k, I, p.gate_wg_per_slot, sg, su, h); break;
    switch (p.gate_D) {
        GU(1, 4) GU(2, 4) GU(3, 4) GU(4, 4) GU(5, 4) GU(6, 2) GU(7, 2) GU(8, 2)
        default: return hipErrorInvalidValue;
    }
#undef GU
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_down(const DecodePlan& p, int E, int H, int I, int nslots, int k, const float* h,
                              const void* const* ep, const int32_t* idx, const float* w, const uint16_t* sd,
                              float* Yp, int* cnt, float* y, hipStream_t s) {
    dim3 grid(nslots * p.down_nrb), block(256);
#define DN(LL, DD, PS) \
    case DD: hipLaunchKernelGGL((k_down<FMT, LL, DD, PS>), grid, block, 0, s, h, ep, idx, w, E, k, nslots, H, I, sd, Yp, cnt, y); break;
    if (p.down_L == 16) {
        switch (p.down_D) {
            DN(16, 1, 4) DN(16, 2, 4) DN(16, 3, 4) DN(16, 4, 4) DN(16, 5, 4) DN(16, 6, 4) DN(16, 7, 4) DN(16, 8, 4)
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.down_D) {
            DN(64, 1, 8) DN(64, 2, 8) DN(64, 3, 8) DN(64, 4, 8) DN(64, 5, 8) DN(64, 6, 8) DN(64, 7, 8) DN(64, 8, 8)
            default: return hipErrorInvalidValue;
        }
    }
#undef DN
    return hipGetLastError();
}

hipError_t launch_decode(int fmt, const DecodePlan& p, int E, int H, int I, int k, const float* x,
                         const void* const* expert_ptrs, const int32_t* idx, const float* w,
                         const uint16_t* sh_gate, const uint16_t* sh_up, const uint16_t* sh_down, float* y,
                         void* ws, hipStream_t s) {
    const int nslots = k + (sh_gate ? 1 : 0);
    char* base = reinterpret_cast<char*>(ws);
    int* cnt = reinterpret_cast<int*>(base);
    float* hbuf = reinterpret_cast<float*>(base + kCounterBytes);
    float* Yp = reinterpret_cast<float*>(base + kCounterBytes + align256((size_t)(k + 1) * I * sizeof(float)));
    hipError_t e;
    if (fmt == kFmtNvfp4) {
        e = launch_gateup<kFmtNvfp4>(p, E, I, nslots, k, x, expert_ptrs, idx, sh_gate, sh_up, hbuf, s);
        if (e != hipSuccess) return e;
        return launch_down<kFmtNvfp4>(p, E, H, I, nslots, k, hbuf, expert_ptrs, idx, w, sh_down, Yp, cnt, y, s);
    }
    e = launch_gateup<kFmtMxfp4>(p, E, I, nslots, k, x, expert_ptrs, idx, sh_gate, sh_up, hbuf, s);
    if (e != hipSuccess) return e;
    return launch_down<kFmtMxfp4>(p, E, H, I, nslots, k, hbuf, expert_ptrs, idx, w, sh_down, Yp, cnt, y, s);
}

// ----------------------------------------------------------------------------
// Dequantisation of one block to fp32 (test support): one thread per code
// byte, the same e2m1 and scale decoders as the GEMVs.
template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ blk, int H, int I, float* __restrict__ gate,
                                                 float* __restrict__ up, float* __restrict__ down) {
    constexpr int G = Fmt<FMT>::G;
    const size_t mat = (size_t)H * I / 2;  // code bytes per matrix
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= 3 * mat) return;
    const int m = (int)(i / mat);
    const size_t b = i - m * mat;
    const int cols = m < 2 ? H : I;
    const size_t r = b / (cols / 2);
    const int c = (int)(b % (cols / 2)) * 2;
    const float sc = scale_to_f32<FMT>(blk[3 * mat + m * (size_t)H * I / G + r * (cols / G) + c / G]);
    const f2v v = fp4x2<0>(blk[i]);
    float* out = m == 0 ? gate : (m == 1 ? up : down);
    out[r * cols + c] = v.x * sc;
    out[r * cols + c + 1] = v.y * sc;
}

hipError_t launch_dequant(int fmt, int H, int I, const void* block, float* gate, float* up, float* down,
                          hipStream_t s) {
    const size_t n = (size_t)3 * H * I / 2;
    dim3 grid((unsigned)((n + 255) / 256)), b(256);
    const uint8_t* blk = reinterpret_cast<const uint8_t*>(block);
    if (fmt == kFmtNvfp4)
        hipLaunchKernelGGL(k_dequant<kFmtNvfp4>, grid, b, 0, s, blk, H, I, gate, up, down);
    else
        hipLaunchKernelGGL(k_dequant<kFmtMxfp4>, grid, b, 0, s, blk, H, I, gate, up, down);
    return hipGetLastError();
}

}  // namespace moe
