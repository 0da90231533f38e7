// Single-token decode kernels for gfx950: the FP4-weight GEMVs of one MoE
// layer ([Q] "The engine", item 4: a single-token SwiGLU expert kernel over
// NVFP4 weights), re-designed for CDNA4:
//  * k_gateup: gate and up rows of every chosen expert (plus the bf16 shared
//    expert) against the LDS-staged activation vector, SiLU*mul epilogue;
//  * k_down: down rows of every chosen expert against its hidden vector,
//    unweighted partial rows per expert;
//  * k_combine: the weighted sum of the partial rows in fixed expert order.
// The GEMVs are HBM-bound: every code byte is read once with coalesced
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
    if (p->down_nrb > kCntRoute - kCntDone) return false;
    return true;
}

struct DecodeArgs {
    const float* x;
    const void* const* expert_ptrs;
    const int32_t* idx;
    const float* w;
    const uint16_t* sh_gate;
    const uint16_t* sh_up;
    const uint16_t* sh_down;
    float* h;    // [(k+1)][I] SwiGLU hidden vectors
    float* Yp;   // [(k+1)][H] unweighted down rows
    float* y;    // [H]
    int E, k, H, I;
    int has_shared;
    int gt_r;    // gate/up tiles per routed slot
    int gt_s;    // gate/up tiles of the shared slot
    int n_gate;  // gate/up workgroups
    int nrb;     // down row blocks
    int sh_sub;  // shared-expert down workgroups per row block
};

// ----------------------------------------------------------------------------
// gate/up rows + SiLU*mul for one tile.
// Wave v handles row pairs pair0 .. pair0+P-1 (gate row i and up row i).
// Lane l reads code dwords l + 64m (m < D) of every row: 8 codes at columns
// 8(l+64m)..+7 whose activations it keeps in registers. Gate and up codes
// ([I][H/2] each) are adjacent in the block, as are their scales; the bf16
// shared expert uses the same lane/column map with 16-byte chunks.
template <int FMT, int D, int P, bool SHARED>
__device__ __forceinline__ void gateup_tile(const DecodeArgs& a, int slot, int pair0, f4v* xs) {
    constexpr int K = 512 * D;     // H
    constexpr int KD = K / 8;      // code dwords per row (= 16-byte bf16 chunks per shared row)
    constexpr int G = Fmt<FMT>::G;
    constexpr int KS = K / G;      // scale bytes per row
    const int tid = threadIdx.x, lane = tid & 63;
    const int I = a.I;
    const int np = min(P, I - pair0);  // wave-uniform; <= 0 for idle waves of the last tile
    const int e = SHARED ? 0 : a.idx[slot];
    // an expert index outside [0, E) poisons this slot instead of reading
    // beyond the pointer table
    const bool bad = !SHARED && (unsigned)e >= (unsigned)a.E;

    // 1. weight loads first (they do not depend on x)
    uint32_t wv[2 * P][D], sv[2 * P][D];
    uint4 v[2 * P][D];
    if (SHARED) {
        const uint4* gq = reinterpret_cast<const uint4*>(a.sh_gate);
        const uint4* uq = reinterpret_cast<const uint4*>(a.sh_up);
#pragma unroll
        for (int r = 0; r < 2 * P; r++) {
            const int p = r % P;
            const size_t row = (size_t)pair0 + p;
            if (p < np) {
#pragma unroll
                for (int m = 0; m < D; m++) v[r][m] = (r < P ? gq : uq)[row * KD + lane + 64 * m];
            }
        }
    } else if (!bad) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.expert_ptrs[e]);
        const uint32_t* codes = reinterpret_cast<const uint32_t*>(blk);
        const uint8_t* scl = blk + (size_t)3 * I * (K / 2);
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
    }

    // 2. x through LDS into registers: lane keeps columns 8(lane+64m)..+7
    for (int i = tid; i < K / 4; i += 256) xs[i] = reinterpret_cast<const f4v*>(a.x)[i];
    __syncthreads();
    if (np > 0) {
        float xr[8 * D];
#pragma unroll
        for (int m = 0; m < D; m++) {
            const f4v p0 = xs[2 * (lane + 64 * m)], p1 = xs[2 * (lane + 64 * m) + 1];
            xr[8 * m + 0] = p0.x; xr[8 * m + 1] = p0.y; xr[8 * m + 2] = p0.z; xr[8 * m + 3] = p0.w;
            xr[8 * m + 4] = p1.x; xr[8 * m + 5] = p1.y; xr[8 * m + 6] = p1.z; xr[8 * m + 7] = p1.w;
        }
        // 3. dot products, row sums, SiLU*mul
        float acc[2 * P];
#pragma unroll
        for (int r = 0; r < 2 * P; r++) {
            float s = 0.f;
            if (r % P < np) {
                if (SHARED) {
#pragma unroll
                    for (int m = 0; m < D; m++) {
                        const float* xx = &xr[8 * m];
                        s = fmaf(bf16_lo(v[r][m].x), xx[0], s); s = fmaf(bf16_hi(v[r][m].x), xx[1], s);
                        s = fmaf(bf16_lo(v[r][m].y), xx[2], s); s = fmaf(bf16_hi(v[r][m].y), xx[3], s);
                        s = fmaf(bf16_lo(v[r][m].z), xx[4], s); s = fmaf(bf16_hi(v[r][m].z), xx[5], s);
                        s = fmaf(bf16_lo(v[r][m].w), xx[6], s); s = fmaf(bf16_hi(v[r][m].w), xx[7], s);
                    }
                } else if (!bad) {
#pragma unroll
                    for (int m = 0; m < D; m++)
                        s = fmaf(scale_to_f32<FMT>(sv[r][m]), dot8_fp4(wv[r][m], &xr[8 * m]), s);
                } else {
                    s = __uint_as_float(0x7FC00000u);
                }
            }
            acc[r] = wave_sum(s);
        }
        if (lane == 0) {
#pragma unroll
            for (int p = 0; p < P; p++)
                if (p < np) a.h[(size_t)slot * I + pair0 + p] = silu_mul(acc[p], acc[P + p]);
        }
    }
}

// ----------------------------------------------------------------------------
// down rows of one slot for one row block, then (last arrival) the combine.
// A row is covered by L lanes (64/L rows per wave pass); lane s of a row
// reads code dwords s + L*m (m < D, while < I/8) and keeps the matching 8D
// hidden values in registers. The weight loads are issued before waiting
// for the slot's hidden vector, so they overlap the gate/up phase.
template <int FMT, int L, int D, int PASSES, bool SHARED>
__device__ __forceinline__ void down_tile(const DecodeArgs& a, int slot, int row_base, f4v* hs) {
    constexpr int G = Fmt<FMT>::G;
    constexpr int RPW = 64 / L;  // rows per wave pass
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H, I = a.I;
    const int KD = I / 8, KS = I / G;
    const int grp = lane / L, s = lane % L;
    const int row0 = row_base + wave * (RPW * PASSES) + grp;  // row of pass q: row0 + q * RPW
    const int e = SHARED ? 0 : a.idx[slot];
    const bool bad = !SHARED && (unsigned)e >= (unsigned)a.E;

    // 1. weight loads
    uint32_t wv[PASSES][D], sv[PASSES][D];
    uint4 v[PASSES][D];
    if (SHARED) {
        const uint4* dq = reinterpret_cast<const uint4*>(a.sh_down);
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const size_t row = (size_t)row0 + q * RPW;
#pragma unroll
            for (int m = 0; m < D; m++)
                if (s + L * m < KD) v[q][m] = dq[row * KD + s + L * m];
        }
    } else if (!bad) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.expert_ptrs[e]);
        const uint32_t* codes = reinterpret_cast<const uint32_t*>(blk + (size_t)I * H);  // after gate, up
        const uint8_t* scl = blk + (size_t)3 * I * H / 2 + (size_t)2 * I * H / G;
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
    }

    // 2. the slot's hidden vector through LDS into registers
    for (int i = tid; i < I / 4; i += 256) hs[i] = reinterpret_cast<const f4v*>(a.h + (size_t)slot * I)[i];
    __syncthreads();
    float hr[8 * D];
#pragma unroll
    for (int m = 0; m < D; m++) {
        const int c = s + L * m;
        f4v p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
        if (c < KD) { p0 = hs[2 * c]; p1 = hs[2 * c + 1]; }
        hr[8 * m + 0] = p0.x; hr[8 * m + 1] = p0.y; hr[8 * m + 2] = p0.z; hr[8 * m + 3] = p0.w;
        hr[8 * m + 4] = p1.x; hr[8 * m + 5] = p1.y; hr[8 * m + 6] = p1.z; hr[8 * m + 7] = p1.w;
    }

    // 3. dot products and row sums
#pragma unroll
    for (int q = 0; q < PASSES; q++) {
        float acc = 0.f;
        if (SHARED) {
#pragma unroll
            for (int m = 0; m < D; m++) {
                if (s + L * m < KD) {
                    const float* xx = &hr[8 * m];
                    acc = fmaf(bf16_lo(v[q][m].x), xx[0], acc); acc = fmaf(bf16_hi(v[q][m].x), xx[1], acc);
                    acc = fmaf(bf16_lo(v[q][m].y), xx[2], acc); acc = fmaf(bf16_hi(v[q][m].y), xx[3], acc);
                    acc = fmaf(bf16_lo(v[q][m].z), xx[4], acc); acc = fmaf(bf16_hi(v[q][m].z), xx[5], acc);
                    acc = fmaf(bf16_lo(v[q][m].w), xx[6], acc); acc = fmaf(bf16_hi(v[q][m].w), xx[7], acc);
                }
            }
        } else if (!bad) {
#pragma unroll
            for (int m = 0; m < D; m++)
                if (s + L * m < KD) acc = fmaf(scale_to_f32<FMT>(sv[q][m]), dot8_fp4(wv[q][m], &hr[8 * m]), acc);
        }
        if (bad) acc = __uint_as_float(0x7FC00000u);
        const float r = (L == 16) ? row16_sum(acc) : wave_sum(acc);
        if (s == 0) a.Yp[(size_t)slot * H + row0 + q * RPW] = r;
    }
}

// ----------------------------------------------------------------------------
// Three launches per call; the kernel boundaries carry the gate/up -> down ->
// combine dependencies (cheaper on this chip than in-kernel device-scope
// hand-offs between workgroups).
template <int FMT, int GD, int GP>
__global__ __launch_bounds__(256) void k_gateup(DecodeArgs a) {
    __shared__ f4v buf[1024];  // x, H <= 4096
    const int bid = blockIdx.x;
    const int ng_r = a.k * a.gt_r;
    if (bid < ng_r) {
        const int slot = bid / a.gt_r, tile = bid % a.gt_r;
        gateup_tile<FMT, GD, GP, false>(a, slot, (tile * 4 + (threadIdx.x >> 6)) * GP, buf);
    } else {
        // shared expert: bf16 rows are 3.5x the bytes of an FP4 row, one pair per wave
        gateup_tile<FMT, GD, 1, true>(a, a.k, (bid - ng_r) * 4 + (threadIdx.x >> 6), buf);
    }
}

template <int FMT, int DL, int DD, int DP>
__global__ __launch_bounds__(256) void k_down(DecodeArgs a) {
    __shared__ f4v buf[1024];  // h, I <= 4096
    constexpr int RPW = 64 / DL;
    constexpr int RB = 4 * RPW * DP;  // rows per routed down workgroup
    const int d = blockIdx.x;
    if (d < a.k * a.nrb) {
        down_tile<FMT, DL, DD, DP, false>(a, d / a.nrb, (d % a.nrb) * RB, buf);
    } else {
        // shared expert: its row blocks are split into sh_sub workgroups of one pass
        down_tile<FMT, DL, DD, 1, true>(a, a.k, (d - a.k * a.nrb) * (4 * RPW), buf);
    }
}

// y[row] = sum_{j<k} w[j] * Yp[j][row] (+ Yp[k][row] for the shared expert),
// in increasing j.
__global__ __launch_bounds__(256) void k_combine(DecodeArgs a) {
    const int row = blockIdx.x * 256 + threadIdx.x;
    if (row >= a.H) return;
    float acc = 0.f;
    for (int j = 0; j < a.k; j++) acc = fmaf(a.w[j], a.Yp[(size_t)j * a.H + row], acc);
    if (a.has_shared) acc += a.Yp[(size_t)a.k * a.H + row];
    a.y[row] = acc;
}

template <int FMT>
static hipError_t launch_expert(const DecodePlan& p, DecodeArgs& a, hipStream_t s) {
    const int n_down = a.k * a.nrb + (a.has_shared ? a.nrb * a.sh_sub : 0);
    dim3 block(256);
#define GU(GD, GP) case GD: hipLaunchKernelGGL((k_gateup<FMT, GD, GP>), dim3(a.n_gate), block, 0, s, a); break;
    switch (p.gate_D) {
        GU(1, 4) GU(2, 4) GU(3, 4) GU(4, 4) GU(5, 4) GU(6, 2) GU(7, 2) GU(8, 2)
        default: return hipErrorInvalidValue;
    }
#undef GU
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
#define DN(DL, DD, DP) case DD: hipLaunchKernelGGL((k_down<FMT, DL, DD, DP>), dim3(n_down), block, 0, s, a); break;
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
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_combine, dim3((a.H + 255) / 256), block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode(int fmt, const DecodePlan& p, int E, int H, int I, int k, const float* x,
                         const void* const* expert_ptrs, const int32_t* idx, const float* w,
                         const uint16_t* sh_gate, const uint16_t* sh_up, const uint16_t* sh_down, float* y,
                         void* ws, hipStream_t s) {
    char* base = reinterpret_cast<char*>(ws);
    DecodeArgs a;
    a.x = x; a.expert_ptrs = expert_ptrs; a.idx = idx; a.w = w;
    a.sh_gate = sh_gate; a.sh_up = sh_up; a.sh_down = sh_down;
    a.h = reinterpret_cast<float*>(base + kCounterBytes);
    a.Yp = reinterpret_cast<float*>(base + kCounterBytes + align256((size_t)(k + 1) * I * sizeof(float)));
    a.y = y;
    a.E = E; a.k = k; a.H = H; a.I = I;
    a.has_shared = sh_gate ? 1 : 0;
    a.gt_r = p.gate_wg_per_slot;
    a.gt_s = (I + 3) / 4;  // shared gate/up: one row pair per wave
    a.n_gate = k * a.gt_r + (a.has_shared ? a.gt_s : 0);
    a.nrb = p.down_nrb;
    a.sh_sub = p.down_RB / (4 * (64 / p.down_L));
    return fmt == kFmtNvfp4 ? launch_expert<kFmtNvfp4>(p, a, s) : launch_expert<kFmtMxfp4>(p, a, s);
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
