// Single-token decode kernels for gfx950: the FP4-weight GEMVs of one MoE
// layer ([Q] "The engine", item 4: a single-token SwiGLU expert kernel over
// NVFP4 weights), re-designed for CDNA4:
//  * gate/up tiles: gate and up rows of a chosen expert (or of the bf16
//    shared expert) against the LDS-staged activation vector, SiLU*mul
//    epilogue;
//  * down tiles: for a block of 8 output rows, one wave per chosen expert
//    (two for the shared expert) against that expert's hidden vector, then
//    the weighted combine in fixed expert order in LDS;
//  * for the fused layer entry point, the router rows share a launch with
//    the shared expert's gate/up (neither depends on the routing), and the
//    top-k runs redundantly at the start of every routed gate/up workgroup.
// Kernel boundaries carry the remaining dependencies (router -> routed
// gate/up -> down): on this chip they are cheaper than in-kernel
// device-scope hand-offs between workgroups.
// The kernels are latency-bound chains of dependent loads, so each level is
// kept short: the expert pointer table is staged in LDS while the routing is
// read, the gate/up launch hands the chosen blocks' addresses to the down
// launch, and every weight load is issued before the first one is used.
// Weights are read with coalesced buffer loads (64 lanes x 4 B contiguous),
// e2m1 pairs are converted by v_cvt_scalef32_pk_f32_fp4, the group scale is
// applied once per 8 codes in registers, and rows are reduced with DPP.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kMaxI = 4096;
constexpr int kDownRB = 8;  // output rows per down workgroup

size_t decode_ws_bytes(int H, int I, int k, int E) {
    (void)H;
    return kCounterBytes + align256((size_t)(k + 1) * I * sizeof(float)) + align256((size_t)E * sizeof(float)) +
           align256((size_t)k * sizeof(void*));
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
    } else {
        p->down_L = 64;
        p->down_D = (KD + 63) / 64;
    }
    p->down_RB = kDownRB;
    if (p->down_D > 8 || H % p->down_RB) return false;
    p->down_nrb = H / p->down_RB;
    return true;
}

struct DecodeArgs {
    const float* x;
    const void* const* expert_ptrs;
    const int32_t* idx;      // routing given to moe_expert_decode
    const float* w;          // routing weights (given, or published by the layer's top-k)
    const uint16_t* sh_gate;
    const uint16_t* sh_up;
    const uint16_t* sh_down;
    const float* Wr;         // router weights (layer)
    float* logits;           // [E] (layer)
    int32_t* idx_out;        // [k] top-k published by the layer entry point
    float* w_out;            // [k]
    const void** sel;        // [k] block addresses of the chosen experts (NULL: invalid index)
    float* h;                // [(k+1)][I] SwiGLU hidden vectors (slot k = shared)
    float* y;                // [H]
    int E, k, H, I;
    int has_shared;
    int gt_r;                // gate/up tiles per routed slot
    int gt_s;                // gate/up tiles of the shared slot
    int n_items;             // down work items: k routed slots + 2 halves of the shared one
    uint32_t block_bytes;
};

__device__ __forceinline__ const void* valid_block(const DecodeArgs& a, const void* const* tbl, int e) {
    return (unsigned)e < (unsigned)a.E ? tbl[e] : nullptr;
}

// ----------------------------------------------------------------------------
// gate/up rows + SiLU*mul for one tile of a routed expert (block `blk`, NULL
// for an invalid index) or of the shared expert, into slot `slot` of h.
// Wave v handles row pairs pair0 .. pair0+P-1 (gate row i and up row i).
// Lane l reads code dwords l + 64m (m < D) of every row: 8 codes at columns
// 8(l+64m)..+7 whose activations it keeps in registers. Gate and up codes
// ([I][H/2] each) are adjacent in the block, as are their scales; the bf16
// shared expert uses the same lane/column map with 16-byte chunks.
template <int FMT, int D, int P, bool SHARED>
__device__ __forceinline__ void gateup_tile(const DecodeArgs& a, int slot, const void* blk, int pair0, f4v* xs) {
    constexpr int K = 512 * D;     // H
    constexpr int KD = K / 8;      // code dwords per row (= 16-byte bf16 chunks per shared row)
    constexpr int G = Fmt<FMT>::G;
    constexpr int KS = K / G;      // scale bytes per row
    const int tid = threadIdx.x, lane = tid & 63;
    const int I = a.I;
    const int np = min(P, I - pair0);  // wave-uniform; <= 0 for idle waves of the last tile
    // an invalid expert index poisons this slot instead of reading anything
    const bool bad = !SHARED && blk == nullptr;

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
        const rsrc_t rb = make_rsrc(blk, a.block_bytes);
        const uint32_t scl = (uint32_t)3 * I * (K / 2);
#pragma unroll
        for (int r = 0; r < 2 * P; r++) {
            const int p = r % P;
            const uint32_t row = (uint32_t)(r / P) * I + pair0 + p;
            if (p < np) {
#pragma unroll
                for (int m = 0; m < D; m++) {
                    const uint32_t c = lane + 64 * m;
                    wv[r][m] = ld_b32(rb, row * (K / 2) + 4 * c);
                    sv[r][m] = ld_b8(rb, scl + row * KS + c * 8 / G);
                }
            }
        }
    }

    // 2. x through LDS into registers: lane keeps columns 8(lane+64m)..+7
    {
        constexpr int NX = (K / 4 + 255) / 256;
        f4v t[NX];
#pragma unroll
        for (int u = 0; u < NX; u++) t[u] = reinterpret_cast<const f4v*>(a.x)[min(tid + 256 * u, K / 4 - 1)];
#pragma unroll
        for (int u = 0; u < NX; u++)
            if (tid + 256 * u < K / 4) xs[tid + 256 * u] = t[u];
    }
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
// Router rows: wave v of workgroup b computes logit row 4b + v, lane reads
// float4 chunks lane + 64m (H = 256 * DV).
template <int DV>
__device__ __forceinline__ void router_rows(const DecodeArgs& a, int wg) {
    const int lane = threadIdx.x & 63, e = 4 * wg + (threadIdx.x >> 6);
    if (e >= a.E) return;
    const f4v* xr = reinterpret_cast<const f4v*>(a.x);
    const f4v* wr = reinterpret_cast<const f4v*>(a.Wr + (size_t)e * (256 * DV));
    f4v p[DV], q[DV];
#pragma unroll
    for (int m = 0; m < DV; m++) { p[m] = wr[lane + 64 * m]; q[m] = xr[lane + 64 * m]; }
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < DV; m++) {
        acc = fmaf(p[m].x, q[m].x, acc); acc = fmaf(p[m].y, q[m].y, acc);
        acc = fmaf(p[m].z, q[m].z, acc); acc = fmaf(p[m].w, q[m].w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) a.logits[e] = acc;
}

// ----------------------------------------------------------------------------
// Down projection of one block of kDownRB output rows, all slots, and the
// combine. Work item j < k: routed slot j, all rows; items k, k+1: the two
// halves of the rows of the bf16 shared expert (its rows carry 3.5x the bytes
// of an FP4 row). Wave v processes items v, v + nwaves, ... A row is covered
// by L lanes (64/L rows per pass); lane s of a row reads code dwords s + L*m
// (m < D, while < I/8) and holds the matching 8D hidden values. Partial rows
// meet in LDS; thread r then forms y[row] = sum_j w[j] * part[j][r]
// (+ shared) in increasing j.
template <int FMT, int L, int D>
__device__ __forceinline__ void down_rows(const DecodeArgs& a, int rb, float (*part)[kDownRB], float* wsh) {
    constexpr int G = Fmt<FMT>::G;
    constexpr int RPW = 64 / L;               // rows per wave pass
    constexpr int PASSES = kDownRB / RPW;     // passes for all rows of the block
    constexpr int QC = PASSES < 4 ? PASSES / 2 : (D >= 7 ? 2 : 4);  // passes per load group (divides PASSES / 2)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int H = a.H, I = a.I, k = a.k;
    const int KD = I / 8, KS = I / G;
    const int grp = lane / L, s = lane % L;
    // the combine weights, read while the weights stream
    if (tid < k) wsh[tid] = a.w[tid];
    for (int item = wave; item < a.n_items; item += nwaves) {
        const bool shared = item >= k;
        const int slot = shared ? k : item;
        const int q0 = shared ? (item - k) * (PASSES / 2) : 0;
        const int nq = shared ? PASSES / 2 : PASSES;  // PASSES is even (2 or 8)
        const void* blk = shared ? nullptr : a.sel[slot];
        const bool bad = !shared && blk == nullptr;
        const int row0 = rb * kDownRB + grp;  // row of pass q: row0 + q * RPW
        // the hidden vector of this item's slot, in registers
        float hr[8 * D];
        const f4v* hp = reinterpret_cast<const f4v*>(a.h + (size_t)slot * I);
#pragma unroll
        for (int m = 0; m < D; m++) {
            const int c = s + L * m;
            f4v p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0;
            if (c < KD) { p0 = hp[2 * c]; p1 = hp[2 * c + 1]; }
            hr[8 * m + 0] = p0.x; hr[8 * m + 1] = p0.y; hr[8 * m + 2] = p0.z; hr[8 * m + 3] = p0.w;
            hr[8 * m + 4] = p1.x; hr[8 * m + 5] = p1.y; hr[8 * m + 6] = p1.z; hr[8 * m + 7] = p1.w;
        }
        const rsrc_t rbuf = make_rsrc(blk, bad || shared ? 0u : a.block_bytes);
        const uint32_t codes = (uint32_t)I * H;  // after gate, up
        const uint32_t scl = (uint32_t)3 * I * H / 2 + (uint32_t)2 * I * H / G;
        const uint4* dq = reinterpret_cast<const uint4*>(a.sh_down);
        // passes in groups of QC (bounded registers), all loads of a group first
        for (int qc = 0; qc < nq; qc += QC) {
            uint32_t wv[QC][D], sv[QC][D];
            uint4 v[QC][D];
#pragma unroll
            for (int q = 0; q < QC; q++) {
                const uint32_t row = (uint32_t)row0 + (q0 + qc + q) * RPW;
                if (shared) {
#pragma unroll
                    for (int m = 0; m < D; m++)
                        if (s + L * m < KD) v[q][m] = dq[(size_t)row * KD + s + L * m];
                } else if (!bad) {
#pragma unroll
                    for (int m = 0; m < D; m++) {
                        const uint32_t c = s + L * m;
                        if (c < (uint32_t)KD) {
                            wv[q][m] = ld_b32(rbuf, codes + row * (I / 2) + 4 * c);
                            sv[q][m] = ld_b8(rbuf, scl + row * KS + c * 8 / G);
                        }
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < QC; q++) {
                float acc = 0.f;
                if (shared) {
#pragma unroll
                    for (int m = 0; m < D; m++) {
                        if (s + L * m < KD) {
                            const float* xx = &hr[8 * m];
                            const uint4 t = v[q][m];
                            acc = fmaf(bf16_lo(t.x), xx[0], acc); acc = fmaf(bf16_hi(t.x), xx[1], acc);
                            acc = fmaf(bf16_lo(t.y), xx[2], acc); acc = fmaf(bf16_hi(t.y), xx[3], acc);
                            acc = fmaf(bf16_lo(t.z), xx[4], acc); acc = fmaf(bf16_hi(t.z), xx[5], acc);
                            acc = fmaf(bf16_lo(t.w), xx[6], acc); acc = fmaf(bf16_hi(t.w), xx[7], acc);
                        }
                    }
                } else if (!bad) {
#pragma unroll
                    for (int m = 0; m < D; m++)
                        if (s + L * m < KD)
                            acc = fmaf(scale_to_f32<FMT>(sv[q][m]), dot8_fp4(wv[q][m], &hr[8 * m]), acc);
                } else {
                    acc = __uint_as_float(0x7FC00000u);
                }
                const float r = (L == 16) ? row16_sum(acc) : wave_sum(acc);
                if (s == 0) part[slot][grp + (q0 + qc + q) * RPW] = r;
            }
        }
    }
    __syncthreads();
    if (tid < kDownRB) {
        float acc = 0.f;
        for (int j = 0; j < k; j++) acc = fmaf(wsh[j], part[j][tid], acc);
        if (a.has_shared) acc += part[k][tid];
        a.y[rb * kDownRB + tid] = acc;
    }
}

// ----------------------------------------------------------------------------
// kernels

// Expert pointer table -> LDS, by all 256 threads of the workgroup, in two
// halves so that other loads can be in flight between them: load_table
// issues the loads, store_table writes LDS (made visible by the caller's
// barrier). E <= kMaxE = 4 * 256.
constexpr int kTableRegs = kMaxE / 256;
__device__ __forceinline__ void load_table(const DecodeArgs& a, const void* (&t)[kTableRegs]) {
#pragma unroll
    for (int u = 0; u < kTableRegs; u++) t[u] = a.expert_ptrs[min((int)threadIdx.x + 256 * u, a.E - 1)];
}
__device__ __forceinline__ void store_table(const DecodeArgs& a, const void* const (&t)[kTableRegs],
                                            const void** tbl) {
#pragma unroll
    for (int u = 0; u < kTableRegs; u++)
        if ((int)threadIdx.x + 256 * u < a.E) tbl[threadIdx.x + 256 * u] = t[u];
}

// moe_expert_decode, launch 1: routed gate/up tiles, then shared ones.
// Workgroup 0 publishes the chosen blocks' addresses for the down launch.
template <int FMT, int GD, int GP>
__global__ __launch_bounds__(256) void k_gateup(DecodeArgs a) {
    __shared__ f4v buf[1024];  // x, H <= 4096
    __shared__ const void* tbl[kMaxE];
    const int bid = blockIdx.x, ng_r = a.k * a.gt_r, v = threadIdx.x >> 6;
    if (bid < ng_r) {
        const int slot = bid / a.gt_r;
        const int e = a.idx[slot];
        const int ej = (bid == 0 && (int)threadIdx.x < a.k) ? a.idx[threadIdx.x] : -1;
        const void* t[kTableRegs];
        load_table(a, t);
        store_table(a, t, tbl);
        __syncthreads();
        if (bid == 0 && (int)threadIdx.x < a.k) a.sel[threadIdx.x] = valid_block(a, tbl, ej);
        gateup_tile<FMT, GD, GP, false>(a, slot, valid_block(a, tbl, e), ((bid % a.gt_r) * 4 + v) * GP, buf);
    } else {
        gateup_tile<FMT, GD, 1, true>(a, a.k, nullptr, (bid - ng_r) * 4 + v, buf);
    }
}

// moe_layer_decode, launch 1: router rows, then the shared expert's gate/up.
template <int FMT, int GD>
__global__ __launch_bounds__(256) void k_router_shared(DecodeArgs a) {
    __shared__ f4v buf[1024];
    const int nr = (a.E + 3) / 4;
    if ((int)blockIdx.x < nr)
        router_rows<2 * GD>(a, blockIdx.x);
    else
        gateup_tile<FMT, GD, 1, true>(a, a.k, nullptr, (blockIdx.x - nr) * 4 + (threadIdx.x >> 6), buf);
}

// moe_layer_decode, launch 2: every workgroup selects the top-k from the
// logits (identically) while the pointer table is staged; workgroup 0
// publishes the routing and the chosen blocks' addresses; then the routed
// gate/up tiles.
template <int FMT, int GD, int GP>
__global__ __launch_bounds__(256) void k_topk_gateup(DecodeArgs a) {
    __shared__ f4v buf[1024];
    __shared__ const void* tbl[kMaxE];
    __shared__ int sel_e;
    const int bid = blockIdx.x, slot = bid / a.gt_r;
    const void* t[kTableRegs];
    load_table(a, t);
    int e = -1;
    float wt = 0.f;
    if (threadIdx.x < 64) {
        topk_select([&](int i) { return a.logits[i]; }, a.E, a.k, e, wt);
        if ((int)threadIdx.x == slot) sel_e = e;
        if (bid == 0 && (int)threadIdx.x < a.k) {
            a.idx_out[threadIdx.x] = e;
            a.w_out[threadIdx.x] = wt;
        }
    }
    store_table(a, t, tbl);
    __syncthreads();
    if (bid == 0 && (int)threadIdx.x < a.k) a.sel[threadIdx.x] = valid_block(a, tbl, e);
    gateup_tile<FMT, GD, GP, false>(a, slot, valid_block(a, tbl, sel_e),
                                    ((bid % a.gt_r) * 4 + (threadIdx.x >> 6)) * GP, buf);
}

// down projection + combine (both entry points): one workgroup per block of
// kDownRB output rows.
// At most 16 waves (1024 threads, 128 VGPRs) where a wave's registers fit in
// 128 (16-lane rows of up to 640 codes); otherwise 8 waves (512 threads, 256
// VGPRs).
constexpr int down_max_waves(int L, int D) { return (L == 16 && D <= 5) ? 16 : 8; }

template <int FMT, int DL, int DD>
__global__ __launch_bounds__(64 * down_max_waves(DL, DD)) void k_down_combine(DecodeArgs a) {
    __shared__ float part[kMaxK + 1][kDownRB];
    __shared__ float wsh[kMaxK];
    down_rows<FMT, DL, DD>(a, blockIdx.x, part, wsh);
}

// ----------------------------------------------------------------------------
template <int FMT>
static hipError_t launch_down(const DecodePlan& p, DecodeArgs& a, hipStream_t s) {
    const int nw = min(down_max_waves(p.down_L, p.down_D), a.n_items);
    dim3 grid(a.H / kDownRB), block(64 * nw);
#define DN(DL, DD) case DD: hipLaunchKernelGGL((k_down_combine<FMT, DL, DD>), grid, block, 0, s, a); break;
    if (p.down_L == 16) {
        switch (p.down_D) {
            DN(16, 1) DN(16, 2) DN(16, 3) DN(16, 4) DN(16, 5) DN(16, 6) DN(16, 7) DN(16, 8)
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.down_D) {
            DN(64, 1) DN(64, 2) DN(64, 3) DN(64, 4) DN(64, 5) DN(64, 6) DN(64, 7) DN(64, 8)
            default: return hipErrorInvalidValue;
        }
    }
#undef DN
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_expert(const DecodePlan& p, DecodeArgs& a, hipStream_t s) {
    const int n_gate = a.k * a.gt_r + (a.has_shared ? a.gt_s : 0);
#define GU(GD, GP) case GD: hipLaunchKernelGGL((k_gateup<FMT, GD, GP>), dim3(n_gate), dim3(256), 0, s, a); break;
    switch (p.gate_D) {
        GU(1, 4) GU(2, 4) GU(3, 4) GU(4, 4) GU(5, 4) GU(6, 2) GU(7, 2) GU(8, 2)
        default: return hipErrorInvalidValue;
    }
#undef GU
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_down<FMT>(p, a, s);
}

template <int FMT>
static hipError_t launch_layer(const DecodePlan& p, DecodeArgs& a, hipStream_t s) {
    const int n1 = (a.E + 3) / 4 + (a.has_shared ? a.gt_s : 0);
#define RS(GD) case GD: hipLaunchKernelGGL((k_router_shared<FMT, GD>), dim3(n1), dim3(256), 0, s, a); break;
    switch (p.gate_D) {
        RS(1) RS(2) RS(3) RS(4) RS(5) RS(6) RS(7) RS(8)
        default: return hipErrorInvalidValue;
    }
#undef RS
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
#define TG(GD, GP) case GD: hipLaunchKernelGGL((k_topk_gateup<FMT, GD, GP>), dim3(a.k * a.gt_r), dim3(256), 0, s, a); break;
    switch (p.gate_D) {
        TG(1, 4) TG(2, 4) TG(3, 4) TG(4, 4) TG(5, 4) TG(6, 2) TG(7, 2) TG(8, 2)
        default: return hipErrorInvalidValue;
    }
#undef TG
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_down<FMT>(p, a, s);
}

static DecodeArgs make_args(const DecodePlan& p, int fmt, int E, int H, int I, int k, const float* x,
                            const void* const* expert_ptrs, const uint16_t* sh_gate, const uint16_t* sh_up,
                            const uint16_t* sh_down, float* y, void* ws) {
    char* base = reinterpret_cast<char*>(ws);
    const size_t h_bytes = align256((size_t)(k + 1) * I * sizeof(float));
    const size_t l_bytes = align256((size_t)E * sizeof(float));
    DecodeArgs a = {};
    a.x = x; a.expert_ptrs = expert_ptrs;
    a.sh_gate = sh_gate; a.sh_up = sh_up; a.sh_down = sh_down;
    a.h = reinterpret_cast<float*>(base + kCounterBytes);
    a.logits = reinterpret_cast<float*>(base + kCounterBytes + h_bytes);
    a.sel = reinterpret_cast<const void**>(base + kCounterBytes + h_bytes + l_bytes);
    a.y = y;
    a.E = E; a.k = k; a.H = H; a.I = I;
    a.has_shared = sh_gate ? 1 : 0;
    a.gt_r = p.gate_wg_per_slot;
    a.gt_s = (I + 3) / 4;  // shared gate/up: one row pair per wave
    a.n_items = k + (a.has_shared ? 2 : 0);
    const size_t n = (size_t)3 * H * I;
    a.block_bytes = (uint32_t)(n / 2 + n / (fmt == kFmtNvfp4 ? 16 : 32));
    return a;
}

hipError_t launch_decode(int fmt, const DecodePlan& p, int E, int H, int I, int k, const float* x,
                         const void* const* expert_ptrs, const int32_t* idx, const float* w,
                         const uint16_t* sh_gate, const uint16_t* sh_up, const uint16_t* sh_down, float* y,
                         void* ws, hipStream_t s) {
    DecodeArgs a = make_args(p, fmt, E, H, I, k, x, expert_ptrs, sh_gate, sh_up, sh_down, y, ws);
    a.idx = idx;
    a.w = w;
    return fmt == kFmtNvfp4 ? launch_expert<kFmtNvfp4>(p, a, s) : launch_expert<kFmtMxfp4>(p, a, s);
}

hipError_t launch_layer_decode(int fmt, const DecodePlan& p, int E, int H, int I, int k, const float* x,
                               const float* Wr, const void* const* expert_ptrs, const uint16_t* sh_gate,
                               const uint16_t* sh_up, const uint16_t* sh_down, float* y, int32_t* idx_out,
                               float* w_out, void* ws, hipStream_t s) {
    DecodeArgs a = make_args(p, fmt, E, H, I, k, x, expert_ptrs, sh_gate, sh_up, sh_down, y, ws);
    a.Wr = Wr;
    a.idx_out = idx_out;
    a.w_out = w_out;
    a.w = w_out;  // the down launch reads the published weights
    return fmt == kFmtNvfp4 ? launch_layer<kFmtNvfp4>(p, a, s) : launch_layer<kFmtMxfp4>(p, a, s);
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
