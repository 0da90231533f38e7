// Single-token decode kernels for gfx950: the FP4-weight GEMVs of one MoE
// layer ([Q] "The engine", item 4: a single-token SwiGLU expert kernel over
// NVFP4 weights), re-designed for CDNA4:
//  * gate/up tiles: gate and up rows of a chosen expert (or of the bf16
//    shared expert) against the LDS-staged activation vector, SiLU*mul
//    epilogue;
//  * down items: a block of 8 output rows of one chosen expert (or of the
//    shared expert) against its hidden vector, per wave; the down launch
//    then forms the weighted combine in fixed expert order in LDS.
// moe_expert_decode is two launches (gate/up, then down + combine);
// moe_layer_decode puts the router GEMV in front of them (three launches),
// and its gate/up launch selects each routed workgroup's expert from the
// router logits itself.
// Kernel boundaries carry the dependencies: on this chip they are cheaper
// than in-kernel device-scope hand-offs between workgroups (an empty launch
// in a graph costs about 1.5 us; a hand-off through device-scope atomics
// several times that).
// The kernels are latency-bound chains of dependent loads, so each level is
// kept short: the loads the weight addresses depend on (the routing or the
// router logits, then the expert pointer table) are issued first, and x
// after them (the memory counter completes in issue order, so a wait for the
// routing never waits for x); the gate/up launch hands the chosen blocks'
// addresses to the down launch, and every weight load of a wave is issued
// before the first one is used.
// Weights are read with coalesced buffer loads (64 lanes x 4 B contiguous),
// e2m1 pairs are converted by v_cvt_scalef32_pk_f32_fp4, the group scale is
// applied once per 8 codes in registers, and rows are reduced with DPP.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kMaxI = 4096;
constexpr int kDownRB = 8;  // output rows per down workgroup
constexpr int kDownNJ = 1;  // routed items per wave in the down launch (16-lane rows)

// Workspace regions after the reserved bytes: h [(k+1)][I], logits [E],
// chosen block addresses [k].
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
    p->gate_P = p->gate_D <= 4 ? 4 : 2;  // 2 pairs per wave at H = 2560: 1 and 4 measured slower
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
    int n_items;             // down-launch items: k routed slots (+ 2 halves of the shared one)
    uint32_t block_bytes;
};

__device__ __forceinline__ const void* valid_block(const DecodeArgs& a, const void* const* tbl, int e) {
    return (unsigned)e < (unsigned)a.E ? tbl[e] : nullptr;
}

// ----------------------------------------------------------------------------
// x (K fp32) on its way to LDS: thread t of the workgroup's 256 loads float4
// chunks t + 256u into registers (load), which are written to LDS later
// (store), after the weight loads have been issued.
template <int K>
struct XStage {
    static constexpr int N = (K / 4 + 255) / 256;
    f4v t[N];
    __device__ __forceinline__ void load(const float* x) {
        const f4v* x4 = reinterpret_cast<const f4v*>(x);
#pragma unroll
        for (int u = 0; u < N; u++) t[u] = x4[min((int)threadIdx.x + 256 * u, K / 4 - 1)];
    }
    __device__ __forceinline__ void store(f4v* xs) const {
#pragma unroll
        for (int u = 0; u < N; u++)
            if ((int)threadIdx.x + 256 * u < K / 4) xs[threadIdx.x + 256 * u] = t[u];
    }
};

// ----------------------------------------------------------------------------
// gate/up rows + SiLU*mul for one tile of a routed expert (block `blk`, NULL
// for an invalid index) or of the shared expert, into slot `slot` of h.
// Wave v handles row pairs pair0 .. pair0+P-1: lanes 0-31 the gate row,
// lanes 32-63 the up row of each pair. Lane s (= lane mod 32) reads 16-code
// chunks c = s + 32m (m < D) of its row: 8 bytes of codes (one NVFP4 scale
// group) with one scale byte, or 32 bytes of bf16 for the shared expert.
// The activations of chunk c come from LDS when the chunk is used, once for
// all P pairs. Gate and up codes ([I][H/2] each) are adjacent in the block,
// as are their scales. xst holds this thread's part of x, already
// requested; every thread of the workgroup calls this (it has a barrier).
template <int FMT, int D, int P, bool SHARED>
__device__ __forceinline__ void gateup_tile(const DecodeArgs& a, int slot, const void* blk, int pair0, f4v* xs,
                                            const XStage<512 * D>& xst) {
    constexpr int K = 512 * D;     // H
    constexpr int G = Fmt<FMT>::G;
    constexpr int KS = K / G;      // scale bytes per row
    const int lane = threadIdx.x & 63, s = lane & 31, half = lane >> 5;  // half 0: gate, 1: up
    const int I = a.I;
    const int np = min(P, I - pair0);  // wave-uniform; <= 0 for idle waves of the last tile
    // an invalid expert index poisons this slot instead of reading anything
    blk = uniform_ptr(blk);
    const bool bad = !SHARED && blk == nullptr;

    // 1. weight loads, unconditional (rows past the last are clamped onto it
    // and their sums dropped; an invalid index gets a buffer of 0 bytes, whose
    // loads return 0 without touching memory), so that the compiler's memory
    // counter waits stay exact
    uint2 wv[P][D];
    uint32_t sv[P][D];
    uint4 v[P][D][2];
    if (SHARED) {
        const uint4* q = reinterpret_cast<const uint4*>(half ? a.sh_up : a.sh_gate);
#pragma unroll
        for (int p = 0; p < P; p++) {
            const size_t row = (size_t)min(pair0 + p, I - 1);
#pragma unroll
            for (int m = 0; m < D; m++) {
                const size_t c = s + 32 * m;
                v[p][m][0] = q[row * (K / 8) + 2 * c];
                v[p][m][1] = q[row * (K / 8) + 2 * c + 1];
            }
        }
    } else {
        const rsrc_t rb = make_rsrc(bad ? (const void*)a.x : blk, bad ? 0u : a.block_bytes);
        const uint32_t scl = (uint32_t)3 * I * (K / 2);
#pragma unroll
        for (int p = 0; p < P; p++) {
            const uint32_t row = (uint32_t)half * I + min(pair0 + p, I - 1);
#pragma unroll
            for (int m = 0; m < D; m++) {
                const uint32_t c = s + 32 * m;
                wv[p][m] = ld_b64(rb, row * (K / 2) + 8 * c);
                sv[p][m] = ld_b8(rb, scl + row * KS + c * 16 / G);
            }
        }
    }

    // 2. x into LDS (it was requested before the weights); the barrier orders
    // LDS only, so the weight loads stay in flight across it
    xst.store(xs);
    lds_barrier();
    if (np > 0) {
        // 3. dot products per chunk (its 16 activations read once for all pairs)
        float acc[P];
#pragma unroll
        for (int p = 0; p < P; p++) acc[p] = 0.f;
#pragma unroll
        for (int m = 0; m < D; m++) {
            const int c = s + 32 * m;
            float xx[16];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const f4v t = xs[4 * c + j];
                xx[4 * j + 0] = t.x; xx[4 * j + 1] = t.y; xx[4 * j + 2] = t.z; xx[4 * j + 3] = t.w;
            }
#pragma unroll
            for (int p = 0; p < P; p++) {
                if (SHARED) {
                    float t = acc[p];
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++) {
                        const uint4 u = v[p][m][h2];
                        const float* x8 = &xx[8 * h2];
                        t = fmaf(bf16_lo(u.x), x8[0], t); t = fmaf(bf16_hi(u.x), x8[1], t);
                        t = fmaf(bf16_lo(u.y), x8[2], t); t = fmaf(bf16_hi(u.y), x8[3], t);
                        t = fmaf(bf16_lo(u.z), x8[4], t); t = fmaf(bf16_hi(u.z), x8[5], t);
                        t = fmaf(bf16_lo(u.w), x8[6], t); t = fmaf(bf16_hi(u.w), x8[7], t);
                    }
                    acc[p] = t;
                } else {
                    acc[p] = fmaf(scale_to_f32<FMT>(sv[p][m]), dot16_fp4(wv[p][m].x, wv[p][m].y, xx), acc[p]);
                }
            }
        }
        // 4. row sums (both rows of a pair in one reduction), SiLU*mul
#pragma unroll
        for (int p = 0; p < P; p++) {
            const float r = row16_sum(acc[p]);
            const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)) +
                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16));
            const float u = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 32)) +
                            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 48));
            if (lane == 0 && p < np)
                a.h[(size_t)slot * I + pair0 + p] = bad ? __uint_as_float(0x7FC00000u) : silu_mul(g, u);
        }
    }
}

// ----------------------------------------------------------------------------
// Down projection, one wave, one item: passes q0 .. q0+nq-1 of row block rb
// (kDownRB rows) of one matrix -- a routed FP4 block (`blk`, NULL for an
// invalid index) or the bf16 shared down -- against h[slot]. A row is
// covered by L lanes (RPW = 64/L rows per pass, pass q holds rows
// rb*kDownRB + grp + q*RPW); lane s of a row reads code dwords s + L*m
// (m < D, while < I/8) and the matching 8 hidden values per dword. The row
// sum of pass q goes to dst[grp + q*RPW] (LDS or global).
// The hidden vector is held in registers, or (hs != NULL) staged in this
// wave's own LDS slice of I floats and read back per column chunk, which
// frees 8D registers.
template <int FMT, int L, int D, bool SHARED, bool HL>
__device__ __forceinline__ void down_item(const DecodeArgs& a, int slot, const void* blk, int rb, int q0, int nq,
                                          float* dst, f4v* hs) {
    constexpr int G = Fmt<FMT>::G;
    constexpr int RPW = 64 / L;               // rows per wave pass
    constexpr int PASSES = kDownRB / RPW;     // passes for all rows of the block
    // passes per load group: it divides nq (all PASSES passes for a routed
    // item, PASSES / 2 for a shared half item), and the shared expert's
    // 16-byte bf16 chunks hold 4x the registers of the FP4 dwords
    constexpr int QC = SHARED ? (PASSES < 4 ? PASSES / 2 : (D >= 7 ? 1 : 2))
                              : (PASSES < 4 ? PASSES : (D >= 7 ? 2 : 4));
    const int lane = threadIdx.x & 63;
    const int H = a.H, I = a.I;
    const int KD = I / 8, KS = I / G;
    const int grp = lane / L, s = lane % L;
    blk = uniform_ptr(blk);
    const bool bad = !SHARED && blk == nullptr;
    const int row0 = rb * kDownRB + grp;
    // the hidden vector of this item's slot (zero past the row's end); every
    // global load below is unconditional, with indices clamped, so that the
    // compiler's memory counter waits stay exact
    const f4v* hp = reinterpret_cast<const f4v*>(a.h + (size_t)slot * I);
    float hr[HL ? 1 : 8 * D];
    if constexpr (HL) {
        constexpr int NU = (2 * L * D + 63) / 64;  // float4 chunks per lane (I/4 <= 2*L*D)
        f4v t[NU];
#pragma unroll
        for (int u = 0; u < NU; u++) t[u] = hp[min(lane + 64 * u, 2 * KD - 1)];
#pragma unroll
        for (int u = 0; u < NU; u++)
            if (lane + 64 * u < 2 * KD) hs[lane + 64 * u] = t[u];
    } else {
#pragma unroll
        for (int m = 0; m < D; m++) {
            const int c = min(s + L * m, KD - 1);
            const f4v p0 = hp[2 * c], p1 = hp[2 * c + 1];
            hr[8 * m + 0] = p0.x; hr[8 * m + 1] = p0.y; hr[8 * m + 2] = p0.z; hr[8 * m + 3] = p0.w;
            hr[8 * m + 4] = p1.x; hr[8 * m + 5] = p1.y; hr[8 * m + 6] = p1.z; hr[8 * m + 7] = p1.w;
        }
    }
    // an invalid index gets a buffer of 0 bytes: its loads return 0 without
    // touching memory, and its rows are poisoned below
    const rsrc_t rbuf = make_rsrc(SHARED || bad ? (const void*)a.x : blk, SHARED || bad ? 0u : a.block_bytes);
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
#pragma unroll
            for (int m = 0; m < D; m++) {
                const uint32_t c = min(s + L * m, KD - 1);
                if (SHARED) {
                    v[q][m] = dq[(size_t)row * KD + c];
                } else {
                    wv[q][m] = ld_b32(rbuf, codes + row * (I / 2) + 4 * c);
                    sv[q][m] = ld_b8(rbuf, scl + row * KS + c * 8 / G);
                }
            }
        }
        float acc[QC];
#pragma unroll
        for (int q = 0; q < QC; q++) acc[q] = 0.f;
        // per column chunk m: its 8 hidden values, then every pass of the group
        // (each pass still accumulates over m in increasing order)
#pragma unroll
        for (int m = 0; m < D; m++) {
            const bool in = s + L * m < KD;  // columns past the row's end leave acc unchanged
            float xx[8];
            if constexpr (HL) {
                const int c = min(s + L * m, KD - 1);
                const f4v p0 = hs[2 * c], p1 = hs[2 * c + 1];
                xx[0] = p0.x; xx[1] = p0.y; xx[2] = p0.z; xx[3] = p0.w;
                xx[4] = p1.x; xx[5] = p1.y; xx[6] = p1.z; xx[7] = p1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) xx[i] = hr[8 * m + i];
            }
#pragma unroll
            for (int q = 0; q < QC; q++) {
                float t = acc[q];
                if (SHARED) {
                    const uint4 u = v[q][m];
                    t = fmaf(bf16_lo(u.x), xx[0], t); t = fmaf(bf16_hi(u.x), xx[1], t);
                    t = fmaf(bf16_lo(u.y), xx[2], t); t = fmaf(bf16_hi(u.y), xx[3], t);
                    t = fmaf(bf16_lo(u.z), xx[4], t); t = fmaf(bf16_hi(u.z), xx[5], t);
                    t = fmaf(bf16_lo(u.w), xx[6], t); t = fmaf(bf16_hi(u.w), xx[7], t);
                } else {
                    t = fmaf(scale_to_f32<FMT>(sv[q][m]), dot8_fp4(wv[q][m], xx), t);
                }
                acc[q] = in ? t : acc[q];
            }
        }
#pragma unroll
        for (int q = 0; q < QC; q++) {
            float r = (L == 16) ? row16_sum(acc[q]) : wave_sum(acc[q]);
            if (bad) r = __uint_as_float(0x7FC00000u);
            if (s == 0) dst[grp + (q0 + qc + q) * RPW] = r;
        }
    }
}

// ----------------------------------------------------------------------------
// Down projection of NJ routed items at once by one wave (16-lane rows, the
// hidden vectors staged in the wave's LDS slices): the same rows, passes and
// arithmetic as down_item for each item, with the loads of all items issued
// before the first is used. Item j: slot[j], block blk[j] (NULL: invalid
// index; an item with slot[j] < 0 is absent), row sums to dst[j].
template <int FMT, int D, int NJ>
__device__ __forceinline__ void down_items16(const DecodeArgs& a, const int (&slot)[NJ], const void* (&blk)[NJ],
                                             int rb, float* const (&dst)[NJ], f4v* hs) {
    constexpr int L = 16, G = Fmt<FMT>::G;
    constexpr int RPW = 64 / L, PASSES = kDownRB / RPW;  // 4 rows per pass, 2 passes
    const int lane = threadIdx.x & 63;
    const int H = a.H, I = a.I;
    const int KD = I / 8, KS = I / G;
    const int grp = lane / L, s = lane % L;
    const int row0 = rb * kDownRB + grp;
    const uint32_t codes = (uint32_t)I * H;
    const uint32_t scl = (uint32_t)3 * I * H / 2 + (uint32_t)2 * I * H / G;
    bool bad[NJ];
    rsrc_t rbuf[NJ];
    // hidden vectors -> LDS (unconditional loads, clamped indices)
    {
        constexpr int NU = (2 * L * D + 63) / 64;
        f4v t[NJ][NU];
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const f4v* hp = reinterpret_cast<const f4v*>(a.h + (size_t)max(slot[j], 0) * I);
#pragma unroll
            for (int u = 0; u < NU; u++) t[j][u] = hp[min(lane + 64 * u, 2 * KD - 1)];
        }
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            blk[j] = uniform_ptr(blk[j]);
            bad[j] = blk[j] == nullptr;
            rbuf[j] = make_rsrc(bad[j] ? (const void*)a.x : blk[j], bad[j] ? 0u : a.block_bytes);
#pragma unroll
            for (int u = 0; u < NU; u++)
                if (lane + 64 * u < 2 * KD) hs[j * (I / 4) + lane + 64 * u] = t[j][u];
        }
    }
    uint32_t wv[NJ][PASSES][D], sv[NJ][PASSES][D];
#pragma unroll
    for (int j = 0; j < NJ; j++)
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const uint32_t row = (uint32_t)row0 + q * RPW;
#pragma unroll
            for (int m = 0; m < D; m++) {
                const uint32_t c = min(s + L * m, KD - 1);
                wv[j][q][m] = ld_b32(rbuf[j], codes + row * (I / 2) + 4 * c);
                sv[j][q][m] = ld_b8(rbuf[j], scl + row * KS + c * 8 / G);
            }
        }
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        float acc[PASSES];
#pragma unroll
        for (int q = 0; q < PASSES; q++) acc[q] = 0.f;
#pragma unroll
        for (int m = 0; m < D; m++) {
            const bool in = s + L * m < KD;
            const int c = min(s + L * m, KD - 1);
            const f4v p0 = hs[j * (I / 4) + 2 * c], p1 = hs[j * (I / 4) + 2 * c + 1];
            const float xx[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int q = 0; q < PASSES; q++) {
                const float t = fmaf(scale_to_f32<FMT>(sv[j][q][m]), dot8_fp4(wv[j][q][m], xx), acc[q]);
                acc[q] = in ? t : acc[q];
            }
        }
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            float r = row16_sum(acc[q]);
            if (bad[j]) r = __uint_as_float(0x7FC00000u);
            if (s == 0 && slot[j] >= 0) dst[j][grp + q * RPW] = r;
        }
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

// moe_layer_decode, launch 1: the router GEMV, one logit row per wave and two
// waves per workgroup (one round of workgroups covers the chip); lane l reads
// float4 chunks l + 64m of the row and of x (H = 256 * DV).
template <int DV>
__global__ __launch_bounds__(128) void k_router(DecodeArgs a) {
    const int lane = threadIdx.x & 63, e = blockIdx.x * 2 + wave_id();
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

// Gate/up launch of both entry points: the routed gate/up tiles, then the
// shared expert's. TNI = 0 (moe_expert_decode): the routing is given, and
// workgroup 0 publishes the chosen blocks' addresses for the down launch.
// TNI > 0 (moe_layer_decode): every routed workgroup selects the experts
// from the router logits (TNI per lane of its first wave, E <= 64 TNI), up to
// its own slot, so that early slots start streaming early; the first
// workgroup of the last slot, which runs all k rounds, publishes the routing,
// the weights and the chosen blocks' addresses. The loads the weight
// addresses depend on go first (the routing or the logits, then the expert
// pointer table, staged in LDS), x after them.
template <int FMT, int GD, int GP, int TNI>
__global__ __launch_bounds__(256) void k_gateup(DecodeArgs a) {
    __shared__ f4v buf[1024];  // x, H <= 4096
    __shared__ const void* tbl[kMaxE];
    __shared__ int sel_e;
    constexpr int NTB = TNI > 0 ? (64 * TNI + 255) / 256 : kTableRegs;  // table entries per thread
    const int bid = blockIdx.x, ng_r = a.k * a.gt_r, t = threadIdx.x;
    if (bid >= ng_r) {
        XStage<512 * GD> xst;
        xst.load(a.x);
        gateup_tile<FMT, GD, 1, true>(a, a.k, nullptr, (bid - ng_r) * 4 + wave_id(), buf, xst);
        return;
    }
    const int slot = bid / a.gt_r;
    float f[TNI > 0 ? TNI : 1];
    int e = -1;    // this lane's chosen expert (for the publisher)
    int eg = 0;    // the slot's expert (given routing)
    if constexpr (TNI > 0) {
        if (t < 64) {
#pragma unroll
            for (int i = 0; i < TNI; i++) f[i] = a.logits[min(t * TNI + i, a.E - 1)];
        }
    } else {
        eg = a.idx[slot];
        e = a.idx[min(t, a.k - 1)];  // used by workgroup 0, threads < k
    }
    const void* tp[NTB];
#pragma unroll
    for (int u = 0; u < NTB; u++) tp[u] = a.expert_ptrs[min(t + 256 * u, a.E - 1)];
    XStage<512 * GD> xst;
    xst.load(a.x);
    const bool publisher = TNI > 0 ? bid == (a.k - 1) * a.gt_r : bid == 0;
    if constexpr (TNI > 0) {
        if (t < 64) {
            float wt;
            topk_select_vals<TNI>(f, a.E, publisher ? a.k : slot + 1, e, wt);
            if (t == slot) sel_e = e;
            if (publisher && t < a.k) {
                a.idx_out[t] = e;
                a.w_out[t] = wt;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < NTB; u++)
        if (t + 256 * u < a.E) tbl[t + 256 * u] = tp[u];
    lds_barrier();
    if (publisher && t < a.k) a.sel[t] = valid_block(a, tbl, e);
    gateup_tile<FMT, GD, GP, false>(a, slot, valid_block(a, tbl, TNI > 0 ? sel_e : eg),
                                    ((bid % a.gt_r) * 4 + wave_id()) * GP, buf, xst);
}

// down projection + combine (both entry points): one workgroup per block of
// kDownRB output rows; wave v takes items v, v + nwaves, ... (item j < k:
// routed slot j; items k, k+1: the two halves of the shared expert's rows).
// Thread r then forms y[row] = sum_j w[j] * part[j][r] (+ the shared row)
// in increasing j.
// At most 16 waves (1024 threads, 128 VGPRs) where a wave's registers fit in
// 128 (16-lane rows of up to 640 codes); 4 waves (512 VGPRs) for the widest
// rows (more than 3584 codes); otherwise 8 waves (512 threads, 256 VGPRs).
constexpr int down_max_waves(int L, int D) { return (L == 16 && D <= 5) ? 16 : (D >= 8 ? 4 : 8); }

// SH: the layer has a shared expert, whose rows are items of this launch.
// PAIRS (16-lane rows,
// when the units fit the workgroup): one unit per wave, routed items two at
// a time plus one wave per shared half, so that several small workgroups
// share a CU and a launch covers the chip in one round. Otherwise waves loop
// over single items.
template <int FMT, int DL, int DD, bool SH, bool PAIRS>
__global__ __launch_bounds__(64 * down_max_waves(DL, DD)) void k_down_combine(DecodeArgs a) {
    __shared__ float part[kMaxK + 1][kDownRB];
    __shared__ float wsh[kMaxK];
    extern __shared__ f4v hsm[];  // 16-lane rows: hidden vectors, I-float slices per wave (dynamic size)
    constexpr bool HL = DL == 16;
    constexpr int PASSES = kDownRB / (64 / DL);
    const int tid = threadIdx.x, wave = wave_id(), nwaves = blockDim.x >> 6;
    const int rb = blockIdx.x, k = a.k;
    // the combine's weights: loaded now, stored to LDS after the items (a
    // store here would hold wave 0's weight loads behind this load)
    const float wt = a.w[min(tid, k - 1)];
    if constexpr (PAIRS) {
        // one unit per wave: kDownNJ routed items (items w, w + npair, ...),
        // then the two halves of the shared expert's rows; the wave's kDownNJ
        // LDS slices hold the hidden vectors
        constexpr int NJ = kDownNJ;
        const int npair = (k + NJ - 1) / NJ;
        f4v* hs = hsm + (size_t)wave * NJ * (a.I / 4);
        if (wave < npair) {
            int sl[NJ];
            const void* bl[NJ];
            float* dd[NJ];
#pragma unroll
            for (int i = 0; i < NJ; i++) {
                sl[i] = wave + i * npair < k ? wave + i * npair : -1;
                bl[i] = sl[i] >= 0 ? a.sel[sl[i]] : nullptr;
                dd[i] = part[max(sl[i], 0)];
            }
            down_items16<FMT, DD, NJ>(a, sl, bl, rb, dd, hs);
        } else if (SH) {
            down_item<FMT, DL, DD, true, true>(a, k, nullptr, rb, (wave - npair) * (PASSES / 2), PASSES / 2,
                                               part[k], hs);
        }
    } else {
        for (int item = wave; item < a.n_items; item += nwaves) {
            f4v* hs = HL ? hsm + (size_t)wave * (a.I / 4) : nullptr;
            if (!SH || item < k)
                down_item<FMT, DL, DD, false, HL>(a, item, a.sel[item], rb, 0, PASSES, part[item], hs);
            else
                down_item<FMT, DL, DD, true, HL>(a, k, nullptr, rb, (item - k) * (PASSES / 2), PASSES / 2, part[k],
                                                 hs);
        }
    }
    if (tid < k) wsh[tid] = wt;
    __syncthreads();
    if (tid < kDownRB) {
        const int row = rb * kDownRB + tid;
        float acc = 0.f;
        for (int j = 0; j < k; j++) acc = fmaf(wsh[j], part[j][tid], acc);
        if (a.has_shared) acc += part[k][tid];
        a.y[row] = acc;
    }
}

// ----------------------------------------------------------------------------
// Streaming forms for large layers. When the chosen experts' weights are
// many times what one round of resident workgroups has in flight, the
// one-shot tiles above run in several rounds, each paying the full memory
// latency. Here a resident grid (one workgroup of four waves per compute
// unit: a wave per SIMD) keeps loads in flight continuously instead.
// A wave covers a weight row with all 64 lanes: lane l reads the 16-byte
// chunks c = l + 64m (32 codes each), so every load instruction reads 1 KB
// of one row contiguously, and the wave keeps the activations of its chunks
// (x, or one hidden vector) in registers for every row it reads.
// gate/up row pairs in flight per wave: 4 for moe_expert_decode, 3 for the
// layer form (whose top-k runs first). Measured at the DeepSeek shape: with
// three workgroups per compute unit 2 and 3 did best (more cost registers and
// resident waves); with one per compute unit 3 and 4 are 2% faster again.
template <bool TOPK>
constexpr int stream_dp() { return TOPK ? 3 : 4; }
constexpr int kStreamRows = 16;  // down rows per workgroup

__device__ __forceinline__ uint32_t ld_b16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// sum over the 32 codes of chunk w (16 bytes) times x[0..31], with the
// chunk's scales: NVFP4 two E4M3 bytes (16 codes each) applied to the two
// partial sums; MXFP4 one UE8M0 byte, handed to the e2m1 conversion itself
// (it multiplies by 2^(byte - 127) exactly: the byte is the exponent field
// of its fp32 scale operand), so the products need no separate scaling.
template <int FMT>
__device__ __forceinline__ float chunk_dot(const uint4& w, uint32_t sc, const float* x, float acc) {
    if constexpr (FMT == kFmtNvfp4) {
        acc = fmaf(e4m3_to_f32(sc & 0xFFu), dot16_fp4(w.x, w.y, x), acc);
        return fmaf(e4m3_to_f32((sc >> 8) & 0xFFu), dot16_fp4(w.z, w.w, x + 16), acc);
    } else {
        const float s = __uint_as_float((sc & 0xFFu) << 23);
        const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const f2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], s, 0);
            const f2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], s, 1);
            const f2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], s, 2);
            const f2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q[i], s, 3);
            acc = fmaf(p0.x, x[8 * i + 0], acc); acc = fmaf(p0.y, x[8 * i + 1], acc);
            acc = fmaf(p1.x, x[8 * i + 2], acc); acc = fmaf(p1.y, x[8 * i + 3], acc);
            acc = fmaf(p2.x, x[8 * i + 4], acc); acc = fmaf(p2.y, x[8 * i + 5], acc);
            acc = fmaf(p3.x, x[8 * i + 6], acc); acc = fmaf(p3.y, x[8 * i + 7], acc);
        }
        return acc;
    }
}

// this lane's activations of chunks lane + 64m: xs[m][0..31] = v[32c ..]
template <int NCH>
__device__ __forceinline__ void load_chunk_acts(const float* v, int nchunk, float (&xs)[NCH][32]) {
    const f4v* v4 = reinterpret_cast<const f4v*>(v);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int m = 0; m < NCH; m++) {
        const int c = min(lane + 64 * m, nchunk - 1);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const f4v t = v4[8 * c + i];
            xs[m][4 * i] = t.x; xs[m][4 * i + 1] = t.y; xs[m][4 * i + 2] = t.z; xs[m][4 * i + 3] = t.w;
        }
    }
}

// cache policy of the weight loads: non-temporal (each weight byte is read
// once per call)
constexpr int kNT = 2;

// c ? a : b as integer arithmetic (the compiler turns some conditionals on
// lane-dependent values into branches)
__device__ __forceinline__ uint32_t sel_u32(bool c, uint32_t a, uint32_t b) {
    const uint32_t m = 0u - (uint32_t)c;
    return (a & m) | (b & ~m);
}
// marks a loaded value as used (the compiler then waits for its load here)
__device__ __forceinline__ void consume(const uint4& v) {
    asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}
__device__ __forceinline__ void consume(uint32_t v) { asm volatile("" ::"v"(v)); }

// gate/up + SiLU*mul, streaming. Units u = slot * I + row (gate row and up
// row of one routed slot) are split into contiguous ranges, one per
// workgroup of the grid (one per compute unit); wave w takes units
// w, w + 4, ... of its workgroup's range, so the four waves sweep adjacent
// rows together, and keeps stream_dp<TOPK>() units of loads in flight. The scales
// of a unit come with one dword per lane (MXFP4: lanes 0-31 the gate row's,
// 32-63 the up row's; NVFP4: one dword of each row) and reach the lanes that
// need them by ds_bpermute. TOPK (moe_layer_decode): the workgroup first
// selects the experts of the slots its range touches from the logits; the
// last workgroup, whose range ends with the last slot, publishes the
// routing. Otherwise (moe_expert_decode) the routing is given and workgroup
// 0 publishes the chosen blocks' addresses for the down launch.
template <int FMT, int NCH, bool TOPK>
__global__ __launch_bounds__(256) void k_gateup_stream(DecodeArgs a) {
    constexpr int G = Fmt<FMT>::G;
    constexpr int DP = stream_dp<TOPK>();
    constexpr int NSC = FMT == kFmtNvfp4 ? 2 : 1;  // scale dwords per lane per unit
    __shared__ const void* blks[kMaxK];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int H = a.H, I = a.I, k = a.k;
    const int nchunk = H / 32;
    const uint32_t KB = (uint32_t)H / 2, KS = (uint32_t)H / G;
    const uint32_t sbase = (uint32_t)3 * I * (H / 2);
    const int U = k * I;
    const long long nwg = gridDim.x, b = blockIdx.x;
    const int wu0 = (int)(U * b / nwg), wu1 = (int)(U * (b + 1) / nwg);
    const int u0 = wu0 + wave, u1 = wu1;
    float xs[NCH][32];
    if constexpr (TOPK) {
        load_chunk_acts<NCH>(a.x, nchunk, xs);  // in flight during the top-k
        // slots this workgroup's range touches: 0 .. need-1
        const int need = wu1 > wu0 ? (wu1 - 1) / I + 1 : 1;
        const bool publisher = blockIdx.x == gridDim.x - 1;
        if (threadIdx.x < 64) {
            int e = -1;
            float wt = 0.f;
            topk_select([&](int i) { return a.logits[i]; }, a.E, publisher ? k : need, e, wt);
            if (lane < k) {
                const void* bp = valid_block(a, a.expert_ptrs, e);
                blks[lane] = bp;
                if (publisher) {
                    a.idx_out[lane] = e;
                    a.w_out[lane] = wt;
                    a.sel[lane] = bp;
                }
            }
        }
    } else {
        if ((int)threadIdx.x < k) {
            const void* bp = valid_block(a, a.expert_ptrs, a.idx[threadIdx.x]);
            blks[threadIdx.x] = bp;
            if (blockIdx.x == 0) a.sel[threadIdx.x] = bp;
        }
    }
    lds_barrier();
    if constexpr (!TOPK) load_chunk_acts<NCH>(a.x, nchunk, xs);  // needed from the first unit on

    const rsrc_t rh = make_rsrc(a.h, (uint32_t)(4 * U));
    uint4 cw[DP][2][NCH];
    uint32_t sw[DP][NSC];
    // loads of unit u into register set d (past the range: out-of-range
    // offsets, zeros without memory traffic; an invalid expert: a buffer of
    // 0 bytes)
    auto issue = [&](int d, int u) {
        const bool on = u < u1;
        const int uu = min(on ? u : u0, U - 1);
        const int slot = uu / I, r = uu % I;
        const void* blk = uniform_ptr(blks[slot]);
        const rsrc_t rs = make_rsrc(blk ? blk : (const void*)a.x, blk ? a.block_bytes : 0u);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const uint32_t row = (uint32_t)(h * I + r);
#pragma unroll
            for (int m = 0; m < NCH; m++) {
                const int c = lane + 64 * m;
                const bool ok = on && c < nchunk;
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, sel_u32(ok, row * KB + 16u * c, kOOB), 0, kNT);
                cw[d][h][m] = uint4{v[0], v[1], v[2], v[3]};
            }
        }
        if constexpr (NSC == 1) {
            const uint32_t row = (uint32_t)((lane >> 5) * I + r), o = 4u * (lane & 31);
            sw[d][0] = ld_b32(rs, sel_u32(on && o < KS, sbase + row * KS + o, kOOB));
        } else {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint32_t row = (uint32_t)(h * I + r), o = 4u * lane;
                sw[d][h] = ld_b32(rs, sel_u32(on && o < KS, sbase + row * KS + o, kOOB));
            }
        }
    };
    // scale bits of chunk c of row h (MXFP4: its byte; NVFP4: its two bytes)
    auto chunk_scale = [&](const uint32_t (&sc)[NSC], int h, int c) -> uint32_t {
        if constexpr (NSC == 1) {
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (h * 32 + (c >> 2)), (int)sc[0]);
            return v >> (8 * (c & 3));
        } else {
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (c >> 1), (int)sc[h]);
            return v >> (16 * (c & 1));
        }
    };
    auto compute = [&](int d, int u) {
        if (u >= u1) {
            // nothing to compute (uniform), but the set's loads are used here
            // as on the other path, so that the compiler's waits after this
            // point stay the same on both
#pragma unroll
            for (int h = 0; h < 2; h++)
#pragma unroll
                for (int m = 0; m < NCH; m++) consume(cw[d][h][m]);
#pragma unroll
            for (int i = 0; i < NSC; i++) consume(sw[d][i]);
            return;
        }
        const int slot = u / I, r = u % I;
        // every scale permute first, so that one LDS wait covers them all
        uint32_t scv[2][NCH];
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int m = 0; m < NCH; m++) scv[h][m] = chunk_scale(sw[d], h, min(lane + 64 * m, nchunk - 1));
        float t[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < NCH; m++) acc = chunk_dot<FMT>(cw[d][h][m], scv[h][m], xs[m], acc);
            t[h] = wave_sum(acc);
        }
        // one store instruction (lanes other than 0 store to an out-of-range
        // offset, which is dropped); integer selects, no branch
        const uint32_t badm = 0u - (uint32_t)(blks[slot] == nullptr);  // all ones: invalid expert -> NaN
        const uint32_t hv = __float_as_uint(silu_mul(t[0], t[1])) | (badm & 0x7FC00000u);
        const uint32_t keep = 0u - (uint32_t)(lane == 0);
        const uint32_t off = 4u * (uint32_t)(slot * I + r);
        __builtin_amdgcn_raw_buffer_store_b32(hv, rh, (off & keep) | (kOOB & ~keep), 0, 0);
    };
    // the empty asm statements keep the units' loads in issue order (the
    // scheduler would otherwise interleave the sets, and the wait for the
    // first set would become a wait for all of them)
#pragma unroll
    for (int d = 0; d < DP; d++) {
        issue(d, u0 + 4 * d);
        asm volatile("" ::: "memory");
    }
    for (int ub = u0; ub < u1; ub += 4 * DP) {
#pragma unroll
        for (int d = 0; d < DP; d++) {
            compute(d, ub + 4 * d);
            issue(d, ub + 4 * (d + DP));
            asm volatile("" ::: "memory");
        }
    }
}

// down projection + combine, streaming form: workgroup = k waves (wave j:
// routed slot j) x kStreamRows output rows. Wave j holds its chunks of h[j]
// in registers and has the loads of all its rows in flight at once. The
// rows' scale bytes are contiguous in the block: one 16-byte load per lane
// brings them to the wave's LDS slice (one-byte loads per chunk measured
// about 1.5x slower for the whole launch), where each lane reads its own.
// The row sums meet in LDS and thread r forms y[row] = sum_j w[j] *
// part[j][r] in increasing j (the same order as k_down_combine).
template <int FMT, int NCH>
__global__ __launch_bounds__(64 * 8) void k_down_stream(DecodeArgs a) {
    constexpr int G = Fmt<FMT>::G;
    constexpr int R = kStreamRows;
    constexpr int SCB = R * 4096 / G;  // scale bytes of R rows, I <= 4096
    __shared__ float part[8][R];
    __shared__ float wsh[8];
    __shared__ __attribute__((aligned(16))) uint8_t scs[8][SCB];
    const int tid = threadIdx.x, lane = tid & 63, j = wave_id();
    const int H = a.H, I = a.I, k = a.k;
    const int nchunk = I / 32;
    const uint32_t KB = (uint32_t)I / 2, KS = (uint32_t)I / G;
    const uint32_t codes0 = (uint32_t)I * H;                                  // down codes [H][I/2]
    const uint32_t scl0 = (uint32_t)3 * I * H / 2 + (uint32_t)2 * I * H / G;  // down scales [H][I/G]
    const int n0 = blockIdx.x * R;
    const void* blk = uniform_ptr(a.sel[j]);
    const bool bad = blk == nullptr;
    const rsrc_t rs = make_rsrc(bad ? (const void*)a.x : blk, bad ? 0u : a.block_bytes);
    uint4 cw[R][NCH];
#pragma unroll
    for (int q = 0; q < R; q++) {
        const uint32_t row = (uint32_t)(n0 + q);
#pragma unroll
        for (int m = 0; m < NCH; m++) {
            const int c = lane + 64 * m;
            const auto v =
                __builtin_amdgcn_raw_buffer_load_b128(rs, sel_u32(c < nchunk, codes0 + row * KB + 16u * c, kOOB), 0, kNT);
            cw[q][m] = uint4{v[0], v[1], v[2], v[3]};
        }
    }
    // scales of rows n0 .. n0+R-1: R*KS contiguous bytes at a 16-byte
    // aligned offset (R*KS = I/4 or I/2, a multiple of 16 as I % 64 == 0)
    constexpr int NSL = (SCB + 1023) / 1024;
    uint4 sl[NSL];
#pragma unroll
    for (int i = 0; i < NSL; i++) {
        const uint32_t o = 16u * (lane + 64 * i);
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, sel_u32(o < R * KS, scl0 + n0 * KS + o, kOOB), 0, 0);
        sl[i] = uint4{v[0], v[1], v[2], v[3]};
    }
    float hs[NCH][32];
    load_chunk_acts<NCH>(a.h + (size_t)j * I, nchunk, hs);
    if (tid < k) wsh[tid] = a.w[tid];
#pragma unroll
    for (int i = 0; i < NSL; i++) {
        const int o = 16 * (lane + 64 * i);
        if (o < SCB) *reinterpret_cast<uint4*>(&scs[j][o]) = sl[i];
    }
    // (this wave's LDS writes and reads stay in order: no barrier needed)
#pragma unroll
    for (int q = 0; q < R; q++) {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < NCH; m++) {
            const int c = min(lane + 64 * m, nchunk - 1);
            const uint32_t so = (uint32_t)q * KS + (FMT == kFmtNvfp4 ? 2u * c : (uint32_t)c);
            const uint32_t sc = FMT == kFmtNvfp4 ? *reinterpret_cast<const uint16_t*>(&scs[j][so]) : scs[j][so];
            acc = chunk_dot<FMT>(cw[q][m], sc, hs[m], acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) part[j][q] = bad ? __uint_as_float(0x7FC00000u) : acc;
    }
    __syncthreads();
    if (tid < R) {
        float acc = 0.f;
        for (int jj = 0; jj < k; jj++) acc = fmaf(wsh[jj], part[jj][tid], acc);
        a.y[n0 + tid] = acc;
    }
}

// The same launch for rows of 65 to 96 chunks (2048 < I <= 3072). Each row's
// first 64 chunks take one load across the wave; the remaining chunks (at
// most 32) of two neighbouring rows share one load, lanes 0-31 the first
// row's and lanes 32-63 the second's. Two rows then cost three loads and
// three chunk products per lane instead of four (a quarter of the general
// form's lanes idle at I = 2880). NH waves share a routed slot, each with
// R / NH of the rows: with k <= 6, two per slot put three waves on every
// SIMD instead of one or two (down 14.05 -> 13.44 us at the DeepSeek shape).
template <int FMT, int NH>
__global__ __launch_bounds__(NH == 2 ? 64 * 12 : 64 * 8) void k_down_stream_pair(DecodeArgs a) {  // NH = 2: k <= 6
    constexpr int G = Fmt<FMT>::G;
    constexpr int R = kStreamRows;
    constexpr int RW = R / NH;              // rows per wave
    constexpr int SCB = RW * 3072 / G;      // scale bytes of RW rows, I <= 3072
    __shared__ float part[8][R];
    __shared__ float wsh[8];
    __shared__ __attribute__((aligned(16))) uint8_t scs[8 * NH][SCB];
    const int tid = threadIdx.x, lane = tid & 63, wv = wave_id();
    const int j = wv / NH, q0w = (wv % NH) * RW;  // routed slot, first row of this wave
    const int H = a.H, I = a.I, k = a.k;
    const int nchunk = I / 32, ntail = nchunk - 64;  // 1 .. 32
    const int hi = lane >> 5, tl = lane & 31;
    const int ct = min(64 + tl, nchunk - 1);  // this lane's tail chunk (clamped)
    const uint32_t KB = (uint32_t)I / 2, KS = (uint32_t)I / G;
    const uint32_t codes0 = (uint32_t)I * H;
    const uint32_t scl0 = (uint32_t)3 * I * H / 2 + (uint32_t)2 * I * H / G;
    const int n0 = blockIdx.x * R + q0w;  // this wave's first output row
    const void* blk = uniform_ptr(a.sel[j]);
    const bool bad = blk == nullptr;
    const rsrc_t rs = make_rsrc(bad ? (const void*)a.x : blk, bad ? 0u : a.block_bytes);
    uint4 cw[RW], cwt[RW / 2];
#pragma unroll
    for (int q = 0; q < RW; q++) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, codes0 + (uint32_t)(n0 + q) * KB + 16u * lane, 0, kNT);
        cw[q] = uint4{v[0], v[1], v[2], v[3]};
    }
#pragma unroll
    for (int p = 0; p < RW / 2; p++) {
        const uint32_t row = (uint32_t)(n0 + 2 * p + hi);
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(
            rs, sel_u32(tl < ntail, codes0 + row * KB + 16u * (64 + tl), kOOB), 0, kNT);
        cwt[p] = uint4{v[0], v[1], v[2], v[3]};
    }
    constexpr int NSL = (SCB + 1023) / 1024;
    uint4 sl[NSL];
#pragma unroll
    for (int i = 0; i < NSL; i++) {
        const uint32_t o = 16u * (lane + 64 * i);
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, sel_u32(o < RW * KS, scl0 + n0 * KS + o, kOOB), 0, 0);
        sl[i] = uint4{v[0], v[1], v[2], v[3]};
    }
    // activations of chunk lane (set 0) and of the tail chunk (set 1)
    float hs[2][32];
    {
        const f4v* v4 = reinterpret_cast<const f4v*>(a.h + (size_t)j * I);
        const int cc[2] = {lane, ct};
#pragma unroll
        for (int m = 0; m < 2; m++)
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const f4v t = v4[8 * cc[m] + i];
                hs[m][4 * i] = t.x; hs[m][4 * i + 1] = t.y; hs[m][4 * i + 2] = t.z; hs[m][4 * i + 3] = t.w;
            }
    }
    if (tid < k) wsh[tid] = a.w[tid];
#pragma unroll
    for (int i = 0; i < NSL; i++) {
        const int o = 16 * (lane + 64 * i);
        if (o < SCB) *reinterpret_cast<uint4*>(&scs[wv][o]) = sl[i];
    }
    auto scale = [&](int q, int c) -> uint32_t {
        const uint32_t so = (uint32_t)q * KS + (FMT == kFmtNvfp4 ? 2u * c : (uint32_t)c);
        return FMT == kFmtNvfp4 ? *reinterpret_cast<const uint16_t*>(&scs[wv][so]) : scs[wv][so];
    };
    // (this wave's LDS writes and reads stay in order: no barrier needed)
#pragma unroll
    for (int p = 0; p < RW / 2; p++) {
        const int q0 = 2 * p, q1 = 2 * p + 1;
        float acc0 = chunk_dot<FMT>(cw[q0], scale(q0, lane), hs[0], 0.f);
        float acc1 = chunk_dot<FMT>(cw[q1], scale(q1, lane), hs[0], 0.f);
        float t = chunk_dot<FMT>(cwt[p], scale(q0 + hi, ct), hs[1], 0.f);
        t = tl < ntail ? t : 0.f;
        acc0 += hi ? 0.f : t;
        acc1 += hi ? t : 0.f;
        acc0 = wave_sum(acc0);
        acc1 = wave_sum(acc1);
        if (lane == 0) {
            part[j][q0w + q0] = bad ? __uint_as_float(0x7FC00000u) : acc0;
            part[j][q0w + q1] = bad ? __uint_as_float(0x7FC00000u) : acc1;
        }
    }
    __syncthreads();
    if (tid < R) {
        float acc = 0.f;
        for (int jj = 0; jj < k; jj++) acc = fmaf(wsh[jj], part[jj][tid], acc);
        a.y[blockIdx.x * R + tid] = acc;
    }
}

// the stream forms serve layers with no shared expert, k <= 8, I % 64 == 0
// and at least 32 MB of gate/up codes per token (H, I <= 4096 as for every
// decode layer)
static bool use_stream(const DecodeArgs& a) {
    return !a.has_shared && a.k <= 8 && (size_t)a.k * a.I * a.H >= ((size_t)32 << 20) && a.H % kStreamRows == 0 &&
           a.I % 64 == 0;
}

// compute units of the current device (0 on error)
static int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
}

template <int FMT, bool TOPK>
static hipError_t launch_stream(DecodeArgs& a, hipStream_t s) {
    const int nch_h = (a.H / 32 + 63) / 64, nch_i = (a.I / 32 + 63) / 64;
    auto gu = nch_h == 1 ? k_gateup_stream<FMT, 1, TOPK> : k_gateup_stream<FMT, 2, TOPK>;
    const int grid = cu_count();
    if (grid <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gu, dim3(grid), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nch_i == 2 && a.I <= 3072) {
        // two waves per routed slot (half its rows each) while that fits 12 waves
        if (a.k <= 6)
            hipLaunchKernelGGL((k_down_stream_pair<FMT, 2>), dim3(a.H / kStreamRows), dim3(128 * a.k), 0, s, a);
        else
            hipLaunchKernelGGL((k_down_stream_pair<FMT, 1>), dim3(a.H / kStreamRows), dim3(64 * a.k), 0, s, a);
        return hipGetLastError();
    }
    auto dn = nch_i == 1 ? k_down_stream<FMT, 1> : k_down_stream<FMT, 2>;
    hipLaunchKernelGGL(dn, dim3(a.H / kStreamRows), dim3(64 * a.k), 0, s, a);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
template <int FMT>
static hipError_t launch_down(const DecodePlan& p, DecodeArgs& a, hipStream_t s) {
    const bool sh = a.n_items > a.k;
    const int maxw = down_max_waves(p.down_L, p.down_D);
    const int units = (a.k + kDownNJ - 1) / kDownNJ + (a.n_items - a.k);  // routed units + shared halves
    const bool pairs = p.down_L == 16 && units <= maxw;
    const int nw = pairs ? units : min(maxw, a.n_items);
    dim3 grid(a.H / kDownRB), block(64 * nw);
    // hidden vectors in LDS for 16-lane rows: two I-float slices per wave
    // (pairs), one otherwise
    const size_t shm = p.down_L == 16 ? (size_t)nw * (pairs ? kDownNJ : 1) * a.I * sizeof(float) : 0;
#define DNV(DL, DD, SH, PR) hipLaunchKernelGGL((k_down_combine<FMT, DL, DD, SH, PR>), grid, block, shm, s, a)
#define DN(DL, DD)                                                   \
    case DD:                                                         \
        if (pairs) {                                                 \
            if (sh) DNV(DL, DD, true, true); else DNV(DL, DD, false, true);   \
        } else {                                                     \
            if (sh) DNV(DL, DD, true, false); else DNV(DL, DD, false, false); \
        }                                                            \
        break;
    if (p.down_L == 16) {
        switch (p.down_D) {
            DN(16, 1) DN(16, 2) DN(16, 3) DN(16, 4) DN(16, 5) DN(16, 6) DN(16, 7) DN(16, 8)
            default: return hipErrorInvalidValue;
        }
    } else {
#undef DN
#define DN(DL, DD)                                                   \
    case DD:                                                         \
        if (sh) DNV(DL, DD, true, false); else DNV(DL, DD, false, false); \
        break;
        switch (p.down_D) {
            DN(64, 1) DN(64, 2) DN(64, 3) DN(64, 4) DN(64, 5) DN(64, 6) DN(64, 7) DN(64, 8)
            default: return hipErrorInvalidValue;
        }
    }
#undef DN
#undef DNV
    return hipGetLastError();
}

// gate/up launch: TNI = 0 (routing given) or the logits per lane of the
// in-kernel top-k (the smallest that holds E)
template <int FMT, int TNI>
static hipError_t launch_gateup(const DecodePlan& p, DecodeArgs& a, hipStream_t s) {
    const int n_gate = a.k * a.gt_r + (a.has_shared ? a.gt_s : 0);
#define GU(GD, GP) case GD: hipLaunchKernelGGL((k_gateup<FMT, GD, GP, TNI>), dim3(n_gate), dim3(256), 0, s, a); break;
    switch (p.gate_D) {
        GU(1, 4) GU(2, 4) GU(3, 4) GU(4, 4) GU(5, 2) GU(6, 2) GU(7, 2) GU(8, 2)
        default: return hipErrorInvalidValue;
    }
#undef GU
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_expert(const DecodePlan& p, DecodeArgs& a, hipStream_t s) {
    if (use_stream(a)) return launch_stream<FMT, false>(a, s);
    hipError_t e = launch_gateup<FMT, 0>(p, a, s);
    if (e != hipSuccess) return e;
    return launch_down<FMT>(p, a, s);
}

template <int FMT>
static hipError_t launch_layer(const DecodePlan& p, DecodeArgs& a, hipStream_t s) {
#define RT(GD) case GD: hipLaunchKernelGGL((k_router<2 * GD>), dim3((a.E + 1) / 2), dim3(128), 0, s, a); break;
    switch (p.gate_D) {
        RT(1) RT(2) RT(3) RT(4) RT(5) RT(6) RT(7) RT(8)
        default: return hipErrorInvalidValue;
    }
#undef RT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (use_stream(a)) return launch_stream<FMT, true>(a, s);
    if (a.E <= 64) e = launch_gateup<FMT, 1>(p, a, s);
    else if (a.E <= 128) e = launch_gateup<FMT, 2>(p, a, s);
    else if (a.E <= 256) e = launch_gateup<FMT, 4>(p, a, s);
    else if (a.E <= 512) e = launch_gateup<FMT, 8>(p, a, s);
    else e = launch_gateup<FMT, 16>(p, a, s);
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
