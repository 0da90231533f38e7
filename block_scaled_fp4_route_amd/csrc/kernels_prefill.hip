// Prefill for gfx950: every prompt token through one MoE layer at once, with
// the token->expert assignments grouped by expert ([Q] "The engine", item 5:
// the whole prompt through each layer, so each expert's weights are read
// once per prompt instead of once per chunk).
//
//  1. k_group_count / k_group_scatter: stable grouping of the T*k
//     assignments a = t*k + j by expert (count, exclusive prefix sum, ordered
//     compaction with ballots: deterministic, no atomics).
//  2. k_tile_list: M-tiles of every expert, heaviest experts first.
//  3. k_quant_x_*: x~ = bf16(x) (NVFP4 layers) or MXFP4 per 32 (MXFP4 layers).
//  4. ragged grouped GEMMs (gate/up with SiLU*mul epilogue, then down):
//     NVFP4 weights are decoded to bf16 in registers and multiplied with
//     v_mfma_f32_16x16x32_bf16; MXFP4 weights and activations go straight into
//     v_mfma_scale_f32_{16x16x128,32x32x64}_f8f6f4 with their E8M0 scales.
//  5. k_combine: out[t] = sum_j w[t][j] * Y[pos(t, j)] in increasing j.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBM_NV = 64;  // NVFP4 M-tile (rows of one expert)
constexpr int kBM_MX = 32;  // MXFP4 M-tile
constexpr int kGroupThreads = 1024;

// ---------------------------------------------------------------------------
// Workspace layout
struct PrefillWs {
    int* count;   // [E]
    int* off;     // [E+1]
    int* perm;    // [T*k] assignment id at each grouped position
    int* pos;     // [T*k] grouped position of each assignment (-1: invalid expert)
    int* tile_e;  // [max_tiles]
    int* tile_m;  // [max_tiles] first row of the tile within its expert
    int* ntiles;  // [1]
    void* xq;     // x~: bf16 [T][H] | MXFP4 codes [T][H/2] + scales [T][H/32]
    void* hq;     // h~: bf16 [T*k][I] | MXFP4 codes [T*k][I/2] + scales [T*k][I/32]
    float* hf;    // MXFP4 only: h before rounding [T*k][I]
    float* Y;     // [T*k][H]
    size_t bytes;
};

static int max_tiles(int fmt, int E, int T, int k) {
    const int bm = fmt == kFmtNvfp4 ? kBM_NV : kBM_MX;
    return E + (T * k + bm - 1) / bm;
}

static PrefillWs prefill_layout(int fmt, int H, int I, int E, int k, int T, void* ws) {
    PrefillWs w = {};
    char* b = reinterpret_cast<char*>(ws);
    size_t o = kCounterBytes;
    auto take = [&](size_t n) { char* p = b ? b + o : nullptr; o += align256(n); return p; };
    const size_t n = (size_t)T * k;
    const int mt = max_tiles(fmt, E, T, k);
    w.count = (int*)take(sizeof(int) * E);
    w.off = (int*)take(sizeof(int) * (E + 1));
    w.perm = (int*)take(sizeof(int) * n);
    w.pos = (int*)take(sizeof(int) * n);
    w.tile_e = (int*)take(sizeof(int) * mt);
    w.tile_m = (int*)take(sizeof(int) * mt);
    w.ntiles = (int*)take(sizeof(int));
    if (fmt == kFmtNvfp4) {
        w.xq = take((size_t)T * H * 2);
        w.hq = take(n * I * 2);
        w.hf = nullptr;
    } else {
        w.xq = take((size_t)T * H / 2 + (size_t)T * H / 32 + 256);
        w.hq = take(n * I / 2 + n * I / 32 + 256);
        w.hf = (float*)take(n * I * sizeof(float));
    }
    w.Y = (float*)take(n * H * sizeof(float));
    w.bytes = o;
    return w;
}

bool prefill_supported(int fmt, int H, int I, int E, int k) {
    if (E < 1 || E > kMaxE || k < 1 || k > kMaxK) return false;
    if (fmt == kFmtNvfp4) return H % 256 == 0 && I % 128 == 0 && H <= 16384 && I <= 16384;
    return H % 256 == 0 && I % 64 == 0 && H <= 16384 && I <= 16384;
}

size_t prefill_ws_bytes(int fmt, int H, int I, int E, int k, int T) {
    return prefill_layout(fmt, H, I, E, k, T, nullptr).bytes;
}

// ---------------------------------------------------------------------------
// 1. grouping

__device__ __forceinline__ int block_sum_int(int v, int* red) {
    // kGroupThreads threads; red has >= 16 ints
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int s = 0;
    for (int i = 0; i < kGroupThreads / 64; i++) s += red[i];
    __syncthreads();
    return s;
}

// grid E: count[e] = #{a : idx[a] == e}; also marks every pos[] invalid.
__global__ __launch_bounds__(kGroupThreads) void k_group_count(const int32_t* __restrict__ idx, int n, int E,
                                                               int* __restrict__ count, int* __restrict__ pos) {
    __shared__ int red[16];
    const int e = blockIdx.x;
    int c = 0;
    for (int a = threadIdx.x; a < n; a += kGroupThreads) c += idx[a] == e;
    c = block_sum_int(c, red);
    if (threadIdx.x == 0) count[e] = c;
    const int lo = (int)((long long)n * e / E), hi = (int)((long long)n * (e + 1) / E);
    for (int a = lo + threadIdx.x; a < hi; a += kGroupThreads) pos[a] = -1;
}

// grid E: off[e] = sum_{e'<e} count[e']; perm[off[e] + r] = the r-th
// assignment (in increasing a) routed to e; pos[a] = its grouped position.
__global__ __launch_bounds__(kGroupThreads) void k_group_scatter(const int32_t* __restrict__ idx, int n, int E,
                                                                 const int* __restrict__ count, int* __restrict__ off,
                                                                 int* __restrict__ perm, int* __restrict__ pos) {
    __shared__ int red[16];
    __shared__ int wtot[16];
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int s = 0;
    for (int i = tid; i < e; i += kGroupThreads) s += count[i];
    const int base = block_sum_int(s, red);
    if (tid == 0) {
        off[e] = base;
        if (e == E - 1) off[E] = base + count[e];
    }
    int running = 0;
    for (int a0 = 0; a0 < n; a0 += kGroupThreads) {
        const int a = a0 + tid;
        const bool match = a < n && idx[a] == e;
        const unsigned long long m = __ballot(match);
        const int lane_pre = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wtot[wave] = __popcll(m);
        __syncthreads();
        int wave_pre = 0, total = 0;
        for (int i = 0; i < kGroupThreads / 64; i++) {
            const int t = wtot[i];
            wave_pre += i < wave ? t : 0;
            total += t;
        }
        if (match) {
            const int p = base + running + wave_pre + lane_pre;
            perm[p] = a;
            pos[a] = p;
        }
        running += total;
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// 2. tile list: experts ordered by row count (descending; ties by index),
// each split into M-tiles of BM rows.
__global__ __launch_bounds__(kGroupThreads) void k_tile_list(const int* __restrict__ count, int E, int BM,
                                                             int* __restrict__ tile_e, int* __restrict__ tile_m,
                                                             int* __restrict__ ntiles) {
    __shared__ int cnt[kMaxE];
    __shared__ int nt_sorted[kMaxE];
    __shared__ int ex_sorted[kMaxE];
    __shared__ int start[kMaxE + 1];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kGroupThreads) cnt[e] = count[e];
    __syncthreads();
    for (int e = tid; e < E; e += kGroupThreads) {
        const int c = cnt[e];
        int rank = 0;
        for (int j = 0; j < E; j++) rank += (cnt[j] > c) || (cnt[j] == c && j < e);
        ex_sorted[rank] = e;
        nt_sorted[rank] = (c + BM - 1) / BM;
    }
    __syncthreads();
    if (tid == 0) {
        int s = 0;
        for (int r = 0; r < E; r++) {
            start[r] = s;
            s += nt_sorted[r];
        }
        start[E] = s;
        ntiles[0] = s;
    }
    __syncthreads();
    for (int r = tid; r < E; r += kGroupThreads) {
        const int e = ex_sorted[r];
        for (int m = 0; m < nt_sorted[r]; m++) {
            tile_e[start[r] + m] = e;
            tile_m[start[r] + m] = m * BM;
        }
    }
}

// ---------------------------------------------------------------------------
// 3. activation rounding

// x~ = bf16(x), round to nearest even (v_cvt_pk_bf16_f32); 8 values per thread.
__global__ __launch_bounds__(256) void k_quant_bf16(const float* __restrict__ x, size_t n8, bf16x8* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4 a = reinterpret_cast<const f32x4*>(x)[2 * i], b = reinterpret_cast<const f32x4*>(x)[2 * i + 1];
    const f32x2 p0 = {a.x, a.y}, p1 = {a.z, a.w}, p2 = {b.x, b.y}, p3 = {b.z, b.w};
    const bf16x2 q0 = __builtin_convertvector(p0, bf16x2), q1 = __builtin_convertvector(p1, bf16x2);
    const bf16x2 q2 = __builtin_convertvector(p2, bf16x2), q3 = __builtin_convertvector(p3, bf16x2);
    bf16x8 o = {q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
    out[i] = o;
}

// e2m1 code of |t| (t already divided by the block scale, exact), ties to
// the even code, saturating at 6 (code 7).
__device__ __forceinline__ uint32_t e2m1_code(float t) {
    return (uint32_t)(t > 0.25f) + (uint32_t)(t >= 0.75f) + (uint32_t)(t > 1.25f) + (uint32_t)(t >= 1.75f) +
           (uint32_t)(t > 2.5f) + (uint32_t)(t >= 3.5f) + (uint32_t)(t > 5.0f);
}

// MXFP4 conversion of rows of n values (OCP MX): one thread per block of 32;
// shared exponent X = floor(log2 max|v|) - 2 from the fp32 exponent field,
// clamped to [-127, 127]; scale byte X + 127 (0 for an all-zero block);
// codes e2m1(|v| / 2^X) with the sign of v. Codes packed two per byte, the
// even element in the low nibble.
__global__ __launch_bounds__(256) void k_quant_mx(const float* __restrict__ src, size_t nblocks,
                                                  uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  float* __restrict__ dequant) {
    const size_t b = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    const f32x4* p = reinterpret_cast<const f32x4*>(src + b * 32);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const f32x4 q = p[i];
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
    int X = 0;
    uint32_t sb = 0;
    if (amax > 0.f) {
        X = (int)((__float_as_uint(amax) >> 23) & 255u) - 127 - 2;
        X = max(-127, min(127, X));
        sb = (uint32_t)(X + 127);
    }
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const float t = fabsf(ldexpf(v[i], -X));
        const uint32_t c = e2m1_code(t) | ((__float_as_uint(v[i]) >> 31) << 3);
        w[i / 8] |= c << (4 * (i % 8));
    }
    uint4 o = {w[0], w[1], w[2], w[3]};
    reinterpret_cast<uint4*>(codes)[b] = o;
    scales[b] = (uint8_t)sb;
    if (dequant) {
        const float s = ue8m0_to_f32(sb);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const f2v d0 = fp4x2<0>(w[i]), d1 = fp4x2<1>(w[i]), d2 = fp4x2<2>(w[i]), d3 = fp4x2<3>(w[i]);
            float* q = dequant + b * 32 + 8 * i;
            q[0] = d0.x * s; q[1] = d0.y * s; q[2] = d1.x * s; q[3] = d1.y * s;
            q[4] = d2.x * s; q[5] = d2.y * s; q[6] = d3.x * s; q[7] = d3.y * s;
        }
    }
}

// ---------------------------------------------------------------------------
// 4a. NVFP4 gate/up: ragged grouped GEMM with bf16 MFMA.
//
// Workgroup = (M-tile of 64 rows of one expert, 128 output columns of I).
// Wave w owns output columns c0 = n0 + 32w .. +32 of BOTH gate and up, so its
// B operand is 4 column blocks of 16 (gate c0, gate c0+16, up c0, up c0+16)
// and SiLU*mul happens in registers. K runs over H in chunks of 128; within a
// chunk lane group g = lane/16 owns K = 32g .. 32g+31 (one 16-byte load of 32
// codes and 2 scale bytes per column block) and MFMA step s consumes its
// elements 8s..8s+7, with the A operand read from LDS under the same
// K mapping (the dot product is order-independent). The codes are decoded
// to bf16 exactly (e2m1 x E4M3 has at most 6 significant bits).
struct GemmArgs {
    const int* tile_e;
    const int* tile_m;
    const int* ntiles;
    const int* count;
    const int* off;
    const int* perm;
    const void* const* expert_ptrs;
    const void* a_src;      // x~ (gate/up) or h~ (down)
    const uint8_t* a_scl;   // MXFP4 activation scales
    void* out;              // h~ (bf16) / h fp32 (MX) for gate/up; Y for down
    float* h_pre;           // optional debug
    float* h_q;             // optional debug (NVFP4)
    int E, H, I, k, NT;     // NT = N-tiles per M-tile
};

constexpr int kALd = 128 + 8;  // LDS row stride (bf16) of an A tile: 128 K + 8 padding

// Decode 8 e2m1 codes (dword d) times scale s to 8 bf16 (exact).
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t d, float s) {
    const f2v a = fp4x2<0>(d), b = fp4x2<1>(d), c = fp4x2<2>(d), e = fp4x2<3>(d);
    const f32x2 p0 = {a.x * s, a.y * s}, p1 = {b.x * s, b.y * s}, p2 = {c.x * s, c.y * s}, p3 = {e.x * s, e.y * s};
    const bf16x2 q0 = __builtin_convertvector(p0, bf16x2), q1 = __builtin_convertvector(p1, bf16x2);
    const bf16x2 q2 = __builtin_convertvector(p2, bf16x2), q3 = __builtin_convertvector(p3, bf16x2);
    bf16x8 o = {q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
    return o;
}

// Shared K loop of the two NVFP4 GEMMs: acc[rb][cb] += A[64 rows] x B[4
// column blocks]^T over K (= KTOT) in chunks of 128. a_row(r) gives the
// element offset of A row r (or -1 for a padding row); b_row(cb) the B
// (weight) row of this lane's column in block cb; codes/scales are the
// weight matrix regions with KTOT/2 code bytes and KTOT/16 scale bytes per row.
template <class AROW>
__device__ __forceinline__ void nv_kloop(f32x4 (&acc)[4][4], const __bf16* __restrict__ A, AROW a_row,
                                         const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scl,
                                         const int (&brow)[4], int KTOT, __bf16* lds) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int g = lane >> 4, m16 = lane & 15;
    // A loader: thread -> (row tid/4, 32-element quarter tid%4)
    const int lr = tid >> 2, lq = tid & 3;
    const int arow = a_row(lr);
    const int nchunks = KTOT / 128;
    uint4 anext[4];
    uint4 bnext[4];
    uint32_t snext[4];
    auto load_chunk = [&](int ch) {
        const int k0 = ch * 128;
        if (arow >= 0) {
            const uint4* src = reinterpret_cast<const uint4*>(A + (size_t)arow + k0 + 32 * lq);
#pragma unroll
            for (int i = 0; i < 4; i++) anext[i] = src[i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) anext[i] = uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
            const size_t r = (size_t)brow[cb];
            bnext[cb] = *reinterpret_cast<const uint4*>(codes + r * (KTOT / 2) + k0 / 2 + 16 * g);
            snext[cb] = *reinterpret_cast<const uint16_t*>(scl + r * (KTOT / 16) + k0 / 16 + 2 * g);
        }
    };
    auto store_a = [&](int buf) {
        __bf16* dst = lds + (size_t)buf * 64 * kALd + lr * kALd + 32 * lq;
#pragma unroll
        for (int i = 0; i < 4; i++) reinterpret_cast<uint4*>(dst)[i] = anext[i];
    };
    load_chunk(0);
    store_a(0);
    __syncthreads();
    for (int ch = 0; ch < nchunks; ch++) {
        const int cur = ch & 1;
        uint4 bc[4];
        uint32_t sc[4];
#pragma unroll
        for (int cb = 0; cb < 4; cb++) { bc[cb] = bnext[cb]; sc[cb] = snext[cb]; }
        if (ch + 1 < nchunks) load_chunk(ch + 1);
        float s_lo[4], s_hi[4];
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
            s_lo[cb] = e4m3_to_f32(sc[cb] & 0xFFu);
            s_hi[cb] = e4m3_to_f32(sc[cb] >> 8);
        }
        const __bf16* At = lds + (size_t)cur * 64 * kALd;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            bf16x8 bf[4];
#pragma unroll
            for (int cb = 0; cb < 4; cb++) {
                const uint32_t d = s == 0 ? bc[cb].x : (s == 1 ? bc[cb].y : (s == 2 ? bc[cb].z : bc[cb].w));
                bf[cb] = dequant8_bf16(d, s < 2 ? s_lo[cb] : s_hi[cb]);
            }
#pragma unroll
            for (int rb = 0; rb < 4; rb++) {
                const bf16x8 af = *reinterpret_cast<const bf16x8*>(At + (16 * rb + m16) * kALd + 32 * g + 8 * s);
#pragma unroll
                for (int cb = 0; cb < 4; cb++)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[cb], acc[rb][cb], 0, 0, 0);
            }
        }
        if (ch + 1 < nchunks) store_a(cur ^ 1);
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void k_gateup_nv(GemmArgs a) {
    __shared__ __bf16 lds[2 * 64 * kALd];
    const int tile = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
    if (tile >= a.ntiles[0]) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = min(kBM_NV, a.count[e] - m0);
    const int base = a.off[e] + m0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I;
    const int c0 = nt * 128 + 32 * wave;
    const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.expert_ptrs[e]);
    const uint8_t* codes = blk;                               // gate rows then up rows, H/2 bytes each
    const uint8_t* scl = blk + (size_t)3 * I * H / 2;         // gate scales then up scales, H/16 each
    const int m16 = lane & 15;
    const int brow[4] = {c0 + m16, c0 + 16 + m16, I + c0 + m16, I + c0 + 16 + m16};
    const __bf16* X = reinterpret_cast<const __bf16*>(a.a_src);
    const int* perm = a.perm;
    const int k = a.k;
    auto a_row = [&](int r) { return r < rows ? (perm[base + r] / k) * H : -1; };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    nv_kloop(acc, X, a_row, codes, scl, brow, H, lds);
    // epilogue: lane holds column c0 + 16 cbg + m16, rows 16 rb + 4 g + i
    __bf16* hq = reinterpret_cast<__bf16*>(a.out);
    const int g = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < 4; rb++)
#pragma unroll
        for (int cbg = 0; cbg < 2; cbg++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = 16 * rb + 4 * g + i;
                if (r < rows) {
                    const float hv = silu_mul(acc[rb][cbg][i], acc[rb][cbg + 2][i]);
                    const __bf16 hb = (__bf16)hv;
                    const size_t o = (size_t)(base + r) * I + c0 + 16 * cbg + m16;
                    hq[o] = hb;
                    if (a.h_pre) a.h_pre[o] = hv;
                    if (a.h_q) a.h_q[o] = (float)hb;
                }
            }
}

// 4b. NVFP4 down: Y[p][n] = sum_i h~[p][i] * Wd[n][i]. Workgroup = (M-tile of
// 64 grouped rows, 256 columns of H); wave w owns columns n0 + 64w .. +64 as
// 4 column blocks of 16. A rows are contiguous grouped rows of h~.
__global__ __launch_bounds__(256) void k_down_nv(GemmArgs a) {
    __shared__ __bf16 lds[2 * 64 * kALd];
    const int tile = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
    if (tile >= a.ntiles[0]) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = min(kBM_NV, a.count[e] - m0);
    const int base = a.off[e] + m0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I;
    const int n0 = nt * 256 + 64 * wave;
    const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.expert_ptrs[e]);
    const uint8_t* codes = blk + (size_t)I * H;                              // down [H][I/2]
    const uint8_t* scl = blk + (size_t)3 * I * H / 2 + (size_t)2 * I * H / 16;  // down scales [H][I/16]
    const int m16 = lane & 15;
    const int brow[4] = {n0 + m16, n0 + 16 + m16, n0 + 32 + m16, n0 + 48 + m16};
    const __bf16* Hq = reinterpret_cast<const __bf16*>(a.a_src);
    auto a_row = [&](int r) { return r < rows ? (base + r) * I : -1; };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    nv_kloop(acc, Hq, a_row, codes, scl, brow, I, lds);
    float* Y = reinterpret_cast<float*>(a.out);
    const int g = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < 4; rb++)
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = 16 * rb + 4 * g + i;
                if (r < rows) Y[(size_t)(base + r) * H + n0 + 16 * cb + m16] = acc[rb][cb][i];
            }
}

// ---------------------------------------------------------------------------
// 4c. MXFP4 gate/up with the scaled FP4 MFMA (16x16x128): workgroup = (M-tile
// of 32 rows = 2 row blocks, 64 output columns of I); wave w owns columns
// n0 + 16w .. +16 of gate and up. Lane l holds row/column l%16 and
// K = k0 + 32(l/16) .. +31: 16 code bytes plus one UE8M0 scale byte, read
// straight from x~ and from the weight rows.
__global__ __launch_bounds__(256) void k_gateup_mx(GemmArgs a) {
    const int tile = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
    if (tile >= a.ntiles[0]) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = min(kBM_MX, a.count[e] - m0);
    const int base = a.off[e] + m0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I, k = a.k;
    const int g = lane >> 4, m16 = lane & 15;
    const int c = nt * 64 + 16 * wave + m16;
    const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.expert_ptrs[e]);
    const uint8_t* gcode = blk + (size_t)c * (H / 2);
    const uint8_t* ucode = blk + (size_t)(I + c) * (H / 2);
    const uint8_t* gscl = blk + (size_t)3 * I * H / 2 + (size_t)c * (H / 32);
    const uint8_t* uscl = blk + (size_t)3 * I * H / 2 + (size_t)(I + c) * (H / 32);
    const uint8_t* xc = reinterpret_cast<const uint8_t*>(a.a_src);
    // A rows of the two row blocks (padding rows read row 0 of the tile: their
    // outputs are discarded)
    int ar[2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
        const int r = 16 * rb + m16;
        ar[rb] = a.perm[base + (r < rows ? r : 0)] / k;
    }
    f32x4 acc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++) acc[rb][0] = acc[rb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < H; k0 += 128) {
        const int kb = k0 + 32 * g;
        const uint4 bg = *reinterpret_cast<const uint4*>(gcode + kb / 2);
        const uint4 bu = *reinterpret_cast<const uint4*>(ucode + kb / 2);
        const int sg = gscl[kb / 32], su = uscl[kb / 32];
        const i32x8 Bg = {(int)bg.x, (int)bg.y, (int)bg.z, (int)bg.w, 0, 0, 0, 0};
        const i32x8 Bu = {(int)bu.x, (int)bu.y, (int)bu.z, (int)bu.w, 0, 0, 0, 0};
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            const uint4 av = *reinterpret_cast<const uint4*>(xc + (size_t)ar[rb] * (H / 2) + kb / 2);
            const int sa = a.a_scl[(size_t)ar[rb] * (H / 32) + kb / 32];
            const i32x8 A = {(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
            acc[rb][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bg, acc[rb][0], 4, 4, 0, sa, 0, sg);
            acc[rb][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bu, acc[rb][1], 4, 4, 0, sa, 0, su);
        }
    }
    // D layout: lane holds column c, rows 16 rb + 4 g + i
    float* hf = reinterpret_cast<float*>(a.out);
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = 16 * rb + 4 * g + i;
            if (r < rows) {
                const float hv = silu_mul(acc[rb][0][i], acc[rb][1][i]);
                const size_t o = (size_t)(base + r) * I + c;
                hf[o] = hv;
                if (a.h_pre) a.h_pre[o] = hv;
            }
        }
}

// 4d. MXFP4 down with the scaled FP4 MFMA (32x32x64): workgroup = (M-tile of
// 32 grouped rows, 256 columns of H); wave w owns 2 column blocks of 32.
// Lane l holds row/column l%32 and K = k0 + 32(l/32) .. +31.
__global__ __launch_bounds__(256) void k_down_mx(GemmArgs a) {
    const int tile = blockIdx.x / a.NT, nt = blockIdx.x % a.NT;
    if (tile >= a.ntiles[0]) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = min(kBM_MX, a.count[e] - m0);
    const int base = a.off[e] + m0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I;
    const int g = lane >> 5, m32 = lane & 31;
    const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.expert_ptrs[e]);
    const uint8_t* dcode = blk + (size_t)I * H;
    const uint8_t* dscl = blk + (size_t)3 * I * H / 2 + (size_t)2 * I * H / 32;
    const int n0 = nt * 256 + 64 * wave;
    const uint8_t* hc = reinterpret_cast<const uint8_t*>(a.a_src);
    const int arow = base + (m32 < rows ? m32 : 0);
    f32x16 acc[2];
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[cb][i] = 0.f;
    for (int k0 = 0; k0 < I; k0 += 64) {
        const int kb = k0 + 32 * g;
        const uint4 av = *reinterpret_cast<const uint4*>(hc + (size_t)arow * (I / 2) + kb / 2);
        const int sa = a.a_scl[(size_t)arow * (I / 32) + kb / 32];
        const i32x8 A = {(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const size_t n = (size_t)n0 + 32 * cb + m32;
            const uint4 bv = *reinterpret_cast<const uint4*>(dcode + n * (I / 2) + kb / 2);
            const int sb = dscl[n * (I / 32) + kb / 32];
            const i32x8 B = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
            acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[cb], 4, 4, 0, sa, 0, sb);
        }
    }
    // D layout: lane holds column l%32; register i -> row 8(i/4) + 4(l/32) + i%4
    float* Y = reinterpret_cast<float*>(a.out);
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int r = 8 * (i / 4) + 4 * g + (i % 4);
            if (r < rows) Y[(size_t)(base + r) * H + n0 + 32 * cb + m32] = acc[cb][i];
        }
}

// ---------------------------------------------------------------------------
// 5. combine: out[t][c] = sum_j w[t][j] * Y[pos[t*k+j]][c], increasing j,
// fp32 accumulate; fp32 out or bf16 (round to nearest even of that sum).
// An assignment with an expert index outside [0, E) has no position and
// turns its token's output NaN.
__global__ __launch_bounds__(256) void k_combine_prefill(const float* __restrict__ Y, const int* __restrict__ pos,
                                                         const float* __restrict__ w, int k, int H, void* out,
                                                         int out_bf16) {
    const int t = blockIdx.y;
    const int c4 = blockIdx.x * 256 + threadIdx.x;  // float4 column
    if (c4 * 4 >= H) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; j++) {
        const int p = pos[t * k + j];
        const float wj = w[t * k + j];
        if (p < 0) {
            acc = f32x4{__uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u),
                        __uint_as_float(0x7FC00000u)};
            continue;
        }
        const f32x4 yv = reinterpret_cast<const f32x4*>(Y + (size_t)p * H)[c4];
        acc.x = fmaf(wj, yv.x, acc.x);
        acc.y = fmaf(wj, yv.y, acc.y);
        acc.z = fmaf(wj, yv.z, acc.z);
        acc.w = fmaf(wj, yv.w, acc.w);
    }
    if (out_bf16) {
        const f32x2 p0 = {acc.x, acc.y}, p1 = {acc.z, acc.w};
        const bf16x2 q0 = __builtin_convertvector(p0, bf16x2), q1 = __builtin_convertvector(p1, bf16x2);
        bf16x2* o = reinterpret_cast<bf16x2*>(reinterpret_cast<__bf16*>(out) + (size_t)t * H + 4 * c4);
        o[0] = q0;
        o[1] = q1;
    } else {
        reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + (size_t)t * H)[c4] = acc;
    }
}

// ---------------------------------------------------------------------------
#define LAUNCH_CHECK()                              \
    do {                                            \
        hipError_t e_ = hipGetLastError();          \
        if (e_ != hipSuccess) return e_;            \
    } while (0)

hipError_t launch_prefill(int fmt, int H, int I, int E, int k, int T, const float* x,
                          const void* const* expert_ptrs, const int32_t* idx, const float* w, void* out,
                          int out_bf16, void* ws, const PrefillDebug* dbg, hipStream_t s) {
    const PrefillWs L = prefill_layout(fmt, H, I, E, k, T, ws);
    const int n = T * k;
    const int BM = fmt == kFmtNvfp4 ? kBM_NV : kBM_MX;
    const int mt = max_tiles(fmt, E, T, k);
    int* perm = dbg && dbg->perm ? dbg->perm : L.perm;
    int* off = dbg && dbg->off ? dbg->off : L.off;

    hipLaunchKernelGGL(k_group_count, dim3(E), dim3(kGroupThreads), 0, s, idx, n, E, L.count, L.pos);
    LAUNCH_CHECK();
    hipLaunchKernelGGL(k_group_scatter, dim3(E), dim3(kGroupThreads), 0, s, idx, n, E, L.count, off, perm, L.pos);
    LAUNCH_CHECK();
    hipLaunchKernelGGL(k_tile_list, dim3(1), dim3(kGroupThreads), 0, s, L.count, E, BM, L.tile_e, L.tile_m, L.ntiles);
    LAUNCH_CHECK();

    GemmArgs ga = {};
    ga.tile_e = L.tile_e; ga.tile_m = L.tile_m; ga.ntiles = L.ntiles; ga.count = L.count; ga.off = off;
    ga.perm = perm; ga.expert_ptrs = expert_ptrs; ga.E = E; ga.H = H; ga.I = I; ga.k = k;
    ga.h_pre = dbg ? dbg->h_pre : nullptr;

    if (fmt == kFmtNvfp4) {
        __bf16* xq = dbg && dbg->x_bf16 ? reinterpret_cast<__bf16*>(dbg->x_bf16) : reinterpret_cast<__bf16*>(L.xq);
        const size_t n8 = (size_t)T * H / 8;
        hipLaunchKernelGGL(k_quant_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, n8,
                           reinterpret_cast<bf16x8*>(xq));
        LAUNCH_CHECK();
        ga.a_src = xq; ga.out = L.hq; ga.h_q = dbg ? dbg->h_q : nullptr; ga.NT = I / 128;
        hipLaunchKernelGGL(k_gateup_nv, dim3(mt * ga.NT), dim3(256), 0, s, ga);
        LAUNCH_CHECK();
        GemmArgs gd = ga;
        gd.a_src = L.hq; gd.out = L.Y; gd.h_pre = nullptr; gd.h_q = nullptr; gd.NT = H / 256;
        hipLaunchKernelGGL(k_down_nv, dim3(mt * gd.NT), dim3(256), 0, s, gd);
        LAUNCH_CHECK();
    } else {
        uint8_t* xc = dbg && dbg->x_codes ? dbg->x_codes : reinterpret_cast<uint8_t*>(L.xq);
        uint8_t* xs = dbg && dbg->x_scales ? dbg->x_scales : reinterpret_cast<uint8_t*>(L.xq) + (size_t)T * H / 2;
        const size_t nbx = (size_t)T * H / 32;
        hipLaunchKernelGGL(k_quant_mx, dim3((unsigned)((nbx + 255) / 256)), dim3(256), 0, s, x, nbx,
                           reinterpret_cast<uint32_t*>(xc), xs, (float*)nullptr);
        LAUNCH_CHECK();
        ga.a_src = xc; ga.a_scl = xs; ga.out = L.hf; ga.NT = I / 64;
        hipLaunchKernelGGL(k_gateup_mx, dim3(mt * ga.NT), dim3(256), 0, s, ga);
        LAUNCH_CHECK();
        uint8_t* hc = reinterpret_cast<uint8_t*>(L.hq);
        uint8_t* hs = hc + (size_t)n * I / 2;
        const size_t nbh = (size_t)n * I / 32;
        hipLaunchKernelGGL(k_quant_mx, dim3((unsigned)((nbh + 255) / 256)), dim3(256), 0, s, L.hf, nbh,
                           reinterpret_cast<uint32_t*>(hc), hs, dbg ? dbg->h_q : (float*)nullptr);
        LAUNCH_CHECK();
        GemmArgs gd = ga;
        gd.a_src = hc; gd.a_scl = hs; gd.out = L.Y; gd.h_pre = nullptr; gd.NT = H / 256;
        hipLaunchKernelGGL(k_down_mx, dim3(mt * gd.NT), dim3(256), 0, s, gd);
        LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(k_combine_prefill, dim3((H / 4 + 255) / 256, T), dim3(256), 0, s, L.Y, L.pos, w, k, H, out,
                       out_bf16);
    return hipGetLastError();
}

}  // namespace moe
