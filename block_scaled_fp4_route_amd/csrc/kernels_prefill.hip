// Prefill for gfx950: every prompt token through one MoE layer at once, with
// the token->expert assignments grouped by expert ([Q] "The engine", item 5:
// the whole prompt through each layer, so each expert's weights are read
// once per prompt instead of once per chunk).
//
//  1. k_group: stable grouping of the T*k assignments a = t*k + j by expert
//     (count, exclusive prefix sum, ordered compaction with ballots:
//     deterministic, no atomics).
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

// The grouped GEMMs address their activation operands with 32-bit buffer
// offsets and use offsets from 0x7FFFFFF0 up as "no load".
bool prefill_tokens_supported(int H, int I, int k, int T) {
    const size_t lim = 0x7FFFFFF0u;
    return (size_t)T * H * 2 < lim && (size_t)T * k * I * 2 < lim && (size_t)T * H * 4 < ((size_t)1 << 32);
}

bool prefill_supported(int fmt, int H, int I, int E, int k) {
    if (E < 1 || E > kMaxE || k < 1 || k > kMaxK) return false;
    if (fmt == kFmtNvfp4) return H % 256 == 0 && I % 128 == 0 && H <= 16384 && I <= 16384;
    return H % 512 == 0 && I % 64 == 0 && H <= 16384 && I <= 16384;
}

size_t prefill_ws_bytes(int fmt, int H, int I, int E, int k, int T) {
    return prefill_layout(fmt, H, I, E, k, T, nullptr).bytes;
}

// ---------------------------------------------------------------------------
// 1. grouping

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// grid E, 1024 threads per expert e, two passes over idx and no dependency
// between workgroups: pass 1 counts lt = #{a : idx[a] < e} (= off[e], the
// exclusive prefix sum of the counts) and eq = #{a : idx[a] == e}; pass 2
// writes perm[off[e] + r] = the r-th assignment (in increasing a) routed to e
// and pos[a] = its grouped position. Assignments whose expert index lies
// outside [0, E) match no workgroup; workgroup e sets pos = -1 for those in
// its slice of the array (a valid entry is only ever written by its expert's
// workgroup, so the writes never collide).
__global__ __launch_bounds__(kGroupThreads) void k_group(const int32_t* __restrict__ idx, int n, int E,
                                                         int* __restrict__ count, int* __restrict__ off,
                                                         int* __restrict__ perm, int* __restrict__ pos) {
    __shared__ int red[2][kGroupThreads / 64];
    __shared__ int wtot[kGroupThreads / 64];
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NW = kGroupThreads / 64;
    int lt = 0, eq = 0;
    for (int a = tid; a < n; a += kGroupThreads) {
        const int v = idx[a];
        lt += (unsigned)v < (unsigned)e;
        eq += v == e;
    }
    lt = wave_sum_int(lt);
    eq = wave_sum_int(eq);
    if (lane == 0) { red[0][wave] = lt; red[1][wave] = eq; }
    __syncthreads();
    int base = 0, cnt = 0;
    for (int i = 0; i < NW; i++) { base += red[0][i]; cnt += red[1][i]; }
    if (tid == 0) {
        off[e] = base;
        count[e] = cnt;
        if (e == E - 1) off[E] = base + cnt;
    }
    const int lo = (int)((long long)n * e / E), hi = (int)((long long)n * (e + 1) / E);
    for (int a = lo + tid; a < hi; a += kGroupThreads)
        if ((unsigned)idx[a] >= (unsigned)E) pos[a] = -1;
    const unsigned long long below = (1ull << lane) - 1ull;
    int running = base;
    for (int a0 = 0; a0 < n; a0 += kGroupThreads) {
        const int a = a0 + tid;
        const bool match = a < n && idx[a] == e;
        const unsigned long long m = __ballot(match);
        if (lane == 0) wtot[wave] = __popcll(m);
        __syncthreads();
        int wave_pre = 0, total = 0;
        for (int i = 0; i < NW; i++) {
            const int t = wtot[i];
            wave_pre += i < wave ? t : 0;
            total += t;
        }
        if (match) {
            const int p = running + wave_pre + __popcll(m & below);
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
    __shared__ int start[kGroupThreads + 1];
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
    // inclusive scan of nt_sorted (Hillis-Steele over kGroupThreads >= E entries)
    int v = tid < E ? nt_sorted[tid] : 0;
    for (int d = 1; d < kGroupThreads; d <<= 1) {
        start[tid] = v;
        __syncthreads();
        if (tid >= d) v += start[tid - d];
        __syncthreads();
    }
    start[tid + 1] = v;          // start[r + 1] = tiles of ranks 0..r
    if (tid == 0) start[0] = 0;
    if (tid == kGroupThreads - 1) ntiles[0] = v;
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
// and SiLU*mul happens in registers. K runs over H in chunks of 256; within a
// chunk each lane group owns a contiguous quarter of K (see nv_kloop), with
// the A operand read from LDS under the same K mapping (the dot product is
// order-independent). The codes are decoded to bf16 exactly (e2m1 x E4M3 has
// at most 6 significant bits).
// Workgroup -> (M-tile, N-tile). Workgroups are dispatched round-robin over
// the 8 XCDs (each with its own L2), so workgroup b runs on XCD b % 8. M-tile
// t goes to XCD t % 8 and all NT N-tiles of an M-tile (the same gathered
// activation rows) to that XCD, one after the other: the tile list is sorted
// heaviest expert first, so dealing M-tiles round-robin spreads the full
// tiles evenly over the XCDs. The grid is 8 * ceil(max_tiles / 8) * NT.
// Returns false for workgroups beyond the real tiles.
__device__ __forceinline__ bool map_tile(int ntiles, int NT, int& tile, int& nt) {
    const int x = blockIdx.x % 8, j = blockIdx.x / 8;
    tile = x + 8 * (j / NT);
    nt = j % NT;
    return tile < ntiles;
}

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
    uint32_t a_bytes;       // bytes of a_src
    uint32_t a_scl_bytes;   // bytes of a_scl (MXFP4)
    uint32_t block_bytes;   // bytes of one expert block
};

// Wait until at most N vector memory operations of this wave are outstanding
// (loads complete in issue order) and this wave's LDS accesses are done, then
// a workgroup barrier. The direct-to-LDS loads have no register result, so
// the compiler cannot place this wait itself, and a fenced barrier would
// drain every outstanding load (the compiler must assume any of them writes
// LDS). The memory clobber keeps the compiler from moving memory accesses
// across it.
template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

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
// column blocks]^T over K (= KTOT) in chunks of BK (128 or 256). A is a
// buffer of a_bytes bytes; a_row(r) gives the element offset of A row r
// (0 <= r < rows). blk is the expert block (block_bytes), codes_off and
// scl_off the byte offsets of the weight matrix's code and scale regions
// (KTOT/2 code bytes and KTOT/16 scale bytes per row), brow[cb] the weight
// row of this lane's column in block cb. Within a chunk, lane group g =
// lane/16 owns K = g*BK/4 .. +BK/4 (one or two 16-byte code loads per column
// block, 2 or 4 scale bytes) and MFMA step s consumes its elements 8s..8s+7;
// the A tile in LDS is read with the same K mapping.
// Pipeline: the A tile of chunk ch+1 goes from memory straight into LDS
// (buffer_load ... lds, no registers) while chunk ch is computed, and the
// weight fragments run two chunks ahead in two register sets (steps go in
// pairs so that the sets have fixed registers). Every step issues the same
// loads; those past the last chunk use an out-of-range offset, which returns
// zeros without touching memory. The compiler can then count outstanding
// loads exactly, and the explicit waits before each barrier cover the LDS
// loads it cannot see. A rows are stored without padding, 16-byte piece p of
// row r at slot r*SPR + (p ^ (r & 7)), which keeps the fragment reads of 8
// consecutive rows on distinct bank groups. Rows past `rows` load row 0
// (their sums are never stored).
constexpr uint32_t kOOB = 0x7FFFFFF0u;  // beyond every buffer here: loads return 0

template <int BK, class AROW>
__device__ __forceinline__ void nv_kloop(f32x4 (&acc)[4][4], const __bf16* __restrict__ A, uint32_t a_bytes,
                                         AROW a_row, int rows, const void* blk, uint32_t block_bytes,
                                         uint32_t codes_off, uint32_t scl_off, const int (&brow)[4], int KTOT,
                                         __bf16* lds) {
    constexpr int SPR = BK / 8;       // 16-byte pieces per A row
    constexpr int NAI = SPR / 4;      // A loads per wave per chunk (64 rows x SPR pieces over 256 lanes)
    constexpr int QK = BK / 4;        // K per lane group
    constexpr int NB = QK / 32;       // 16-byte code loads per column block (1 or 2)
    constexpr int NS = QK / 8;        // MFMA steps per chunk (4 or 8)
    constexpr int NBL = 4 * (NB + 1); // weight loads per lane per chunk (codes + scales)
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, m16 = lane & 15;
    const rsrc_t ra = make_rsrc(A, a_bytes);
    const rsrc_t rb = make_rsrc(blk, block_bytes);
    // this lane's A loads: LDS slot P = (wave*NAI + i)*64 + lane
    uint32_t aoff[NAI];
#pragma unroll
    for (int i = 0; i < NAI; i++) {
        const int P = (wave * NAI + i) * 64 + lane, r = P / SPR, q = P % SPR;
        aoff[i] = 2u * (uint32_t)(a_row(r < rows ? r : 0) + 8 * (q ^ (r & 7)));
    }
    uint32_t boff[4], soff[4];
#pragma unroll
    for (int cb = 0; cb < 4; cb++) {
        boff[cb] = codes_off + (uint32_t)brow[cb] * (KTOT / 2) + (QK / 2) * g;
        soff[cb] = scl_off + (uint32_t)brow[cb] * (KTOT / 16) + (QK / 16) * g;
    }
    const int nchunks = KTOT / BK;
    auto issue_a = [&](int ch, int buf) {
        const bool on = ch < nchunks;
#pragma unroll
        for (int i = 0; i < NAI; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(lds + (size_t)buf * 64 * BK + (size_t)(wave * NAI + i) * 64 * 8),
                16, on ? aoff[i] + 2u * ch * BK : kOOB, 0, 0, 0);
    };
    auto load_b = [&](int ch, uint4 (&bw)[4][NB], uint32_t (&bs)[4]) {
        const bool on = ch < nchunks;
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
#pragma unroll
            for (int i = 0; i < NB; i++) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rb, on ? boff[cb] + ch * (BK / 2) + 16 * i : kOOB, 0, 0);
                bw[cb][i] = uint4{v[0], v[1], v[2], v[3]};
            }
            const uint32_t so = on ? soff[cb] + ch * (BK / 16) : kOOB;
            bs[cb] = NB == 1 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, so, 0, 0)
                             : __builtin_amdgcn_raw_buffer_load_b32(rb, so, 0, 0);
        }
    };
    uint4 b0[4][NB], b1[4][NB];
    uint32_t s0[4], s1[4];
    issue_a(0, 0);
    load_b(0, b0, s0);
    load_b(1, b1, s1);
    vm_wait_barrier<NBL>();  // A(0) (and B(0)) landed
    // one chunk: take its weights out of set (bw, bs), refill the set with
    // chunk ch+2, load A(ch+1) into the other LDS buffer, compute, then wait
    // for A(ch+1): the barrier also ends every wave's reads of this chunk's
    // buffer, which A(ch+2) overwrites
    auto step = [&](int ch, uint4 (&bw)[4][NB], uint32_t (&bs)[4]) {
        uint4 bc[4][NB];
        uint32_t sc[4];
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
#pragma unroll
            for (int i = 0; i < NB; i++) bc[cb][i] = bw[cb][i];
            sc[cb] = bs[cb];
        }
        issue_a(ch + 1, (ch + 1) & 1);
        load_b(ch + 2, bw, bs);
        if (ch < nchunks) {
            const __bf16* At = lds + (size_t)(ch & 1) * 64 * BK;
#pragma unroll
            for (int s = 0; s < NS; s++) {
                bf16x8 bf[4];
#pragma unroll
                for (int cb = 0; cb < 4; cb++) {
                    const uint4 q = bc[cb][s / 4];
                    const uint32_t d = (s & 3) == 0 ? q.x : ((s & 3) == 1 ? q.y : ((s & 3) == 2 ? q.z : q.w));
                    const float sv = e4m3_to_f32((sc[cb] >> (8 * (s / 2))) & 0xFFu);
                    bf[cb] = dequant8_bf16(d, sv);
                }
                const int p = (QK / 8) * g + s;  // 16-byte piece of the fragment
#pragma unroll
                for (int rb = 0; rb < 4; rb++) {
                    if (16 * rb < rows) {  // uniform: skip padding row blocks of a short tile
                        const int r = 16 * rb + m16;
                        const bf16x8 af = *reinterpret_cast<const bf16x8*>(At + (r * SPR + (p ^ (r & 7))) * 8);
#pragma unroll
                        for (int cb = 0; cb < 4; cb++)
                            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[cb], acc[rb][cb], 0, 0, 0);
                    }
                }
            }
        }
        vm_wait_barrier<NBL>();
    };
    for (int ch = 0; ch < nchunks; ch += 2) {
        step(ch, b0, s0);
        step(ch + 1, b1, s1);
    }
}

constexpr int kBKGate = 256;  // K chunk of the gate/up GEMM (K = H)
constexpr int kBKDown = 128;  // K chunk of the down GEMM (K = I)

__global__ __launch_bounds__(256) void k_gateup_nv(GemmArgs a) {
    __shared__ __bf16 lds[2 * 64 * kBKGate];
    int tile, nt;
    if (!map_tile(a.ntiles[0], a.NT, tile, nt)) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = min(kBM_NV, a.count[e] - m0);
    const int base = a.off[e] + m0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I;
    const int c0 = nt * 128 + 32 * wave;
    const void* blk = a.expert_ptrs[e];
    const uint32_t codes_off = 0;                             // gate rows then up rows, H/2 bytes each
    const uint32_t scl_off = (uint32_t)3 * I * H / 2;         // gate scales then up scales, H/16 each
    const int m16 = lane & 15;
    const int brow[4] = {c0 + m16, c0 + 16 + m16, I + c0 + m16, I + c0 + 16 + m16};
    const __bf16* X = reinterpret_cast<const __bf16*>(a.a_src);
    const int* perm = a.perm;
    const int k = a.k;
    auto a_row = [&](int r) { return (perm[base + r] / k) * H; };  // 0 <= r < rows
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    nv_kloop<kBKGate>(acc, X, a.a_bytes, a_row, rows, blk, a.block_bytes, codes_off, scl_off, brow, H, lds);
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
    __shared__ __bf16 lds[2 * 64 * kBKDown];
    int tile, nt;
    if (!map_tile(a.ntiles[0], a.NT, tile, nt)) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = min(kBM_NV, a.count[e] - m0);
    const int base = a.off[e] + m0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I;
    const int n0 = nt * 256 + 64 * wave;
    const void* blk = a.expert_ptrs[e];
    const uint32_t codes_off = (uint32_t)I * H;                                  // down [H][I/2]
    const uint32_t scl_off = (uint32_t)3 * I * H / 2 + (uint32_t)2 * I * H / 16;  // down scales [H][I/16]
    const int m16 = lane & 15;
    const int brow[4] = {n0 + m16, n0 + 16 + m16, n0 + 32 + m16, n0 + 48 + m16};
    const __bf16* Hq = reinterpret_cast<const __bf16*>(a.a_src);
    auto a_row = [&](int r) { return (base + r) * I; };  // 0 <= r < rows
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    nv_kloop<kBKDown>(acc, Hq, a.a_bytes, a_row, rows, blk, a.block_bytes, codes_off, scl_off, brow, I, lds);
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
// of 32 rows = 2 row blocks, 64*NCB output columns of I); wave w owns NCB
// column blocks of 16 of gate and of up, so one activation fragment feeds
// 2*NCB MFMAs. Lane l holds row/column l%16 and K = k0 + 32(l/16) .. +31:
// 16 code bytes plus one UE8M0 scale byte, read straight from x~ and from
// the weight rows. KU K-steps of loads are in flight ahead of the MFMAs.
template <int NCB, int KU>
__global__ __launch_bounds__(256) void k_gateup_mx(GemmArgs a) {
    int tile, nt;
    if (!map_tile(a.ntiles[0], a.NT, tile, nt)) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = min(kBM_MX, a.count[e] - m0);
    const int base = a.off[e] + m0;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int H = a.H, I = a.I, k = a.k;
    const int g = lane >> 4, m16 = lane & 15;
    const int cbase = nt * 64 * NCB + 16 * NCB * wave + m16;
    const rsrc_t rw = make_rsrc(a.expert_ptrs[e], a.block_bytes);
    const rsrc_t rx = make_rsrc(a.a_src, a.a_bytes);
    const rsrc_t rxs = make_rsrc(a.a_scl, a.a_scl_bytes);
    const uint32_t scl0 = (uint32_t)3 * I * H / 2;
    // A rows of the two row blocks (padding rows read row 0 of the tile:
    // their outputs are discarded)
    uint32_t ar[2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
        const int r = 16 * rb + m16;
        ar[rb] = a.perm[base + (r < rows ? r : 0)] / k;
    }
    const int nrb = rows > 16 ? 2 : 1;  // wave-uniform
    f32x4 acc[2][2 * NCB];
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int j = 0; j < 2 * NCB; j++) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // B rows: j < NCB gate column blocks, j >= NCB up column blocks
    uint32_t brow[2 * NCB];
#pragma unroll
    for (int j = 0; j < 2 * NCB; j++) brow[j] = (uint32_t)(j < NCB ? 0 : I) + cbase + 16 * (j % NCB);
    uint4 bv[2][KU][2 * NCB], av[2][KU][2];
    int sb[2][KU][2 * NCB], sa[2][KU][2];
    const int nsteps = H / 128;
    // every group issues the same loads (steps past the end use an
    // out-of-range offset: zeros, no memory traffic), so the compiler's
    // memory counter waits stay exact and one group stays in flight while
    // the other is computed
    auto load = [&](int buf, int kg) {
#pragma unroll
        for (int u = 0; u < KU; u++) {
            const bool on = kg + u < nsteps;
            const uint32_t kb = (uint32_t)(kg + u) * 128 + 32 * g;
#pragma unroll
            for (int j = 0; j < 2 * NCB; j++) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, on ? brow[j] * (H / 2) + kb / 2 : kOOB, 0, 0);
                bv[buf][u][j] = uint4{v[0], v[1], v[2], v[3]};
                sb[buf][u][j] = (int)ld_b8(rw, on ? scl0 + brow[j] * (H / 32) + kb / 32 : kOOB);
            }
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, on ? ar[rb] * (H / 2) + kb / 2 : kOOB, 0, 0);
                av[buf][u][rb] = uint4{v[0], v[1], v[2], v[3]};
                sa[buf][u][rb] = (int)ld_b8(rxs, on ? ar[rb] * (H / 32) + kb / 32 : kOOB);
            }
        }
    };
    auto compute = [&](int buf, int kg) {
#pragma unroll
        for (int u = 0; u < KU; u++) {
#pragma unroll
            for (int rb = 0; rb < 2; rb++) {
                if (rb < nrb && kg + u < nsteps) {  // uniform: padding row block, steps past the end
                    const uint4 v = av[buf][u][rb];
                    const i32x8 A = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
#pragma unroll
                    for (int j = 0; j < 2 * NCB; j++) {
                        const uint4 w = bv[buf][u][j];
                        const i32x8 B = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
                        acc[rb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[rb][j], 4, 4, 0,
                                                                                      sa[buf][u][rb], 0, sb[buf][u][j]);
                    }
                }
            }
        }
    };
    // two K groups per iteration so that both register buffers have
    // compile-time indices
    load(0, 0);
    for (int kg = 0; kg < nsteps; kg += 2 * KU) {
        load(1, kg + KU);
        compute(0, kg);
        load(0, kg + 2 * KU);
        compute(1, kg + KU);
    }
    // D layout: lane holds column cbase + 16 j, rows 16 rb + 4 g + i
    float* hf = reinterpret_cast<float*>(a.out);
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int j = 0; j < NCB; j++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = 16 * rb + 4 * g + i;
                if (r < rows) {
                    const float hv = silu_mul(acc[rb][j][i], acc[rb][NCB + j][i]);
                    const size_t o = (size_t)(base + r) * I + cbase + 16 * j;
                    hf[o] = hv;
                    if (a.h_pre) a.h_pre[o] = hv;
                }
            }
}

// 4d. MXFP4 down with the scaled FP4 MFMA (32x32x64): workgroup = (M-tile of
// 32 grouped rows, 256 columns of H); wave w owns 2 column blocks of 32.
// Lane l holds row/column l%32 and K = k0 + 32(l/32) .. +31.
__global__ __launch_bounds__(256) void k_down_mx(GemmArgs a) {
    int tile, nt;
    if (!map_tile(a.ntiles[0], a.NT, tile, nt)) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = min(kBM_MX, a.count[e] - m0);
    const int base = a.off[e] + m0;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int H = a.H, I = a.I;
    const int g = lane >> 5, m32 = lane & 31;
    const rsrc_t rw = make_rsrc(a.expert_ptrs[e], a.block_bytes);
    const rsrc_t rh = make_rsrc(a.a_src, a.a_bytes);
    const rsrc_t rhs = make_rsrc(a.a_scl, a.a_scl_bytes);
    const uint32_t dcode = (uint32_t)I * H;
    const uint32_t dscl = (uint32_t)3 * I * H / 2 + (uint32_t)2 * I * H / 32;
    const int n0 = nt * 256 + 64 * wave;
    const uint32_t arow = base + (m32 < rows ? m32 : 0);
    f32x16 acc[2];
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
        for (int i = 0; i < 16; i++) acc[cb][i] = 0.f;
    constexpr int KU = 5;  // K steps per group (I = 2880: 45 steps)
    uint4 av[2][KU], bv[2][KU][2];
    int sa[2][KU], sb[2][KU][2];
    const int nsteps = I / 64;
    // every group issues the same loads (steps past the end use an
    // out-of-range offset: zeros, no memory traffic), so that the compiler's
    // memory counter waits stay exact
    auto load = [&](int buf, int kg) {
#pragma unroll
        for (int u = 0; u < KU; u++) {
            const bool on = kg + u < nsteps;
            const uint32_t kb = (uint32_t)(kg + u) * 64 + 32 * g;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rh, on ? arow * (I / 2) + kb / 2 : kOOB, 0, 0);
            av[buf][u] = uint4{v[0], v[1], v[2], v[3]};
            sa[buf][u] = (int)ld_b8(rhs, on ? arow * (I / 32) + kb / 32 : kOOB);
#pragma unroll
            for (int cb = 0; cb < 2; cb++) {
                const uint32_t n = (uint32_t)n0 + 32 * cb + m32;
                const auto w = __builtin_amdgcn_raw_buffer_load_b128(rw, on ? dcode + n * (I / 2) + kb / 2 : kOOB, 0, 0);
                bv[buf][u][cb] = uint4{w[0], w[1], w[2], w[3]};
                sb[buf][u][cb] = (int)ld_b8(rw, on ? dscl + n * (I / 32) + kb / 32 : kOOB);
            }
        }
    };
    auto compute = [&](int buf, int kg) {
#pragma unroll
        for (int u = 0; u < KU; u++) {
            if (kg + u < nsteps) {
                const uint4 v = av[buf][u];
                const i32x8 A = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
#pragma unroll
                for (int cb = 0; cb < 2; cb++) {
                    const uint4 w = bv[buf][u][cb];
                    const i32x8 B = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
                    acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[cb], 4, 4, 0, sa[buf][u], 0,
                                                                              sb[buf][u][cb]);
                }
            }
        }
    };
    load(0, 0);
    for (int kg = 0; kg < nsteps; kg += 2 * KU) {
        load(1, kg + KU);
        compute(0, kg);
        load(0, kg + 2 * KU);
        compute(1, kg + KU);
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
// grid of the grouped GEMMs (see map_tile): every XCD's M-tiles times NT
static unsigned gemm_grid(int max_mtiles, int NT) { return (unsigned)(8 * ((max_mtiles + 7) / 8) * NT); }

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

    hipLaunchKernelGGL(k_group, dim3(E), dim3(kGroupThreads), 0, s, idx, n, E, L.count, off, perm, L.pos);
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
        ga.a_bytes = (uint32_t)((size_t)T * H * 2);
        ga.block_bytes = (uint32_t)((size_t)3 * H * I / 2 + (size_t)3 * H * I / 16);
        hipLaunchKernelGGL(k_gateup_nv, dim3(gemm_grid(mt, ga.NT)), dim3(256), 0, s, ga);
        LAUNCH_CHECK();
        GemmArgs gd = ga;
        gd.a_src = L.hq; gd.out = L.Y; gd.h_pre = nullptr; gd.h_q = nullptr; gd.NT = H / 256;
        gd.a_bytes = (uint32_t)((size_t)n * I * 2);
        hipLaunchKernelGGL(k_down_nv, dim3(gemm_grid(mt, gd.NT)), dim3(256), 0, s, gd);
        LAUNCH_CHECK();
    } else {
        uint8_t* xc = dbg && dbg->x_codes ? dbg->x_codes : reinterpret_cast<uint8_t*>(L.xq);
        uint8_t* xs = dbg && dbg->x_scales ? dbg->x_scales : reinterpret_cast<uint8_t*>(L.xq) + (size_t)T * H / 2;
        const size_t nbx = (size_t)T * H / 32;
        hipLaunchKernelGGL(k_quant_mx, dim3((unsigned)((nbx + 255) / 256)), dim3(256), 0, s, x, nbx,
                           reinterpret_cast<uint32_t*>(xc), xs, (float*)nullptr);
        LAUNCH_CHECK();
        ga.a_src = xc; ga.a_scl = xs; ga.out = L.hf;
        ga.a_bytes = (uint32_t)((size_t)T * H / 2);
        ga.a_scl_bytes = (uint32_t)((size_t)T * H / 32);
        ga.block_bytes = (uint32_t)((size_t)3 * H * I / 2 + (size_t)3 * H * I / 32);
        if (I % 192 == 0) {
            ga.NT = I / 192;
            hipLaunchKernelGGL((k_gateup_mx<3, 2>), dim3(gemm_grid(mt, ga.NT)), dim3(256), 0, s, ga);
        } else {
            ga.NT = I / 64;
            hipLaunchKernelGGL((k_gateup_mx<1, 4>), dim3(gemm_grid(mt, ga.NT)), dim3(256), 0, s, ga);
        }
        LAUNCH_CHECK();
        uint8_t* hc = reinterpret_cast<uint8_t*>(L.hq);
        uint8_t* hs = hc + (size_t)n * I / 2;
        const size_t nbh = (size_t)n * I / 32;
        hipLaunchKernelGGL(k_quant_mx, dim3((unsigned)((nbh + 255) / 256)), dim3(256), 0, s, L.hf, nbh,
                           reinterpret_cast<uint32_t*>(hc), hs, dbg ? dbg->h_q : (float*)nullptr);
        LAUNCH_CHECK();
        GemmArgs gd = ga;
        gd.a_src = hc; gd.a_scl = hs; gd.out = L.Y; gd.h_pre = nullptr; gd.NT = H / 256;
        gd.a_bytes = (uint32_t)((size_t)n * I / 2);
        gd.a_scl_bytes = (uint32_t)((size_t)n * I / 32);
        hipLaunchKernelGGL(k_down_mx, dim3(gemm_grid(mt, gd.NT)), dim3(256), 0, s, gd);
        LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(k_combine_prefill, dim3((H / 4 + 255) / 256, T), dim3(256), 0, s, L.Y, L.pos, w, k, H, out,
                       out_bf16);
    return hipGetLastError();
}

}  // namespace moe
