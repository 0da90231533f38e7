// Prefill for gfx950: every prompt token through one MoE layer at once, with
// the token->expert assignments grouped by expert ([Q] "The engine", item 5:
// the whole prompt through each layer, so each expert's weights are read
// once per prompt instead of once per chunk).
//
//  1. grouping (k_front): stable grouping of the T*k assignments a = t*k + j
//     by expert (count, exclusive prefix sum, ordered compaction with
//     ballots: deterministic, no atomics).
//  2. tile list (k_front, beside the grouping): M-tiles of every expert,
//     heaviest experts first.
//  3. activation rounding (k_front, beside the grouping; k_quant_mx for h):
//     x~ = bf16(x) (NVFP4 layers; held for the GEMM as fp16 times a power of
//     two per token, exactly) or MXFP4 per 32 (MXFP4 layers).
//  4. ragged grouped GEMMs (gate/up with SiLU*mul epilogue, then down):
//     NVFP4 weights are decoded in registers, exactly, to fp16 for gate/up
//     (v_mfma_f32_16x16x32_f16) and to bf16 for down against h~
//     (v_mfma_f32_16x16x32_bf16); MXFP4 weights (streamed through an LDS ring)
//     and activations go straight into v_mfma_scale_f32_16x16x128_f8f6f4
//     with their E8M0 scales.
//  5. k_combine: out[t] = sum_j w[t][j] * Y[pos(t, j)] in increasing j.
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kBM_NV = 64;    // NVFP4 M-tile (rows of one expert)
constexpr int kBM_NV2 = 128;  // NVFP4 M-tile of the heavy experts
constexpr int kNV2Min = 65;   // rows from which an expert is heavy (more than one 64-row tile)
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
    void* rec;    // [max_tiles] TileRec (MXFP4 GEMMs)
    void* xq;     // x~: scaled fp16 [T][H] | MXFP4 codes [T][H/2] + scales [T][H/32]
    int* xexp;    // NVFP4: [T] power-of-two exponent of each row of the fp16 x~
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
    w.rec = take(16 * (size_t)mt);
    if (fmt == kFmtNvfp4) {
        w.xq = take((size_t)T * H * 2);
        w.xexp = (int*)take(sizeof(int) * (size_t)T);
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

// G = ceil(E/4) workgroups of 1024 threads; workgroup b handles the experts e0 = 4b ..
// e0+3 (those below E) and no workgroup depends on another. Wave w owns the
// contiguous slice [n*w/16, n*(w+1)/16) of the assignments a = t*k + j; its
// lane l takes a = lo + 64*i + l, so the order (i, l) is increasing a. Each
// pass issues all of a wave's loads of up to kGroupPer entries per lane
// together (one memory latency per pass for n <= 16*64*kGroupPer). Pass 1
// counts lt = #{a : idx[a] < e0} (summed over the workgroup: off[e0], the
// exclusive prefix sum of the counts) and eq[d] = #{a : idx[a] == e0 + d}
// per wave; one barrier gives every wave the matches of the waves before it.
// Pass 2 writes perm[off[e] + r] = the r-th assignment (in increasing a)
// routed to e and pos[a] = its grouped position. Assignments whose expert
// index lies outside [0, E) match no expert; workgroup b sets pos = -1 for
// those in its slice [n*b/G, n*(b+1)/G) of the array (G workgroups; a valid
// entry is only ever written by its expert's workgroup, so the writes never
// collide).
constexpr int kGroupPer = 24;
constexpr int kGroupExperts = 4;

__device__ __forceinline__ void group_block(const int32_t* __restrict__ idx, int n, int E, int* __restrict__ count,
                                            int* __restrict__ off, int* __restrict__ perm, int* __restrict__ pos,
                                            int bid, int G) {
    constexpr int NW = kGroupThreads / 64, ND = kGroupExperts;
    __shared__ int red_lt[NW], red_eq[ND][NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e0 = ND * bid;
    const int lo = (int)((long long)n * wave / NW), hi = (int)((long long)n * (wave + 1) / NW);
    int lt = 0, eq[ND] = {};
    for (int a0 = lo; a0 < hi; a0 += 64 * kGroupPer) {
        int v[kGroupPer];
#pragma unroll
        for (int i = 0; i < kGroupPer; i++) {
            const int a = a0 + 64 * i + lane;
            v[i] = a < hi ? idx[a] : E;
        }
#pragma unroll
        for (int i = 0; i < kGroupPer; i++) {
            lt += (unsigned)v[i] < (unsigned)e0;
#pragma unroll
            for (int d = 0; d < ND; d++) eq[d] += v[i] == e0 + d && e0 + d < E;
        }
    }
    lt = wave_sum_int(lt);
#pragma unroll
    for (int d = 0; d < ND; d++) eq[d] = wave_sum_int(eq[d]);
    if (lane == 0) {
        red_lt[wave] = lt;
#pragma unroll
        for (int d = 0; d < ND; d++) red_eq[d][wave] = eq[d];
    }
    __syncthreads();
    int base = 0, mine = 0;
    for (int i = 0; i < NW; i++) base += red_lt[i];
    int running[ND];
#pragma unroll
    for (int d = 0; d < ND; d++) {
        int cnt = 0, pre = 0;
        for (int i = 0; i < NW; i++) {
            cnt += red_eq[d][i];
            pre += i < wave ? red_eq[d][i] : 0;
        }
        running[d] = base + pre;
        mine += red_eq[d][wave];
        if (tid == 0 && e0 + d < E) {
            off[e0 + d] = base;
            count[e0 + d] = cnt;
            if (e0 + d == E - 1) off[E] = base + cnt;
        }
        base += cnt;
    }
    const int slo = (int)((long long)n * bid / G), shi = (int)((long long)n * (bid + 1) / G);
    for (int a = slo + tid; a < shi; a += kGroupThreads)
        if ((unsigned)idx[a] >= (unsigned)E) pos[a] = -1;
    if (mine == 0) return;  // wave-uniform: this wave's slice holds no match
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int a0 = lo; a0 < hi; a0 += 64 * kGroupPer) {
        int v[kGroupPer];
#pragma unroll
        for (int i = 0; i < kGroupPer; i++) {
            const int a = a0 + 64 * i + lane;
            v[i] = a < hi ? idx[a] : E;
        }
#pragma unroll
        for (int i = 0; i < kGroupPer; i++) {
            const int a = a0 + 64 * i + lane;
#pragma unroll
            for (int d = 0; d < ND; d++) {
                const bool match = v[i] == e0 + d && e0 + d < E;
                const unsigned long long m = __ballot(match);
                if (match) {
                    const int p = running[d] + __popcll(m & below);
                    perm[p] = a;
                    pos[a] = p;
                }
                running[d] += __popcll(m);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 2. tile list: experts ordered by row count (descending; ties by index),
// each split into M-tiles of BM rows, or of BM2 rows if it has at least
// BM2min (BM2 = 0: one height); the tiles in that order are then placed in
// the slots so that each XCD runs a contiguous part of the heavy experts'
// tiles (the slot order below). One workgroup of 1024 threads, which counts
// the rows of every expert itself (an LDS histogram of idx), so that it
// depends on nothing but the routing and runs beside the grouping.
//
// With rec != nullptr it also writes one record per slot of the max_tiles
// slots: the expert block, the first grouped row and the row count of the
// tile (row count 0 for slots past the last tile), so a GEMM workgroup finds
// everything it needs with one load.
struct TileRec {
    const uint8_t* blk;  // expert block
    int base;            // first grouped row
    int rows;            // rows of the tile; 0: no tile in this slot
};
static_assert(sizeof(TileRec) == 16, "tile record is 16 bytes");

__device__ __forceinline__ void tile_list_block(const int32_t* __restrict__ idx, int n, int E, int BM, int BM2,
                                                int BM2min, int* __restrict__ tile_e, int* __restrict__ tile_m,
                                                int* __restrict__ ntiles, TileRec* __restrict__ rec, int max_slots,
                                                const void* const* __restrict__ expert_ptrs) {
    static_assert(kMaxE <= kGroupThreads, "one thread per expert in the scans");
    __shared__ int cnt[kMaxE];
    __shared__ int offs[kMaxE];
    __shared__ uint4 key4[kMaxE / 4];
    __shared__ int rank[kMaxE];
    __shared__ int nt_sorted[kMaxE];
    __shared__ int ex_sorted[kMaxE];
    __shared__ int start[kGroupThreads + 1];
    unsigned* key = reinterpret_cast<unsigned*>(key4);
    const int tid = threadIdx.x;
    const int E4 = (E + 3) / 4;
    // rows per expert (assignments with an index outside [0, E) count nowhere)
    for (int e = tid; e < E; e += kGroupThreads) cnt[e] = 0;
    __syncthreads();
    for (int a0 = 0; a0 < n; a0 += kGroupThreads * kGroupPer) {
        int v[kGroupPer];
#pragma unroll
        for (int i = 0; i < kGroupPer; i++) {
            const int a = a0 + kGroupThreads * i + tid;
            v[i] = a < n ? idx[a] : -1;
        }
#pragma unroll
        for (int i = 0; i < kGroupPer; i++)
            if ((unsigned)v[i] < (unsigned)E) atomicAdd(&cnt[v[i]], 1);
    }
    __syncthreads();
    // inclusive scan over threads (Hillis-Steele; kGroupThreads >= E entries)
    auto scan = [&](int v) {
        for (int d = 1; d < kGroupThreads; d <<= 1) {
            start[tid] = v;
            __syncthreads();
            if (tid >= d) v += start[tid - d];
            __syncthreads();
        }
        return v;
    };
    if (rec) {
        // first grouped row of every expert (the grouping's exclusive prefix sum)
        const int c = tid < E ? cnt[tid] : 0;
        const int inc = scan(c);
        if (tid < E) offs[tid] = inc - c;
    }
    // key: larger count first, then lower index (counts clamped to 22 bits,
    // which only coarsens the order of the tile list)
    for (int e = tid; e < 4 * E4; e += kGroupThreads) {
        int c = 0;
        if (e < E) {
            c = cnt[e];
            rank[e] = 0;
        }
        key[e] = e < E ? ((0x3FFFFFu - (unsigned)min(c, 0x3FFFFF)) << 10) | (unsigned)e : 0xFFFFFFFFu;
    }
    __syncthreads();
    // rank[e] = #{j : key[j] < key[e]}, the comparisons split into P parts
    // over all threads (the loop is bound by VALU issue)
    const int P = max(1, kGroupThreads / E);
    for (int u = tid; u < E * P; u += kGroupThreads) {
        const int e = u % E, part = u / E;
        const unsigned ke = key[e];
        int r = 0;
#pragma unroll 4
        for (int j4 = part * E4 / P; j4 < (part + 1) * E4 / P; j4++) {
            const uint4 q = key4[j4];
            r += (q.x < ke) + (q.y < ke) + (q.z < ke) + (q.w < ke);
        }
        atomicAdd(&rank[e], r);
    }
    __syncthreads();
    auto height = [&](int c) { return BM2 > 0 && c >= BM2min ? BM2 : BM; };
    for (int e = tid; e < E; e += kGroupThreads) {
        ex_sorted[rank[e]] = e;
        nt_sorted[rank[e]] = (cnt[e] + height(cnt[e]) - 1) / height(cnt[e]);
    }
    __syncthreads();
    // inclusive scan of nt_sorted
    const int v = scan(tid < E ? nt_sorted[tid] : 0);
    start[tid + 1] = v;          // start[r + 1] = tiles of ranks 0..r
    if (tid == 0) start[0] = 0;
    if (tid == kGroupThreads - 1) ntiles[0] = v;
    __syncthreads();
    // heavy experts (more than one tile) are the ranks 0 .. R-1, their nh
    // tiles the first in rank order
    const int R = __syncthreads_count(tid < E && nt_sorted[tid] >= 2);
    const int used = start[E], nh = start[R];
    // slot -> tile index in rank order. The GEMM workgroups of slot s run on
    // XCD s % 8, and slot 8i + x is XCD x's i-th tile. Every XCD holds n =
    // used/8 tiles (one more for the first used % 8), so the slots below
    // `used` are exactly the tiles. Of them, XCD x takes a contiguous run of
    // the heavy tiles (hx = nh/8, one more for the first nh % 8 XCDs), so
    // that the tiles of one heavy expert share few L2s, spread evenly over
    // its n positions with a heavy tile first (position i is heavy when
    // ceil((i+1) hx / n) > ceil(i hx / n)): the heavy tiles are bound by
    // their MFMAs, the single tiles by their weight loads, and mixed they
    // overlap. The rest are single tiles dealt in rounds (round j: one to
    // every XCD that still has room, in XCD order), which keeps their mix of
    // heights even across XCDs, taken alternately from the largest and the
    // smallest left, which keeps it even along each XCD's sequence.
    auto order = [&](int sl) {
        const int x = sl & 7, i = sl >> 3;
        const int hq = nh >> 3, hr = nh & 7, nq = used >> 3, nr = used & 7;
        const int hx = hq + (x < hr), n = nq + (x < nr);
        const int c0 = (i * hx + n - 1) / n, c1 = ((i + 1) * hx + n - 1) / n;
        if (c1 > c0) return x * hq + min(x, hr) + c0;
        const int j = i - c0;
        int q = 0;
#pragma unroll
        for (int y = 0; y < 8; y++) {
            const int sy = nq + (y < nr) - hq - (y < hr);  // single tiles of XCD y
            q += min(sy, j) + (y < x && sy > j);
        }
        // blocks of 8 (a round) alternate between the largest and the
        // smallest single tiles left
        const int ns = used - nh, f = ((q >> 4) << 3) + (q & 7);
        return nh + (((q >> 3) & 1) ? ns - 1 - f : f);
    };
    // one thread per tile slot: the rank r of its tile u is the last with
    // start[r] <= u
    const int slots = rec ? max_slots : used;
    for (int sl = tid; sl < slots; sl += kGroupThreads) {
        if (sl >= used) {
            TileRec t;
            t.blk = nullptr;
            t.base = 0;
            t.rows = 0;
            rec[sl] = t;
            continue;
        }
        const int u = order(sl);
        int lo = 0, hi = E - 1;  // start[lo] <= u < start[hi + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (start[mid] <= u) lo = mid; else hi = mid - 1;
        }
        const int e = ex_sorted[lo], bm = height(cnt[e]), m = u - start[lo];
        tile_e[sl] = e;
        tile_m[sl] = m * bm;
        if (rec) {
            TileRec t;
            t.blk = reinterpret_cast<const uint8_t*>(expert_ptrs[e]);
            t.base = offs[e] + m * bm;
            t.rows = min(bm, cnt[e] - m * bm);
            rec[sl] = t;
        }
    }
}

// ---------------------------------------------------------------------------
// 3. activation rounding

// NVFP4 layers: x~ = bf16(x) (round to nearest even), handed to the gate/up
// GEMM as fp16 times a power of two per token: one wave per row finds
// m = the largest finite |x~| of the row and picks t with m * 2^t in
// [2^14, 2^15) (t = 0 for a row with no nonzero finite value). Every bf16
// value of the row with |x~| * 2^t >= 2^-14 is then an fp16 normal and
// converts exactly (8 significant bits into 11), and nothing overflows; the
// GEMM multiplies its sums by 2^-t. Only values more than 2^28 below the
// row's largest can lose bits (fp16 subnormals), a change of at most 2^-25 of
// the row maximum per element. Non-finite values pass through. The bf16
// values themselves go to xdbg when it is given.
// One wave per row, the row read twice (the second pass from L2) in blocks
// of 16 float4 per lane whose loads are all issued before the first use.
constexpr int kQuantBlk = 16;
__device__ __forceinline__ void quant_f16_row(const float* __restrict__ x, int T, int H, f16x2* __restrict__ out,
                                              int* __restrict__ xexp, bf16x2* __restrict__ xdbg, int row) {
    const int lane = threadIdx.x & 63, H4 = H / 4;
    if (row >= T) return;
    const f32x4* xr = reinterpret_cast<const f32x4*>(x + (size_t)row * H);
    auto to_bf16 = [](const f32x4 a, bf16x2& q0, bf16x2& q1) {
        const f32x2 p0 = {a.x, a.y}, p1 = {a.z, a.w};
        q0 = __builtin_convertvector(p0, bf16x2);
        q1 = __builtin_convertvector(p1, bf16x2);
    };
    float m = 0.f;
    for (int b0 = 0; b0 < H4; b0 += 64 * kQuantBlk) {
        f32x4 v[kQuantBlk];
#pragma unroll
        for (int u = 0; u < kQuantBlk; u++) v[u] = xr[min(b0 + lane + 64 * u, H4 - 1)];
#pragma unroll
        for (int u = 0; u < kQuantBlk; u++) {
            bf16x2 q0, q1;
            to_bf16(v[u], q0, q1);
            const float a[4] = {fabsf((float)q0.x), fabsf((float)q0.y), fabsf((float)q1.x), fabsf((float)q1.y)};
#pragma unroll
            for (int c = 0; c < 4; c++) m = a[c] <= 3.4028235e38f ? fmaxf(m, a[c]) : m;  // finite only (NaN: false)
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    int e = 0;
    if (m > 0.f) frexpf(m, &e);  // m in [2^(e-1), 2^e)
    const int t = m > 0.f ? 15 - e : 0;
    if (lane == 0) xexp[row] = t;
    f16x2* o = out + (size_t)row * (H / 2);
    for (int b0 = 0; b0 < H4; b0 += 64 * kQuantBlk) {
        f32x4 v[kQuantBlk];
#pragma unroll
        for (int u = 0; u < kQuantBlk; u++) v[u] = xr[min(b0 + lane + 64 * u, H4 - 1)];
#pragma unroll
        for (int u = 0; u < kQuantBlk; u++) {
            const int i = b0 + lane + 64 * u;
            if (i < H4) {
                bf16x2 q0, q1;
                to_bf16(v[u], q0, q1);
                if (xdbg) {
                    xdbg[(size_t)row * (H / 2) + 2 * i] = q0;
                    xdbg[(size_t)row * (H / 2) + 2 * i + 1] = q1;
                }
                const f32x2 p0 = {ldexpf((float)q0.x, t), ldexpf((float)q0.y, t)};
                const f32x2 p1 = {ldexpf((float)q1.x, t), ldexpf((float)q1.y, t)};
                o[2 * i] = __builtin_convertvector(p0, f16x2);
                o[2 * i + 1] = __builtin_convertvector(p1, f16x2);
            }
        }
    }
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
__device__ __forceinline__ void quant_mx_block(const float* __restrict__ src, size_t nblocks,
                                               uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                               float* __restrict__ dequant, size_t b) {
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

// The rounding of h (MXFP4 layers) between the two GEMMs: one thread per
// block of 32.
__global__ __launch_bounds__(256) void k_quant_mx(const float* __restrict__ src, size_t nblocks,
                                                  uint32_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  float* __restrict__ dequant) {
    quant_mx_block(src, nblocks, codes, scales, dequant, (size_t)blockIdx.x * 256 + threadIdx.x);
}

// The first launch of a prefill call: the tile list, the grouping and the
// rounding of x, which depend only on the routing and x, side by side.
// Workgroup 0 builds the tile list (tile_list_block, first: the GEMMs wait on
// it longest); workgroups 1 .. G (G = ceil(E/4)) group the assignments
// (group_block); the workgroups after them round x: 16 rows each, one per
// wave (NVFP4), or 1024 MX blocks, one per thread (MXFP4).
struct FrontArgs {
    const int32_t* idx;
    int n, E, G;
    int* count;
    int* off;
    int* perm;
    int* pos;
    const float* x;
    int T, H;
    f16x2* xq;         // NVFP4: fp16 x~ [T][H]
    int* xexp;         // NVFP4: [T]
    bf16x2* xdbg;      // NVFP4: bf16 x~ (debug) or null
    uint32_t* xcodes;  // MXFP4: codes [T][H/2]
    uint8_t* xscales;  // MXFP4: scales [T][H/32]
    size_t nbx;        // MXFP4: blocks of 32 in x
    int BM, BM2, BM2min;  // tile heights (tile_list_block)
    int* tile_e;
    int* tile_m;
    int* ntiles;
    TileRec* rec;
    int max_slots;
    const void* const* expert_ptrs;
    int* done;         // NVFP4: the GEMM launch's tile counters (4 ints per tile slot), cleared here
};

template <bool NV>
__global__ __launch_bounds__(kGroupThreads) void k_front(FrontArgs f) {
    const int b = (int)blockIdx.x - 1;
    if (b < 0) {
        if (f.done)
            for (int i = threadIdx.x; i < 4 * f.max_slots; i += kGroupThreads) f.done[i] = 0;
        tile_list_block(f.idx, f.n, f.E, f.BM, f.BM2, f.BM2min, f.tile_e, f.tile_m, f.ntiles, f.rec, f.max_slots,
                        f.expert_ptrs);
    } else if (b < f.G) {
        group_block(f.idx, f.n, f.E, f.count, f.off, f.perm, f.pos, b, f.G);
    } else if constexpr (NV) {
        quant_f16_row(f.x, f.T, f.H, f.xq, f.xexp, f.xdbg, (b - f.G) * (kGroupThreads / 64) + wave_id());
    } else {
        quant_mx_block(f.x, f.nbx, f.xcodes, f.xscales, nullptr, (size_t)(b - f.G) * kGroupThreads + threadIdx.x);
    }
}

// ---------------------------------------------------------------------------
// 4a. NVFP4 gate/up: ragged grouped GEMM with fp16 MFMA.
//
// Workgroup = (M-tile of one expert, 128 output columns of I). M-tiles are
// 128 rows for the experts that have more than 64 rows and 64 rows for the
// rest: a decoded weight fragment then serves up to 8 row blocks, which halves
// the decode work and the weight loads per MFMA of the heavy experts (an
// expert of 65-128 rows decodes its weights once instead of twice).
// Wave w owns output columns c0 = n0 + 32w .. +32 of BOTH gate and up, so its
// B operand is 4 column blocks of 16 (gate c0, gate c0+16, up c0, up c0+16)
// and SiLU*mul happens in registers. K runs over H in chunks of 256 (128 for
// the 128-row tiles, whose A tile then takes the same LDS); within a
// chunk each lane group owns a contiguous quarter of K (see nv_kloop), with
// the A operand read from LDS under the same K mapping (the dot product is
// order-independent). The codes are decoded to fp16 exactly (e2m1 x E4M3 has
// at most 6 significant bits and lies in the fp16 normal range); fp16 takes
// two instructions per two codes (conversion, packed multiply) where bf16
// takes four, since the hardware conversion applies only the exponent of a
// scale and gfx950 has no packed bf16 multiply. x~ comes as fp16 times 2^t
// per token (the front launch), and the epilogue multiplies the sums by 2^-t.
// Workgroup -> (M-tile, N-tile). Workgroups are dispatched round-robin over
// the 8 XCDs (each with its own L2), so workgroup b runs on XCD b % 8. M-tile
// t goes to XCD t % 8 and all NT N-tiles of an M-tile (the same gathered
// activation rows) to that XCD, one after the other; the tile list puts the
// tiles of a heavy expert in few XCDs' slots and balances the tiles per XCD
// (tile_list_block). The grid is 8 * ceil(max_tiles / 8) * NT.
// bid: the workgroup's index within its part of the launch (the down part
// of the GEMM launch starts at a multiple of 8, so a tile's gate/up and down
// workgroups share an XCD). Returns false for workgroups beyond the real
// tiles.
__device__ __forceinline__ bool map_tile_b(int bid, int ntiles, int NT, int& tile, int& nt) {
    const int x = bid % 8, j = bid / 8;
    tile = x + 8 * (j / NT);
    nt = j % NT;
    return tile < ntiles;
}
__device__ __forceinline__ bool map_tile(int ntiles, int NT, int& tile, int& nt) {
    return map_tile_b((int)blockIdx.x, ntiles, NT, tile, nt);
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
    const int* xexp;        // NVFP4 gate/up: per-token exponent of the fp16 x~
    uint32_t block_bytes;   // bytes of one expert block
    const TileRec* rec;     // MXFP4: tile records
    int mt;                 // MXFP4: record slots
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

// Decode 8 e2m1 codes (dword d) times scale s to 8 fp16 (exact: a code has
// at most 2 significant bits and an E4M3 scale 4, and |code * scale| lies in
// [2^-10, 2688], inside the fp16 normal range).
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t d, _Float16 s) {
    const f16x2 ss = {s, s};
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * ss;
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * ss;
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * ss;
    const f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * ss;
    f16x8 o = {a.x, a.y, b.x, b.y, c.x, c.y, e.x, e.y};
    return o;
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

// Shared K loop of the two NVFP4 GEMMs: acc[rb][cb] += A[16 RB rows] x B[4
// column blocks]^T over K (= KTOT) in chunks of BK (128 or 256), the A tile
// staged in LDS as MR rows (16, 32, 64 or 128; RB <= MR/16) per chunk: a tile
// of 1 or 2 row blocks loads only those rows (each A load instruction
// writes LDS even where its rows are past the tile's end). A is a
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
// consecutive rows on distinct bank groups. Rows past `rows` take the
// out-of-range offset (zeros, no memory traffic; their sums are never stored).
// SL: the block scales of the workgroup's weight rows were staged in LDS
// before the loop (slds: the scale bytes of column block cb's row, as stored,
// at srow[cb] * KTOT/16), so the loop loads only codes from memory. A scale
// load from memory takes a whole cache line for 2-4 bytes of each row; staged,
// the rows' scales arrive as contiguous lines once.

// 16-byte buffer load straight into LDS: lane l writes lds + 16*l (lds is
// wave-uniform).
__device__ __forceinline__ void load_lds16(rsrc_t r, uint8_t* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// Compiler ordering point: memory accesses stay on their side of it, and
// code that uses a or b after it cannot be scheduled before it.
__device__ __forceinline__ void order_point(int& a, int& b) { asm volatile("" : "+v"(a), "+v"(b)::"memory"); }

// SR (gate/up tiles that do not stage all their scales): the scales go
// through a ring of two 8 KB halves at slds, each holding one group of
// chunks' scale bytes of the workgroup's 256 weight rows (4 chunks of 128 or
// 2 of 256: slice row r's 32 bytes at r*32; gate rows sr_g0.., up rows
// sr_u0.., srow as for SL), staged one group ahead with 1 KB loads of 32
// contiguous bytes per row.
template <int BK, int RB, int MR, bool SL, bool F16, bool SR, class AROW>
__device__ __forceinline__ void nv_kloop(f32x4 (&acc)[RB][4], const __bf16* __restrict__ A, uint32_t a_bytes,
                                         AROW a_row, int rows, const void* blk, uint32_t block_bytes,
                                         uint32_t codes_off, uint32_t scl_off, const int (&brow)[4], int KTOT,
                                         __bf16* lds, const uint8_t* slds, const int (&srow)[4], int sr_g0 = 0,
                                         int sr_u0 = 0) {
    constexpr int SPR = BK / 8;       // 16-byte pieces per A row
    constexpr int NAI = MR * SPR / 256;  // A loads per wave per chunk (MR rows x SPR pieces over 256 lanes)
    static_assert(NAI >= 1 && NAI * 256 == MR * SPR && RB * 16 <= MR, "A tile shape");
    constexpr int QK = BK / 4;        // K per lane group
    constexpr int NB = QK / 32;       // 16-byte code loads per column block (1 or 2)
    constexpr int NS = QK / 8;        // MFMA steps per chunk (4 or 8)
    constexpr int NBL = SL || SR ? 4 * NB : 4 * (NB + 1);  // weight loads per lane per chunk (codes [+ scales])
    constexpr int GS = 4 / NB;  // chunks per scale group (32 bytes per row)
    static_assert(!SR || (!SL && (NB == 1 ? RB >= 8 : RB < 8)), "scale ring: one weight set per 128-wide chunk group, two per 256-wide");
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, m16 = lane & 15;
    const rsrc_t ra = make_rsrc(A, a_bytes);
    const rsrc_t rb = make_rsrc(blk, block_bytes);
    // this lane's A loads: LDS slot P = (wave*NAI + i)*64 + lane
    uint32_t aoff[NAI];
    bool aon[NAI];
#pragma unroll
    for (int i = 0; i < NAI; i++) {
        const int P = (wave * NAI + i) * 64 + lane, r = P / SPR, q = P % SPR;
        aon[i] = r < rows;
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
                ra, (__attribute__((address_space(3))) void*)(lds + (size_t)buf * MR * BK + (size_t)(wave * NAI + i) * 64 * 8),
                16, on && aon[i] ? aoff[i] + 2u * ch * BK : kOOB, 0, 0, 0);
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
            if constexpr (!SL && !SR) {
                const uint32_t so = on ? soff[cb] + ch * (BK / 16) : kOOB;
                bs[cb] = NB == 1 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, so, 0, 0)
                                 : __builtin_amdgcn_raw_buffer_load_b32(rb, so, 0, 0);
            }
        }
    };
    // scale ring (SR): group G = chunks GS*G .. GS*G+GS-1 -> half G & 1; two
    // 1 KB loads per wave (slice rows (2 wave + i) * 32 .. +31, 32 bytes each)
    uint8_t* const srb = const_cast<uint8_t*>(slds);
    auto stage = [&](int G) {
        if constexpr (SR) {
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int P = (wave * 2 + i) * 64 + lane, r = P >> 1, q = P & 1;
                const uint32_t row = r < 128 ? (uint32_t)(sr_g0 + r) : (uint32_t)(sr_u0 + r - 128);
                const uint32_t b = 32u * G + 16u * q;
                load_lds16(rb, srb + (G & 1) * 8192 + (wave * 2 + i) * 1024,
                           b < (uint32_t)(KTOT / 16) ? scl_off + row * (KTOT / 16) + b : kOOB);
            }
        }
    };
    // weight register sets: two (chunks ch+1 and ch+2 in flight), or one for
    // 8 row blocks, whose accumulators leave no room for a second set
    constexpr int NSET = RB >= 8 ? 1 : 2;
    uint4 b0[4][NB], b1[4][NB];
    uint32_t s0[4], s1[4];
    stage(0);  // older than A(0): the first wait covers it
    issue_a(0, 0);
    load_b(0, b0, s0);
    if constexpr (NSET > 1) load_b(1, b1, s1);
    vm_wait_barrier<NBL>();  // A(0) landed
    // one chunk: take its weights out of set (bw, bs), refill the set with
    // chunk ch+NSET, load A(ch+1) into the other LDS buffer, compute, then wait
    // for A(ch+1): the barrier also ends every wave's reads of this chunk's
    // buffer, which A(ch+2) overwrites
    auto step = [&](int ch, uint4 (&bw)[4][NB], uint32_t (&bs)[4], auto stg) {
        constexpr bool STG = decltype(stg)::value;  // this step stages the next scale group
        uint4 bc[4][NB];
        uint32_t sc[4];
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
#pragma unroll
            for (int i = 0; i < NB; i++) bc[cb][i] = bw[cb][i];
            if constexpr (SR) {
                const uint8_t* sp = srb + ((ch / GS) & 1) * 8192 + srow[cb] * 32 + (ch % GS) * (BK / 16) + (QK / 16) * g;
                sc[cb] = NB == 1 ? (uint32_t)*reinterpret_cast<const uint16_t*>(sp) : *reinterpret_cast<const uint32_t*>(sp);
            } else if constexpr (SL) {
                const uint8_t* sp = slds + srow[cb] * (KTOT / 16) + ch * (BK / 16) + (QK / 16) * g;
                sc[cb] = NB == 1 ? (uint32_t)*reinterpret_cast<const uint16_t*>(sp) : *reinterpret_cast<const uint32_t*>(sp);
            } else {
                sc[cb] = bs[cb];
            }
        }
        issue_a(ch + 1, (ch + 1) & 1);
        if constexpr (STG) stage(ch / GS + 1);  // into the half group ch/GS - 1 used
        load_b(ch + NSET, bw, bs);
        if (ch < nchunks) {
            const __bf16* At = lds + (size_t)(ch & 1) * MR * BK;
#pragma unroll
            for (int s = 0; s < NS; s++) {
                // the A fragments of all row blocks first, so their LDS
                // latency hides behind the decode
                const int p = (QK / 8) * g + s;  // 16-byte piece of the fragment
                // fragments as 16-byte vectors of the operand type
                typedef std::conditional_t<F16, f16x8, bf16x8> opv;
                opv af[RB];
#pragma unroll
                for (int rb = 0; rb < RB; rb++) {
                    const int r = 16 * rb + m16;
                    af[rb] = *reinterpret_cast<const opv*>(At + (r * SPR + (p ^ (r & 7))) * 8);
                }
                // no branches inside a chunk: the MFMAs of column block cb can
                // issue between the decode instructions of block cb+1
#pragma unroll
                for (int cb = 0; cb < 4; cb++) {
                    const uint4 q = bc[cb][s / 4];
                    const uint32_t d = (s & 3) == 0 ? q.x : ((s & 3) == 1 ? q.y : ((s & 3) == 2 ? q.z : q.w));
                    const float sv = e4m3_to_f32((sc[cb] >> (8 * (s / 2))) & 0xFFu);
                    if constexpr (F16) {
                        const f16x8 bf = dequant8_f16(d, (_Float16)sv);
#pragma unroll
                        for (int rb = 0; rb < RB; rb++)
                            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[rb], bf, acc[rb][cb], 0, 0, 0);
                    } else {
                        const bf16x8 bf = dequant8_bf16(d, sv);
#pragma unroll
                        for (int rb = 0; rb < RB; rb++)
                            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rb], bf, acc[rb][cb], 0, 0, 0);
                    }
                }
            }
        }
        // A(ch+1) landed (younger: the staged scales, if any, and B(ch+NSET))
        vm_wait_barrier<STG ? NBL + 2 : NBL>();
    };
    using Y = std::integral_constant<bool, true>;
    using N = std::integral_constant<bool, false>;
    if constexpr (NSET > 1 && SR) {
        for (int ch = 0; ch < nchunks; ch += 2) {
            step(ch, b0, s0, Y{});
            step(ch + 1, b1, s1, N{});
        }
    } else if constexpr (NSET > 1) {
        for (int ch = 0; ch < nchunks; ch += 2) {
            step(ch, b0, s0, N{});
            step(ch + 1, b1, s1, N{});
        }
    } else if constexpr (SR) {
        for (int ch = 0; ch < nchunks; ch += 4) {
            step(ch, b0, s0, Y{});
            step(ch + 1, b0, s0, N{});
            step(ch + 2, b0, s0, N{});
            step(ch + 3, b0, s0, N{});
        }
    } else {
        for (int ch = 0; ch < nchunks; ch++) step(ch, b0, s0, N{});
    }
}

constexpr int kBKGate = 256;  // K chunk of the gate/up GEMM (K = H)
constexpr int kBKDown = 128;  // K chunk of the down GEMM (K = I)
constexpr int kDownSclMaxI = 1024;  // I up to which the down GEMM stages its scales (see 4b)
// staged gate/up scale bytes that fit after 32 KB of A tiles in the GEMM
// launch's LDS (2 * kBM_NV2 * kBKDown bf16 + 256 * kDownSclMaxI / 16 bytes)
constexpr int kGateSclMax = 2 * kBM_NV2 * kBKDown * 2 + 256 * kDownSclMaxI / 16 - 32768;

// One gate/up tile: RB row blocks of the tile's rows, K chunks of BK, the A
// tile staged as MR rows.
// SL: the scales of the workgroup's 256 weight rows (gate columns n0 .. +128
// then the matching up columns, H/16 bytes each, two contiguous ranges of
// the block) are staged in LDS at lds + 32 KB first (tiles of up to 32 rows,
// whose A tiles take the first 32 KB; 16 H bytes), so the K loop loads only
// codes from memory.
template <int RB, int BK, int MR, bool SL>
__device__ __forceinline__ void gateup_nv_tile(const GemmArgs& a, __bf16* lds, int e, int base, int rows, int nt) {
    static_assert(!SL || 2 * MR * BK * 2 <= 32768, "staged scales follow the A tiles");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I;
    const int c0 = nt * 128 + 32 * wave;
    const void* blk = a.expert_ptrs[e];
    const uint32_t codes_off = 0;                             // gate rows then up rows, H/2 bytes each
    const uint32_t scl_off = (uint32_t)3 * I * H / 2;         // gate scales then up scales, H/16 each
    const int m16 = lane & 15;
    const int brow[4] = {c0 + m16, c0 + 16 + m16, I + c0 + m16, I + c0 + 16 + m16};
    // slice row of each column block's scales: gate rows 0..127, up rows 128..255
    const int cl = 32 * wave + m16;
    const int srow[4] = {cl, cl + 16, 128 + cl, 128 + cl + 16};
    uint8_t* sl = reinterpret_cast<uint8_t*>(lds) + 32768;
    if constexpr (SL) {
        // 1 KB loads, older than the K loop's first loads (its first wait
        // covers them)
        const uint32_t SB = (uint32_t)H / 16, half = 128 * SB;
        const uint32_t g0 = scl_off + (uint32_t)(nt * 128) * SB, u0 = scl_off + (uint32_t)(I + nt * 128) * SB;
        const rsrc_t rw = make_rsrc(blk, a.block_bytes);
        for (uint32_t ii = wave; ii * 1024 < 2 * half; ii += 4) {
            const uint32_t b = ii * 1024 + 16 * lane;
            load_lds16(rw, sl + ii * 1024, b < half ? g0 + b : (b < 2 * half ? u0 + (b - half) : kOOB));
        }
    }
    const __bf16* X = reinterpret_cast<const __bf16*>(a.a_src);
    const int* perm = a.perm;
    const int k = a.k;
    auto a_row = [&](int r) { return (perm[base + r] / k) * H; };  // 0 <= r < rows
    f32x4 acc[RB][4];
#pragma unroll
    for (int i = 0; i < RB; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // without staged scales (A tiles of up to 64 KB): the scales go through a
    // 16 KB ring after 64 KB
    constexpr bool SR = !SL;
    nv_kloop<BK, RB, MR, SL, true, SR>(acc, X, a.a_bytes, a_row, rows, blk, a.block_bytes, codes_off, scl_off, brow, H,
                                       lds, SR ? reinterpret_cast<uint8_t*>(lds) + 65536 : sl, srow, nt * 128,
                                       I + nt * 128);
    // epilogue: lane holds column c0 + 16 cbg + m16, rows 16 rb + 4 g + i;
    // the sums carry the row's 2^t of the fp16 x~ (exact to undo)
    __bf16* hq = reinterpret_cast<__bf16*>(a.out);
    const int g = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
        int nt_[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = 16 * rb + 4 * g + i;
            nt_[i] = -a.xexp[perm[base + min(r, rows - 1)] / k];
        }
#pragma unroll
        for (int cbg = 0; cbg < 2; cbg++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = 16 * rb + 4 * g + i;
                if (r < rows) {
                    const float hv = silu_mul(ldexpf(acc[rb][cbg][i], nt_[i]), ldexpf(acc[rb][cbg + 2][i], nt_[i]));
                    const __bf16 hb = (__bf16)hv;
                    const size_t o = (size_t)(base + r) * I + c0 + 16 * cbg + m16;
                    hq[o] = hb;
                    if (a.h_pre) a.h_pre[o] = hv;
                    if (a.h_q) a.h_q[o] = (float)hb;
                }
            }
    }
}

// Rows of tile (e, m0): tiles are kBM_NV2 rows high for experts with at least
// kNV2Min rows, kBM_NV otherwise (the tile list's rule).
__device__ __forceinline__ int nv_tile_rows(const GemmArgs& a, int e, int m0) {
    const int c = a.count[e];
    return min(c >= kNV2Min ? kBM_NV2 : kBM_NV, c - m0);
}

// The gate/up part of workgroup bid of the GEMM launch (lds: 2 * 64 *
// kBKGate bf16); returns its tile, or -1 if it has none.
__device__ __forceinline__ int gateup_part(const GemmArgs& a, __bf16* lds, int bid) {
    static_assert(2 * 64 * kBKGate == 2 * kBM_NV2 * 128, "one LDS size for both tile heights");
    int tile, nt;
    if (!map_tile_b(bid, a.ntiles[0], a.NT, tile, nt)) return -1;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = nv_tile_rows(a, e, m0);
    const int base = a.off[e] + m0;
    // the K loop is specialised on the tile's row blocks (wave-uniform); a
    // 128-row tile takes 128-wide K chunks so that its A tile fits the same LDS
    // tiles of up to 32 rows stage their scales where the LDS holds them
    // (16 H bytes after the 32 KB of A tiles, within the launch's 80 KB)
    const bool sl_fits = 16 * a.H <= kGateSclMax;
    if (rows <= 16) {
        if (sl_fits)
            gateup_nv_tile<1, kBKGate, 16, true>(a, lds, e, base, rows, nt);
        else
            gateup_nv_tile<1, kBKGate, 16, false>(a, lds, e, base, rows, nt);
    } else if (rows <= 32) {
        if (sl_fits)
            gateup_nv_tile<2, kBKGate, 32, true>(a, lds, e, base, rows, nt);
        else
            gateup_nv_tile<2, kBKGate, 32, false>(a, lds, e, base, rows, nt);
    } else if (rows <= 48) {
        gateup_nv_tile<3, kBKGate, 48, false>(a, lds, e, base, rows, nt);
    } else if (rows <= 64) {
        gateup_nv_tile<4, kBKGate, 64, false>(a, lds, e, base, rows, nt);
    } else {
        gateup_nv_tile<8, 128, kBM_NV2, false>(a, lds, e, base, rows, nt);
    }
    return tile;
}

// 4b. NVFP4 down: Y[p][n] = sum_i h~[p][i] * Wd[n][i]. Workgroup = (M-tile of
// 64 or 128 grouped rows, 256 columns of H); wave w owns columns n0 + 64w .. +64 as
// 4 column blocks of 16. A rows are contiguous grouped rows of h~.
// SL (I <= kDownSclMaxI): the scales of the 256 weight rows (I/16 bytes each,
// contiguous in the block) are staged in LDS first; the K loop then reads
// only codes from memory.

template <int RB, int MR, bool SL>
__device__ __forceinline__ void down_nv_tile(const GemmArgs& a, __bf16* lds, const uint8_t* sl, int e, int base,
                                             int rows, int nt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H, I = a.I;
    const int n0 = nt * 256 + 64 * wave;
    const void* blk = a.expert_ptrs[e];
    const uint32_t codes_off = (uint32_t)I * H;                                  // down [H][I/2]
    const uint32_t scl_off = (uint32_t)3 * I * H / 2 + (uint32_t)2 * I * H / 16;  // down scales [H][I/16]
    const int m16 = lane & 15;
    const int brow[4] = {n0 + m16, n0 + 16 + m16, n0 + 32 + m16, n0 + 48 + m16};
    const int srow[4] = {brow[0] - nt * 256, brow[1] - nt * 256, brow[2] - nt * 256, brow[3] - nt * 256};
    const __bf16* Hq = reinterpret_cast<const __bf16*>(a.a_src);
    auto a_row = [&](int r) { return (base + r) * I; };  // 0 <= r < rows
    f32x4 acc[RB][4];
#pragma unroll
    for (int i = 0; i < RB; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    nv_kloop<kBKDown, RB, MR, SL, false, false>(acc, Hq, a.a_bytes, a_row, rows, blk, a.block_bytes, codes_off, scl_off, brow, I, lds,
                                  sl, srow);
    float* Y = reinterpret_cast<float*>(a.out);
    const int g = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < RB; rb++)
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = 16 * rb + 4 * g + i;
                if (r < rows) Y[(size_t)(base + r) * H + n0 + 16 * cb + m16] = acc[rb][cb][i];
            }
}

// Bound of the down part's wait for its tile's h~, in polls of ~256 cycles
// (~0.4 s): a wait that ends unmet poisons the tile's outputs with NaN.
// (The debug controls can lower the bound and make every wait unmet.)
constexpr int kTileWaitPolls = 1 << 22;

// The down part of workgroup bid of the GEMM launch (lds: 2 * kBM_NV2 *
// kBKDown bf16; sl: 256 * kDownSclMaxI / 16 bytes). It first waits until
// done[4 * tile] reaches `need`, the count of the tile's gate/up workgroups.
template <bool SL>
__device__ __forceinline__ void down_part(const GemmArgs& a, __bf16* lds, uint8_t* sl, int bid, const int* done,
                                          int need, int max_polls) {
    int tile, nt;
    if (!map_tile_b(bid, a.ntiles[0], a.NT, tile, nt)) return;
    const int e = a.tile_e[tile], m0 = a.tile_m[tile];
    const int rows = nv_tile_rows(a, e, m0);
    const int base = a.off[e] + m0;
    // the outcome of thread 0's wait goes to every thread through the first
    // LDS word (no extra LDS: the second barrier keeps the A tiles from
    // overwriting it before every thread has read it)
    int* flag = reinterpret_cast<int*>(lds);
    if (threadIdx.x == 0) {
        int c = 0, polls = 0;
        while ((c = __hip_atomic_load(done + 4 * tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < need &&
               ++polls < max_polls)
            __builtin_amdgcn_s_sleep(4);
        *flag = c >= need;
    }
    __syncthreads();
    const bool ready = *flag != 0;
    __syncthreads();
    // h~ was written on this XCD (same L2, see k_gemms_nv); no stale line of
    // it may remain in this compute unit's L1
    asm volatile("buffer_inv sc0" ::: "memory");
    if (!ready) {
        float* Y = reinterpret_cast<float*>(a.out);
        for (int i = threadIdx.x; i < rows * 256; i += 256)
            Y[(size_t)(base + i / 256) * a.H + nt * 256 + i % 256] = __uint_as_float(0x7FC00000u);
        return;
    }
    if constexpr (SL) {
        // 1 KB loads of the rows' scales; they are older than the K loop's
        // first loads, so its first wait covers them
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const uint32_t SB = (uint32_t)a.I / 16, tot = 256 * SB;
        const uint32_t s0 = (uint32_t)3 * a.I * a.H / 2 + (uint32_t)2 * a.I * a.H / 16 + (uint32_t)(nt * 256) * SB;
        const rsrc_t rw = make_rsrc(a.expert_ptrs[e], a.block_bytes);
        for (uint32_t ii = wave; ii * 1024 < tot; ii += 4) {
            const uint32_t b = ii * 1024 + 16 * lane;
            load_lds16(rw, sl + ii * 1024, b < tot ? s0 + b : kOOB);
        }
    }
    if (rows <= 16)
        down_nv_tile<1, 16, SL>(a, lds, sl, e, base, rows, nt);
    else if (rows <= 32)
        down_nv_tile<2, 32, SL>(a, lds, sl, e, base, rows, nt);
    else if (rows <= 48)
        down_nv_tile<3, 48, SL>(a, lds, sl, e, base, rows, nt);
    else if (rows <= 64)
        down_nv_tile<4, 64, SL>(a, lds, sl, e, base, rows, nt);
    else
        down_nv_tile<8, kBM_NV2, SL>(a, lds, sl, e, base, rows, nt);
}

// ---------------------------------------------------------------------------
// 4c. The two NVFP4 GEMMs in one launch. Workgroups 0 .. ngu-1 run gate/up
// (gateup_part), workgroups ngu .. the down GEMM of the same tiles; ngu
// is a multiple of 8. Down workgroup (tile t, N-tile) starts only once the
// NT gate/up workgroups of tile t have published its h~ rows: each of those
// waits until its own stores have reached L2, then adds 1 to done[4t] (an
// atomic in L2); the down workgroup polls that counter (bounded) and
// invalidates its L1 before loading h~. No L2 write-back or invalidation is
// needed: with workgroup b on XCD b % 8 (the dispatcher deals workgroups
// round-robin over the XCDs; with 1, 2 or 4 XCDs the same congruence holds),
// a tile's gate/up and down workgroups have equal indices mod 8 and share
// one L2, and every h~ element is written once per call. The dispatcher
// starts workgroups in index order, so every gate/up workgroup has started
// before the first down workgroup waits: the waits end. The down work of
// the heavy tiles (first in the list) then fills the gate/up tail. done[] is
// cleared by the front launch.
struct GemmPair {
    GemmArgs gu, dn;
    int ngu;
    int* done;
    int need;       // publications a down tile waits for (NT of gate/up; more: a control)
    int max_polls;  // bound of each wait
};
template <bool SL>
__global__ __launch_bounds__(256, 2) void k_gemms_nv(GemmPair f) {
    // gate/up: 64 KB of A tiles; down: 64 KB of A tiles + the staged scales
    __shared__ __attribute__((aligned(16))) __bf16 lds[2 * kBM_NV2 * kBKDown + 256 * kDownSclMaxI / 16 / 2];
    static_assert(2 * 64 * kBKGate == 2 * kBM_NV2 * kBKDown, "one A-tile LDS size for both GEMMs");
    const int b = (int)blockIdx.x;
    if (b < f.ngu) {
        const int tile = gateup_part(f.gu, lds, b);
        if (tile < 0) return;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's h~ stores have reached L2
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(f.done + 4 * tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        down_part<SL>(f.dn, lds, reinterpret_cast<uint8_t*>(lds + 2 * kBM_NV2 * kBKDown), b - f.ngu, f.done, f.need,
                      f.max_polls);
    }
}

// ---------------------------------------------------------------------------
// 4d. MXFP4 grouped GEMMs: v_mfma_scale_f32_16x16x128_f8f6f4 on the e2m1
// codes of both operands with their UE8M0 block scales (a design choice of
// this library: the FP4 weights go to the matrix cores as stored, never
// widened). With a few tokens per expert these GEMMs stream the expert
// weights once, so the kernel is built around reading weight rows the way
// HBM likes best: whole row segments, contiguous.
//
// Workgroup = (tile of <= 32 grouped rows of one expert, 64 weight rows).
// gate/up (GU): weight rows 0..31 are gate rows c0..c0+31, rows 32..63 the
// up rows of the same columns, so SiLU*mul pairs stay in the workgroup;
// down: weight rows n0..n0+63 of Wd.
// The weight rows go through an LDS ring of NBUF chunk buffers, CB bytes of
// every row per chunk, with buffer_load ... lds (16 bytes per lane, no
// registers): one instruction covers 1024/CB rows, CB contiguous bytes each.
// Piece p (16 bytes = one 32-code MX block) of row r sits at slot
// r*SPR + (p ^ (r & 15)), so the 16 rows of an MFMA operand read (one piece
// each) fall on distinct bank groups. The block scales of the 64 rows are
// loaded once into LDS at the start.
// K split: the four waves take different K steps of every chunk (SPW steps
// of 128 each) for all 64 rows and both row blocks, so every activation
// fragment is loaded once per workgroup; the partial sums meet in LDS at the
// end. Activation fragments (A: lane = row l%16, 32 codes of K slot l/16 and
// their scale byte) are read straight from x~/h~ with buffer loads.
// The dot product does not depend on the order of K, so K slot g of the step
// (c, w, t) is MX block b = c*SPR + 4*(w*SPW + t) + g for both operands.
// Blocks past the end of the row (b >= K/32) load A from an out-of-range
// offset (zero codes, scale byte 0) and clamp the B scale to the last block
// of the row, so they add exact zeros.
// Pipeline: chunk group j = (weight chunk j, A fragments of chunk j) is
// issued NBUF-1 chunks ahead; every group has the same loads (out-of-range
// past the end), so "group c has landed" is a fixed count of younger loads.
// Each ring buffer is its own LDS array, so the compiler's own waits before
// an LDS read only cover the loads into that buffer.
template <bool GU, int CB, int NBUF, int SCLB>
__global__ __launch_bounds__(256) void k_mx_stream(GemmArgs a) {
    constexpr int SPR = CB / 16;        // pieces (MX blocks) per row per chunk
    constexpr int CKB = 64 * CB;        // bytes per ring buffer
    constexpr int NI = CKB / 1024 / 4;  // weight loads per wave per chunk
    constexpr int SPW = CB / 256;       // K steps of 128 per wave per chunk
    constexpr int NA = 2 * (SPW + 1);   // activation loads per wave per chunk (2 row blocks)
    static_assert(NBUF >= 2 && NBUF <= 4 && (SPW == 1 || SPW == 2) && SPR >= 16, "ring shape");
    static_assert(!GU || SPW == 2, "gate/up streams 512-byte row chunks");
    static_assert(GU || SPW == 1, "down streams 256-byte row chunks");
    __shared__ __attribute__((aligned(16))) uint8_t q0[CKB];
    __shared__ __attribute__((aligned(16))) uint8_t q1[CKB];
    __shared__ __attribute__((aligned(16))) uint8_t q2[NBUF > 2 ? CKB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t q3[NBUF > 3 ? CKB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t scl[SCLB];
    uint8_t* const ring[4] = {q0, q1, q2, q3};

    // workgroup -> (tile, N-tile): see map_tile
    const int xcd = blockIdx.x % 8, jj = blockIdx.x / 8;
    const int tile = xcd + 8 * (jj / a.NT), nt = jj % a.NT;
    if (tile >= a.mt) return;
    const TileRec tr = a.rec[tile];
    if (tr.rows <= 0) return;
    const int rows = tr.rows, base = tr.base;
    const int nrb = rows > 16 ? 2 : 1;

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, m16 = lane & 15;
    const int H = a.H, I = a.I;
    const uint32_t KB = GU ? (uint32_t)H / 2 : (uint32_t)I / 2;  // code bytes per weight row
    const uint32_t SB = KB / 16;                                // scale bytes per row = MX blocks per row
    const int nch = (int)((KB + CB - 1) / CB);
    const int c0 = GU ? 32 * nt : 64 * nt;  // first output column (GU: of I; down: of H)

    const rsrc_t rw = make_rsrc(tr.blk, a.block_bytes);
    const rsrc_t rx = make_rsrc(a.a_src, a.a_bytes);
    const rsrc_t rxs = make_rsrc(a.a_scl, a.a_scl_bytes);

    // activation rows of the two row blocks (rows past the tile read its
    // first row; their sums are never stored). GU rows come from perm: the
    // loads are issued here, the row offsets formed after the first weight
    // loads are out (see the prologue).
    int arow[2];
#pragma unroll
    for (int rb = 0; rb < 2; rb++) {
        const int m = 16 * rb + m16;
        const int r = m < rows ? m : 0;
        arow[rb] = GU ? a.perm[base + r] : base + r;
    }
    uint32_t aoff[2], asoff[2];
    auto set_rows = [&]() {
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            const uint32_t ar = GU ? (uint32_t)(arow[rb] / a.k) : (uint32_t)arow[rb];
            aoff[rb] = ar * KB;
            asoff[rb] = ar * SB;
        }
    };

    // scales of the 64 weight rows -> scl: [64][SB]; GU rows are 16-byte
    // pieces, piece p of row r stored at r*PPR + (p ^ (r & smask)); down rows
    // (SB bytes, any even count) are stored as they are.
    const uint32_t code0 = GU ? 0u : (uint32_t)I * H;
    const uint32_t PPR = SB / 16;
    const uint32_t smask = GU ? (min(PPR & (~PPR + 1u), 8u) - 1u) : 0u;
    {
        const uint32_t sbase = (uint32_t)3 * I * H / 2;
        const uint32_t nsl = (64 * SB + 1023) / 1024;  // 1 KB loads for the whole area
        for (uint32_t ii = wave; ii < nsl; ii += 4) {
            uint32_t o;
            if (GU) {
                const uint32_t P = ii * 64 + lane, r = P / PPR, sp = P % PPR, p = sp ^ (r & smask);
                const uint32_t row = (r < 32 ? 0u : (uint32_t)I) + c0 + (r & 31);
                o = r < 64 ? sbase + row * SB + 16 * p : kOOB;
            } else {
                const uint32_t b = ii * 1024 + 16 * lane;
                o = b < 64 * SB ? sbase + (uint32_t)2 * I * H / 32 + (uint32_t)c0 * SB + b : kOOB;
            }
            load_lds16(rw, scl + ii * 1024, o);
        }
    }
    // (these loads are older than chunk group 0, so the wait for group 0
    // covers them)

    // this lane's weight loads: ring slot q = (wave*NI + i)*64 + lane
    uint32_t woff[NI], wcol[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const uint32_t q = (uint32_t)(wave * NI + i) * 64 + lane, r = q / SPR, sp = q % SPR, p = sp ^ (r & 15u);
        const uint32_t row = GU ? (r < 32 ? 0u : (uint32_t)I) + c0 + (r & 31) : (uint32_t)c0 + r;
        wcol[i] = 16 * p;
        woff[i] = code0 + row * KB + 16 * p;
    }

    // register sets for the activation fragments of NBUF chunks
    uint4 av[NBUF][2][SPW];
    uint32_t as[NBUF][2][SPW];
    auto issue_w = [&](int c, int u) {
#pragma unroll
        for (int i = 0; i < NI; i++) {
            const bool on = c < nch && (uint32_t)c * CB + wcol[i] < KB;
            load_lds16(rw, ring[u] + (wave * NI + i) * 1024, on ? woff[i] + (uint32_t)c * CB : kOOB);
        }
    };
    auto issue_a = [&](int c, int u) {
#pragma unroll
        for (int rb = 0; rb < 2; rb++) {
            const bool onr = rb < nrb && c < nch;
#pragma unroll
            for (int t = 0; t < SPW; t++) {
                const uint32_t b = (uint32_t)c * SPR + 4 * (wave * SPW + t) + g;
                const bool on = onr && b < SB;
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, on ? aoff[rb] + 16 * b : kOOB, 0, 0);
                av[u][rb][t] = uint4{v[0], v[1], v[2], v[3]};
            }
            if constexpr (SPW == 2) {
                // the 8 scale bytes of the wave's two steps (SB is a multiple of 16)
                const uint32_t b0 = (uint32_t)c * SPR + 8 * wave;
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(rxs, onr && b0 < SB ? asoff[rb] + b0 : kOOB, 0, 0);
                as[u][rb][0] = (v[0] >> (8 * g)) & 0xFFu;
                as[u][rb][1] = (v[1] >> (8 * g)) & 0xFFu;
            } else {
                const uint32_t b = (uint32_t)c * SPR + 4 * wave + g;
                as[u][rb][0] = ld_b8(rxs, onr && b < SB ? asoff[rb] + b : kOOB);
            }
        }
    };

    f32x4 acc[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int c, int u) {
        const uint8_t* B = ring[u];
#pragma unroll
        for (int t = 0; t < SPW; t++) {
            const uint32_t bfirst = (uint32_t)c * SPR + 4 * (wave * SPW + t);
            if (c < nch && bfirst < SB) {  // uniform: steps wholly past the row end add nothing
                const uint32_t p = 4 * (wave * SPW + t) + g;  // piece within the chunk
                const uint32_t b = min(bfirst + g, SB - 1);  // scale of the block (clamped)
                i32x8 Bf[4];
                int sb[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t r = 16 * j + m16;
                    const uint4 w = *reinterpret_cast<const uint4*>(B + (r * SPR + (p ^ (r & 15u))) * 16);
                    Bf[j] = i32x8{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
                    uint32_t so;
                    if (GU) {
                        const uint32_t pp = b / 16;
                        so = r * SB + 16 * (pp ^ (r & smask)) + (b & 15);
                    } else {
                        so = r * SB + b;
                    }
                    sb[j] = scl[so];
                }
#pragma unroll
                for (int rb = 0; rb < 2; rb++) {
                    if (rb < nrb) {  // uniform
                        const uint4 v = av[u][rb][t];
                        const i32x8 A = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            acc[rb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                A, Bf[j], acc[rb][j], 4, 4, 0, (int)as[u][rb][t], 0, sb[j]);
                    }
                }
            }
        }
    };

    // prologue: groups 0 .. NBUF-2. The asm statements keep the groups in
    // order, and keep the row offsets (which wait for the perm loads) behind
    // the first weight loads.
    issue_w(0, 0);
    order_point(arow[0], arow[1]);
    set_rows();
    issue_a(0, 0);
#pragma unroll
    for (int j = 1; j < NBUF - 1; j++) {
        asm volatile("" ::: "memory");
        issue_w(j, j);
        issue_a(j, j);
    }
    for (int cc = 0; cc < nch; cc += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; u++) {
            const int c = cc + u;
            // group c landed in every wave; every wave is done with chunk c-1,
            // whose buffer group c+NBUF-1 overwrites
            vm_wait_barrier<(NBUF - 2) * (NI + NA)>();
            issue_w(c + NBUF - 1, (u + NBUF - 1) % NBUF);
            issue_a(c + NBUF - 1, (u + NBUF - 1) % NBUF);
            compute(c, u);
        }
    }
    vm_wait_barrier<0>();  // no load (out-of-range tail groups included) still writes LDS

    // partial sums of the four waves -> LDS (8 KB per wave), then the sums
    uint8_t* red = CKB >= 32768 ? q0 + wave * 8192 : (wave < 2 ? q0 + wave * 8192 : q1 + (wave - 2) * 8192);
#pragma unroll
    for (int rb = 0; rb < 2; rb++)
        if (rb < nrb)
#pragma unroll
            for (int j = 0; j < 4; j++)
                *reinterpret_cast<f32x4*>(red + ((rb * 4 + j) * 64 + lane) * 16) = acc[rb][j];
    __syncthreads();
    auto part = [&](int w, int rb, int j) -> f32x4 {
        const uint8_t* rw8 = CKB >= 32768 ? q0 + w * 8192 : (w < 2 ? q0 + w * 8192 : q1 + (w - 2) * 8192);
        return *reinterpret_cast<const f32x4*>(rw8 + ((rb * 4 + j) * 64 + lane) * 16);
    };
    const int rb = wave >> 1;
    if (rb >= nrb) return;
    if (GU) {
        // thread: row block rb, gate column block cj (0/1) and its up block
        const int cj = wave & 1;
        f32x4 gs = part(0, rb, cj), us = part(0, rb, cj + 2);
#pragma unroll
        for (int w = 1; w < 4; w++) {
            gs += part(w, rb, cj);
            us += part(w, rb, cj + 2);
        }
        float* hf = reinterpret_cast<float*>(a.out);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int r = 16 * rb + 4 * g + i;
            if (r < rows) {
                const float hv = silu_mul(gs[i], us[i]);
                const size_t o = (size_t)(base + r) * I + c0 + 16 * cj + m16;
                hf[o] = hv;
                if (a.h_pre) a.h_pre[o] = hv;
            }
        }
    } else {
        float* Y = reinterpret_cast<float*>(a.out);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int j = 2 * (wave & 1) + h;
            f32x4 ys = part(0, rb, j);
#pragma unroll
            for (int w = 1; w < 4; w++) ys += part(w, rb, j);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = 16 * rb + 4 * g + i;
                if (r < rows) Y[(size_t)(base + r) * H + c0 + 16 * j + m16] = ys[i];
            }
        }
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
    // groups of up to 8 assignments: all their Y loads first, then the sums
    // in increasing j
    constexpr int NG = 8;
    for (int j0 = 0; j0 < k; j0 += NG) {
        int pv[NG];
        float wv[NG];
#pragma unroll
        for (int i = 0; i < NG; i++) {
            pv[i] = pos[t * k + min(j0 + i, k - 1)];
            wv[i] = w[t * k + min(j0 + i, k - 1)];
        }
        __builtin_amdgcn_sched_barrier(0);  // the positions' and weights' loads issue together, before the rows'
        f32x4 yv[NG];
#pragma unroll
        for (int i = 0; i < NG; i++) yv[i] = reinterpret_cast<const f32x4*>(Y + (size_t)max(pv[i], 0) * H)[c4];
#pragma unroll
        for (int i = 0; i < NG; i++) {
            const int j = j0 + i;
            if (j >= k) break;
            const float wj = wv[i];
            if (pv[i] < 0) {
                acc = f32x4{__uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u), __uint_as_float(0x7FC00000u),
                            __uint_as_float(0x7FC00000u)};
                continue;
            }
            acc.x = fmaf(wj, yv[i].x, acc.x);
            acc.y = fmaf(wj, yv[i].y, acc.y);
            acc.z = fmaf(wj, yv[i].z, acc.z);
            acc.w = fmaf(wj, yv[i].w, acc.w);
        }
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

    FrontArgs fa = {};
    fa.idx = idx; fa.n = n; fa.E = E; fa.G = (E + kGroupExperts - 1) / kGroupExperts;
    fa.count = L.count; fa.off = off; fa.perm = perm; fa.pos = L.pos;
    fa.x = x; fa.T = T; fa.H = H;
    TileRec* rec = fmt == kFmtMxfp4 ? reinterpret_cast<TileRec*>(L.rec) : nullptr;
    fa.BM = BM; fa.BM2 = fmt == kFmtNvfp4 ? kBM_NV2 : 0; fa.BM2min = kNV2Min;
    fa.tile_e = L.tile_e; fa.tile_m = L.tile_m; fa.ntiles = L.ntiles; fa.rec = rec; fa.max_slots = mt;
    fa.expert_ptrs = expert_ptrs;
    fa.done = fmt == kFmtNvfp4 ? reinterpret_cast<int*>(L.rec) : nullptr;
    uint8_t* xc = dbg && dbg->x_codes ? dbg->x_codes : reinterpret_cast<uint8_t*>(L.xq);
    uint8_t* xs = dbg && dbg->x_scales ? dbg->x_scales : reinterpret_cast<uint8_t*>(L.xq) + (size_t)T * H / 2;
    if (fmt == kFmtNvfp4) {
        fa.xq = reinterpret_cast<f16x2*>(L.xq); fa.xexp = L.xexp;
        fa.xdbg = dbg && dbg->x_bf16 ? reinterpret_cast<bf16x2*>(dbg->x_bf16) : (bf16x2*)nullptr;
        const int nq = (T + kGroupThreads / 64 - 1) / (kGroupThreads / 64);
        hipLaunchKernelGGL(k_front<true>, dim3((unsigned)(1 + fa.G + nq)), dim3(kGroupThreads), 0, s, fa);
    } else {
        fa.xcodes = reinterpret_cast<uint32_t*>(xc); fa.xscales = xs; fa.nbx = (size_t)T * H / 32;
        const int nq = (int)((fa.nbx + kGroupThreads - 1) / kGroupThreads);
        hipLaunchKernelGGL(k_front<false>, dim3((unsigned)(1 + fa.G + nq)), dim3(kGroupThreads), 0, s, fa);
    }
    LAUNCH_CHECK();

    GemmArgs ga = {};
    ga.tile_e = L.tile_e; ga.tile_m = L.tile_m; ga.ntiles = L.ntiles; ga.count = L.count; ga.off = off;
    ga.perm = perm; ga.expert_ptrs = expert_ptrs; ga.E = E; ga.H = H; ga.I = I; ga.k = k;
    ga.h_pre = dbg ? dbg->h_pre : nullptr;

    if (fmt == kFmtNvfp4) {
        ga.a_src = L.xq;
        ga.xexp = L.xexp; ga.out = L.hq; ga.h_q = dbg ? dbg->h_q : nullptr; ga.NT = I / 128;
        ga.a_bytes = (uint32_t)((size_t)T * H * 2);
        ga.block_bytes = (uint32_t)((size_t)3 * H * I / 2 + (size_t)3 * H * I / 16);
        GemmArgs gd = ga;
        gd.a_src = L.hq; gd.out = L.Y; gd.h_pre = nullptr; gd.h_q = nullptr; gd.NT = H / 256;
        gd.a_bytes = (uint32_t)((size_t)n * I * 2);
        GemmPair gp;
        gp.gu = ga; gp.dn = gd; gp.ngu = (int)gemm_grid(mt, ga.NT); gp.done = reinterpret_cast<int*>(L.rec);
        gp.need = ga.NT + (dbg && dbg->tile_wait_unmet ? 1 : 0);
        gp.max_polls = dbg && dbg->tile_wait_polls > 0 ? dbg->tile_wait_polls : kTileWaitPolls;
        const dim3 grid((unsigned)gp.ngu + gemm_grid(mt, gd.NT));
        if (I <= kDownSclMaxI)
            hipLaunchKernelGGL(k_gemms_nv<true>, grid, dim3(256), 0, s, gp);
        else
            hipLaunchKernelGGL(k_gemms_nv<false>, grid, dim3(256), 0, s, gp);
        LAUNCH_CHECK();
    } else {
        ga.a_src = xc; ga.a_scl = xs; ga.out = L.hf;
        ga.a_bytes = (uint32_t)((size_t)T * H / 2);
        ga.a_scl_bytes = (uint32_t)((size_t)T * H / 32);
        ga.block_bytes = (uint32_t)((size_t)3 * H * I / 2 + (size_t)3 * H * I / 32);
        ga.rec = rec;
        ga.mt = mt;
        ga.NT = I / 32;
        if (2 * H <= 8192)
            hipLaunchKernelGGL((k_mx_stream<true, 512, 2, 8192>), dim3(gemm_grid(mt, ga.NT)), dim3(256), 0, s, ga);
        else
            hipLaunchKernelGGL((k_mx_stream<true, 512, 2, 32768>), dim3(gemm_grid(mt, ga.NT)), dim3(256), 0, s, ga);
        LAUNCH_CHECK();
        uint8_t* hc = reinterpret_cast<uint8_t*>(L.hq);
        uint8_t* hs = hc + (size_t)n * I / 2;
        const size_t nbh = (size_t)n * I / 32;
        hipLaunchKernelGGL(k_quant_mx, dim3((unsigned)((nbh + 255) / 256)), dim3(256), 0, s, L.hf, nbh,
                           reinterpret_cast<uint32_t*>(hc), hs, dbg ? dbg->h_q : (float*)nullptr);
        LAUNCH_CHECK();
        GemmArgs gd = ga;
        gd.a_src = hc; gd.a_scl = hs; gd.out = L.Y; gd.h_pre = nullptr;
        gd.a_bytes = (uint32_t)((size_t)n * I / 2);
        gd.a_scl_bytes = (uint32_t)((size_t)n * I / 32);
        gd.NT = H / 64;
        if (2 * I <= 8192)
            hipLaunchKernelGGL((k_mx_stream<false, 256, 3, 8192>), dim3(gemm_grid(mt, gd.NT)), dim3(256), 0, s, gd);
        else
            hipLaunchKernelGGL((k_mx_stream<false, 256, 3, 32768>), dim3(gemm_grid(mt, gd.NT)), dim3(256), 0, s, gd);
        LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(k_combine_prefill, dim3((H / 4 + 255) / 256, T), dim3(256), 0, s, L.Y, L.pos, w, k, H, out,
                       out_bf16);
    return hipGetLastError();
}

}  // namespace moe
