// Router for gfx950: logits = Wr x (fp32), then top-k and the softmax
// weights renormalised over the chosen k, computed on the device so the
// chosen experts never travel to the host (the pages' engine read them back
// once per layer, [Q] "Where the time actually goes").
//  * k_route_logits + k_route_topk (T <= 16): one wave per (expert row,
//    token) so the E x H fp32 router matrix streams from HBM over the whole
//    chip, then one wave per token runs the top-k.
//  * k_route_tokens (T > 16): one workgroup per token computes all E logits
//    into LDS and runs the top-k itself.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

size_t route_ws_bytes(int T, int E) { return kCounterBytes + align256((size_t)T * E * sizeof(float)); }

bool route_supported(int H, int E, int k) { return H % 256 == 0 && H <= 8192 && E >= 1 && E <= kMaxE && k >= 1 && k <= kMaxK && k <= E; }

// grid (E, T), 64 threads: one wave per (expert row, token), H = 256 * DV
// (lane reads float4 chunks lane + 64m), so the E x H fp32 router matrix
// streams from HBM over the whole chip.
template <int DV>
__global__ __launch_bounds__(64) void k_route_logits(const float* __restrict__ x, const float* __restrict__ Wr, int E,
                                                     float* __restrict__ logits) {
    constexpr int H = 256 * DV;
    const int lane = threadIdx.x, e = blockIdx.x, t = blockIdx.y;
    const f4v* xr = reinterpret_cast<const f4v*>(x + (size_t)t * H);
    const f4v* wr = reinterpret_cast<const f4v*>(Wr + (size_t)e * H);
    f4v a[DV], b[DV];
#pragma unroll
    for (int m = 0; m < DV; m++) { a[m] = wr[lane + 64 * m]; b[m] = xr[lane + 64 * m]; }
    float acc = 0.f;
#pragma unroll
    for (int m = 0; m < DV; m++) {
        acc = fmaf(a[m].x, b[m].x, acc); acc = fmaf(a[m].y, b[m].y, acc);
        acc = fmaf(a[m].z, b[m].z, acc); acc = fmaf(a[m].w, b[m].w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[(size_t)t * E + e] = acc;
}

// grid T, 64 threads: the top-k of one token's logits (the kernel boundary
// after k_route_logits makes every logit visible).
__global__ __launch_bounds__(64) void k_route_topk(const float* __restrict__ logits, int E, int k,
                                                   int32_t* __restrict__ idx, float* __restrict__ w) {
    const float* lt = logits + (size_t)blockIdx.x * E;
    topk_wave([&](int i) { return lt[i]; }, E, k, idx + (size_t)blockIdx.x * k, w + (size_t)blockIdx.x * k);
}

// grid T, 256 threads: one token per workgroup.
template <int DV>
__global__ __launch_bounds__(256) void k_route_tokens(const float* __restrict__ x, const float* __restrict__ Wr, int E,
                                                      int k, float* __restrict__ logits_out, int32_t* __restrict__ idx,
                                                      float* __restrict__ w) {
    constexpr int H = 256 * DV;
    __shared__ float ls[kMaxE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, t = blockIdx.x;
    const f4v* xr = reinterpret_cast<const f4v*>(x + (size_t)t * H);
    f4v b[DV];
#pragma unroll
    for (int m = 0; m < DV; m++) b[m] = xr[lane + 64 * m];
    for (int e = wave; e < E; e += 4) {
        const f4v* wr = reinterpret_cast<const f4v*>(Wr + (size_t)e * H);
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < DV; m++) {
            const f4v a = wr[lane + 64 * m];
            acc = fmaf(a.x, b[m].x, acc); acc = fmaf(a.y, b[m].y, acc);
            acc = fmaf(a.z, b[m].z, acc); acc = fmaf(a.w, b[m].w, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) ls[e] = acc;
    }
    __syncthreads();
    if (logits_out)
        for (int e = tid; e < E; e += 256) logits_out[(size_t)t * E + e] = ls[e];
    if (wave == 0) topk_wave([&](int i) { return ls[i]; }, E, k, idx + (size_t)t * k, w + (size_t)t * k);
}

hipError_t launch_route(int H, int E, int k, int T, const float* x, const float* Wr, int32_t* idx, float* w,
                        float* logits_out, void* ws, hipStream_t s) {
    char* base = reinterpret_cast<char*>(ws);
    const int DV = H / 256;
    if (T <= kRouteSplitMaxT) {
        float* lg = logits_out ? logits_out : reinterpret_cast<float*>(base + kCounterBytes);
        dim3 grid(E, T), block(64);
#define RS(D) \
    case D: hipLaunchKernelGGL((k_route_logits<D>), grid, block, 0, s, x, Wr, E, lg); break;
        switch (DV) {
            RS(1) RS(2) RS(3) RS(4) RS(5) RS(6) RS(7) RS(8) RS(9) RS(10) RS(11) RS(12) RS(13) RS(14) RS(15) RS(16)
            RS(17) RS(18) RS(19) RS(20) RS(21) RS(22) RS(23) RS(24) RS(25) RS(26) RS(27) RS(28) RS(29) RS(30) RS(31) RS(32)
            default: return hipErrorInvalidValue;
        }
#undef RS
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_route_topk, dim3(T), dim3(64), 0, s, lg, E, k, idx, w);
    } else {
        dim3 grid(T), block(256);
#define RT(D) \
    case D: hipLaunchKernelGGL((k_route_tokens<D>), grid, block, 0, s, x, Wr, E, k, logits_out, idx, w); break;
        switch (DV) {
            RT(1) RT(2) RT(3) RT(4) RT(5) RT(6) RT(7) RT(8) RT(9) RT(10) RT(11) RT(12) RT(13) RT(14) RT(15) RT(16)
            RT(17) RT(18) RT(19) RT(20) RT(21) RT(22) RT(23) RT(24) RT(25) RT(26) RT(27) RT(28) RT(29) RT(30) RT(31) RT(32)
            default: return hipErrorInvalidValue;
        }
#undef RT
    }
    return hipGetLastError();
}

}  // namespace moe
