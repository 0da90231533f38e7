// Speculative expert prefetch ([Q] "The engine", item 3 and [D] "Making it
// faster": guess the next layer's experts while this layer computes and move
// them closer before they are needed).
//
// On this machine every expert is already in HBM; "closer" is the 256 MB
// last-level cache (MALL) shared by the chip: k_prefetch reads the guessed
// experts' blocks with plain loads while the current layer runs on another
// stream, so the next layer's expert kernels find them in the MALL. The
// guess itself is moe_route with the next layer's router on this layer's
// input. Every loaded word goes into an XOR checksum per 64 KiB chunk (the
// kernel's only output), which makes the read observable and testable.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kPrefetchLoads = 16;                              // 16-byte loads per thread
constexpr uint32_t kPrefetchChunk = 256u * 16u * kPrefetchLoads;  // 64 KiB per workgroup

int prefetch_chunks(size_t block_bytes) { return (int)((block_bytes + kPrefetchChunk - 1) / kPrefetchChunk); }

// Workgroup b reads chunk c = b % nchunks of the block of expert idx[b / nchunks]
// (all loads issued before the first use; past the block's end the buffer
// returns zeros) and writes the XOR of the chunk's 32-bit words to sink[b];
// an index outside [0, E) reads nothing and writes 0. (Four workgroups per
// expert walking their chunks in a loop measured slower beside a decode.)
__global__ __launch_bounds__(256) void k_prefetch(const void* const* __restrict__ ptrs, const int32_t* __restrict__ idx,
                                                  int E, uint32_t block_bytes, int nchunks, uint32_t* __restrict__ sink) {
    __shared__ uint32_t red[4];
    const int j = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
    const int e = __builtin_amdgcn_readfirstlane(idx[j]);
    const bool ok = (unsigned)e < (unsigned)E;
    const void* blk = ok ? ptrs[e] : nullptr;
    const rsrc_t r = make_rsrc(ok ? blk : (const void*)sink, ok ? block_bytes : 0u);
    const uint32_t base = (uint32_t)c * kPrefetchChunk + 16u * threadIdx.x;
    uint4 v[kPrefetchLoads];
#pragma unroll
    for (int u = 0; u < kPrefetchLoads; u++) {
        const auto q = __builtin_amdgcn_raw_buffer_load_b128(r, base + 4096u * u, 0, 0);
        v[u] = uint4{q[0], q[1], q[2], q[3]};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kPrefetchLoads; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

hipError_t launch_prefetch(const void* const* ptrs, const int32_t* idx, int n, int E, size_t block_bytes,
                           uint32_t* sink, hipStream_t s) {
    const int nch = prefetch_chunks(block_bytes);
    hipLaunchKernelGGL(k_prefetch, dim3((unsigned)(n * nch)), dim3(256), 0, s, ptrs, idx, E, (uint32_t)block_bytes,
                       nch, sink);
    return hipGetLastError();
}

}  // namespace moe
