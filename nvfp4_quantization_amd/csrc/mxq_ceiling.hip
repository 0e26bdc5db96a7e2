// mxq_ceiling.hip -- the HBM ceilings the benchmark measures beside the quantizers
// (libmxq_ceiling.so, not part of the quantization ABI): a streaming read and a
// streaming copy, hand-written for gfx950 in the access pattern the quantizers use
// (16-byte loads per lane, whole 64-byte-aligned rows of a work-group per
// instruction, many loads in flight per lane).  Their rates bound what any kernel
// that moves the same bytes can reach on the box.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;          // 16-byte loads in flight per lane
constexpr int64_t kChunk = (int64_t)kThreads * kUnroll * 16;   // bytes per work-group step

// Reads n16 16-byte words of src (grid-strided chunks of kChunk bytes) and writes one
// word per work-group (the XOR of what it read), so that no load can be dropped.
__global__ __launch_bounds__(kThreads) void k_read(const u32x4v* __restrict__ src, int64_t n16,
                                                   uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * (kChunk / 16); base < n16; base += (int64_t)gridDim.x * (kChunk / 16)) {
        u32x4v v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads + threadIdx.x;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4v{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    __shared__ uint32_t red[kThreads / 64];
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// dst[i] = src[i] for n16 16-byte words (loads and stores non-temporal).
__global__ __launch_bounds__(kThreads) void k_copy(const u32x4v* __restrict__ src, u32x4v* __restrict__ dst,
                                                   int64_t n16) {
    for (int64_t base = (int64_t)blockIdx.x * (kChunk / 16); base < n16; base += (int64_t)gridDim.x * (kChunk / 16)) {
        u32x4v v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads + threadIdx.x;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4v{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + (int64_t)u * kThreads + threadIdx.x;
            if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

}  // namespace

extern "C" {

// Work-groups a launch uses (the sink of mxq_ceiling_read needs this many words).
int mxq_ceiling_grid(void) { return 4096; }

// Reads `bytes` (a multiple of 16; src 16-byte aligned) on the stream.  0 on success.
int mxq_ceiling_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
    hipLaunchKernelGGL(k_read, dim3(mxq_ceiling_grid()), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4v*>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Copies `bytes` (a multiple of 16; both 16-byte aligned) on the stream.  0 on success.
int mxq_ceiling_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || ((reinterpret_cast<uintptr_t>(src) |
                                                          reinterpret_cast<uintptr_t>(dst)) & 15))
        return 1;
    hipLaunchKernelGGL(k_copy, dim3(mxq_ceiling_grid()), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4v*>(src), static_cast<u32x4v*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
