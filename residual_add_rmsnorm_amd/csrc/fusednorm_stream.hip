// Streaming ceilings for the measurement harness: how fast this GPU reads HBM,
// and copies it, with plain 16-byte vector accesses and nothing else. They put
// a measured ceiling next to the published 8 TB/s when the epilogues' achieved
// bandwidth is reported; no epilogue uses them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fusednorm.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPerThread = 4;                               // vectors per thread
constexpr int64_t kChunk = (int64_t)kThreads * kPerThread;  // vectors per workgroup (16 KiB)

// Workgroup b reads vectors [b * kChunk, (b + 1) * kChunk): each thread issues
// its kPerThread loads (lane-contiguous, so every wave access is 1 KiB of
// consecutive bytes) before combining them. The combined value is stored only
// if it equals a constant no input of the harness produces; the branch keeps
// the loads from being removed.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const u32x4* __restrict__ src,
                                                               uint32_t* __restrict__ sink) {
    const int64_t base = (int64_t)blockIdx.x * kChunk + threadIdx.x;
    u32x4 v[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) v[k] = __builtin_nontemporal_load(&src[base + k * kThreads]);
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ void __launch_bounds__(kThreads) stream_copy_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst) {
    const int64_t base = (int64_t)blockIdx.x * kChunk + threadIdx.x;
    u32x4 v[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) v[k] = __builtin_nontemporal_load(&src[base + k * kThreads]);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) __builtin_nontemporal_store(v[k], &dst[base + k * kThreads]);
}

int check_stream_args(const void* a, const void* b, int64_t bytes) {
    if (!a || !b || bytes <= 0) return FUSEDNORM_ERR_INVALID_ARGUMENT;
    if (bytes % (kChunk * 16) != 0 || bytes / (kChunk * 16) > 0x7FFFFFFF)
        return FUSEDNORM_ERR_UNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(b) % 16)
        return FUSEDNORM_ERR_UNSUPPORTED;
    return FUSEDNORM_OK;
}

int launch_status() {
    return hipGetLastError() == hipSuccess ? FUSEDNORM_OK : FUSEDNORM_ERR_HIP;
}

}  // namespace

extern "C" {

int fusednorm_stream_read(const void* src, int64_t bytes, void* sink, void* stream) {
    if (int s = check_stream_args(src, sink, bytes)) return s;
    (void)hipGetLastError();
    const unsigned grid = (unsigned)(bytes / (kChunk * 16));
    stream_read_kernel<<<grid, kThreads, 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(src),
                                                                   static_cast<uint32_t*>(sink));
    return launch_status();
}

int fusednorm_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (int s = check_stream_args(src, dst, bytes)) return s;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes) return FUSEDNORM_ERR_UNSUPPORTED;
    (void)hipGetLastError();
    const unsigned grid = (unsigned)(bytes / (kChunk * 16));
    stream_copy_kernel<<<grid, kThreads, 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(src),
                                                                   static_cast<u32x4*>(dst));
    return launch_status();
}

}  // extern "C"
