// Streaming ceilings for the measurement harness: how fast this GPU reads HBM,
// copies it, and moves a given mix of read and write streams, with plain
// 16-byte vector accesses and nothing else. They put a measured ceiling next
// to the published 8 TB/s when the epilogues' achieved bandwidth is reported;
// no epilogue uses them.
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


// ---------------------------------------------------------------- mixed streams
// The bytes of one epilogue launch without its arithmetic: per row, n_src
// source rows in and n_dst destination rows out. One workgroup of 256 threads
// per row (grid-stride past 2^20 rows); lane l owns the row's 16-byte vectors
// l, l + 256, ... (VPT of them), so every wave access is 1 KiB of consecutive
// bytes; two source rows are in flight at a time. The row's destination
// stores are issued together after a workgroup barrier, each lane storing only
// within each destination row. All accesses go through buffer resources sized
// to the row, so lanes past a row's end read zeros.
constexpr int kMixMaxSrc = 16;
constexpr int kMixMaxDst = 4;
constexpr int kMixThreads = 256;
constexpr int kMixMaxVpt = 8;           // rows of up to 32 KiB
constexpr int64_t kMixMaxGrid = 1 << 20;

struct MixArgs {
    const u32x4* src[kMixMaxSrc];
    u32x4* dst[kMixMaxDst];
    uint32_t dst_bytes[kMixMaxDst];
    int64_t src_stride;                 // in 16-byte vectors
    uint32_t src_bytes;
    int n_src;
    int n_dst;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mix_row(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int VPT>
__global__ void __launch_bounds__(kMixThreads) stream_mix_kernel(MixArgs a, int64_t rows) {
    uint32_t off[VPT];
#pragma unroll
    for (int s = 0; s < VPT; ++s) off[s] = (uint32_t)(s * kMixThreads + threadIdx.x) * 16u;
    auto issue = [&](int k, int64_t r, u32x4 (&v)[VPT]) {
        const __amdgpu_buffer_rsrc_t rs = mix_row(a.src[k] + r * a.src_stride, a.src_bytes);
#pragma unroll
        for (int s = 0; s < VPT; ++s) v[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, off[s], 0, 2);
    };
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        u32x4 ring[2][VPT];
        u32x4 acc[VPT];
#pragma unroll
        for (int s = 0; s < VPT; ++s) acc[s] = u32x4{0u, 0u, 0u, 0u};
        issue(0, r, ring[0]);
        if (a.n_src > 1) issue(1, r, ring[1]);
        for (int base = 0; base < a.n_src; base += 2) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int k = base + j;
                if (k < a.n_src) {
#pragma unroll
                    for (int s = 0; s < VPT; ++s) acc[s] ^= ring[j][s];
                    if (k + 2 < a.n_src) issue(k + 2, r, ring[j]);
                }
            }
        }
        __syncthreads();
        for (int d = 0; d < a.n_dst; ++d) {
            const __amdgpu_buffer_rsrc_t rs =
                mix_row(a.dst[d] + r * (a.dst_bytes[d] / 16u), a.dst_bytes[d]);
#pragma unroll
            for (int s = 0; s < VPT; ++s)
                if (off[s] < a.dst_bytes[d])  // lanes past the destination row issue no store
                    __builtin_amdgcn_raw_buffer_store_b128(acc[s], rs, off[s], 0, 2);
        }
    }
}

template <int VPT>
hipError_t launch_mix(const MixArgs& a, int64_t rows, hipStream_t stream) {
    const int64_t grid = rows < kMixMaxGrid ? rows : kMixMaxGrid;
    stream_mix_kernel<VPT><<<dim3((unsigned)grid), dim3(kMixThreads), 0, stream>>>(a, rows);
    return hipGetLastError();
}

struct Range {
    uintptr_t lo, hi;
};
bool overlap(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi; }

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


int fusednorm_stream_mix(const void* const* src, int n_src, int64_t src_row_bytes,
                         int64_t src_stride, void* const* dst, const int64_t* dst_row_bytes,
                         int n_dst, int64_t rows, void* stream) {
    if (!src || !dst || !dst_row_bytes || n_src < 1 || n_src > kMixMaxSrc || n_dst < 1 ||
        n_dst > kMixMaxDst || rows < 0 || src_row_bytes <= 0 || src_stride <= 0)
        return FUSEDNORM_ERR_INVALID_ARGUMENT;
    for (int k = 0; k < n_src; ++k)
        if (!src[k]) return FUSEDNORM_ERR_INVALID_ARGUMENT;
    for (int k = 0; k < n_dst; ++k)
        if (!dst[k] || dst_row_bytes[k] <= 0) return FUSEDNORM_ERR_INVALID_ARGUMENT;
    if (src_row_bytes % 16 || src_row_bytes > (int64_t)kMixMaxVpt * kMixThreads * 16 ||
        src_stride % 16 || src_stride < src_row_bytes || rows > 0x7FFFFFFF)
        return FUSEDNORM_ERR_UNSUPPORTED;
    MixArgs a{};
    Range in[kMixMaxSrc], out[kMixMaxDst];
    for (int k = 0; k < n_src; ++k) {
        if (reinterpret_cast<uintptr_t>(src[k]) % 16) return FUSEDNORM_ERR_UNSUPPORTED;
        a.src[k] = static_cast<const u32x4*>(src[k]);
        const uintptr_t lo = reinterpret_cast<uintptr_t>(src[k]);
        in[k] = Range{lo, lo + (uintptr_t)(rows > 0 ? (rows - 1) * src_stride + src_row_bytes : 0)};
    }
    for (int k = 0; k < n_dst; ++k) {
        if (dst_row_bytes[k] % 16 || dst_row_bytes[k] > src_row_bytes ||
            reinterpret_cast<uintptr_t>(dst[k]) % 16)
            return FUSEDNORM_ERR_UNSUPPORTED;
        a.dst[k] = static_cast<u32x4*>(dst[k]);
        a.dst_bytes[k] = (uint32_t)dst_row_bytes[k];
        const uintptr_t lo = reinterpret_cast<uintptr_t>(dst[k]);
        out[k] = Range{lo, lo + (uintptr_t)(rows * dst_row_bytes[k])};
        for (int j = 0; j < n_src; ++j)
            if (overlap(out[k], in[j])) return FUSEDNORM_ERR_UNSUPPORTED;
        for (int j = 0; j < k; ++j)
            if (overlap(out[k], out[j])) return FUSEDNORM_ERR_UNSUPPORTED;
    }
    if (rows == 0) return FUSEDNORM_OK;
    a.src_stride = src_stride / 16;
    a.src_bytes = (uint32_t)src_row_bytes;
    a.n_src = n_src;
    a.n_dst = n_dst;
    (void)hipGetLastError();
    const int vpt = (int)((src_row_bytes / 16 + kMixThreads - 1) / kMixThreads);
    hipError_t e;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (vpt) {
        case 1: e = launch_mix<1>(a, rows, s); break;
        case 2: e = launch_mix<2>(a, rows, s); break;
        case 3: e = launch_mix<3>(a, rows, s); break;
        case 4: e = launch_mix<4>(a, rows, s); break;
        case 5: e = launch_mix<5>(a, rows, s); break;
        case 6: e = launch_mix<6>(a, rows, s); break;
        case 7: e = launch_mix<7>(a, rows, s); break;
        default: e = launch_mix<8>(a, rows, s); break;
    }
    return e == hipSuccess ? FUSEDNORM_OK : FUSEDNORM_ERR_HIP;
}

}  // extern "C"
