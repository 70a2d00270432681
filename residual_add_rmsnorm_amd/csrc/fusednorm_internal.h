// Internal declarations shared by the kernels and the C-ABI layer of
// libfusednorm. Not installed; the public interface is include/fusednorm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fusednorm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 8 bf16 = 16 bytes
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // 8 e4m3 codes = 8 bytes

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;   // 1024 threads per workgroup
constexpr int kMaxPartials = 16;
constexpr int kMaxVpt = 8;      // 16-byte vectors per lane per token
constexpr int kMaxGroups = 128;  // 1x128 FP8 groups in the widest row (16384)
// The fused epilogue keeps CH*VPT prefetched 16-byte vectors per lane (CH =
// partial buffers loaded together); beyond this the kernel would spill.
constexpr int kMaxLoadsPerLane = 16;

// Largest workgroup each variant is compiled for. More vectors per lane (and,
// for the fused epilogue, more partials loaded together) hold more loads in
// flight and need more VGPRs: a 1024-thread workgroup leaves 128 VGPRs per
// lane, 512 threads 256, 256 threads 512.
constexpr __host__ __device__ int max_threads_for(int vpt) {
    return vpt <= 2 ? 1024 : (vpt <= 4 ? 512 : 256);
}
constexpr __host__ __device__ int max_threads_for(int vpt, int ch) {
    return (vpt <= 2 && vpt * ch <= 8) ? 1024 : (vpt <= 4 ? 512 : 256);
}

enum EpilogueMode { kModeNorm = 0, kModeQuantToken = 1, kModeQuantBlock = 2, kModeQuantStatic = 3 };
// kQkQuant: local means, plus 1x128 e4m3 of the normalised segment 1.
enum QkMode { kQkLocal = 0, kQkSupplied = 1, kQkStats = 2, kQkQuant = 3 };

struct EpilogueArgs {
    const u32x4* partials[kMaxPartials];  // P row-major bf16 [T, H]
    const u32x4* residual;                // bf16 [T, H]
    const u32x4* weight;                  // bf16 [H]
    u32x4* residual_out;                  // bf16 [T, H]
    u32x4* norm_out;                      // bf16 [T, H] or null
    u32x2* quant_out;                     // e4m3 [T, H] (FP8 modes)
    float* scale_out;                     // fp32 [T] or [T, H/128] (dynamic FP8 modes)
    const float* static_scale;            // fp32 [1] (static FP8 mode)
    int P;
    int nvec;                             // H / 8
    uint32_t row_bytes;                   // H * 2
    int groups;                           // H / 128 (block FP8)
    float h;                              // H as fp32 (exact for H <= 2^24)
    float eps;
};

// The QK norm, its one-segment form (sharded-hidden RMSNorm) and the MLA
// all-gather epilogue: each row holds segment 1 (q, nq vectors) then, when
// segments == 2, segment 2 (k, nk vectors); anything after them is not read.
struct QkArgs {
    const uint16_t* qkv;                  // bf16 rows
    int64_t row_stride;                   // elements
    const u32x4* wq;                      // bf16 [q_size]
    const u32x4* wk;                      // bf16 [kv_size] (segments == 2)
    u32x4* q_out;                         // bf16 [T, q_size] (may be null in kQkQuant)
    u32x4* k_out;                         // bf16 [T, kv_size] (segments == 2)
    u32x2* quant_out;                     // e4m3 [T, q_size] (kQkQuant)
    float* scale_out;                     // fp32 [T, q_size / 128] (kQkQuant)
    const float* var_in;                  // fp32 [T, segments] (supplied mode)
    float* var_out;                       // fp32 [T, segments] (statistics mode)
    int segments;                         // 1 or 2
    int nq;                               // q_size / 8
    int nk;                               // kv_size / 8 (0 when segments == 1)
    float q_size;
    float kv_size;                        // 1 when segments == 1 (unused)
    int groups;                           // q_size / 128 (kQkQuant)
    float tp_world;
    float eps;                            // segment 1
    float eps_k;                          // segment 2
};

struct LaunchShape {
    int vpt;      // 16-byte vectors per lane
    int threads;  // workgroup size, a multiple of 64
    int ch;       // fused epilogue: partial buffers loaded together (2 or 4)
    int per_cu;   // 0: one workgroup per token; k > 0: at most k resident
                  // workgroups per CU, each looping over tokens
};

// Launch shape of the fused epilogue for T rows of nvec 16-byte vectors and P
// partial buffers, and of the QK norm for T rows of nvec vectors, on a device
// with `cus` compute units. The shape decides only speed; every shape
// computes the same result. A shape with vpt == 0 means none fits.
LaunchShape pick_epilogue_shape(int nvec, int P, int64_t T, int cus);
LaunchShape pick_qk_shape(int nvec, int64_t T, int cus);

// Compute units of the current device (cached per device).
hipError_t device_cus(int* cus);

hipError_t launch_epilogue(const EpilogueArgs& a, EpilogueMode mode, int64_t T, LaunchShape s,
                           hipStream_t stream);
hipError_t launch_qk(const QkArgs& a, QkMode mode, int64_t T, LaunchShape s, hipStream_t stream);
hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

}  // namespace fusednorm
