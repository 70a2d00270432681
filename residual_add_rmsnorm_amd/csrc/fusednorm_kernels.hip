// Device code of libfusednorm: the fused tensor-parallel epilogue
// (sum of P partial buffers + residual + RMSNorm, optionally OCP e4m3 with a
// per-token or per-1x128-group scale) and the MiniMax QK RMSNorm, for gfx950.
//
// What is computed follows the tokenspeed triton.py page, section "AMD Triton
// All-Reduce + RMSNorm" (amd_allreduce_residual_rmsnorm_kernel), the fusion
// patterns named in the tokenspeed trtllm.py page, section "Pattern enums",
// and the vLLM minimax_rms_norm/rms_norm_tp page (_minimax_qk_var_kernel,
// _minimax_rms_apply_kernel). How it is computed is designed for CDNA4:
//
//   * one workgroup per token; the row is cut into 16-byte vectors (8 bf16)
//     and vector i belongs to lane i mod blockDim, slot i / blockDim, so every
//     wave-wide load or store covers 1 KiB of consecutive bytes;
//   * every load a lane needs for its token (P partials, residual, weight) is
//     issued before the first add: a wave keeps (P+2)*VPT 16-byte requests in
//     flight to HBM;
//   * the fp32 row stays in VGPRs between the reduction and the normalisation;
//     sums and maxima are reduced inside a wave with DPP row permutes plus two
//     cross-row lane shuffles, then across the token's waves through LDS;
//   * a 1x128 FP8 group is 16 consecutive vectors = 16 consecutive lanes of
//     one wave = one DPP row, so a group's amax needs no LDS;
//   * stores are 16-byte (bf16) and 8-byte (e4m3) vectors made with gfx950's
//     packed conversions v_cvt_pk_bf16_f32 and v_cvt_pk_fp8_f32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fusednorm_internal.h"

namespace fusednorm {
namespace {

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even), element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float (&f)[8]) {
    u32x4 r;
    r.x = pack_bf16x2(f[0], f[1]);
    r.y = pack_bf16x2(f[2], f[3]);
    r.z = pack_bf16x2(f[4], f[5]);
    r.w = pack_bf16x2(f[6], f[7]);
    return r;
}

// OCP e4m3 of four values already clamped to [-448, 448], round to nearest
// even; value k lands in byte k.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

__device__ __forceinline__ u32x2 pack_e4m3x8(const float (&r)[8]) {
    u32x2 q;
    q.x = pack_e4m3x4(clamp448(r[0]), clamp448(r[1]), clamp448(r[2]), clamp448(r[3]));
    q.y = pack_e4m3x4(clamp448(r[4]), clamp448(r[5]), clamp448(r[6]), clamp448(r[7]));
    return q;
}

// ---------------------------------------------------------------- global memory

// Read-once streams (partials, residual, qkv) and write-once outputs use
// non-temporal accesses so they do not displace the weight vector, which
// every token of the launch re-reads.
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_stream(u32x2* p, u32x2 v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// ---------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

struct Sum { __device__ float operator()(float a, float b) const { return a + b; } };
struct Max { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// Reduction over each row of 16 lanes; every lane of the row ends with the
// row's result. quad_perm [1,0,3,2] and [2,3,0,1] combine within quads,
// row_half_mirror pairs the two quads of a half-row, row_mirror the halves.
template <class Op>
__device__ __forceinline__ float row16_reduce(float v, Op op) {
    v = op(v, dpp<0xB1>(v));
    v = op(v, dpp<0x4E>(v));
    v = op(v, dpp<0x141>(v));
    v = op(v, dpp<0x140>(v));
    return v;
}

template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
    v = row16_reduce(v, op);
    v = op(v, __shfl_xor(v, 16));
    v = op(v, __shfl_xor(v, 32));
    return v;
}

// Workgroup reduction of a sum s and, when TWO, a second value m combined with
// Op2. Every thread receives the same results; waves are combined in order.
template <bool TWO, class Op2>
__device__ __forceinline__ void block_reduce(float& s, float& m, Op2 op2) {
    __shared__ float red[2][kMaxWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    s = wave_reduce(s, Sum{});
    if (TWO) m = wave_reduce(m, op2);
    if (nwaves == 1) return;
    if (lane == 0) {
        red[0][wave] = s;
        if (TWO) red[1][wave] = m;
    }
    __syncthreads();
    s = red[0][0];
    if (TWO) m = red[1][0];
    for (int w = 1; w < nwaves; ++w) {
        s += red[0][w];
        if (TWO) m = op2(m, red[1][w]);
    }
}

__device__ __forceinline__ float sumsq8(const float (&f)[8]) {
    return ((f[0] * f[0] + f[1] * f[1]) + (f[2] * f[2] + f[3] * f[3])) +
           ((f[4] * f[4] + f[5] * f[5]) + (f[6] * f[6] + f[7] * f[7]));
}

template <int N>
__device__ __forceinline__ float tree_sum(float (&v)[N]) {
#pragma unroll
    for (int width = 1; width < N; width *= 2)
#pragma unroll
        for (int s = 0; s + width < N; s += 2 * width) v[s] += v[s + width];
    return v[0];
}

// ---------------------------------------------------------------- fused epilogue

// Adds partial buffers P0 .. P0+N-1 to the fp32 accumulators, in partial
// order. All N*VPT loads are issued before the first add.
template <int N, int P0, int VPT>
__device__ __forceinline__ void add_partials(const EpilogueArgs& a, int64_t row, int tid, int nthr,
                                             const bool (&valid)[VPT], float (&x)[VPT][8]) {
    u32x4 v[N][VPT];
#pragma unroll
    for (int k = 0; k < N; ++k)
#pragma unroll
        for (int s = 0; s < VPT; ++s)
            v[k][s] = valid[s] ? load_stream(a.partials[P0 + k] + row + s * nthr + tid) : zero4();
#pragma unroll
    for (int k = 0; k < N; ++k)
#pragma unroll
        for (int s = 0; s < VPT; ++s) {
            float f[8];
            unpack8(v[k][s], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[s][e] += f[e];
        }
}

// Adds exactly n partials (1 <= n <= N) starting at partial P0.
template <int N, int P0, int VPT>
__device__ __forceinline__ void add_partials_upto(int n, const EpilogueArgs& a, int64_t row, int tid,
                                                  int nthr, const bool (&valid)[VPT],
                                                  float (&x)[VPT][8]) {
    if constexpr (N == 1) {
        add_partials<1, P0>(a, row, tid, nthr, valid, x);
    } else {
        if (n == N) add_partials<N, P0>(a, row, tid, nthr, valid, x);
        else add_partials_upto<N - 1, P0>(n, a, row, tid, nthr, valid, x);
    }
}

// Adds partials P0 .. P-1 in chunks of CH buffers; one chunk's loads are in
// flight together, so a kernel compiled for chunk CH holds CH*VPT vectors of
// loads in registers.
template <int CH, int P0, int VPT>
__device__ __forceinline__ void add_all_partials(int P, const EpilogueArgs& a, int64_t row, int tid,
                                                 int nthr, const bool (&valid)[VPT],
                                                 float (&x)[VPT][8]) {
    if constexpr (P0 < kMaxPartials) {
        if (P > P0) {
            const int n = P - P0;
            if constexpr (CH == 1) {
                add_partials<1, P0>(a, row, tid, nthr, valid, x);
            } else {
                if (n >= CH) add_partials<CH, P0>(a, row, tid, nthr, valid, x);
                else add_partials_upto<CH - 1, P0>(n, a, row, tid, nthr, valid, x);
            }
            add_all_partials<CH, P0 + CH>(P, a, row, tid, nthr, valid, x);
        }
    }
}

// Multiplier taking x*w to the e4m3 grid, 448 / max|x*w|, or 0 for an all-zero
// token or group. For maxima so small that 448/max would overflow fp32, both
// the maximum and x*w are first scaled by 2^64 (exact: a power of two).
struct QuantScale {
    float pre;   // applied to x*w before qmul
    float qmul;
};

__device__ __forceinline__ QuantScale quant_scale(float xw_max) {
    QuantScale q{1.0f, 0.0f};
    if (xw_max > 0.0f) {
        float m = xw_max;
        if (m < 0x1p-100f) {
            q.pre = 0x1p64f;
            m *= q.pre;
        }
        q.qmul = 448.0f / m;
    }
    return q;
}

template <int VPT, int MODE, int CH>
__global__ void __launch_bounds__(max_threads_for(VPT)) fused_epilogue_kernel(EpilogueArgs a) {
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int64_t t = blockIdx.x;
    const int64_t row = t * a.nvec;  // start of the token's row, in 16-byte vectors

    bool valid[VPT];
    u32x4 res[VPT], wv[VPT];
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        const int i = s * nthr + tid;
        valid[s] = i < a.nvec;
        res[s] = valid[s] ? load_stream(a.residual + row + i) : zero4();
        wv[s] = valid[s] ? a.weight[i] : zero4();
    }

    // x = (((0 + p_0) + p_1) + ... + p_{P-1}) + residual, in fp32.
    float x[VPT][8];
#pragma unroll
    for (int s = 0; s < VPT; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[s][e] = 0.0f;
    add_all_partials<CH, 0>(a.P, a, row, tid, nthr, valid, x);
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        float r[8];
        unpack8(res[s], r);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[s][e] += r[e];
    }

    // Token statistics: sum of x^2 and, for per-token FP8, max |x*w|.
    float part[VPT];
    float xw_max = 0.0f;
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        part[s] = sumsq8(x[s]);
        if (MODE == kModeQuantToken) {
            float w[8];
            unpack8(wv[s], w);
#pragma unroll
            for (int e = 0; e < 8; ++e) xw_max = fmaxf(xw_max, fabsf(x[s][e] * w[e]));
        }
    }
    float ss = tree_sum(part);
    block_reduce<MODE == kModeQuantToken>(ss, xw_max, Max{});
    const float inv = rsqrtf(ss / a.h + a.eps);

    // y / (amax_y / 448) = 448 * x*w / max|x*w|: the rsqrt cancels, so the
    // codes come straight from x*w.
    QuantScale token_q{1.0f, 0.0f};
    if (MODE == kModeQuantToken) {
        token_q = quant_scale(xw_max);
        if (tid == 0) a.scale_out[t] = (xw_max * inv) / 448.0f;
    }

#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        const int i = s * nthr + tid;
        float w[8], xw[8];
        unpack8(wv[s], w);
#pragma unroll
        for (int e = 0; e < 8; ++e) xw[e] = x[s][e] * w[e];

        QuantScale q = token_q;
        float group_max = 0.0f;
        if (MODE == kModeQuantBlock) {
            // every lane takes part: the 16 lanes of this DPP row hold one group
#pragma unroll
            for (int e = 0; e < 8; ++e) group_max = fmaxf(group_max, fabsf(xw[e]));
            group_max = row16_reduce(group_max, Max{});
            q = quant_scale(group_max);
        }
        if (valid[s]) {
            store_stream(a.residual_out + row + i, pack_bf16x8(x[s]));
            if (a.norm_out) {
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (x[s][e] * inv) * w[e];
                store_stream(a.norm_out + row + i, pack_bf16x8(y));
            }
            if (MODE != kModeNorm) {
                float r[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = (xw[e] * q.pre) * q.qmul;
                u32x2 codes = pack_e4m3x8(r);
                if (q.qmul == 0.0f) codes = u32x2{0u, 0u};  // all-zero token or group: +0 codes
                store_stream(a.quant_out + row + i, codes);
                if (MODE == kModeQuantBlock && (tid & 15) == 0)
                    a.scale_out[t * a.groups + i / 16] = (group_max * inv) / 448.0f;
            }
        }
    }
}

// ---------------------------------------------------------------- QK RMSNorm

template <int VPT, int MODE>
__global__ void __launch_bounds__(max_threads_for(VPT)) qk_norm_kernel(QkArgs a) {
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int64_t t = blockIdx.x;
    const int nv = a.nq + a.nk;
    // q then k lie back to back at the start of the row: one span of nv vectors.
    const u32x4* src = reinterpret_cast<const u32x4*>(a.qkv + t * a.row_stride);

    bool valid[VPT];
    u32x4 raw[VPT];
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        const int i = s * nthr + tid;
        valid[s] = i < nv;
        raw[s] = valid[s] ? load_stream(src + i) : zero4();
    }

    float var_q, var_k;
    if (MODE == kQkSupplied) {
        const float2 v = a.var_in[t];
        var_q = v.x;
        var_k = v.y;
    } else {
        float sq[VPT], sk[VPT];
#pragma unroll
        for (int s = 0; s < VPT; ++s) {
            const int i = s * nthr + tid;
            float f[8];
            unpack8(raw[s], f);
            const float v = sumsq8(f);
            sq[s] = i < a.nq ? v : 0.0f;
            sk[s] = i < a.nq ? 0.0f : v;
        }
        float tq = tree_sum(sq), tk = tree_sum(sk);
        block_reduce<true>(tq, tk, Sum{});
        var_q = tq / a.q_size;
        var_k = tk / a.kv_size;
        if (MODE == kQkStats) {
            if (tid == 0) a.var_out[t] = make_float2(var_q, var_k);
            return;
        }
    }
    const float inv_q = rsqrtf(var_q / a.tp_world + a.eps);
    const float inv_k = rsqrtf(var_k / a.tp_world + a.eps);

#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        const int i = s * nthr + tid;
        if (valid[s]) {
            const bool is_q = i < a.nq;
            const u32x4 wraw = is_q ? a.wq[i] : a.wk[i - a.nq];
            const float inv = is_q ? inv_q : inv_k;
            float f[8], w[8], y[8];
            unpack8(raw[s], f);
            unpack8(wraw, w);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (f[e] * inv) * w[e];
            u32x4* dst = is_q ? a.q_out + t * a.nq + i : a.k_out + t * a.nk + (i - a.nq);
            store_stream(dst, pack_bf16x8(y));
        }
    }
}

// ---------------------------------------------------------------- e4m3 encode

__global__ void __launch_bounds__(256) e4m3_encode_kernel(const float* in, uint8_t* out, int64_t n) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of 8 values
    const int64_t base = g * 8;
    if (base >= n) return;
    if (base + 8 <= n) {
        const float4 lo = reinterpret_cast<const float4*>(in)[2 * g];
        const float4 hi = reinterpret_cast<const float4*>(in)[2 * g + 1];
        const float r[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        reinterpret_cast<u32x2*>(out)[g] = pack_e4m3x8(r);
        return;
    }
    for (int64_t j = base; j < n; ++j)
        out[j] = (uint8_t)(pack_e4m3x4(clamp448(in[j]), 0.0f, 0.0f, 0.0f) & 0xFFu);
}

// ---------------------------------------------------------------- dispatch

template <int VPT, int CH>
void launch_epilogue_ch(const EpilogueArgs& a, EpilogueMode mode, dim3 grid, dim3 block,
                        hipStream_t stream) {
    switch (mode) {
        case kModeNorm:
            fused_epilogue_kernel<VPT, kModeNorm, CH><<<grid, block, 0, stream>>>(a);
            break;
        case kModeQuantToken:
            fused_epilogue_kernel<VPT, kModeQuantToken, CH><<<grid, block, 0, stream>>>(a);
            break;
        default:
            fused_epilogue_kernel<VPT, kModeQuantBlock, CH><<<grid, block, 0, stream>>>(a);
            break;
    }
}

template <int VPT>
hipError_t launch_epilogue_vpt(const EpilogueArgs& a, EpilogueMode mode, int64_t T, int threads,
                               hipStream_t stream) {
    const dim3 grid((unsigned)T), block((unsigned)threads);
    // chunk of partial buffers loaded together: 2, 4 or 8
    if (a.P <= 2) launch_epilogue_ch<VPT, 2>(a, mode, grid, block, stream);
    else if (a.P <= 4) launch_epilogue_ch<VPT, 4>(a, mode, grid, block, stream);
    else launch_epilogue_ch<VPT, 8>(a, mode, grid, block, stream);
    return hipGetLastError();
}

template <int VPT>
hipError_t launch_qk_vpt(const QkArgs& a, QkMode mode, int64_t T, int threads, hipStream_t stream) {
    const dim3 grid((unsigned)T), block((unsigned)threads);
    switch (mode) {
        case kQkLocal: qk_norm_kernel<VPT, kQkLocal><<<grid, block, 0, stream>>>(a); break;
        case kQkSupplied: qk_norm_kernel<VPT, kQkSupplied><<<grid, block, 0, stream>>>(a); break;
        default: qk_norm_kernel<VPT, kQkStats><<<grid, block, 0, stream>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace

LaunchShape pick_shape(int nvec) {
    // Fewest idle lanes first, then the workgroup size nearest 256 threads.
    LaunchShape best{1, 64};
    long best_waste = -1, best_dist = 0;
    for (int vpt = 1; vpt <= kMaxVpt; ++vpt) {
        const int lanes = (nvec + vpt - 1) / vpt;
        const int threads = ((lanes + kWave - 1) / kWave) * kWave;
        if (threads > max_threads_for(vpt)) continue;
        const long waste = (long)threads * vpt - nvec;
        const long dist = threads > 256 ? threads - 256 : 256 - threads;
        if (best_waste < 0 || waste < best_waste || (waste == best_waste && dist < best_dist)) {
            best = LaunchShape{vpt, threads};
            best_waste = waste;
            best_dist = dist;
        }
    }
    return best;
}

hipError_t launch_epilogue(const EpilogueArgs& a, EpilogueMode mode, int64_t T, LaunchShape s,
                           hipStream_t stream) {
    switch (s.vpt) {
        case 1: return launch_epilogue_vpt<1>(a, mode, T, s.threads, stream);
        case 2: return launch_epilogue_vpt<2>(a, mode, T, s.threads, stream);
        case 3: return launch_epilogue_vpt<3>(a, mode, T, s.threads, stream);
        case 4: return launch_epilogue_vpt<4>(a, mode, T, s.threads, stream);
        case 5: return launch_epilogue_vpt<5>(a, mode, T, s.threads, stream);
        case 6: return launch_epilogue_vpt<6>(a, mode, T, s.threads, stream);
        case 7: return launch_epilogue_vpt<7>(a, mode, T, s.threads, stream);
        case 8: return launch_epilogue_vpt<8>(a, mode, T, s.threads, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_qk(const QkArgs& a, QkMode mode, int64_t T, LaunchShape s, hipStream_t stream) {
    switch (s.vpt) {
        case 1: return launch_qk_vpt<1>(a, mode, T, s.threads, stream);
        case 2: return launch_qk_vpt<2>(a, mode, T, s.threads, stream);
        case 3: return launch_qk_vpt<3>(a, mode, T, s.threads, stream);
        case 4: return launch_qk_vpt<4>(a, mode, T, s.threads, stream);
        case 5: return launch_qk_vpt<5>(a, mode, T, s.threads, stream);
        case 6: return launch_qk_vpt<6>(a, mode, T, s.threads, stream);
        case 7: return launch_qk_vpt<7>(a, mode, T, s.threads, stream);
        case 8: return launch_qk_vpt<8>(a, mode, T, s.threads, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
    const int64_t groups = (n + 7) / 8;
    const int64_t blocks = (groups + 255) / 256;
    e4m3_encode_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(in, out, n);
    return hipGetLastError();
}

}  // namespace fusednorm
