// Device code of libfusednorm, for gfx950: the fused tensor-parallel epilogue
// (sum of P partial buffers + residual + RMSNorm, optionally OCP e4m3 with a
// per-token, per-1x128-group or static scale; also the reduce-scatter form
// with an extra addend) and the RMSNorms over row segments: the MiniMax QK
// norm, its one-segment (hidden-sharded) form and the MLA all-gather epilogue.
//
// What is computed follows the tokenspeed triton.py page, section "AMD Triton
// All-Reduce + RMSNorm" (amd_allreduce_residual_rmsnorm_kernel), the fusion
// patterns named in the tokenspeed trtllm.py page, sections "Pattern enums",
// "AllReduce fusion", "AllGather fusion" and "ReduceScatter fusion", and the
// vLLM minimax_rms_norm/rms_norm_tp page (_minimax_qk_var_kernel,
// _minimax_rms_apply_kernel). How it is computed is designed for CDNA4:
//
//   * the grid: one workgroup per token, the hardware dispatcher keeping every
//     CU filled as workgroups finish; for wide rows with few tokens per CU,
//     two resident workgroups per CU, each looping over tokens and issuing the
//     next token's loads as soon as the current token's sum is formed;
//   * a token's row is cut into 16-byte vectors (8 bf16); vector i belongs to
//     lane i mod blockDim, slot i / blockDim, so every wave-wide access covers
//     1 KiB of consecutive bytes, read and written through per-row buffer
//     resources with the non-temporal policy (lanes past the row end read
//     zeros and issue no stores; the hardware range check of the resources
//     bounds every access to its row);
//   * the fp32 row stays in VGPRs between the reduction and the normalisation;
//     sums and maxima are reduced inside a wave with DPP row permutes plus two
//     cross-row lane shuffles, then across the token's waves through LDS;
//   * a 1x128 FP8 group is 16 consecutive vectors = 16 consecutive lanes of
//     one wave = one DPP row, so a group's amax needs no LDS; in the fused
//     epilogue the amaxes go to LDS before the token's reduction barrier and
//     the token's scale row is stored after it by one instruction, one lane
//     per group (16 bytes from each wave at different times, into cache lines
//     shared with neighbouring tokens' rows written from other XCDs, measured
//     1.3% slower on the 16384 x 7168 launch);
//   * stores are 16-byte (bf16) and 8-byte (e4m3) vectors made with gfx950's
//     packed conversions v_cvt_pk_bf16_f32 and v_cvt_pk_fp8_f32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

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

// Token rows are read and written through buffer resources: a resource covers
// one row of one stream (wave-uniform, held in SGPRs) and each lane adds its
// byte offset, the same offset for every stream of the row. The hardware range
// check of the resource makes a lane past the end of the row read zeros and
// drop its stores, so a row access can never touch memory outside that row.
// Read-once inputs and write-once outputs carry the non-temporal policy bit so
// they do not displace the weights, which every token re-reads.
constexpr int kBufferFormat = 0x00020000;  // buffer descriptor word 3 for gfx9-family raw access
constexpr int kPolicyStream = 2;           // cache policy: nt (sc0 = bit 0, nt = bit 1, sc1 = bit 4)

struct Row {
    __amdgpu_buffer_rsrc_t rsrc;
};

__device__ __forceinline__ Row make_row(const void* base, uint32_t bytes) {
    return Row{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                                 kBufferFormat)};
}
__device__ __forceinline__ u32x4 load16(Row r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r.rsrc, off, 0, kPolicyStream);
}
__device__ __forceinline__ void store16(Row r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r.rsrc, off, 0, kPolicyStream);
}
__device__ __forceinline__ void store8(Row r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r.rsrc, off, 0, kPolicyStream);
}

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
// A workgroup that loops over tokens alternates between two LDS buffers
// (buf = token parity): a wave can only come back to a buffer after the next
// token's barrier, which every wave reaches after reading this one.
template <bool TWO, class Op2>
__device__ __forceinline__ void block_reduce(float& s, float& m, Op2 op2, int buf) {
    __shared__ float red[2][2][kMaxWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    s = wave_reduce(s, Sum{});
    if (TWO) m = wave_reduce(m, op2);
    if (nwaves == 1) return;
    if (lane == 0) {
        red[buf][0][wave] = s;
        if (TWO) red[buf][1][wave] = m;
    }
    __syncthreads();
    s = red[buf][0][0];
    if (TWO) m = red[buf][1][0];
    for (int w = 1; w < nwaves; ++w) {
        s += red[buf][0][w];
        if (TWO) m = op2(m, red[buf][1][w]);
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
__device__ __forceinline__ void add_partials(const EpilogueArgs& a, int64_t row,
                                             const uint32_t (&off)[VPT], float (&x)[VPT][8]) {
    u32x4 v[N][VPT];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const Row r = make_row(a.partials[P0 + k] + row, a.row_bytes);
#pragma unroll
        for (int s = 0; s < VPT; ++s) v[k][s] = load16(r, off[s]);
    }
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
__device__ __forceinline__ void add_partials_upto(int n, const EpilogueArgs& a, int64_t row,
                                                  const uint32_t (&off)[VPT], float (&x)[VPT][8]) {
    if constexpr (N == 1) {
        add_partials<1, P0>(a, row, off, x);
    } else {
        if (n == N) add_partials<N, P0>(a, row, off, x);
        else add_partials_upto<N - 1, P0>(n, a, row, off, x);
    }
}

// Adds partials P0 .. P-1 in chunks of CH buffers; one chunk's loads are in
// flight together, so a kernel compiled for chunk CH holds CH*VPT vectors of
// loads in registers.
template <int CH, int P0, int VPT>
__device__ __forceinline__ void add_all_partials(int P, const EpilogueArgs& a, int64_t row,
                                                 const uint32_t (&off)[VPT], float (&x)[VPT][8]) {
    if constexpr (P0 < kMaxPartials) {
        if (P > P0) {
            const int n = P - P0;
            if constexpr (CH == 1) {
                add_partials<1, P0>(a, row, off, x);
            } else {
                if (n >= CH) add_partials<CH, P0>(a, row, off, x);
                else add_partials_upto<CH - 1, P0>(n, a, row, off, x);
            }
            add_all_partials<CH, P0 + CH>(P, a, row, off, x);
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

// The loads of one token that are issued ahead of its arithmetic: the first
// chunk of up to CH partial buffers and the residual.
template <int VPT, int CH>
struct TokenLoads {
    u32x4 part[CH][VPT];
    u32x4 res[VPT];
};

template <int VPT, int CH>
__device__ __forceinline__ void issue_token_loads(const EpilogueArgs& a, int n0, int64_t row,
                                                  const uint32_t (&off)[VPT],
                                                  TokenLoads<VPT, CH>& L) {
#pragma unroll
    for (int k = 0; k < CH; ++k)
        if (k < n0) {
            const Row r = make_row(a.partials[k] + row, a.row_bytes);
#pragma unroll
            for (int s = 0; s < VPT; ++s) L.part[k][s] = load16(r, off[s]);
        }
    const Row r = make_row(a.residual + row, a.row_bytes);
#pragma unroll
    for (int s = 0; s < VPT; ++s) L.res[s] = load16(r, off[s]);
}

// x = (((0 + p_0) + p_1) + ... + p_{P-1}) + residual, in fp32: the first chunk
// from the loads already in flight, any further partials (P > CH) loaded here
// two at a time, which keeps their registers off the prefetch's budget.
template <int VPT, int CH>
__device__ __forceinline__ void sum_token(const EpilogueArgs& a, int n0, int64_t row,
                                          const uint32_t (&off)[VPT],
                                          const TokenLoads<VPT, CH>& L, float (&x)[VPT][8]) {
#pragma unroll
    for (int s = 0; s < VPT; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[s][e] = 0.0f;
#pragma unroll
    for (int k = 0; k < CH; ++k)
        if (k < n0) {
#pragma unroll
            for (int s = 0; s < VPT; ++s) {
                float f[8];
                unpack8(L.part[k][s], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[s][e] += f[e];
            }
        }
    add_all_partials<2, CH>(a.P, a, row, off, x);
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        float r[8];
        unpack8(L.res[s], r);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[s][e] += r[e];
    }
}

// The fused epilogue. Workgroup b handles tokens b, b + gridDim.x, ... The
// first chunk of partial buffers and the residual are loaded together, any
// further partials two buffers at a time; when the grid is smaller than T, the
// next token's first loads are issued as soon as the current token's sum is
// formed, so they are in flight while the current token is reduced,
// normalised and stored.
template <int VPT, int MODE, int CH>
__global__ void __launch_bounds__(max_threads_for(VPT, CH))
fused_epilogue_kernel(EpilogueArgs a, int64_t T) {
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int n0 = a.P < CH ? a.P : CH;

    bool valid[VPT];
    uint32_t off[VPT];  // byte offset of the lane's vector in slot s, within a bf16 row
    u32x4 wv[VPT];      // the weight: loaded once, used for every token of the workgroup
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        const int i = s * nthr + tid;
        valid[s] = i < a.nvec;
        off[s] = (uint32_t)i * 16u;
        wv[s] = valid[s] ? a.weight[i] : zero4();
    }

    // static FP8: one dequantisation scale s for the tensor; codes from y * (1/s)
    const float static_rcp = MODE == kModeQuantStatic ? 1.0f / *a.static_scale : 0.0f;
    // block FP8: each group's max |x*w|, published by the reduction's barrier
    // so that the token's scale row is stored by one instruction (two buffers:
    // a token's maxima are written before its barrier, read after it)
    __shared__ float row_gmax[2][MODE == kModeQuantBlock ? kMaxGroups : 1];

    int64_t t = blockIdx.x;  // the host launches at most T workgroups
    TokenLoads<VPT, CH> L;
    issue_token_loads(a, n0, t * a.nvec, off, L);
    for (int parity = 0;; parity ^= 1) {
        const int64_t row = t * a.nvec;  // start of the token's row, in 16-byte vectors
        float x[VPT][8];
        sum_token(a, n0, row, off, L, x);
        const int64_t t_next = t + gridDim.x;
        const bool more = t_next < T;
        if (more) issue_token_loads(a, n0, t_next * a.nvec, off, L);

        // Token statistics: sum of x^2 and, for per-token FP8, max |x*w|; for
        // block FP8 the max |x*w| of each 1x128 group (the 16 lanes of one DPP
        // row in one slot; every lane takes part, lanes past the row hold 0).
        float part[VPT];
        float xw_max = 0.0f;
        float group_max[VPT];
#pragma unroll
        for (int s = 0; s < VPT; ++s) {
            part[s] = sumsq8(x[s]);
            if (MODE == kModeQuantToken || MODE == kModeQuantBlock) {
                float w[8];
                unpack8(wv[s], w);
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[s][e] * w[e]));
                if (MODE == kModeQuantToken) xw_max = fmaxf(xw_max, m);
                if (MODE == kModeQuantBlock) {
                    group_max[s] = row16_reduce(m, Max{});
                    if (valid[s] && (tid & 15) == 0) row_gmax[parity][(s * nthr + tid) / 16] = group_max[s];
                }
            }
        }
        float ss = tree_sum(part);
        block_reduce<MODE == kModeQuantToken>(ss, xw_max, Max{}, parity);
        const float inv = rsqrtf(ss / a.h + a.eps);
        // One contiguous store of the token's scale row. Written a few bytes
        // per wave instead, pieces of a row whose cache lines it shares with
        // neighbouring tokens' rows (written from other XCDs) cost time at the
        // memory side. The reduction above crosses a barrier only when the
        // workgroup has several waves; a one-wave workgroup takes one here.
        if (MODE == kModeQuantBlock) {
            if (nthr == kWave) __syncthreads();
            if (tid < a.groups) a.scale_out[t * a.groups + tid] = (row_gmax[parity][tid] * inv) / 448.0f;
        }

        // y / (amax_y / 448) = 448 * x*w / max|x*w|: the rsqrt cancels, so the
        // codes come straight from x*w.
        QuantScale token_q{1.0f, 0.0f};
        if (MODE == kModeQuantToken) {
            token_q = quant_scale(xw_max);
            if (tid == 0) a.scale_out[t] = (xw_max * inv) / 448.0f;
        }

        const Row out_res = make_row(a.residual_out + row, a.row_bytes);
        const Row out_norm = a.norm_out ? make_row(a.norm_out + row, a.row_bytes) : out_res;
        const Row out_q = MODE != kModeNorm ? make_row(a.quant_out + row, a.row_bytes / 2u) : out_res;
#pragma unroll
        for (int s = 0; s < VPT; ++s) {
            float w[8], xw[8];
            unpack8(wv[s], w);
#pragma unroll
            for (int e = 0; e < 8; ++e) xw[e] = x[s][e] * w[e];

            const QuantScale q = MODE == kModeQuantBlock ? quant_scale(group_max[s]) : token_q;
            // lanes past the end of the row (valid[s] false) issue no stores
            if (!valid[s]) continue;
            store16(out_res, off[s], pack_bf16x8(x[s]));
            if (a.norm_out) {
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (x[s][e] * inv) * w[e];
                store16(out_norm, off[s], pack_bf16x8(y));
            }
            if (MODE == kModeQuantStatic) {
                float r[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = ((x[s][e] * inv) * w[e]) * static_rcp;
                store8(out_q, off[s] / 2u, pack_e4m3x8(r));
            } else if (MODE != kModeNorm) {
                float r[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = (xw[e] * q.pre) * q.qmul;
                u32x2 codes = pack_e4m3x8(r);
                if (q.qmul == 0.0f) codes = u32x2{0u, 0u};  // all-zero token or group: +0 codes
                store8(out_q, off[s] / 2u, codes);
            }
        }
        if (!more) break;
        t = t_next;
    }
}

// ---------------------------------------------------------------- QK RMSNorm

// The QK norm family. Workgroup b handles row b (and b + gridDim.x, ... when
// the grid is smaller than T).
template <int VPT, int MODE>
__global__ void __launch_bounds__(max_threads_for(VPT)) qk_norm_kernel(QkArgs a, int64_t T) {
    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int nv = a.nq + a.nk;

    // q then k lie back to back at the start of each row: one span of nv vectors.
    bool valid[VPT], is_q[VPT];
    uint32_t off[VPT];  // byte offset of the lane's vector in slot s, within a row
    u32x4 wv[VPT];      // the q or k weight of each vector, loaded once
#pragma unroll
    for (int s = 0; s < VPT; ++s) {
        const int i = s * nthr + tid;
        valid[s] = i < nv;
        is_q[s] = i < a.nq;
        off[s] = (uint32_t)i * 16u;
        wv[s] = !valid[s] ? zero4() : is_q[s] ? a.wq[i] : a.wk[i - a.nq];
    }

    const int seg = a.segments;
    const uint32_t qk_bytes = (uint32_t)nv * 16u;  // q and k; v is never read
    int parity = 0;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x, parity ^= 1) {
        u32x4 raw[VPT];  // lanes past the row read zeros
        {
            const Row src = make_row(a.qkv + t * a.row_stride, qk_bytes);
#pragma unroll
            for (int s = 0; s < VPT; ++s) raw[s] = load16(src, off[s]);
        }
        float2 var_in = make_float2(0.0f, 0.0f);
        if (MODE == kQkSupplied) {
            var_in.x = a.var_in[t * seg];
            if (seg == 2) var_in.y = a.var_in[t * seg + 1];
        }

        float var_q, var_k;
        if (MODE == kQkSupplied) {
            var_q = var_in.x;
            var_k = var_in.y;
        } else {
            float sq[VPT], sk[VPT];
#pragma unroll
            for (int s = 0; s < VPT; ++s) {
                float f[8];
                unpack8(raw[s], f);
                const float v = sumsq8(f);
                sq[s] = is_q[s] ? v : 0.0f;
                sk[s] = is_q[s] ? 0.0f : v;
            }
            float tq = tree_sum(sq), tk = tree_sum(sk);
            block_reduce<true>(tq, tk, Sum{}, parity);
            var_q = tq / a.q_size;
            var_k = tk / a.kv_size;
        }
        if (MODE == kQkStats) {
            if (tid == 0) {
                a.var_out[t * seg] = var_q;
                if (seg == 2) a.var_out[t * seg + 1] = var_k;
            }
        } else {
            const float inv_q = rsqrtf(var_q / a.tp_world + a.eps);
            const float inv_k = rsqrtf(var_k / a.tp_world + a.eps_k);
            // a null q_out (quantised q only) and the k output of one segment
            // get resources of zero bytes, and are never stored to
            const Row out_q = a.q_out ? make_row(a.q_out + t * a.nq, (uint32_t)a.nq * 16u)
                                      : make_row(a.k_out, 0u);
            const Row out_k = seg == 2 ? make_row(a.k_out + t * a.nk, (uint32_t)a.nk * 16u)
                                       : make_row(a.q_out, 0u);
            const Row out_c = MODE == kQkQuant ? make_row(a.quant_out + t * a.nq, (uint32_t)a.nq * 8u)
                                               : out_k;
            const bool want_q = a.q_out != nullptr;
#pragma unroll
            for (int s = 0; s < VPT; ++s) {
                const float inv = is_q[s] ? inv_q : inv_k;
                float f[8], w[8], y[8];
                unpack8(raw[s], f);
                unpack8(wv[s], w);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (f[e] * inv) * w[e];
                // each lane issues only the store that applies to its vector
                // (a wave's vectors are all q or all k except at the one wave
                // that straddles the boundary, so the branch rarely diverges)
                if (is_q[s]) {
                    if (want_q) store16(out_q, off[s], pack_bf16x8(y));
                } else if (valid[s]) {
                    store16(out_k, off[s] - (uint32_t)a.nq * 16u, pack_bf16x8(y));
                }
                if (MODE == kQkQuant) {
                    // A 1x128 group is the 16 lanes of one DPP row in one slot;
                    // q_size is a multiple of 128, so no group reaches into k.
                    // As in the fused epilogue the codes come from x*w, which
                    // the rsqrt multiplies away.
                    float xw[8], r[8];
                    float gmax = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        xw[e] = f[e] * w[e];
                        gmax = fmaxf(gmax, fabsf(xw[e]));
                    }
                    gmax = row16_reduce(gmax, Max{});
                    const QuantScale q = quant_scale(gmax);
#pragma unroll
                    for (int e = 0; e < 8; ++e) r[e] = (xw[e] * q.pre) * q.qmul;
                    u32x2 codes = pack_e4m3x8(r);
                    if (q.qmul == 0.0f) codes = u32x2{0u, 0u};  // all-zero group: +0 codes
                    if (is_q[s]) store8(out_c, off[s] / 2u, codes);
                    const int i = s * nthr + tid;
                    if (is_q[s] && (tid & 15) == 0)
                        a.scale_out[t * a.groups + i / 16] = (gmax * inv_q) / 448.0f;
                }
            }
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

// Compute units of the current device, and workgroups of `kernel` that fit
// on one CU at once (0 when no kernel is given); cached per device, kernel
// and workgroup size.
struct Residency {
    int cus;
    int per_cu;
};

hipError_t residency(const void* kernel, int threads, Residency* out) {
    struct Entry {
        int device;
        const void* kernel;
        int threads;
        Residency r;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry& c : cache)
            if (c.device == dev && c.kernel == kernel && c.threads == threads) {
                *out = c.r;
                return hipSuccess;
            }
    }
    Residency r{0, 0};
    if (kernel) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&r.per_cu, kernel, threads, 0);
        if (e != hipSuccess) return e;
        if (r.per_cu < 1) r.per_cu = 1;
    }
    e = hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (r.cus < 1) r.cus = 1;
    std::lock_guard<std::mutex> lock(mu);
    cache.push_back(Entry{dev, kernel, threads, r});
    *out = r;
    return hipSuccess;
}

// per_cu == 0: one workgroup per token (past kMaxGrid tokens, each workgroup
// also takes tokens blockIdx.x + gridDim.x, ...; a dispatch counts its
// work-items in 32 bits). per_cu > 0: at most per_cu resident workgroups per
// CU, each looping over tokens. Never more workgroups than tokens.
constexpr int64_t kMaxGrid = 1 << 20;

template <typename Args>
hipError_t launch_tokens(void (*kernel)(Args, int64_t), const Args& a, int64_t T, int threads,
                         int per_cu, hipStream_t stream) {
    int64_t cap = kMaxGrid;
    if (per_cu > 0) {
        Residency r{};
        hipError_t e = residency(reinterpret_cast<const void*>(kernel), threads, &r);
        if (e != hipSuccess) return e;
        cap = (int64_t)r.cus * (r.per_cu < per_cu ? r.per_cu : per_cu);
    }
    const int64_t grid = T < cap ? T : cap;
    kernel<<<dim3((unsigned)grid), dim3((unsigned)threads), 0, stream>>>(a, T);
    return hipGetLastError();
}

template <int VPT, int CH>
hipError_t launch_epilogue_ch(const EpilogueArgs& a, EpilogueMode mode, int64_t T, int threads,
                              int per_cu, hipStream_t stream) {
    if constexpr (VPT * CH > kMaxLoadsPerLane) {
        return hipErrorInvalidValue;  // never picked: see pick_epilogue_shape
    } else {
        switch (mode) {
            case kModeNorm:
                return launch_tokens(fused_epilogue_kernel<VPT, kModeNorm, CH>, a, T, threads,
                                     per_cu, stream);
            case kModeQuantToken:
                return launch_tokens(fused_epilogue_kernel<VPT, kModeQuantToken, CH>, a, T,
                                     threads, per_cu, stream);
            case kModeQuantBlock:
                return launch_tokens(fused_epilogue_kernel<VPT, kModeQuantBlock, CH>, a, T,
                                     threads, per_cu, stream);
            default:
                return launch_tokens(fused_epilogue_kernel<VPT, kModeQuantStatic, CH>, a, T,
                                     threads, per_cu, stream);
        }
    }
}

template <int VPT>
hipError_t launch_epilogue_vpt(const EpilogueArgs& a, EpilogueMode mode, int64_t T, int threads,
                               int ch, int per_cu, hipStream_t stream) {
    switch (ch) {
        case 2: return launch_epilogue_ch<VPT, 2>(a, mode, T, threads, per_cu, stream);
        case 4: return launch_epilogue_ch<VPT, 4>(a, mode, T, threads, per_cu, stream);
        default: return hipErrorInvalidValue;  // the pickers choose 2 or 4
    }
}

template <int VPT>
hipError_t launch_qk_vpt(const QkArgs& a, QkMode mode, int64_t T, int threads, hipStream_t stream) {
    switch (mode) {
        case kQkLocal: return launch_tokens(qk_norm_kernel<VPT, kQkLocal>, a, T, threads, 0, stream);
        case kQkSupplied:
            return launch_tokens(qk_norm_kernel<VPT, kQkSupplied>, a, T, threads, 0, stream);
        case kQkStats:
            return launch_tokens(qk_norm_kernel<VPT, kQkStats>, a, T, threads, 0, stream);
        default: return launch_tokens(qk_norm_kernel<VPT, kQkQuant>, a, T, threads, 0, stream);
    }
}

}  // namespace

hipError_t device_cus(int* cus) {
    Residency r{};
    hipError_t e = residency(nullptr, 0, &r);
    *cus = r.cus;
    return e;
}

hipError_t launch_epilogue(const EpilogueArgs& a, EpilogueMode mode, int64_t T, LaunchShape s,
                           hipStream_t stream) {
    switch (s.vpt) {
        case 1: return launch_epilogue_vpt<1>(a, mode, T, s.threads, s.ch, s.per_cu, stream);
        case 2: return launch_epilogue_vpt<2>(a, mode, T, s.threads, s.ch, s.per_cu, stream);
        case 3: return launch_epilogue_vpt<3>(a, mode, T, s.threads, s.ch, s.per_cu, stream);
        case 4: return launch_epilogue_vpt<4>(a, mode, T, s.threads, s.ch, s.per_cu, stream);
        case 5: return launch_epilogue_vpt<5>(a, mode, T, s.threads, s.ch, s.per_cu, stream);
        case 6: return launch_epilogue_vpt<6>(a, mode, T, s.threads, s.ch, s.per_cu, stream);
        case 7: return launch_epilogue_vpt<7>(a, mode, T, s.threads, s.ch, s.per_cu, stream);
        case 8: return launch_epilogue_vpt<8>(a, mode, T, s.threads, s.ch, s.per_cu, stream);
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
