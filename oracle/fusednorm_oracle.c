/*
 * CPU oracle for the fused tensor-parallel epilogue and the MiniMax QK RMSNorm.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it. It shares no code, header, table or constant
 * with the HIP library.
 *
 * Plain C, one token per loop iteration, OpenMP over tokens only; a result
 * never depends on the thread count. Floating point is fp64 everywhere except
 * the partial sum, whose precision and order the pages fix (see orc_row_sum).
 *
 * Pages cited (by title and section):
 *   [TS-TRITON]  lightseekorg--tokenspeed, tokenspeed_kernel/ops/communication/
 *                triton.py, section "AMD Triton All-Reduce + RMSNorm",
 *                function amd_allreduce_residual_rmsnorm_kernel.
 *   [TS-TRTLLM]  lightseekorg--tokenspeed, tokenspeed_kernel/thirdparty/cuda/
 *                trtllm.py, sections "Pattern enums", "AllReduce fusion",
 *                "AllGather fusion", "MiniMax QK fused AR + RMSNorm".
 *   [VLLM-QK]    vLLM API docs, vllm.model_executor.layers.minimax_rms_norm.
 *                rms_norm_tp: _minimax_qk_norm_tp_eager, _minimax_qk_var_kernel,
 *                _minimax_rms_apply_kernel.
 *
 * Readings where the pages are silent (bf16 rounding mode, the FP8 format and
 * scale convention, ties, zero rows) are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NOMEM 2

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits. */
/* It is the upper half of an IEEE binary32, so decoding is a 16-bit shift.   */
/* ------------------------------------------------------------------------ */

double orc_bf16_decode(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Nearest bf16 to v, ties to the even stored mantissa (round-to-nearest-even,
 * the reading taken for every fp32 -> bf16 store on the pages, which store fp32
 * values into bf16 tensors without naming a mode). NaN -> 0x7FC0. */
uint16_t orc_bf16_encode(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    int e2;
    frexp(a, &e2);            /* a = f * 2^e2, f in [0.5, 1) */
    int ue = e2 - 1;          /* a lies in [2^ue, 2^(ue+1)) */
    if (ue > 127) return (uint16_t)(sign | 0x7F80);
    if (ue < -126) ue = -126; /* subnormals share the spacing of the lowest binade */
    /* Representable values in this binade are n * 2^(ue-7), n = 128..255
     * (n = 0..127 for subnormals). */
    double q = ldexp(a, 7 - ue); /* exact: scaling by a power of two */
    double n = floor(q);
    double rem = q - n;
    if (rem > 0.5 || (rem == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
    /* Bit patterns of non-negative bf16 values increase with the value, and
     * n = 256 rolls over into the next binade (or to +inf above 2^127). */
    long bits = ((long)(ue + 127) << 7) + ((long)n - 128);
    return (uint16_t)(sign | (uint16_t)bits);
}

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa     */
/* bits; no infinities; S.1111.111 is NaN; largest finite value 448.          */
/* ------------------------------------------------------------------------ */

double orc_e4m3_decode(uint8_t code) {
    int s = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                 /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);  /* normal */
    return s ? -v : v;
}

/* Largest code c in [0, 126] with decode(c) <= a, for 0 <= a <= 448. The 127
 * finite non-negative codes decode to strictly increasing values. */
static int orc_e4m3_floor_code(double a) {
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (orc_e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* Nearest e4m3 code to r after clamping |r| to 448 (saturating), ties to the
 * code with an even mantissa LSB; the sign bit is copied, so a negative value
 * that rounds to zero gives 0x80. NaN -> 0x7F. */
uint8_t orc_e4m3_encode(double r) {
    if (isnan(r)) return 0x7F;
    uint8_t sign = signbit(r) ? 0x80 : 0;
    double a = fabs(r);
    if (a > 448.0) a = 448.0;
    int c = orc_e4m3_floor_code(a);
    if (c < 126) {
        double lo = orc_e4m3_decode((uint8_t)c), hi = orc_e4m3_decode((uint8_t)(c + 1));
        double dlo = a - lo, dhi = hi - a;
        if (dhi < dlo || (dhi == dlo && (c & 1))) c += 1;
    }
    return (uint8_t)(sign | (uint8_t)c);
}

/* 1 when |r| (clamped to 448) lies within 2^-19 * m of the midpoint m between
 * the two finite codes around it. A value that close to a rounding boundary
 * may land on either side once a kernel's own fp32 roundings of r (a few fp32
 * ulps, under 2^-21 relative) are applied, so an off-by-one code there is an
 * expected difference, counted rather than failed. */
uint8_t orc_e4m3_near_tie(double r) {
    double a = fabs(r);
    if (isnan(a)) return 0;
    if (a > 448.0) a = 448.0;
    int c = orc_e4m3_floor_code(a);
    if (c >= 126) c = 125; /* 448 itself: the nearest midpoint lies below it */
    double m = 0.5 * (orc_e4m3_decode((uint8_t)c) + orc_e4m3_decode((uint8_t)(c + 1)));
    return fabs(a - m) <= ldexp(m, -19) ? 1 : 0;
}

/* Element-wise array forms, for the tests. */
void orc_bf16_encode_array(const double* v, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_encode(v[i]);
}
void orc_bf16_decode_array(const uint16_t* b, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_decode(b[i]);
}
void orc_e4m3_encode_array(const double* v, uint8_t* out, uint8_t* near_tie, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        out[i] = orc_e4m3_encode(v[i]);
        if (near_tie) near_tie[i] = orc_e4m3_near_tie(v[i]);
    }
}
void orc_e4m3_decode_array(const uint8_t* c, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]);
}

/* ------------------------------------------------------------------------ */
/* Fused epilogue, one token row at a time.                                  */
/* ------------------------------------------------------------------------ */

/* Steps 1-2, partial sum and residual add, per [TS-TRITON]: an fp32
 * accumulator starts at zero, each peer's bf16 value is widened to fp32 and
 * added in peer order, then the widened residual is added; the result is the
 * updated residual. The pages fix this precision (fp32 accumulate, in peer
 * order) so the oracle performs exactly those fp32 additions; every later step
 * runs in fp64. */
static void orc_row_sum(const uint16_t* const* partials, int P, const uint16_t* residual,
                        int64_t row_off, int64_t H, float* x) {
    for (int64_t j = 0; j < H; ++j) {
        float acc = 0.0f;
        for (int p = 0; p < P; ++p) acc += (float)orc_bf16_decode(partials[p][row_off + j]);
        x[j] = acc + (float)orc_bf16_decode(residual[row_off + j]);
    }
}

/* Steps 3-4 per [TS-TRITON]: mean of x^2 over the true width H, rsqrt of the
 * mean plus eps (eps is the fp32 value handed in), then x * scale * weight. */
static double orc_row_inv_rms(const float* x, int64_t H, float eps) {
    double ss = 0.0;
    for (int64_t j = 0; j < H; ++j) ss += (double)x[j] * (double)x[j];
    double ms = ss / (double)H;
    return 1.0 / sqrt(ms + (double)eps);
}

static int orc_check_common(const uint16_t* const* partials, int P, const uint16_t* residual,
                            const uint16_t* weight, int64_t T, int64_t H) {
    if (P < 1 || !partials || !residual || !weight || T < 0 || H <= 0) return ORC_ERR_ARG;
    for (int p = 0; p < P; ++p) if (!partials[p]) return ORC_ERR_ARG;
    return ORC_OK;
}

/* Scale convention for the FP8 epilogues (pages silent; plain reading of an
 * absmax scale): s = amax / 448 is the dequantisation multiplier, so y ~ code*s,
 * and the quantised value is y / s = 448 * y / amax, clamped and rounded to the
 * nearest e4m3 code. A block whose amax is 0 gets s = 0 and all-zero codes. */
static void orc_quant_block(const double* y, int64_t n, uint8_t* codes, uint8_t* near_tie,
                            float* scale, double* r_out) {
    double amax = 0.0;
    for (int64_t j = 0; j < n; ++j) if (fabs(y[j]) > amax) amax = fabs(y[j]);
    if (amax == 0.0) {
        *scale = 0.0f;
        for (int64_t j = 0; j < n; ++j) {
            codes[j] = 0x00;
            if (near_tie) near_tie[j] = 0;
            if (r_out) r_out[j] = 0.0;
        }
        return;
    }
    *scale = (float)(amax / 448.0);
    for (int64_t j = 0; j < n; ++j) {
        double r = 448.0 * y[j] / amax;
        codes[j] = orc_e4m3_encode(r);
        if (near_tie) near_tie[j] = orc_e4m3_near_tie(r);
        if (r_out) r_out[j] = r;
    }
}

/* The fused epilogue on T tokens of width H:
 *   x = fp32 partial sum + residual            -> residual_out = bf16(x)
 *   y = x * rsqrt(mean(x^2) + eps) * weight    -> norm_out     = bf16(y)
 * and, when codes != NULL, FP8 quantisation of fp32 y (never of bf16(y)):
 *   group_size == 0: one scale per token  (pattern kARResidualRMSNormFP8Quant)
 *   group_size  > 0: one scale per run of group_size consecutive channels of a
 *                    token (pattern kARResidualRMSNormFP8BlockWiseQuant; the
 *                    pages use 128), scales row-major [T, H/group_size].
 * Pattern names from [TS-TRTLLM] "Pattern enums". Any output pointer may be
 * NULL. x_out (fp32 [T,H]) exposes the updated residual before its bf16
 * rounding, y_out / r_out (fp64 [T,H]) the normalised values and the values
 * handed to the e4m3 rounding. */
int orc_fused_add_rmsnorm(const uint16_t* const* partials, int P, const uint16_t* residual,
                          const uint16_t* weight, int64_t T, int64_t H, float eps,
                          int64_t group_size,
                          uint16_t* norm_out, uint16_t* residual_out,
                          uint8_t* codes, float* scales, uint8_t* near_tie,
                          float* x_out, double* y_out, double* r_out) {
    if (orc_check_common(partials, P, residual, weight, T, H) != ORC_OK) return ORC_ERR_ARG;
    if (group_size < 0 || (group_size > 0 && H % group_size != 0)) return ORC_ERR_ARG;
    if (codes && !scales) return ORC_ERR_ARG;
    int64_t n_groups = group_size > 0 ? H / group_size : 1;
    int64_t g_len = group_size > 0 ? group_size : H;
    int err = ORC_OK;
#pragma omp parallel
    {
        float* x = (float*)malloc((size_t)H * sizeof(float));
        double* y = (double*)malloc((size_t)H * sizeof(double));
        double* r = (double*)malloc((size_t)H * sizeof(double));
        if (!x || !y || !r) {
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            if (!x || !y || !r) continue;
            int64_t off = t * H;
            orc_row_sum(partials, P, residual, off, H, x);
            double inv = orc_row_inv_rms(x, H, eps);
            for (int64_t j = 0; j < H; ++j)
                y[j] = (double)x[j] * inv * orc_bf16_decode(weight[j]);
            for (int64_t j = 0; j < H; ++j) {
                if (residual_out) residual_out[off + j] = orc_bf16_encode((double)x[j]);
                if (norm_out) norm_out[off + j] = orc_bf16_encode(y[j]);
                if (x_out) x_out[off + j] = x[j];
                if (y_out) y_out[off + j] = y[j];
            }
            if (codes) {
                for (int64_t g = 0; g < n_groups; ++g)
                    orc_quant_block(y + g * g_len, g_len, codes + off + g * g_len,
                                    near_tie ? near_tie + off + g * g_len : NULL,
                                    scales + t * n_groups + g, r + g * g_len);
                if (r_out) memcpy(r_out + off, r, (size_t)H * sizeof(double));
            }
        }
        free(x);
        free(y);
        free(r);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* MiniMax QK RMSNorm, per [VLLM-QK] and [TS-TRTLLM] "MiniMax QK fused AR +   */
/* RMSNorm". A token's packed row at qkv + t*row_stride holds q (q_size), then */
/* k (kv_size), then v (kv_size, never read).                                  */
/* ------------------------------------------------------------------------ */

/* The TP-pre stage (_minimax_qk_var_kernel): local means of squares of the q
 * and k segments, means[2t] = mean(q^2), means[2t+1] = mean(k^2), in fp64. */
int orc_qk_means(const uint16_t* qkv, int64_t T, int64_t row_stride, int64_t q_size,
                 int64_t kv_size, double* means) {
    if (!qkv || !means || T < 0 || q_size <= 0 || kv_size <= 0 ||
        row_stride < q_size + kv_size)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* row = qkv + t * row_stride;
        double sq = 0.0, sk = 0.0;
        for (int64_t j = 0; j < q_size; ++j) {
            double v = orc_bf16_decode(row[j]);
            sq += v * v;
        }
        for (int64_t j = 0; j < kv_size; ++j) {
            double v = orc_bf16_decode(row[q_size + j]);
            sk += v * v;
        }
        means[2 * t] = sq / (double)q_size;
        means[2 * t + 1] = sk / (double)kv_size;
    }
    return ORC_OK;
}

/* The TP-post stage (_minimax_rms_apply_kernel) and the eager definition
 * (_minimax_qk_norm_tp_eager): out = x * rsqrt(var / tp_world + eps) * w, per
 * segment, where var is the local mean (var_in == NULL, tp_world must be 1) or
 * var_in[t] = the sum over tp_world shards of their local means (fp32 [T,2]),
 * so var / tp_world is the mean over the whole row. Outputs are contiguous
 * [T, q_size] and [T, kv_size]. yq / yk (fp64, nullable) expose the values
 * before rounding. */
int orc_qk_rmsnorm(const uint16_t* qkv, int64_t T, int64_t row_stride, int64_t q_size,
                   int64_t kv_size, const uint16_t* q_weight, const uint16_t* k_weight,
                   float eps, int tp_world, const float* var_in,
                   uint16_t* q_out, uint16_t* k_out, double* yq, double* yk) {
    if (!qkv || !q_weight || !k_weight || !q_out || !k_out || T < 0 || q_size <= 0 ||
        kv_size <= 0 || row_stride < q_size + kv_size || tp_world < 1 ||
        (!var_in && tp_world != 1))
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* row = qkv + t * row_stride;
        double vq, vk;
        if (var_in) {
            vq = (double)var_in[2 * t];
            vk = (double)var_in[2 * t + 1];
        } else {
            double sq = 0.0, sk = 0.0;
            for (int64_t j = 0; j < q_size; ++j) {
                double v = orc_bf16_decode(row[j]);
                sq += v * v;
            }
            for (int64_t j = 0; j < kv_size; ++j) {
                double v = orc_bf16_decode(row[q_size + j]);
                sk += v * v;
            }
            vq = sq / (double)q_size;
            vk = sk / (double)kv_size;
        }
        double inv_q = 1.0 / sqrt(vq / (double)tp_world + (double)eps);
        double inv_k = 1.0 / sqrt(vk / (double)tp_world + (double)eps);
        for (int64_t j = 0; j < q_size; ++j) {
            double y = orc_bf16_decode(row[j]) * inv_q * orc_bf16_decode(q_weight[j]);
            q_out[t * q_size + j] = orc_bf16_encode(y);
            if (yq) yq[t * q_size + j] = y;
        }
        for (int64_t j = 0; j < kv_size; ++j) {
            double y = orc_bf16_decode(row[q_size + j]) * inv_k * orc_bf16_decode(k_weight[j]);
            k_out[t * kv_size + j] = orc_bf16_encode(y);
            if (yk) yk[t * kv_size + j] = y;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Sharded-hidden RMSNorm: one matrix whose hidden dimension is split over   */
/* tp_world ranks ([TS-TRTLLM] "MiniMax QK fused AR + RMSNorm":              */
/* minimax_allreduce_rms, the single-matrix form; the two stages around the  */
/* all-reduce follow [VLLM-QK]). A token's row at x + t*row_stride holds this */
/* rank's H_local channels.                                                   */
/* ------------------------------------------------------------------------ */

/* The pre stage: local mean of squares of each row, means[t] (fp64). */
int orc_sharded_means(const uint16_t* x, int64_t T, int64_t row_stride, int64_t H,
                      double* means) {
    if (!x || !means || T < 0 || H <= 0 || row_stride < H) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* row = x + t * row_stride;
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = orc_bf16_decode(row[j]);
            ss += v * v;
        }
        means[t] = ss / (double)H;
    }
    return ORC_OK;
}

/* The post stage: out = x * rsqrt(var / tp_world + eps) * w, where var is the
 * local mean (var_in == NULL, tp_world must be 1) or var_in[t] = the sum over
 * the tp_world ranks of their local means (fp32 [T]). out is contiguous
 * [T, H]; y (fp64, nullable) exposes the values before rounding. */
int orc_sharded_rmsnorm(const uint16_t* x, int64_t T, int64_t row_stride, int64_t H,
                        const uint16_t* weight, float eps, int tp_world, const float* var_in,
                        uint16_t* out, double* y) {
    if (!x || !weight || !out || T < 0 || H <= 0 || row_stride < H || tp_world < 1 ||
        (!var_in && tp_world != 1))
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* row = x + t * row_stride;
        double var;
        if (var_in) {
            var = (double)var_in[t];
        } else {
            double ss = 0.0;
            for (int64_t j = 0; j < H; ++j) {
                double v = orc_bf16_decode(row[j]);
                ss += v * v;
            }
            var = ss / (double)H;
        }
        double inv = 1.0 / sqrt(var / (double)tp_world + (double)eps);
        for (int64_t j = 0; j < H; ++j) {
            double v = orc_bf16_decode(row[j]) * inv * orc_bf16_decode(weight[j]);
            out[t * H + j] = orc_bf16_encode(v);
            if (y) y[t * H + j] = v;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Fused epilogue with a static FP8 scale: the scale_factor argument of       */
/* [TS-TRTLLM] "AllReduce fusion" (one fp32 value for the whole tensor). The */
/* pages do not say whether it multiplies or divides; as for the dynamic     */
/* variants it is taken as the dequantisation multiplier, y ~ code * s, so   */
/* the quantised value is y / s, clamped to +-448 and rounded to the nearest */
/* e4m3 code (ties to even). No scale is written.                            */
/* ------------------------------------------------------------------------ */
int orc_fused_add_rmsnorm_static(const uint16_t* const* partials, int P, const uint16_t* residual,
                                 const uint16_t* weight, int64_t T, int64_t H, float eps,
                                 float scale, uint16_t* norm_out, uint16_t* residual_out,
                                 uint8_t* codes, uint8_t* near_tie, double* y_out,
                                 double* r_out) {
    if (orc_check_common(partials, P, residual, weight, T, H) != ORC_OK) return ORC_ERR_ARG;
    if (!codes || !(scale > 0.0f) || isinf(scale)) return ORC_ERR_ARG;
    const double s = (double)scale;
    int err = ORC_OK;
#pragma omp parallel
    {
        float* x = (float*)malloc((size_t)H * sizeof(float));
        if (!x) {
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            if (!x) continue;
            int64_t off = t * H;
            orc_row_sum(partials, P, residual, off, H, x);
            double inv = orc_row_inv_rms(x, H, eps);
            for (int64_t j = 0; j < H; ++j) {
                double y = (double)x[j] * inv * orc_bf16_decode(weight[j]);
                double r = y / s;
                if (residual_out) residual_out[off + j] = orc_bf16_encode((double)x[j]);
                if (norm_out) norm_out[off + j] = orc_bf16_encode(y);
                codes[off + j] = orc_e4m3_encode(r);
                if (near_tie) near_tie[off + j] = orc_e4m3_near_tie(r);
                if (y_out) y_out[off + j] = y;
                if (r_out) r_out[off + j] = r;
            }
        }
        free(x);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* All-gather epilogue for MLA ([TS-TRTLLM] "AllGather fusion":             */
/* trtllm_allgather_fusion, patterns kAllGatherfusedRMS and                  */
/* kAllGatherfusedRMSFP8BlockWiseQuant). Each gathered row holds the         */
/* q_lora_rank segment x, then the kv_lora_rank segment y, then the rope part */
/* (never read). Two RMSNorms with their own weight and eps:                 */
/*   x_out = bf16(x * rsqrt(mean(x^2) + x_eps) * x_gamma)                     */
/*   y_out = bf16(y * rsqrt(mean(y^2) + y_eps) * y_gamma)                     */
/* and, when codes != NULL, 1x128 e4m3 of the fp64 normalised x with one     */
/* scale per group (scales [T, q_lora_rank/128]), as in the block variant of */
/* the fused epilogue. x_out may be NULL; y_out may not.                     */
/* ------------------------------------------------------------------------ */
int orc_ag_dual_rmsnorm(const uint16_t* rows, int64_t T, int64_t row_stride, int64_t q_rank,
                        int64_t kv_rank, const uint16_t* x_gamma, const uint16_t* y_gamma,
                        float x_eps, float y_eps, uint16_t* x_out, uint16_t* y_out,
                        uint8_t* codes, float* scales, uint8_t* near_tie, double* yx,
                        double* yy) {
    if (!rows || !x_gamma || !y_gamma || !y_out || T < 0 || q_rank <= 0 || kv_rank <= 0 ||
        row_stride < q_rank + kv_rank)
        return ORC_ERR_ARG;
    if (codes && (!scales || q_rank % 128 != 0)) return ORC_ERR_ARG;
    const int64_t groups = q_rank / 128;
    int err = ORC_OK;
#pragma omp parallel
    {
        double* vx = (double*)malloc((size_t)q_rank * sizeof(double));
        if (!vx) {
#pragma omp atomic write
            err = ORC_ERR_NOMEM;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            if (!vx) continue;
            const uint16_t* row = rows + t * row_stride;
            double sx = 0.0, sy = 0.0;
            for (int64_t j = 0; j < q_rank; ++j) {
                double v = orc_bf16_decode(row[j]);
                sx += v * v;
            }
            for (int64_t j = 0; j < kv_rank; ++j) {
                double v = orc_bf16_decode(row[q_rank + j]);
                sy += v * v;
            }
            double inv_x = 1.0 / sqrt(sx / (double)q_rank + (double)x_eps);
            double inv_y = 1.0 / sqrt(sy / (double)kv_rank + (double)y_eps);
            for (int64_t j = 0; j < q_rank; ++j) {
                vx[j] = orc_bf16_decode(row[j]) * inv_x * orc_bf16_decode(x_gamma[j]);
                if (x_out) x_out[t * q_rank + j] = orc_bf16_encode(vx[j]);
                if (yx) yx[t * q_rank + j] = vx[j];
            }
            for (int64_t j = 0; j < kv_rank; ++j) {
                double v = orc_bf16_decode(row[q_rank + j]) * inv_y * orc_bf16_decode(y_gamma[j]);
                y_out[t * kv_rank + j] = orc_bf16_encode(v);
                if (yy) yy[t * kv_rank + j] = v;
            }
            if (codes)
                for (int64_t g = 0; g < groups; ++g)
                    orc_quant_block(vx + g * 128, 128, codes + t * q_rank + g * 128,
                                    near_tie ? near_tie + t * q_rank + g * 128 : NULL,
                                    scales + t * groups + g, NULL);
        }
        free(vx);
    }
    return err;
}
