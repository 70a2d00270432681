/*
 * libfusednorm -- the fused epilogue that follows a tensor-parallel reduction,
 * and the MiniMax-style QK RMSNorm, as hand-written HIP kernels for gfx950
 * (MI355X), behind a C ABI.
 *
 * Pages this interface follows (cited by title and section):
 *   [TS-TRITON]  lightseekorg--tokenspeed, tokenspeed_kernel/ops/communication/
 *                triton.py, section "AMD Triton All-Reduce + RMSNorm"
 *                (amd_allreduce_residual_rmsnorm_kernel and its dispatcher
 *                allreduce_residual_rmsnorm / allreduce_residual_rmsnorm_can_run).
 *   [TS-TRTLLM]  lightseekorg--tokenspeed, tokenspeed_kernel/thirdparty/cuda/
 *                trtllm.py, sections "Pattern enums" (AllReduceFusionPattern,
 *                AllGatherFusionPattern, ReduceScatterFusionPattern),
 *                "AllReduce fusion" (trtllm_allreduce_fusion and its static
 *                scale_factor), "AllGather fusion" (trtllm_allgather_fusion, the
 *                128-wide FP8 block), "ReduceScatter fusion"
 *                (trtllm_reducescatter_fusion) and "MiniMax QK fused AR +
 *                RMSNorm" (minimax_allreduce_rms_qk, minimax_allreduce_rms).
 *   [VLLM-QK]    vLLM API docs, vllm.model_executor.layers.minimax_rms_norm.
 *                rms_norm_tp (_minimax_qk_norm_tp_eager, _minimax_qk_var_kernel,
 *                _minimax_rms_apply_kernel).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to row-major data. bf16 travels as
 *     16-bit storage, FP8 as one byte per value in OCP E4M3 ("e4m3fn": bias 7,
 *     largest finite 448, no infinities, S.1111.111 = NaN).
 *   - The caller owns and allocates every buffer; the library allocates no
 *     device memory and never synchronises. Its only state is a small host-side
 *     cache, per device, of the CU count and the kernels' occupancy (filled on
 *     first use, guarded by a mutex) and the calling thread's last error text.
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) on
 *     the current device; results are ready when that stream reaches the work.
 *     Calls are thread-safe and reentrant.
 *   - Every argument is validated before anything is launched; on any error
 *     nothing is launched and nothing is written. T == 0 (n == 0) is valid:
 *     once the scalar arguments are checked the call returns FUSEDNORM_OK
 *     without examining any buffer (empty tensors may pass NULL) and launches
 *     nothing.
 *   - bf16 outputs are rounded to nearest, ties to even. Arithmetic is fp32.
 *   - Overlap: no output may overlap any input or another output, with one
 *     exception: residual_out may be exactly residual_in (in-place update).
 *     Partial overlaps that the library can detect from the address ranges are
 *     rejected with FUSEDNORM_ERR_UNSUPPORTED.
 *   - NaN or Inf inputs are outside the contract. With eps == 0 an all-zero
 *     token has no defined norm (0 * rsqrt(0)) and its outputs are NaN.
 *
 * Besides the entry points of the method, the library exports three
 * measurement aids (fusednorm_stream_read / _copy / _mix, at the end of this
 * file): plain streaming kernels that measure what HBM delivers for a given
 * read/write mix, reported next to the epilogues' bandwidth. They compute
 * nothing of the method.
 */
#ifndef FUSEDNORM_H
#define FUSEDNORM_H

#include <stdint.h>

/* The functions declared below are the library's whole dynamic interface: it
 * is built with hidden default visibility, and this macro exports exactly
 * them. */
#if defined(__GNUC__) || defined(__clang__)
#define FUSEDNORM_API __attribute__((visibility("default")))
#else
#define FUSEDNORM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define FUSEDNORM_VERSION 10100 /* major*10000 + minor*100 + patch */
#define FUSEDNORM_MAX_PARTIALS 16
#define FUSEDNORM_MAX_HIDDEN 16384
#define FUSEDNORM_FP8_GROUP 128

typedef enum {
    FUSEDNORM_OK = 0,
    /* A required pointer is NULL, a count or size is out of range, eps is
     * negative or not finite, or tp_world is inconsistent with var_in. The
     * [TS-TRTLLM] wrappers assert on such arguments. */
    FUSEDNORM_ERR_INVALID_ARGUMENT = 1,
    /* Well-formed but outside what the kernels handle: widths not a multiple
     * of 8 elements, H above FUSEDNORM_MAX_HIDDEN, pointers not 16-byte
     * aligned, an FP8 group other than 128, partially overlapping buffers. The
     * [TS-TRITON] dispatcher returns (None, None, None, None) for unsupported
     * inputs so the caller can take another path; this code plays that role. */
    FUSEDNORM_ERR_UNSUPPORTED = 2,
    /* The HIP runtime reported an error when the kernel was enqueued. */
    FUSEDNORM_ERR_HIP = 3
} fusednorm_status;

/*
 * fused_add_rmsnorm -- pattern kARResidualRMSNorm ([TS-TRTLLM] "Pattern enums";
 * the computation is [TS-TRITON] amd_allreduce_residual_rmsnorm_kernel with the
 * P peer buffers already resident in this GPU's memory).
 *
 * For every token t < T and channel j < H:
 *   x[t,j]            = ((0 + p_0[t,j]) + p_1[t,j] + ... + p_{P-1}[t,j]) + residual_in[t,j]
 *                       (fp32 accumulation in partial order 0..P-1, then the residual)
 *   residual_out[t,j] = bf16(x[t,j])
 *   norm_out[t,j]     = bf16( x[t,j] * rsqrt(mean_j(x[t,:]^2) + eps) * weight[j] )
 * The mean uses the fp32 x, not bf16(x), and divides by the true H.
 *
 *   partials      HOST array of P device pointers, each bf16 [T, H], 16-B aligned
 *   P             1 .. FUSEDNORM_MAX_PARTIALS
 *   residual_in   bf16 [T, H]
 *   weight        bf16 [H] per-channel RMSNorm weight (used as w, not 1 + w)
 *   T, H          tokens (>= 0) and hidden width (8 .. 16384, multiple of 8)
 *   eps           >= 0, added to the mean of squares inside the rsqrt
 *   norm_out      bf16 [T, H], required
 *   residual_out  bf16 [T, H], required; may equal residual_in
 *   stream        hipStream_t or NULL
 * Returns a fusednorm_status.
 */
FUSEDNORM_API int fused_add_rmsnorm(const void* const* partials, int P, const void* residual_in,
                                    const void* weight, int64_t T, int64_t H, float eps,
                                    void* norm_out, void* residual_out, void* stream);

/*
 * fused_add_rmsnorm_quant_fp8 -- pattern kARResidualRMSNormFP8Quant (with
 * norm_out != NULL it also covers kARResidualRMSNormOutFP8Quant), [TS-TRTLLM]
 * "Pattern enums". The fused epilogue above, then dynamic per-token FP8:
 *   y[t,j]         = x[t,j] * rsqrt(mean_j(x[t,:]^2) + eps) * weight[j]   (fp32)
 *   amax[t]        = max_j |y[t,j]|
 *   scale_out[t]   = amax[t] / 448        (dequantisation multiplier: y ~ code * scale)
 *   quant_out[t,j] = e4m3( clamp(y[t,j] / scale_out[t], -448, 448) ), nearest, ties to even
 * The fp32 y is quantised, never bf16(y). A token whose amax is 0 gets scale 0
 * and all codes 0x00.
 *
 *   norm_out      bf16 [T, H] or NULL (not written)
 *   residual_out  bf16 [T, H], required; may equal residual_in
 *   quant_out     e4m3 [T, H], 16-B aligned, required
 *   scale_out     fp32 [T], 4-B aligned, required
 * Other arguments as for fused_add_rmsnorm.
 */
FUSEDNORM_API int fused_add_rmsnorm_quant_fp8(const void* const* partials, int P,
                                              const void* residual_in, const void* weight,
                                              int64_t T, int64_t H, float eps, void* norm_out,
                                              void* residual_out, void* quant_out, float* scale_out,
                                              void* stream);

/*
 * fused_add_rmsnorm_quant_fp8_block -- pattern kARResidualRMSNormFP8BlockWiseQuant
 * ([TS-TRTLLM] "Pattern enums"; the 128-wide block from "AllGather fusion").
 * As fused_add_rmsnorm_quant_fp8, but with one scale per group g of
 * group_size consecutive channels of a token:
 *   amax[t,g]          = max_{j in [g*128, g*128+128)} |y[t,j]|
 *   scale_out[t,g]     = amax[t,g] / 448
 *   quant_out[t,j]     = e4m3( clamp(y[t,j] / scale_out[t,g], -448, 448) )
 *
 *   group_size    must be FUSEDNORM_FP8_GROUP (128); H must be a multiple of it
 *   scale_out     fp32 [T, H/128] row-major, 4-B aligned, required
 * Other arguments as for fused_add_rmsnorm_quant_fp8.
 */
FUSEDNORM_API int fused_add_rmsnorm_quant_fp8_block(const void* const* partials, int P,
                                                    const void* residual_in, const void* weight,
                                                    int64_t T, int64_t H, float eps, int group_size,
                                                    void* norm_out, void* residual_out,
                                                    void* quant_out, float* scale_out,
                                                    void* stream);

/*
 * fused_add_rmsnorm_quant_fp8_static -- pattern kARResidualRMSNormFP8Quant with
 * the static fp32 scale_factor of [TS-TRTLLM] "AllReduce fusion" (one value for
 * the whole tensor; with norm_out != NULL also kARResidualRMSNormOutFP8Quant).
 * The scale is the dequantisation multiplier, as for the dynamic variants:
 *   quant_out[t,j] = e4m3( clamp(y[t,j] / scale, -448, 448) ), nearest, ties to even
 * with y as in fused_add_rmsnorm_quant_fp8; no scale is written.
 *
 *   scale_factor  DEVICE pointer to one fp32, 4-B aligned; must be finite and > 0
 *                 (read by the kernel, so the host cannot check its value)
 *   norm_out      bf16 [T, H] or NULL;  quant_out e4m3 [T, H], 16-B aligned
 * Other arguments as for fused_add_rmsnorm.
 */
FUSEDNORM_API int fused_add_rmsnorm_quant_fp8_static(const void* const* partials, int P,
                                                     const void* residual_in, const void* weight,
                                                     int64_t T, int64_t H, float eps,
                                                     const float* scale_factor, void* norm_out,
                                                     void* residual_out, void* quant_out,
                                                     void* stream);

/*
 * fused_rs_epilogue -- the epilogue of a reduce-scatter fusion
 * ([TS-TRTLLM] "ReduceScatter fusion": trtllm_reducescatter_fusion; pattern
 * codes from ReduceScatterFusionPattern in "Pattern enums") on this GPU's
 * token slice. Rows [token_offset, token_offset + T) of the P partial buffers
 * are summed in fp32 in partial order, then add_in (patterns 7, 8) and the
 * residual are added, in that order; then RMSNorm and the pattern's step:
 *   1 kRSResidualRMSNorm                     norm_out (required)
 *   2 kRSResidualRMSNormFP8Quant             quant_out with the static scale_factor
 *   4 kRSResidualRMSNormOutFP8Quant          as 2, plus norm_out (required)
 *   6 kRSResidualRMSNormFP8BlockWiseQuant    quant_out + scale_out [T, H/128], norm_out optional
 *   7 kRSAddResidualRMSNormFP8BlockWiseQuant as 6, with add_in
 *   8 kRSAddResidualRMSNorm                  as 1, with add_in
 * Patterns 0 (the bare collective) and 3, 5 (FP4) return FUSEDNORM_ERR_UNSUPPORTED.
 * Outputs a pattern does not write (quant_out and scale_out for 1 and 8,
 * scale_out for 2 and 4) and scale_factor outside 2 and 4 are ignored and may be
 * NULL; the bare reduce-scattered sum is not written.
 *
 *   partials      HOST array of P device pointers, each bf16 [token_num, H] with
 *                 token_num >= token_offset + T (the caller guarantees it)
 *   add_in        bf16 [T, H] for patterns 7 and 8, else NULL; P <= 15 with add_in
 *   residual_in, residual_out, norm_out, quant_out  [T, H] of this slice
 *   scale_factor  DEVICE fp32 [1] for patterns 2 and 4 (as
 *                 fused_add_rmsnorm_quant_fp8_static), else ignored
 * Other arguments as for fused_add_rmsnorm and its FP8 variants.
 */
FUSEDNORM_API int fused_rs_epilogue(int pattern, const void* const* partials, int P,
                                    int64_t token_offset, const void* add_in,
                                    const void* residual_in, const void* weight, int64_t T,
                                    int64_t H, float eps, const float* scale_factor, void* norm_out,
                                    void* residual_out, void* quant_out, float* scale_out,
                                    void* stream);

/*
 * ag_dual_rmsnorm -- the epilogue of the all-gather fusion for MLA on the
 * gathered rows ([TS-TRTLLM] "AllGather fusion": trtllm_allgather_fusion with
 * AllGatherFusionPattern 1 kAllGatherfusedRMS and 2
 * kAllGatherfusedRMSFP8BlockWiseQuant; the gather itself is not part of this
 * library). Token t's row starts at rows + t * row_stride and holds x
 * (q_lora_rank elements), then y (kv_lora_rank), then the rope part (never read
 * or written). Per token, in fp32:
 *   x_norm_out[t,:] = bf16( x * rsqrt(mean(x^2) + x_eps) * x_gamma )
 *   y_norm_out[t,:] = bf16( y * rsqrt(mean(y^2) + y_eps) * y_gamma )
 * and, for pattern 2, the normalised x (before rounding to bf16) in 1x128 FP8
 * groups as fused_add_rmsnorm_quant_fp8_block: for each group g of 128,
 *   scale_out[t,g] = max|x_norm| / 448,
 *   quant_out[t,j] = e4m3( x_norm[j] / scale_out[t,g] )   (zero group: codes 0)
 *
 *   pattern       1: x_norm_out and y_norm_out; quant_out, scale_out NULL
 *                 2: y_norm_out, quant_out, scale_out; x_norm_out optional (NULL: not written)
 *                 0 (the bare all-gather) returns FUSEDNORM_ERR_UNSUPPORTED
 *   rows          bf16, 16-B aligned; row_stride (elements) a multiple of 8 and
 *                 >= q_lora_rank + kv_lora_rank
 *   q_lora_rank   multiple of 8 (of 128 for pattern 2); kv_lora_rank multiple of
 *                 8; their sum <= 16384
 *   x_gamma       bf16 [q_lora_rank];  y_gamma bf16 [kv_lora_rank]; 16-B aligned
 *   x_eps, y_eps  >= 0
 *   x_norm_out    bf16 [T, q_lora_rank];  y_norm_out bf16 [T, kv_lora_rank]
 *   quant_out     e4m3 [T, q_lora_rank], 8-B aligned
 *   scale_out     fp32 [T, q_lora_rank / 128], 4-B aligned
 */
FUSEDNORM_API int ag_dual_rmsnorm(int pattern, const void* rows, int64_t T, int64_t row_stride,
                                  int64_t q_lora_rank, int64_t kv_lora_rank, const void* x_gamma,
                                  const void* y_gamma, float x_eps, float y_eps, void* x_norm_out,
                                  void* y_norm_out, void* quant_out, float* scale_out,
                                  void* stream);

/*
 * qk_rmsnorm -- the MiniMax QK RMSNorm under tensor parallelism ([VLLM-QK]
 * _minimax_qk_norm_tp_eager and _minimax_rms_apply_kernel; [TS-TRTLLM]
 * minimax_allreduce_rms_qk for the contiguous outputs).
 *
 * Token t's row starts at qkv + t * row_stride and holds q (q_size elements),
 * then k (kv_size), then v (kv_size; never read or written). Per token:
 *   var_q, var_k = var_in[t,0], var_in[t,1]           if var_in != NULL
 *                = mean(q^2), mean(k^2) (fp32)         if var_in == NULL (tp_world must be 1)
 *   q_out[t,:] = bf16( q * rsqrt(var_q / tp_world + eps) * q_weight )
 *   k_out[t,:] = bf16( k * rsqrt(var_k / tp_world + eps) * k_weight )
 * var_in holds, per token, the sum over tp_world shards of each shard's local
 * mean of squares (what the all-reduce of qk_rmsnorm_var's output yields), so
 * var / tp_world is the mean over the whole row.
 *
 *   qkv           bf16, 16-B aligned; row_stride (elements) a multiple of 8 and
 *                 >= q_size + kv_size
 *   T             tokens (>= 0)
 *   q_size        multiple of 8, > 0;  kv_size multiple of 8, > 0;
 *                 q_size + kv_size <= 16384
 *   q_weight      bf16 [q_size];  k_weight bf16 [kv_size]
 *   eps           >= 0
 *   tp_world      >= 1
 *   var_in        fp32 [T, 2], 8-B aligned, or NULL
 *   q_out         bf16 [T, q_size] contiguous;  k_out bf16 [T, kv_size] contiguous
 */
FUSEDNORM_API int qk_rmsnorm(const void* qkv, int64_t T, int64_t row_stride, int64_t q_size,
                             int64_t kv_size, const void* q_weight, const void* k_weight, float eps,
                             int tp_world, const float* var_in, void* q_out, void* k_out,
                             void* stream);

/*
 * qk_rmsnorm_var -- the tensor-parallel "pre" stage of the QK norm ([VLLM-QK]
 * _minimax_qk_var_kernel): per token, the local means of squares of the q and k
 * segments, accumulated in fp32:
 *   var_out[t,0] = mean(q^2),  var_out[t,1] = mean(k^2)
 * Summing var_out over the shards of a row (the all-reduce, not part of this
 * library) gives qk_rmsnorm's var_in.
 *
 *   var_out       fp32 [T, 2], 8-B aligned
 * Other arguments as for qk_rmsnorm.
 */
FUSEDNORM_API int qk_rmsnorm_var(const void* qkv, int64_t T, int64_t row_stride, int64_t q_size,
                                 int64_t kv_size, float* var_out, void* stream);

/*
 * sharded_rmsnorm -- RMSNorm of one matrix whose hidden dimension is split over
 * tp_world ranks: the single-matrix form of the MiniMax norm ([TS-TRTLLM]
 * "MiniMax QK fused AR + RMSNorm": minimax_allreduce_rms, input [T, H/nranks]
 * with a bf16 weight of that width), computed as the post stage that follows
 * the all-reduce of the ranks' local means ([VLLM-QK] structure). Per token:
 *   var    = var_in[t]            if var_in != NULL (the sum of the ranks' local means)
 *          = mean(x[t,:]^2) (fp32) if var_in == NULL (tp_world must be 1)
 *   out[t,:] = bf16( x[t,:] * rsqrt(var / tp_world + eps) * weight )
 *
 *   x             bf16 rows at x + t*row_stride, 16-B aligned; H and row_stride
 *                 multiples of 8, H <= row_stride, H <= 16384
 *   weight        bf16 [H];  var_in fp32 [T], 4-B aligned, or NULL
 *   out           bf16 [T, H] contiguous
 */
FUSEDNORM_API int sharded_rmsnorm(const void* x, int64_t T, int64_t row_stride, int64_t H,
                                  const void* weight, float eps, int tp_world, const float* var_in,
                                  void* out, void* stream);

/*
 * sharded_rmsnorm_var -- the pre stage of sharded_rmsnorm ([VLLM-QK]
 * _minimax_qk_var_kernel's form for one segment): var_out[t] = mean(x[t,:H]^2),
 * accumulated in fp32. Summing var_out over the ranks (the all-reduce, not part
 * of this library) gives sharded_rmsnorm's var_in.
 *
 *   var_out       fp32 [T], 4-B aligned
 */
FUSEDNORM_API int sharded_rmsnorm_var(const void* x, int64_t T, int64_t row_stride, int64_t H,
                                      float* var_out, void* stream);

/*
 * fusednorm_e4m3_encode -- element-wise fp32 -> OCP E4M3 with exactly the
 * conversion the FP8 epilogues use (clamp to [-448, 448], round to nearest,
 * ties to even, sign kept, so a negative value that rounds to zero is 0x80).
 * It exposes that conversion so it can be checked on its own.
 *
 *   in    fp32 [n], 16-B aligned;  out  uint8 [n], 16-B aligned;  n >= 0
 */
FUSEDNORM_API int fusednorm_e4m3_encode(const float* in, void* out, int64_t n, void* stream);

/*
 * Measurement aids (not part of the method): plain streaming kernels that give
 * the HBM ceiling next to which the epilogues' bandwidth is reported.
 *   fusednorm_stream_read  reads `bytes` from src with 16-byte vector loads;
 *                          sink (4 bytes, device) is written only in a case
 *                          that no ordinary input reaches
 *   fusednorm_stream_copy  copies `bytes` from src to dst (no overlap)
 * bytes must be a positive multiple of 16 KiB; pointers 16-B aligned.
 *
 *   fusednorm_stream_mix   the same bytes as one epilogue launch, moved with
 *                          no arithmetic: for each of `rows` rows r it reads
 *                          n_src source rows (source k: src_row_bytes bytes at
 *                          src[k] + r * src_stride bytes) and writes n_dst
 *                          destination rows (destination k: dst_row_bytes[k]
 *                          bytes at dst[k] + r * dst_row_bytes[k]), each a
 *                          byte mix of the sources (XOR of the first
 *                          dst_row_bytes[k] bytes of every source row). One
 *                          workgroup per row, 16-byte vectors, the source rows
 *                          read two at a time, the row's stores issued together.
 *                          src and dst are host arrays of device pointers.
 *     1 <= n_src <= 16, 1 <= n_dst <= 4, rows >= 0 (0: nothing launched);
 *     src_row_bytes a multiple of 16 in [16, 32768]; src_stride a multiple of
 *     16, >= src_row_bytes; every dst_row_bytes[k] a multiple of 16 in
 *     [16, src_row_bytes]; pointers 16-B aligned; no destination overlaps a
 *     source or another destination.
 *
 * Returns FUSEDNORM_ERR_INVALID_ARGUMENT for NULL pointers, counts out of
 * range or bytes <= 0, FUSEDNORM_ERR_UNSUPPORTED for other unsupported sizes,
 * alignment or overlap, FUSEDNORM_ERR_HIP for a launch error. They do not set
 * fusednorm_last_error.
 */
FUSEDNORM_API int fusednorm_stream_read(const void* src, int64_t bytes, void* sink, void* stream);
FUSEDNORM_API int fusednorm_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);
FUSEDNORM_API int fusednorm_stream_mix(const void* const* src, int n_src, int64_t src_row_bytes,
                                       int64_t src_stride, void* const* dst,
                                       const int64_t* dst_row_bytes, int n_dst, int64_t rows,
                                       void* stream);

/* Static description of a status code. Never NULL. */
FUSEDNORM_API const char* fusednorm_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread (which
 * argument failed which check); "" when there is none. Valid until the next
 * call on that thread. */
FUSEDNORM_API const char* fusednorm_last_error(void);

/* FUSEDNORM_VERSION of the built library. */
FUSEDNORM_API int fusednorm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FUSEDNORM_H */
