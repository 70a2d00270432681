// C-ABI entry points of libfusednorm (declared in include/fusednorm.h).
//
// Every argument is checked on the host before anything touches the HIP
// runtime, so invalid calls return a status without launching or writing
// anything, also on a machine without a GPU. The checks mirror the pages'
// supported-input contract: the tokenspeed triton.py page, section "AMD Triton
// All-Reduce + RMSNorm" (allreduce_residual_rmsnorm_can_run: bf16, contiguous,
// 2-D, matching shapes; the dispatcher returns no result for unsupported
// inputs) and the 128-element FP8 block of the tokenspeed trtllm.py page,
// section "AllGather fusion".
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <hip/hip_runtime.h>

#include "fusednorm.h"
#include "fusednorm_internal.h"

static_assert(FUSEDNORM_MAX_HIDDEN / FUSEDNORM_FP8_GROUP <= fusednorm::kMaxGroups,
              "the kernels gather a row's 1x128 scales in a fixed LDS array");

namespace {

using fusednorm::u32x2;
using fusednorm::u32x4;

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return FUSEDNORM_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range [lo, hi) of a buffer.
struct Span {
    uintptr_t lo, hi;
    const char* name;
};

Span span(const void* p, int64_t bytes, const char* name) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0), name};
}

bool intersects(const Span& a, const Span& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Outputs must not overlap inputs or each other. The one allowed alias is an
// input and an output that are the same buffer exactly (`same_ok` pairs).
int check_overlaps(const Span* in, int n_in, const Span* out, int n_out, int alias_in,
                   int alias_out) {
    for (int o = 0; o < n_out; ++o) {
        for (int i = 0; i < n_in; ++i) {
            if (!intersects(out[o], in[i])) continue;
            if (i == alias_in && o == alias_out && out[o].lo == in[i].lo && out[o].hi == in[i].hi)
                continue;
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "%s overlaps %s", out[o].name, in[i].name);
        }
        for (int p = o + 1; p < n_out; ++p)
            if (intersects(out[o], out[p]))
                return fail(FUSEDNORM_ERR_UNSUPPORTED, "%s overlaps %s", out[o].name, out[p].name);
    }
    return FUSEDNORM_OK;
}

int check_eps(float eps) {
    if (!(eps >= 0.0f) || !isfinite(eps))
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    return FUSEDNORM_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(FUSEDNORM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

enum class Quant { None, Token, Block, Static };

int fused_common(const void* const* partials_in, int P, const void* residual_in, const void* weight,
                 int64_t T, int64_t H, float eps, int group_size, void* norm_out,
                 void* residual_out, void* quant_out, float* scale_out, void* stream, Quant quant,
                 const float* static_scale = nullptr, int64_t token_offset = 0,
                 const void* add_in = nullptr) {
    // ---- scalar arguments
    if (P < 1 || P > FUSEDNORM_MAX_PARTIALS)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "P = %d outside [1, %d]", P,
                    FUSEDNORM_MAX_PARTIALS);
    if (T < 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
    if (H <= 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "H = %lld <= 0", (long long)H);
    if (int s = check_eps(eps)) return s;
    if (H % 8 != 0)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "H = %lld is not a multiple of 8", (long long)H);
    if (H > FUSEDNORM_MAX_HIDDEN)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "H = %lld above %d", (long long)H,
                    FUSEDNORM_MAX_HIDDEN);
    if (T > 0x7FFFFFFF) return fail(FUSEDNORM_ERR_UNSUPPORTED, "T above 2^31 - 1");
    if (quant == Quant::Block) {
        if (group_size != FUSEDNORM_FP8_GROUP)
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "group_size = %d (only %d)", group_size,
                        FUSEDNORM_FP8_GROUP);
        if (H % FUSEDNORM_FP8_GROUP != 0)
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "H = %lld is not a multiple of %d",
                        (long long)H, FUSEDNORM_FP8_GROUP);
    }
    if (token_offset < 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "token_offset < 0");
    if (add_in && P + 1 > FUSEDNORM_MAX_PARTIALS)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "P = %d leaves no room for add_in (at most %d)",
                    P, FUSEDNORM_MAX_PARTIALS - 1);
    if (T == 0) return ok();  // nothing to read or write: buffers are not examined
    // ---- buffers
    if (!partials_in) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "partials is NULL");
    for (int p = 0; p < P; ++p)
        if (!partials_in[p]) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "partials[%d] is NULL", p);
    // The rows the kernel reads: each partial from token_offset on, then add_in as
    // one more addend after the partials (before the residual).
    const void* partials[FUSEDNORM_MAX_PARTIALS];
    for (int p = 0; p < P; ++p)
        partials[p] = static_cast<const char*>(partials_in[p]) + token_offset * H * 2;
    if (add_in) partials[P++] = add_in;
    if (!residual_in) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "residual_in is NULL");
    if (!weight) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "weight is NULL");
    if (!residual_out) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "residual_out is NULL");
    if (quant == Quant::None && !norm_out)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "norm_out is NULL");
    if (quant != Quant::None && !quant_out)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "quant_out is NULL");
    if ((quant == Quant::Token || quant == Quant::Block) && !scale_out)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "scale_out is NULL");
    if (quant == Quant::Static && !static_scale)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "scale_factor is NULL");
    if (static_scale && !aligned(static_scale, 4))
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "scale_factor not 4-byte aligned");
    for (int p = 0; p < P; ++p)
        if (!aligned(partials[p], 16))
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "partials[%d] not 16-byte aligned", p);
    if (!aligned(residual_in, 16)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "residual_in not 16-byte aligned");
    if (!aligned(weight, 16)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "weight not 16-byte aligned");
    if (!aligned(residual_out, 16)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "residual_out not 16-byte aligned");
    if (norm_out && !aligned(norm_out, 16)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "norm_out not 16-byte aligned");
    if (quant_out && !aligned(quant_out, 16)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "quant_out not 16-byte aligned");
    if (scale_out && !aligned(scale_out, 4)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "scale_out not 4-byte aligned");
    // ---- buffer overlap
    const int64_t row_bytes = H * 2;
    Span in[FUSEDNORM_MAX_PARTIALS + 3];
    int n_in = 0;
    for (int p = 0; p < P; ++p)
        in[n_in++] = span(partials[p], T * row_bytes, add_in && p == P - 1 ? "add_in" : "a partial");
    const int residual_idx = n_in;
    in[n_in++] = span(residual_in, T * row_bytes, "residual_in");
    in[n_in++] = span(weight, row_bytes, "weight");
    Span out[4];
    int n_out = 0;
    out[n_out++] = span(residual_out, T * row_bytes, "residual_out");
    if (norm_out) out[n_out++] = span(norm_out, T * row_bytes, "norm_out");
    if (quant == Quant::Static) in[n_in++] = span(static_scale, 4, "scale_factor");
    if (quant != Quant::None) out[n_out++] = span(quant_out, T * H, "quant_out");
    if (quant == Quant::Token || quant == Quant::Block) {
        const int64_t scales = quant == Quant::Token ? T : T * (H / FUSEDNORM_FP8_GROUP);
        out[n_out++] = span(scale_out, scales * 4, "scale_out");
    }
    if (int s = check_overlaps(in, n_in, out, n_out, residual_idx, 0)) return s;

    // ---- launch
    fusednorm::EpilogueArgs a{};
    for (int p = 0; p < P; ++p) a.partials[p] = static_cast<const u32x4*>(partials[p]);
    a.residual = static_cast<const u32x4*>(residual_in);
    a.weight = static_cast<const u32x4*>(weight);
    a.residual_out = static_cast<u32x4*>(residual_out);
    a.norm_out = static_cast<u32x4*>(norm_out);
    a.quant_out = static_cast<u32x2*>(quant_out);
    a.scale_out = scale_out;
    a.static_scale = static_scale;
    a.P = P;
    a.nvec = (int)(H / 8);
    a.row_bytes = (uint32_t)(H * 2);
    a.groups = (int)(H / FUSEDNORM_FP8_GROUP);
    a.h = (float)H;
    a.eps = eps;
    const fusednorm::EpilogueMode mode = quant == Quant::None    ? fusednorm::kModeNorm
                                         : quant == Quant::Token ? fusednorm::kModeQuantToken
                                         : quant == Quant::Block ? fusednorm::kModeQuantBlock
                                                                 : fusednorm::kModeQuantStatic;
    (void)hipGetLastError();  // start from a clean error state
    int cus = 0;
    if (hipError_t e = fusednorm::device_cus(&cus)) return hip_status(e, "device query");
    const fusednorm::LaunchShape shape = fusednorm::pick_epilogue_shape(a.nvec, P, T, cus);
    if (shape.vpt == 0)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "no launch shape covers H = %lld", (long long)H);
    return hip_status(fusednorm::launch_epilogue(a, mode, T, shape, (hipStream_t)stream),
                      "kernel launch");
}

int qk_common(const void* qkv, int64_t T, int64_t row_stride, int64_t q_size, int64_t kv_size,
              const void* q_weight, const void* k_weight, float eps, int tp_world,
              const float* var_in, void* q_out, void* k_out, float* var_out, void* stream,
              fusednorm::QkMode mode) {
    const bool stats = mode == fusednorm::kQkStats;
    if (T < 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
    if (q_size <= 0 || kv_size <= 0)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "q_size and kv_size must be > 0");
    if (row_stride <= 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "row_stride must be > 0");
    if (!stats) {
        if (int s = check_eps(eps)) return s;
        if (tp_world < 1) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "tp_world = %d < 1", tp_world);
        if (!var_in && tp_world != 1)
            return fail(FUSEDNORM_ERR_INVALID_ARGUMENT,
                        "tp_world = %d needs var_in (the sum of the shards' means)", tp_world);
    }
    if (q_size % 8 || kv_size % 8 || row_stride % 8)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "q_size, kv_size and row_stride must be multiples of 8");
    if (row_stride < q_size + kv_size)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "row_stride %lld < q_size + kv_size", (long long)row_stride);
    if (q_size + kv_size > FUSEDNORM_MAX_HIDDEN)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "q_size + kv_size above %d", FUSEDNORM_MAX_HIDDEN);
    if (T > 0x7FFFFFFF) return fail(FUSEDNORM_ERR_UNSUPPORTED, "T above 2^31 - 1");
    if (T == 0) return ok();  // nothing to read or write: buffers are not examined
    if (!qkv) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "qkv is NULL");
    if (stats) {
        if (!var_out) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "var_out is NULL");
    } else {
        if (!q_weight || !k_weight)
            return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "q_weight / k_weight is NULL");
        if (!q_out || !k_out) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "q_out / k_out is NULL");
    }
    if (!aligned(qkv, 16)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "qkv not 16-byte aligned");
    if (!stats) {
        if (!aligned(q_weight, 16) || !aligned(k_weight, 16))
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "q_weight / k_weight not 16-byte aligned");
        if (!aligned(q_out, 16) || !aligned(k_out, 16))
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "q_out / k_out not 16-byte aligned");
        if (var_in && !aligned(var_in, 8))
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "var_in not 8-byte aligned");
    } else if (!aligned(var_out, 8)) {
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "var_out not 8-byte aligned");
    }
    const int64_t qkv_bytes = ((T - 1) * row_stride + q_size + kv_size) * 2;
    Span in[4];
    int n_in = 0;
    in[n_in++] = span(qkv, qkv_bytes, "qkv");
    Span out[2];
    int n_out = 0;
    if (stats) {
        out[n_out++] = span(var_out, T * 8, "var_out");
    } else {
        in[n_in++] = span(q_weight, q_size * 2, "q_weight");
        in[n_in++] = span(k_weight, kv_size * 2, "k_weight");
        if (var_in) in[n_in++] = span(var_in, T * 8, "var_in");
        out[n_out++] = span(q_out, T * q_size * 2, "q_out");
        out[n_out++] = span(k_out, T * kv_size * 2, "k_out");
    }
    if (int s = check_overlaps(in, n_in, out, n_out, -1, -1)) return s;

    fusednorm::QkArgs a{};
    a.qkv = static_cast<const uint16_t*>(qkv);
    a.row_stride = row_stride;
    a.wq = static_cast<const u32x4*>(q_weight);
    a.wk = static_cast<const u32x4*>(k_weight);
    a.q_out = static_cast<u32x4*>(q_out);
    a.k_out = static_cast<u32x4*>(k_out);
    a.var_in = var_in;
    a.var_out = var_out;
    a.segments = 2;
    a.nq = (int)(q_size / 8);
    a.nk = (int)(kv_size / 8);
    a.q_size = (float)q_size;
    a.kv_size = (float)kv_size;
    a.tp_world = (float)tp_world;
    a.eps = eps;
    a.eps_k = eps;
    if (!stats) mode = var_in ? fusednorm::kQkSupplied : fusednorm::kQkLocal;
    (void)hipGetLastError();
    int cus = 0;
    if (hipError_t e = fusednorm::device_cus(&cus)) return hip_status(e, "device query");
    const fusednorm::LaunchShape shape = fusednorm::pick_qk_shape(a.nq + a.nk, T, cus);
    if (shape.vpt == 0)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "no launch shape covers q_size + kv_size");
    return hip_status(fusednorm::launch_qk(a, mode, T, shape, (hipStream_t)stream), "kernel launch");
}

int sharded_common(const void* x, int64_t T, int64_t row_stride, int64_t H, const void* weight,
                   float eps, int tp_world, const float* var_in, void* out, float* var_out,
                   void* stream, fusednorm::QkMode mode) {
    const bool stats = mode == fusednorm::kQkStats;
    if (T < 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
    if (H <= 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "H = %lld <= 0", (long long)H);
    if (row_stride <= 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "row_stride must be > 0");
    if (!stats) {
        if (int s = check_eps(eps)) return s;
        if (tp_world < 1) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "tp_world = %d < 1", tp_world);
        if (!var_in && tp_world != 1)
            return fail(FUSEDNORM_ERR_INVALID_ARGUMENT,
                        "tp_world = %d needs var_in (the sum of the ranks' means)", tp_world);
    }
    if (H % 8 || row_stride % 8)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "H and row_stride must be multiples of 8");
    if (row_stride < H)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "row_stride %lld < H", (long long)row_stride);
    if (H > FUSEDNORM_MAX_HIDDEN)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "H = %lld above %d", (long long)H, FUSEDNORM_MAX_HIDDEN);
    if (T > 0x7FFFFFFF) return fail(FUSEDNORM_ERR_UNSUPPORTED, "T above 2^31 - 1");
    if (T == 0) return ok();  // nothing to read or write: buffers are not examined
    if (!x) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "x is NULL");
    if (stats) {
        if (!var_out) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "var_out is NULL");
        if (!aligned(var_out, 4)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "var_out not 4-byte aligned");
    } else {
        if (!weight) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "weight is NULL");
        if (!out) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "out is NULL");
        if (!aligned(weight, 16) || !aligned(out, 16))
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "weight / out not 16-byte aligned");
        if (var_in && !aligned(var_in, 4))
            return fail(FUSEDNORM_ERR_UNSUPPORTED, "var_in not 4-byte aligned");
    }
    if (!aligned(x, 16)) return fail(FUSEDNORM_ERR_UNSUPPORTED, "x not 16-byte aligned");
    Span in[3];
    int n_in = 0;
    in[n_in++] = span(x, ((T - 1) * row_stride + H) * 2, "x");
    Span o[1];
    if (stats) {
        o[0] = span(var_out, T * 4, "var_out");
    } else {
        in[n_in++] = span(weight, H * 2, "weight");
        if (var_in) in[n_in++] = span(var_in, T * 4, "var_in");
        o[0] = span(out, T * H * 2, "out");
    }
    if (int s = check_overlaps(in, n_in, o, 1, -1, -1)) return s;

    fusednorm::QkArgs a{};
    a.qkv = static_cast<const uint16_t*>(x);
    a.row_stride = row_stride;
    a.wq = static_cast<const u32x4*>(weight);
    a.wk = static_cast<const u32x4*>(weight);
    a.q_out = static_cast<u32x4*>(out);
    a.k_out = nullptr;
    a.var_in = var_in;
    a.var_out = var_out;
    a.segments = 1;
    a.nq = (int)(H / 8);
    a.nk = 0;
    a.q_size = (float)H;
    a.kv_size = 1.0f;
    a.tp_world = (float)tp_world;
    a.eps = eps;
    a.eps_k = eps;
    if (!stats) mode = var_in ? fusednorm::kQkSupplied : fusednorm::kQkLocal;
    (void)hipGetLastError();
    int cus = 0;
    if (hipError_t e = fusednorm::device_cus(&cus)) return hip_status(e, "device query");
    const fusednorm::LaunchShape shape = fusednorm::pick_qk_shape(a.nq, T, cus);
    if (shape.vpt == 0) return fail(FUSEDNORM_ERR_UNSUPPORTED, "no launch shape covers H");
    return hip_status(fusednorm::launch_qk(a, mode, T, shape, (hipStream_t)stream), "kernel launch");
}

int ag_common(int pattern, const void* rows, int64_t T, int64_t row_stride, int64_t q_rank,
              int64_t kv_rank, const void* x_gamma, const void* y_gamma, float x_eps, float y_eps,
              void* x_out, void* y_out, void* quant_out, float* scale_out, void* stream) {
    if (pattern == 0)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "pattern 0 (a bare all-gather) is not implemented");
    if (pattern != 1 && pattern != 2)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "pattern %d is not an all-gather pattern",
                    pattern);
    const bool quant = pattern == 2;
    if (T < 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
    if (q_rank <= 0 || kv_rank <= 0)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "q_lora_rank and kv_lora_rank must be > 0");
    if (row_stride <= 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "row_stride must be > 0");
    if (int s = check_eps(x_eps)) return s;
    if (int s = check_eps(y_eps)) return s;
    if (q_rank % 8 || kv_rank % 8 || row_stride % 8)
        return fail(FUSEDNORM_ERR_UNSUPPORTED,
                    "q_lora_rank, kv_lora_rank and row_stride must be multiples of 8");
    if (quant && q_rank % FUSEDNORM_FP8_GROUP)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "q_lora_rank must be a multiple of %d",
                    FUSEDNORM_FP8_GROUP);
    if (row_stride < q_rank + kv_rank)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "row_stride %lld < q_lora_rank + kv_lora_rank",
                    (long long)row_stride);
    if (q_rank + kv_rank > FUSEDNORM_MAX_HIDDEN)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "q_lora_rank + kv_lora_rank above %d",
                    FUSEDNORM_MAX_HIDDEN);
    if (T > 0x7FFFFFFF) return fail(FUSEDNORM_ERR_UNSUPPORTED, "T above 2^31 - 1");
    if (T == 0) return ok();  // nothing to read or write: buffers are not examined
    if (!rows) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "rows is NULL");
    if (!x_gamma || !y_gamma)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "x_gamma / y_gamma is NULL");
    if (!y_out) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "y_norm_out is NULL");
    if (quant) {
        if (!quant_out || !scale_out)
            return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "pattern 2 needs quant_out and scale_out");
    } else {
        if (!x_out) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "x_norm_out is NULL");
        if (quant_out || scale_out)
            return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "pattern 1 writes no quant_out / scale_out");
    }
    if (!aligned(rows, 16) || !aligned(x_gamma, 16) || !aligned(y_gamma, 16) ||
        !aligned(y_out, 16) || (x_out && !aligned(x_out, 16)))
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "rows, gammas and outputs must be 16-byte aligned");
    if (quant && (!aligned(quant_out, 8) || !aligned(scale_out, 4)))
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "quant_out / scale_out misaligned");
    const int64_t groups = q_rank / FUSEDNORM_FP8_GROUP;
    Span in[3] = {span(rows, ((T - 1) * row_stride + q_rank + kv_rank) * 2, "rows"),
                  span(x_gamma, q_rank * 2, "x_gamma"), span(y_gamma, kv_rank * 2, "y_gamma")};
    Span out[4];
    int n_out = 0;
    out[n_out++] = span(y_out, T * kv_rank * 2, "y_norm_out");
    if (x_out) out[n_out++] = span(x_out, T * q_rank * 2, "x_norm_out");
    if (quant) {
        out[n_out++] = span(quant_out, T * q_rank, "quant_out");
        out[n_out++] = span(scale_out, T * groups * 4, "scale_out");
    }
    if (int s = check_overlaps(in, 3, out, n_out, -1, -1)) return s;

    fusednorm::QkArgs a{};
    a.qkv = static_cast<const uint16_t*>(rows);
    a.row_stride = row_stride;
    a.wq = static_cast<const u32x4*>(x_gamma);
    a.wk = static_cast<const u32x4*>(y_gamma);
    a.q_out = static_cast<u32x4*>(x_out);
    a.k_out = static_cast<u32x4*>(y_out);
    a.quant_out = static_cast<u32x2*>(quant_out);
    a.scale_out = scale_out;
    a.segments = 2;
    a.nq = (int)(q_rank / 8);
    a.nk = (int)(kv_rank / 8);
    a.groups = (int)groups;
    a.q_size = (float)q_rank;
    a.kv_size = (float)kv_rank;
    a.tp_world = 1.0f;
    a.eps = x_eps;
    a.eps_k = y_eps;
    (void)hipGetLastError();
    int cus = 0;
    if (hipError_t e = fusednorm::device_cus(&cus)) return hip_status(e, "device query");
    const fusednorm::LaunchShape shape = fusednorm::pick_qk_shape(a.nq + a.nk, T, cus);
    if (shape.vpt == 0)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "no launch shape covers q_lora_rank + kv_lora_rank");
    return hip_status(fusednorm::launch_qk(a, quant ? fusednorm::kQkQuant : fusednorm::kQkLocal, T,
                                           shape, (hipStream_t)stream),
                      "kernel launch");
}

}  // namespace

extern "C" {

int fused_add_rmsnorm(const void* const* partials, int P, const void* residual_in,
                      const void* weight, int64_t T, int64_t H, float eps, void* norm_out,
                      void* residual_out, void* stream) {
    return fused_common(partials, P, residual_in, weight, T, H, eps, 0, norm_out, residual_out,
                        nullptr, nullptr, stream, Quant::None);
}

int fused_add_rmsnorm_quant_fp8(const void* const* partials, int P, const void* residual_in,
                                const void* weight, int64_t T, int64_t H, float eps,
                                void* norm_out, void* residual_out, void* quant_out,
                                float* scale_out, void* stream) {
    return fused_common(partials, P, residual_in, weight, T, H, eps, 0, norm_out, residual_out,
                        quant_out, scale_out, stream, Quant::Token);
}

int fused_add_rmsnorm_quant_fp8_block(const void* const* partials, int P,
                                      const void* residual_in, const void* weight, int64_t T,
                                      int64_t H, float eps, int group_size, void* norm_out,
                                      void* residual_out, void* quant_out, float* scale_out,
                                      void* stream) {
    return fused_common(partials, P, residual_in, weight, T, H, eps, group_size, norm_out,
                        residual_out, quant_out, scale_out, stream, Quant::Block);
}

int fused_add_rmsnorm_quant_fp8_static(const void* const* partials, int P,
                                       const void* residual_in, const void* weight, int64_t T,
                                       int64_t H, float eps, const float* scale_factor,
                                       void* norm_out, void* residual_out, void* quant_out,
                                       void* stream) {
    return fused_common(partials, P, residual_in, weight, T, H, eps, 0, norm_out, residual_out,
                        quant_out, nullptr, stream, Quant::Static, scale_factor);
}

int fused_rs_epilogue(int pattern, const void* const* partials, int P, int64_t token_offset,
                      const void* add_in, const void* residual_in, const void* weight, int64_t T,
                      int64_t H, float eps, const float* scale_factor, void* norm_out,
                      void* residual_out, void* quant_out, float* scale_out, void* stream) {
    const bool add = pattern == 7 || pattern == 8;
    if (pattern == 0 || pattern == 3 || pattern == 5)
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "pattern %d is not implemented", pattern);
    if (pattern < 0 || pattern > 8)
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "pattern %d is not a reduce-scatter pattern",
                    pattern);
    if (T > 0 && add != (add_in != nullptr))
        return fail(FUSEDNORM_ERR_INVALID_ARGUMENT,
                    add ? "pattern %d needs add_in" : "pattern %d takes no add_in", pattern);
    switch (pattern) {
        case 1:
        case 8:
            return fused_common(partials, P, residual_in, weight, T, H, eps, 0, norm_out,
                                residual_out, nullptr, nullptr, stream, Quant::None, nullptr,
                                token_offset, add_in);
        case 2:
        case 4:
            if (pattern == 2 && norm_out)
                return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "pattern 2 writes no norm_out");
            if (pattern == 4 && !norm_out && T > 0)
                return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "pattern 4 needs norm_out");
            return fused_common(partials, P, residual_in, weight, T, H, eps, 0, norm_out,
                                residual_out, quant_out, nullptr, stream, Quant::Static,
                                scale_factor, token_offset, add_in);
        default:  // 6 and 7: 1x128 block FP8
            return fused_common(partials, P, residual_in, weight, T, H, eps, FUSEDNORM_FP8_GROUP,
                                norm_out, residual_out, quant_out, scale_out, stream, Quant::Block,
                                nullptr, token_offset, add_in);
    }
}

int qk_rmsnorm(const void* qkv, int64_t T, int64_t row_stride, int64_t q_size, int64_t kv_size,
               const void* q_weight, const void* k_weight, float eps, int tp_world,
               const float* var_in, void* q_out, void* k_out, void* stream) {
    return qk_common(qkv, T, row_stride, q_size, kv_size, q_weight, k_weight, eps, tp_world,
                     var_in, q_out, k_out, nullptr, stream, fusednorm::kQkLocal);
}

int qk_rmsnorm_var(const void* qkv, int64_t T, int64_t row_stride, int64_t q_size,
                   int64_t kv_size, float* var_out, void* stream) {
    return qk_common(qkv, T, row_stride, q_size, kv_size, nullptr, nullptr, 0.0f, 1, nullptr,
                     nullptr, nullptr, var_out, stream, fusednorm::kQkStats);
}

int sharded_rmsnorm(const void* x, int64_t T, int64_t row_stride, int64_t H, const void* weight,
                    float eps, int tp_world, const float* var_in, void* out, void* stream) {
    return sharded_common(x, T, row_stride, H, weight, eps, tp_world, var_in, out, nullptr, stream,
                          fusednorm::kQkLocal);
}

int sharded_rmsnorm_var(const void* x, int64_t T, int64_t row_stride, int64_t H, float* var_out,
                        void* stream) {
    return sharded_common(x, T, row_stride, H, nullptr, 0.0f, 1, nullptr, nullptr, var_out, stream,
                          fusednorm::kQkStats);
}

int ag_dual_rmsnorm(int pattern, const void* rows, int64_t T, int64_t row_stride,
                    int64_t q_lora_rank, int64_t kv_lora_rank, const void* x_gamma,
                    const void* y_gamma, float x_eps, float y_eps, void* x_norm_out,
                    void* y_norm_out, void* quant_out, float* scale_out, void* stream) {
    return ag_common(pattern, rows, T, row_stride, q_lora_rank, kv_lora_rank, x_gamma, y_gamma,
                     x_eps, y_eps, x_norm_out, y_norm_out, quant_out, scale_out, stream);
}

int fusednorm_e4m3_encode(const float* in, void* out, int64_t n, void* stream) {
    if (n < 0) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "n < 0");
    if (n == 0) return ok();
    if (!in || !out) return fail(FUSEDNORM_ERR_INVALID_ARGUMENT, "in / out is NULL");
    if (!aligned(in, 16) || !aligned(out, 16))
        return fail(FUSEDNORM_ERR_UNSUPPORTED, "in / out not 16-byte aligned");
    const Span i = span(in, n * 4, "in"), o = span(out, n, "out");
    if (int s = check_overlaps(&i, 1, &o, 1, -1, -1)) return s;
    if ((n + 7) / 8 > (int64_t)0x7FFFFFFF * 256) return fail(FUSEDNORM_ERR_UNSUPPORTED, "n too large");
    (void)hipGetLastError();
    return hip_status(fusednorm::launch_e4m3_encode(in, static_cast<uint8_t*>(out), n,
                                                    (hipStream_t)stream),
                      "kernel launch");
}

const char* fusednorm_status_string(int status) {
    switch (status) {
        case FUSEDNORM_OK: return "ok";
        case FUSEDNORM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case FUSEDNORM_ERR_UNSUPPORTED: return "unsupported input";
        case FUSEDNORM_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* fusednorm_last_error(void) { return g_last_error; }

int fusednorm_version(void) { return FUSEDNORM_VERSION; }

}  // extern "C"
