// Launch shapes of libfusednorm's kernels: for a row of nvec 16-byte vectors,
// P partial buffers and T tokens on a device with `cus` compute units, which
// workgroup size, vectors per lane, partials per load chunk and grid the fused
// epilogue and the QK-family kernel run with. Host-only: the shape decides
// only speed (every shape computes the same result), and the rules below are
// the ones measured fastest on MI355X with inputs out of cache.
#include "fusednorm_internal.h"

namespace fusednorm {
namespace {

int round_up_wave(int n) { return (n + kWave - 1) / kWave * kWave; }

}  // namespace

LaunchShape pick_epilogue_shape(int nvec, int P, int64_t T, int cus) {
    if (T <= cus) {
        // Fewer tokens than CUs: each token is one workgroup's whole job, so
        // spread it over as many lanes as fit (fewest vectors per lane), with
        // up to four partial buffers' loads in flight at once.
        for (int ch = P <= 2 ? 2 : 4; ch >= 2; ch /= 2) {
            for (int vpt = 1; vpt <= kMaxVpt && vpt * ch <= kMaxLoadsPerLane; ++vpt) {
                const int threads = round_up_wave((nvec + vpt - 1) / vpt);
                if (threads <= max_threads_for(vpt, ch)) return LaunchShape{vpt, threads, ch, 0};
            }
        }
        return LaunchShape{0, 0, 0, 0};
    }
    // Many tokens: 256 threads (fewer for rows of fewer than 256 vectors),
    // partials two buffers at a time. Measured on MI355X, inputs out of cache,
    // rows of 2048 to 8192 elements with 2 and 8 partials: for rows of at
    // least 14 KiB (896 vectors) and at most 8 tokens per CU, two resident
    // workgroups per CU that loop over tokens and prefetch the next token's
    // loads were up to 8% faster (the ramp-up and the tail are a large share
    // of such a launch), and with 8 or more partials two vectors per lane on
    // half-row-wide workgroups were 1% to 3% faster again; with more tokens
    // per CU, or narrower rows, one workgroup per token was 3% to 20% faster.
    if (nvec >= 896 && T <= 8 * (int64_t)cus) {
        if (P >= 8 && nvec % 128 == 0 && nvec / 2 <= max_threads_for(2, 2))
            return LaunchShape{2, nvec / 2, 2, 2};
        const int vpt = (nvec + 255) / 256;
        if (vpt > kMaxVpt) return LaunchShape{0, 0, 0, 0};
        return LaunchShape{vpt, 256, 2, 2};
    }
    const int threads = round_up_wave(nvec < 256 ? nvec : 256);
    const int vpt = (nvec + threads - 1) / threads;
    if (vpt > kMaxVpt) return LaunchShape{0, 0, 0, 0};
    return LaunchShape{vpt, threads, 2, 0};
}

LaunchShape pick_qk_shape(int nvec, int64_t T, int cus) {
    if (T <= cus) {
        for (int vpt = 1; vpt <= kMaxVpt; ++vpt) {
            const int threads = round_up_wave((nvec + vpt - 1) / vpt);
            if (threads <= max_threads_for(vpt)) return LaunchShape{vpt, threads, 0, 0};
        }
        return LaunchShape{0, 0, 0, 0};
    }
    // Many tokens: at least two vectors per lane and at most 256 threads.
    // Measured on MI355X: 128 threads x 2 for 4 KB rows (the MLA rows with FP8
    // of the q part, the hidden-sharded RMSNorm), 256 x 4 for the 14 KB q | k
    // rows of the QK norm, each the fastest or within 1% of it.
    const int half = (nvec + 1) / 2;
    const int threads = round_up_wave(half < 256 ? half : 256);
    const int vpt = (nvec + threads - 1) / threads;
    if (vpt > kMaxVpt) return LaunchShape{0, 0, 0, 0};
    return LaunchShape{vpt, threads, 0, 0};
}

}  // namespace fusednorm
