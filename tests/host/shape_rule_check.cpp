// Host-side check of the launch-shape pickers (fusednorm_launch_policy.cpp,
// host code only, no GPU needed): every shape they return must be one the
// kernels are compiled for and cover the row, and the persistent grid must be
// picked exactly where the rule says. Prints "ok" or the first violation.
#include "fusednorm_internal.h"

#include <cstdio>

using namespace fusednorm;

static int fail(const char* what, int nvec, int P, long long T, int cus, LaunchShape s) {
    std::printf("FAIL %s: nvec=%d P=%d T=%lld cus=%d -> vpt=%d threads=%d ch=%d per_cu=%d\n", what,
                nvec, P, T, cus, s.vpt, s.threads, s.ch, s.per_cu);
    return 1;
}

int main() {
    const int cus_list[] = {80, 256, 304};
    const long long Ts[] = {1, 2, 255, 256, 257, 1000, 2048, 2049, 4096, 1 << 20, (1 << 20) + 37};
    for (int cus : cus_list) {
        for (int nvec = 1; nvec <= 2048; ++nvec) {
            for (int P = 1; P <= 16; ++P) {
                for (long long T : Ts) {
                    const LaunchShape s = pick_epilogue_shape(nvec, P, T, cus);
                    if (s.vpt < 1 || s.vpt > kMaxVpt) return fail("vpt out of range", nvec, P, T, cus, s);
                    if (s.threads < kWave || s.threads % kWave) return fail("threads not whole waves", nvec, P, T, cus, s);
                    if (s.ch != 2 && s.ch != 4) return fail("chunk not 2 or 4", nvec, P, T, cus, s);
                    if (s.vpt * s.ch > kMaxLoadsPerLane) return fail("too many loads per lane", nvec, P, T, cus, s);
                    if (s.threads > max_threads_for(s.vpt, s.ch)) return fail("above the variant's workgroup bound", nvec, P, T, cus, s);
                    if ((long long)s.vpt * s.threads < nvec) return fail("row not covered", nvec, P, T, cus, s);
                    if (s.threads / kWave > kMaxWaves) return fail("more waves than the LDS reduction holds", nvec, P, T, cus, s);
                    // block FP8 (rows of whole 1x128 groups): the token's scale row is
                    // gathered in LDS and stored one lane per group
                    if (nvec % 16 == 0 && nvec / 16 > s.threads) return fail("fewer lanes than 1x128 groups", nvec, P, T, cus, s);
                    if (nvec % 16 == 0 && nvec / 16 > kMaxGroups) return fail("more groups than the LDS row holds", nvec, P, T, cus, s);
                    const bool persistent = T > cus && nvec >= 896 && T <= 8LL * cus;
                    if ((s.per_cu != 0) != persistent) return fail("persistent grid against the rule", nvec, P, T, cus, s);
                    if (s.per_cu != 0 && s.per_cu != 2) return fail("resident workgroups per CU", nvec, P, T, cus, s);
                }
            }
            for (long long T : Ts) {
                const LaunchShape q = pick_qk_shape(nvec, T, cus);
                if (q.vpt < 1 || q.vpt > kMaxVpt) return fail("qk vpt out of range", nvec, 0, T, cus, q);
                if (q.threads < kWave || q.threads % kWave) return fail("qk threads not whole waves", nvec, 0, T, cus, q);
                if (q.threads > max_threads_for(q.vpt)) return fail("qk above the variant's workgroup bound", nvec, 0, T, cus, q);
                if ((long long)q.vpt * q.threads < nvec) return fail("qk row not covered", nvec, 0, T, cus, q);
                if (q.per_cu != 0) return fail("qk persistent", nvec, 0, T, cus, q);
            }
        }
    }
    std::printf("ok\n");
    return 0;
}
