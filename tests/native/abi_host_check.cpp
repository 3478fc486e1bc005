// abi_host_check.cpp -- drives every C entry point of include/swa_sink.h on
// the CPU (with the kernel launchers replaced by launch_stubs.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer: argument validation, size
// arithmetic, kernel choice and workspace sizing, over fixed cases and a
// seeded sweep of valid, invalid and extreme arguments.  Exit status 0 when
// every check holds; the sanitizers abort on the first memory or UB error.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "swa_sink.h"

extern int g_launches;

namespace {

int failures = 0;
void expect(bool ok, const char *what, long line) {
    if (!ok) {
        std::fprintf(stderr, "check failed (line %ld): %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// Dummy device pointers: never dereferenced by host code.
void *const P = reinterpret_cast<void *>(uintptr_t{1} << 20);
float *const F = reinterpret_cast<float *>(uintptr_t{1} << 21);
const int32_t *const I = reinterpret_cast<const int32_t *>(uintptr_t{1} << 22);
void *const MIS = reinterpret_cast<void *>((uintptr_t{1} << 20) + 8);   // 8-byte aligned only

// Calls must either fail before launching anything or succeed.
void one_call(int rc, int before, bool empty_ok, const char *name) {
    const int launched = g_launches - before;
    if (rc != SWA_OK) {
        if (launched != 0) std::fprintf(stderr, "%s: error %d after a launch\n", name, rc);
        EXPECT(launched == 0);
        EXPECT(rc >= SWA_ERR_SCRATCH && rc <= SWA_ERR_NULL);
    } else {
        EXPECT(launched >= (empty_ok ? 0 : 1));
    }
}

void fixed_cases() {
    int n0 = g_launches;
    // prefill: the 32K workload and its error cases
    EXPECT(swa_sink_prefill(P, P, P, F, P, F, 1, 64, 8, 32768, 128, 128, SWA_BF16, nullptr) == SWA_OK);
    EXPECT(g_launches == n0 + 1);
    EXPECT(swa_sink_prefill(nullptr, P, P, F, P, F, 1, 64, 8, 32768, 128, 128, 1, nullptr) == SWA_ERR_NULL);
    EXPECT(swa_sink_prefill(P, P, P, F, P, F, 1, 64, 7, 32768, 128, 128, 1, nullptr) == SWA_ERR_SHAPE);
    EXPECT(swa_sink_prefill(P, P, P, F, P, F, 1, 64, 8, 32768, 96, 128, 1, nullptr) == SWA_ERR_UNSUPPORTED);
    EXPECT(swa_sink_prefill(P, P, P, F, P, F, 1, 64, 8, 32768, 128, 128, 7, nullptr) == SWA_ERR_UNSUPPORTED);
    EXPECT(swa_sink_prefill(MIS, P, P, F, P, F, 1, 64, 8, 32768, 128, 128, 1, nullptr) == SWA_ERR_UNSUPPORTED);
    EXPECT(swa_sink_prefill(P, P, P, F, P, F, 1, 64, 8, 0, 128, 128, 1, nullptr) == SWA_OK);
    EXPECT(swa_sink_prefill(P, P, P, F, P, F, 1, 64, 8, INT_MAX, 128, 128, 1, nullptr) == SWA_ERR_SHAPE);
    // decode, ring decode
    n0 = g_launches;
    EXPECT(swa_sink_decode(P, P, P, F, P, F, 256, 64, 8, 4, 128, 128, I, SWA_BF16, nullptr) == SWA_OK);
    EXPECT(swa_sink_decode_ring(P, P, P, F, P, F, 256, 64, 8, 4, 128, 131, 128, I, 1, nullptr) == SWA_OK);
    EXPECT(g_launches == n0 + 2);
    EXPECT(swa_sink_decode(P, P, P, F, P, F, 256, 64, 8, 129, 128, 128, I, 1, nullptr) == SWA_ERR_SHAPE);
    EXPECT(swa_sink_decode_ring(P, P, P, F, P, F, 256, 64, 8, 4, 128, 127, 128, I, 1, nullptr) == SWA_ERR_SHAPE);
    // global: workspace exactly as queried, one byte short, and missing
    const size_t ws = global_sink_attn_workspace_bytes(8, 64, 8, 1, 262144, 128);
    EXPECT(ws > 0);
    EXPECT(global_sink_attn(P, P, P, F, P, F, 8, 64, 8, 1, 262144, 128, P, ws, 1, nullptr) == SWA_OK);
    EXPECT(global_sink_attn(P, P, P, F, P, F, 8, 64, 8, 1, 262144, 128, P, ws - 1, 1, nullptr) == SWA_ERR_WORKSPACE);
    EXPECT(global_sink_attn(P, P, P, F, P, F, 8, 64, 8, 1, 262144, 128, nullptr, 0, 1, nullptr) == SWA_ERR_WORKSPACE);
    EXPECT(global_sink_attn_workspace_bytes(1, 64, 8, 65536, 65536, 128) == 0);
    EXPECT(global_sink_attn_noalloc(P, P, P, F, P, F, 8, 64, 8, 1, 262144, 128, 1, nullptr) == SWA_OK);
    EXPECT(global_sink_attn_noalloc(P, P, P, F, P, F, 4096, 64, 8, 1, 65536, 128, 1, nullptr) == SWA_ERR_SCRATCH);
    // backward
    const size_t bws = swa_sink_backward_workspace_bytes(1, 64, 32768);
    EXPECT(bws == 4ull * 64 * (2 * 32768 + 1024));
    EXPECT(swa_sink_backward(P, P, P, F, P, F, P, P, P, P, F, 1, 64, 8, 32768, 128, 128, P, bws, 1, nullptr) == SWA_OK);
    EXPECT(swa_sink_backward(P, P, P, F, P, F, P, P, P, P, F, 1, 64, 8, 32768, 128, 128, P, bws - 4, 1, nullptr) == SWA_ERR_WORKSPACE);
    // block maxima, RoPE append, packed prefill
    EXPECT(global_sink_attn_block_max(P, P, P, F, P, F, F, 128, 1, 64, 8, 65536, 65536, 128, 1, nullptr) == SWA_OK);
    EXPECT(global_sink_attn_block_max(P, P, P, F, P, F, F, 48, 1, 64, 8, 65536, 65536, 128, 1, nullptr) == SWA_ERR_SHAPE);
    EXPECT(swa_sink_rope_append(P, P, P, P, P, P, I, 256, 64, 8, 4, 131, 128, 1e6, 1, nullptr) == SWA_OK);
    EXPECT(swa_sink_rope_append(P, P, P, P, P, P, I, 256, 64, 8, 4, 131, 128, 1.0, 1, nullptr) == SWA_ERR_UNSUPPORTED);
    EXPECT(swa_sink_prefill_varlen(P, P, P, F, P, F, I, 16, 8192, 56476, 64, 8, 128, 128, 1, nullptr) == SWA_OK);
    for (int code = SWA_ERR_SCRATCH; code <= SWA_OK; ++code) EXPECT(swa_sink_strerror(code) != nullptr);
}

// Seeded sweep over argument grids that include every boundary value.
void sweep(int n_calls) {
    std::mt19937_64 rng(20260);
    const std::vector<int> Bs = {-1, 0, 1, 2, 3, 255, 256, 65535, 65536};
    const std::vector<int> Hs = {-1, 0, 1, 2, 6, 8, 16, 64, 65535, 65536};
    const std::vector<int> Ss = {-1, 0, 1, 31, 32, 33, 127, 128, 129, 4097, 32768, 262144,
                                 1 << 21, (1 << 30) + 1, INT_MAX - 31, INT_MAX};
    const std::vector<int> Ds = {-1, 0, 1, 32, 64, 96, 128, 256};
    const std::vector<int> Ws = {-1, 0, 1, 2, 33, 97, 98, 128, 129, 130, 4096, INT_MAX};
    const std::vector<int> dts = {-1, 0, 1, 2};
    const std::vector<void *> ptrs = {P, P, P, nullptr, MIS};
    // Valid-looking choices, so that most calls get past the cheap checks and
    // exercise the size arithmetic with boundary values.
    const std::vector<int> Bv = {1, 2, 3, 255, 256, 65535};
    const std::vector<int> Hqv = {8, 16, 64}, Hkvv = {1, 2, 8}, Dv = {64, 128}, dtv = {0, 1};
    auto pick = [&](const auto &v) { return v[rng() % v.size()]; };
    auto mix = [&](const auto &good, const auto &any) { return (rng() % 4) ? pick(good) : pick(any); };
    for (int it = 0; it < n_calls; ++it) {
        const int B = mix(Bv, Bs), Hq = mix(Hqv, Hs), Hkv = mix(Hkvv, Hs);
        const int S = pick(Ss), S2 = (rng() % 2) ? S : pick(Ss);
        const int D = mix(Dv, Ds), W = pick(Ws), W2 = pick(Ws), dt = mix(dtv, dts), T = pick(Ws);
        void *q = (rng() % 8) ? P : pick(ptrs), *k = (rng() % 8) ? P : pick(ptrs);
        void *o = (rng() % 8) ? P : pick(ptrs), *w = (rng() % 4) ? P : pick(ptrs);
        float *f = (rng() % 8) ? F : nullptr;
        const int32_t *cl = (rng() % 4) ? I : nullptr;
        const size_t wsb = (rng() % 2) ? SIZE_MAX : (size_t)(rng() % (1u << 30));
        const int before = g_launches;
        switch (it % 11) {
        case 0: one_call(swa_sink_prefill(q, k, P, F, o, f, B, Hq, Hkv, S, D, W, dt, nullptr),
                         before, true, "prefill"); break;
        case 1: one_call(swa_sink_decode(q, k, P, F, o, f, B, Hq, Hkv, T, W, D, cl, dt, nullptr),
                         before, true, "decode"); break;
        case 2: one_call(swa_sink_decode_ring(q, k, P, F, o, f, B, Hq, Hkv, T, W, W2, D, cl, dt,
                                              nullptr), before, true, "decode_ring"); break;
        case 3: (void)global_sink_attn_workspace_bytes(B, Hq, Hkv, S, S2, D);
                one_call(global_sink_attn(q, k, P, F, o, f, B, Hq, Hkv, S, S2, D, w, wsb, dt,
                                          nullptr), before, true, "global"); break;
        case 4: one_call(global_sink_attn_noalloc(q, k, P, F, o, f, B, Hq, Hkv, S, S2, D, dt,
                                                  nullptr), before, true, "noalloc"); break;
        case 5: one_call(global_sink_attn_block_max(q, k, P, F, o, f, f, W, B, Hq, Hkv, S, S2, D,
                                                    dt, nullptr), before, true, "block_max"); break;
        case 6: (void)swa_sink_backward_workspace_bytes(B, Hq, S);
                one_call(swa_sink_backward(q, k, P, F, o, f, P, P, P, P, f, B, Hq, Hkv, S, D, W,
                                           w, wsb, dt, nullptr), before, true, "backward"); break;
        case 7: one_call(swa_sink_rope_append(q, k, P, o, P, P, cl, B, Hq, Hkv, T, W, D,
                                              (rng() % 3) ? 1e4 : -1.0, dt, nullptr),
                         before, true, "rope_append"); break;
        case 8: one_call(swa_sink_prefill_varlen(q, k, P, F, o, f, cl ? cl : nullptr, B, S, S2, Hq,
                                                 Hkv, D, W, dt, nullptr), before, true, "varlen"); break;
        case 9: (void)swa_sink_strerror(static_cast<int>(rng() % 20) - 10); break;
        default: (void)global_sink_attn_workspace_bytes(B, Hq, Hkv, S, S2, D);
                 (void)swa_sink_backward_workspace_bytes(B, Hq, S); break;
        }
    }
}

}  // namespace

int main() {
    fixed_cases();
    sweep(2000000);
    std::printf("abi host check: %d failures, %d launches\n", failures, g_launches);
    return failures == 0 ? 0 : 1;
}
