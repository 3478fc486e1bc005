// launch_stubs.cpp -- stand-ins for the kernel launchers (csrc/*.hip device
// code), so that the C entry points (api.hip) and the host planning code
// (plan.hip) can be built as plain C++ with sanitizers and driven on a CPU.
// Each stub checks that the arguments the entry point forwards are the
// validated ones, counts the call and reports success.  No device memory is
// touched: the tensor pointers are dummies.
#include <cstdio>
#include <cstdlib>

#include "launch.h"

int g_launches = 0;

namespace {
void need(bool ok, const char *what) {
    if (!ok) {
        std::fprintf(stderr, "launcher received invalid arguments: %s\n", what);
        std::abort();
    }
}
void prefill_ok(const swa::PrefillArgs &a) {
    need(a.q && a.k && a.v && a.sink && a.out, "null tensor");
    need(a.B >= 1 && a.Hq >= 1 && a.Hkv >= 1 && a.Hq % a.Hkv == 0, "heads");
    need(a.S >= 1 && a.S_kv >= a.S && a.window >= 1, "rows");
    need(a.D == 64 || a.D == 128, "head dim");
}
void decode_ok(const swa::DecodeArgs &a) {
    need(a.q && a.kcache && a.vcache && a.sink && a.out, "null tensor");
    need(a.B >= 1 && a.Hq % a.Hkv == 0 && a.T >= 1 && a.T <= a.R && a.W <= a.R, "sizes");
    need(a.D == 64 || a.D == 128, "head dim");
}
}  // namespace

namespace swa {
hipError_t launch_rope_append(const AppendArgs &a, bool, hipStream_t) {
    need(a.B >= 1 && a.T >= 1 && a.T <= a.R && a.theta > 1.0, "append sizes");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_prefill_ring_bf16(const PrefillArgs &a, hipStream_t) {
    prefill_ok(a);
    need(prefill_ring_supported(a.window, a.Hq / a.Hkv), "ring kernel chosen outside its range");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_stream_bf16(const PrefillArgs &a, hipStream_t) {
    prefill_ok(a);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_stream_bf16_block_max(const PrefillArgs &a, float *bmax, int block_k, hipStream_t) {
    prefill_ok(a);
    need(bmax != nullptr && block_k >= 32 && block_k % 32 == 0, "block max");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_ring_decode_bf16(const DecodeArgs &a, hipStream_t) {
    decode_ok(a);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_splitkv_bf16(const PrefillArgs &a, void *ws, hipStream_t) {
    prefill_ok(a);
    need(ws != nullptr, "workspace");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_splitkv_bf16_static(const PrefillArgs &a, hipStream_t) {
    prefill_ok(a);
    need(splitkv_workspace_bytes(a.B, a.Hq, a.Hkv, a.S, a.S_kv, a.D) <= kStaticScratchBytes,
         "static scratch too small");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_backward_pre(const BackwardArgs &, hipStream_t, bool) { return hipSuccess; }
hipError_t launch_backward_dsink(const BackwardArgs &, hipStream_t) { return hipSuccess; }
hipError_t launch_backward_f32(const BackwardArgs &a, hipStream_t) {
    need(a.ws_dsum && a.ws_l2 && a.ws_part && a.window >= 1 && a.window <= a.S, "backward");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_backward_bf16(const BackwardArgs &a, hipStream_t s) {
    return launch_backward_f32(a, s);
}
hipError_t launch_generic_f32_linear(const PrefillArgs &a, hipStream_t) {
    prefill_ok(a);
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_generic_f32_ring(const DecodeArgs &a, hipStream_t) {
    decode_ok(a);
    ++g_launches;
    return hipSuccess;
}
}  // namespace swa
