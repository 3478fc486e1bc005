// plan.hip -- host-only launch planning shared by the entry points and the
// kernel launchers: which kernel serves a call, how long a sequence slice
// one buffer descriptor can cover, how global decode is split over the keys
// and how much workspace each path needs.  No device code: this file also
// builds as plain C++ (with api.hip) for the sanitizer test of the host side.
#include <algorithm>

#include "launch.h"

namespace swa {

// Largest chunk (a multiple of 32 positions) whose buffer windows stay below
// 2^31 bytes: q/out rows [c0, c1) of all heads, k/v rows [r0, c1) of one KV
// head including the (ntw-1)-tile halo.
int prefill_chunk_cap(int Hq, int Hkv, int D, int ntw) {
    constexpr long kTile = 32;
    const long limit = 1L << 31;
    const long q_rows = limit / ((long)Hq * D * 2);
    const long kv_rows = limit / ((long)Hkv * D * 2) - kTile * (ntw - 1);
    const long rows = q_rows < kv_rows ? q_rows : kv_rows;
    return (int)(rows < kTile ? kTile : (rows / kTile) * kTile);
}

// The LDS-ring prefill serves windows spanning exactly five 32-key tiles
// with one wave per query head of a GQA group.
bool prefill_ring_supported(int window, int G) {
    const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
    return window >= 98 && window <= 129 && g_ok;
}

// Global decode: enough splits over the keys that about 2048 waves (two per
// SIMD) each stream one key range; ranges are whole 32-key chunks, and one
// split's buffer window (kps rows of all KV heads) stays below 2^31 bytes.
SplitPlan plan_split(int B, int Hq, int Hkv, int S_q, int S_kv, int D) {
    constexpr long kTargetWaves = 2048;
    constexpr int ck = 32;
    const int G = Hq / Hkv;
    const int n_ct = (G * S_q + 31) / 32;
    const long pairs = (long)B * Hkv * n_ct;
    const int max_splits = (S_kv + ck - 1) / ck;
    int want = (int)((kTargetWaves + pairs - 1) / pairs);
    want = std::max(1, std::min(want, max_splits));
    int kps = (S_kv + want - 1) / want;
    kps = ((kps + ck - 1) / ck) * ck;
    const long cap = ((1L << 31) / ((long)Hkv * D * 2)) / ck * ck;
    if (kps > cap) kps = (int)cap;
    const int n_splits = (S_kv + kps - 1) / kps;
    return {n_splits, kps, n_ct};
}

int splitkv_num_splits(int B, int Hq, int Hkv, int S_q, int S_kv) {
    return plan_split(B, Hq, Hkv, S_q, S_kv, 128).n_splits;
}

// Short query blocks (at most 64 (token, head) columns per KV head) are split
// over the keys; longer ones take the streaming kernel.
bool splitkv_preferred(int Hq, int Hkv, int S_q, int S_kv) {
    (void)S_kv;
    return (long)(Hq / Hkv) * S_q <= 64;
}

// Partial records (acc[D], m, l) per (split, sequence, head, query row).
size_t splitkv_workspace_bytes(int B, int Hq, int Hkv, int S_q, int S_kv, int D) {
    const SplitPlan p = plan_split(B, Hq, Hkv, S_q, S_kv, D);
    return (size_t)p.n_splits * B * Hq * S_q * (D + 2) * sizeof(float);
}

// Backward workspace: D_i and lse*log2(e) per (sequence, head, row), and one
// sink-gradient partial per 32-row tile.
size_t backward_workspace_bytes(int B, int Hq, int S) {
    const size_t tiles = (size_t)(S + kBackwardRows - 1) / kBackwardRows;
    return 4 * (size_t)B * Hq * (2 * (size_t)S + tiles);
}

}  // namespace swa
