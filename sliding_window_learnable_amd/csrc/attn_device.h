// attn_device.h -- device building blocks shared by the gfx950 attention
// kernels: bf16 MFMA tiles, operand layouts, LDS staging and the
// sink-seeded softmax state.
//
// MFMA tile used everywhere: v_mfma_f32_32x32x16_bf16 (64-lane wavefront).
//   A (32 x 16): lane l holds row (l & 31), k-elements 8*(l >> 5) + e, e = 0..7
//   B (16 x 32): lane l holds col (l & 31), k-elements 8*(l >> 5) + e
//   C (32 x 32): lane l holds col (l & 31), rows 8*(r >> 2) + 4*(l >> 5) + (r & 3)
//                for accumulator register r = 0..15.
// Scores are computed transposed, S^T = K Q^T (rows = keys, cols = queries),
// so that every lane owns one query column: row reductions become in-lane
// reductions plus one exchange with lane l ^ 32, and the score registers are
// already laid out as the B operand of the next product O^T = V^T P^T.
// To make that hand-off free, the A rows of S^T are fed keys in the order
//   row m = 8j + 4h + c  <-  key 16*(j >> 1) + 8*h + 4*(j & 1) + c
// after which accumulator register r of lane l holds the key
//   16*(r >> 3) + 8*(l >> 5) + (r & 7)
// i.e. registers 0..7 are 8 consecutive keys = one B operand of a K=16 step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// An empty asm that reads x: the compiler waits here for the load that
// produced x, so no wait for it is left to land inside a later loop (where
// it would also wait for that loop's own prefetches).
template <class V>
__device__ __forceinline__ void retire(const V &x) {
    asm volatile("" ::"v"(x));
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// Key index (0..31 within a 32-key tile) that A row m of S^T is fed with.
__device__ __forceinline__ int score_row_key(int m) {
    const int j = m >> 3, h = (m >> 2) & 1, c = m & 3;
    return 16 * (j >> 1) + 8 * h + 4 * (j & 1) + c;
}

// Key index (0..31) held by accumulator register r of lane `lane` in S^T.
__device__ __forceinline__ int score_reg_key(int r, int lane) {
    return 16 * (r >> 3) + 8 * (lane >> 5) + (r & 7);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16 &p, int half) {
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (bf16)p[8 * half + e];
    return b;
}

__device__ __forceinline__ float wave_xor32_max(float x) {
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_xor32_sum(float x) {
    return x + __shfl_xor(x, 32);
}

// Work-group barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its outstanding global loads and stores (which
// __syncthreads() would also drain), so prefetches and output stores stay
// in flight across it.  The memory clobber keeps the compiler from moving
// LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Waits for this wave's LDS operations while holding the data registers of
// the LDS writes just issued: the compiler treats a write's data registers
// as free once the write has issued, but under load (matrix products still
// in flight, bank-conflicted lanes) the LDS unit can read them later than
// the next instructions that reuse them.  Naming them as operands keeps
// them intact until the writes are complete.
template <class V, int N>
__device__ __forceinline__ void lds_settle(const V (&w)[N]) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "lds_settle holds 1, 2, 4 or 8 registers");
    if constexpr (N == 8)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     :
                     : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]),
                       "v"(w[6]), "v"(w[7])
                     : "memory");
    else if constexpr (N == 4)
        asm volatile("s_waitcnt lgkmcnt(0)" : : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]) : "memory");
    else if constexpr (N == 2)
        asm volatile("s_waitcnt lgkmcnt(0)" : : "v"(w[0]), "v"(w[1]) : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : : "v"(w[0]) : "memory");
}

// Waits until at most N vector memory operations of this wave are
// outstanding, holding the registers in w until then: the data registers
// of earlier 16-byte stores, which the store may read after the
// instructions that follow it (the compiler treats them as free once the
// store has issued).  N counts the operations issued after those stores.
template <int N, class V, int K>
__device__ __forceinline__ void hold_until_done(const V (&w)[K]) {
    static_assert(K == 4 || K == 8, "hold_until_done holds 4 or 8 registers");
    if constexpr (K == 8)
        asm volatile("s_waitcnt vmcnt(%8)"
                     :
                     : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]),
                       "v"(w[6]), "v"(w[7]), "n"(N)
                     : "memory");
    else
        asm volatile("s_waitcnt vmcnt(%4)" : : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "n"(N)
                     : "memory");
}

// ---------------------------------------------------------------------------
// Buffer addressing.  A 128-bit resource (base, byte range) lives in SGPRs,
// each lane supplies one 32-bit byte offset, uniform offsets go in an SGPR.
// Loads past the range return zeros and stores past it are dropped, so tile
// edges need no clamping or branches.  (Word 3 = 0x00020000 is the raw,
// untyped 32-bit buffer format of the CDNA family.)
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ bf16x8 buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_store16(bf16x8 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, 0);
}
// Streaming store (cache policy "nt"): output written once and not read
// back by this kernel.  Whole 128-byte segments only.
__device__ __forceinline__ void buf_store16_nt(bf16x8 v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, 2);
}
__device__ __forceinline__ void buf_store_f32(float v, rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, 0);
}
// A byte offset beyond any range a descriptor here can have: stores to it
// are dropped, loads from it return zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Largest power of two dividing G, capped at 8: waves per work-group when
// one wave serves one query head of a GQA group.
// Operand tiles copied straight into LDS (Q, dO, K, V rows) are unpadded
// rows whose 16-byte chunks are XOR-swizzled by row (chunk c of row r sits
// at c ^ swz(r)), so that both the row reads of score products (16 rows,
// one chunk) and the transposing reads of value / gradient products (4 rows
// x 32 dims per 32 lanes) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: in each 16-lane group, lane j supplies the address of
// 4 bf16 (row j/4, dims 4(j%4)..+3 of a 16-dim span); lane i receives the
// element at dim i of each of the 4 rows.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16 *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
    return __builtin_bit_cast(bf16x4, r);
}
// The same read at an LDS byte address.
__device__ __forceinline__ bf16x4 lds_read_tr_at(uint32_t a) {
    const s16x4 r =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(size_t)a);
    return __builtin_bit_cast(bf16x4, r);
}
// 16 bytes at an LDS byte address.
__device__ __forceinline__ bf16x8 lds_read16_at(uint32_t a) {
    return *(__attribute__((address_space(3))) const bf16x8 *)(size_t)a;
}
// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(__attribute__((address_space(3))) const void *)p;
}

// Buffer descriptor as four scalar dwords (raw buffer, num_records bytes).
__device__ __forceinline__ u32x4 sgpr_rsrc(const void *base, uint32_t bytes) {
    const unsigned long long p = (unsigned long long)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((unsigned)p);
    r[1] = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// ---------------------------------------------------------------------------
// LDS poisoning, for debug builds (-DSWA_LDS_POISON; never in the product
// library).  Every kernel fills its LDS with NaN patterns on entry, and every
// buffer->LDS copy first overwrites the 16 bytes per lane it is about to
// fill: a read of LDS that no copy or store has reached yet -- a slot read
// before its copy landed (a missing wait or barrier), a tile never staged,
// a stale slot index -- then yields NaN in the results instead of plausible
// old values.  Results of a correct kernel are bit-identical either way.
// ---------------------------------------------------------------------------
#ifdef SWA_LDS_POISON
constexpr bool kLdsPoison = true;
#else
constexpr bool kLdsPoison = false;
#endif
constexpr uint32_t kPoisonWord = 0x7FC17FC1u;   // two bf16 NaNs, also an fp32 NaN

// Whole-work-group fill of an LDS object, then a barrier.  Every wave of the
// work-group must call it (before any early return).
template <class T>
__device__ __forceinline__ void lds_poison_all(T &obj) {
    if constexpr (kLdsPoison) {
        uint32_t *w = reinterpret_cast<uint32_t *>(&obj);
        for (unsigned i = threadIdx.x; i < sizeof(T) / 4; i += blockDim.x) w[i] = kPoisonWord;
        __syncthreads();
    }
}
// One wave's fill of its own LDS object (no barrier: only this wave uses it).
template <class T>
__device__ __forceinline__ void lds_poison_wave(T &obj) {
    if constexpr (kLdsPoison) {
        uint32_t *w = reinterpret_cast<uint32_t *>(&obj);
        for (unsigned i = threadIdx.x & 63; i < sizeof(T) / 4; i += 64) w[i] = kPoisonWord;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}
// The 16 bytes a copy of this lane will write at LDS address lds + 16 * lane.
__device__ __forceinline__ void lds_poison_lane16_at(uint32_t lds) {
    if constexpr (kLdsPoison) {
        const unsigned la = lds + 16u * (threadIdx.x & 63);
        u32x4 p;
        p[0] = p[1] = p[2] = p[3] = kPoisonWord;
        asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(la), "v"(p) : "memory");
    }
}
__device__ __forceinline__ void lds_poison_lane16(const void *lds) {
    lds_poison_lane16_at((unsigned)(size_t)(__attribute__((address_space(3))) const void *)lds);
}

// Buffer -> LDS copy (no registers): lane l's 16 bytes at voff land at
// lds + 16 l; out-of-range dwords land as zero.  Written as asm so that the
// compiler does not wait for every copy before each LDS read (it cannot
// tell the copies' targets from the tiles being read); the copies are
// waited for explicitly (vmcnt) before the barrier that publishes them.
// m0 is reserved to the compiler, which uses it for nothing in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(u32x4 r, const void *lds, uint32_t voff) {
    lds_poison_lane16(lds);
    const unsigned la = __builtin_amdgcn_readfirstlane(
        (unsigned)(size_t)(__attribute__((address_space(3))) const void *)lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(la),
                 "v"(voff), "s"(r)
                 : "memory", "m0");
}
// The same copy to an LDS byte address, with a uniform byte offset added
// in the scalar offset field (no per-lane add); and with the non-temporal
// cache policy, for data read exactly once in whole cache lines per
// instruction.
__device__ __forceinline__ void dma16_at(u32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
    lds_poison_lane16_at(lds);
    const unsigned la = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(la),
                 "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma16_nt_at(u32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
    lds_poison_lane16_at(lds);
    const unsigned la = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds" ::"s"(la),
                 "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__host__ __device__ constexpr int waves_for_group(int G) {
    return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

}  // namespace swa
