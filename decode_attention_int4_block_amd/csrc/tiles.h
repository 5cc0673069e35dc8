// Building blocks shared by the decode and the prefill attention kernels:
// MFMA operand packing, the exact fp16 hi/lo split, wave-uniform and
// constant-space loads, the direct global->LDS step copies and their waits.
#pragma once

#include <hip/hip_fp16.h>

#include "common.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

constexpr int kStages = 3;
constexpr int kStageBytes = 4352;       // 4 x 1 KB codes + 256 B params
constexpr int kDmaPerStep = 5;

// Stage layout of the params (INT4: tokens 0..31 of the step; INT8: entries 0..15).
constexpr int kStKP = 4096;             // key (scale, zero) of token t at kStKP + 4 t
constexpr int kStVP = 4224;             // value (scale, zero) of token t at kStVP + 4 t

__device__ inline floatx4 mfma16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline half8 pack8(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
    u32x4 u = {a0, a1, a2, a3};
    return __builtin_bit_cast(half8, u);
}

// f16 pair of (a, b), round to nearest (keeps f16 subnormals: the lo parts
// of small values live there).
__device__ inline uint32_t f16x2(float a, float b) {
    const half2v h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

__device__ inline float h_lo(uint32_t w) { return (float)__builtin_bit_cast(half2v, w)[0]; }
__device__ inline float h_hi(uint32_t w) { return (float)__builtin_bit_cast(half2v, w)[1]; }

// hi = f16(a / S, b / S), lo = f16(a - S hi, b - S hi): S hi + lo carries ~21
// bits of a and b, and lo keeps absolute steps of 2^-24 for small values.
// lo must be taken against the very f16 values packed into hi: the compiler
// would otherwise re-derive them from a and b (e.g. by fusing the product that
// formed a into a single-rounding f16 conversion), and where the two roundings
// differ, hi + lo misses a by one f16 step of hi.  The empty asm makes the
// packed word opaque.
template <int S>
__device__ inline void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    constexpr float inv = 1.0f / S;
    hi = f16x2(a * inv, b * inv);
    uint32_t h = hi;
    __asm__("" : "+v"(h));
    lo = f16x2(fmaf(h_lo(h), -(float)S, a), fmaf(h_hi(h), -(float)S, b));
}

__device__ inline float bf16f(uint32_t b) { return __uint_as_float(b << 16); }

template <typename T>
__device__ inline T ldg(const void *p) { return *reinterpret_cast<const T *>(p); }

typedef __attribute__((address_space(3))) void *lds_ptr;

// Values every lane holds the same copy of, made visibly wave-uniform so that
// the loads they index become scalar loads.
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uni64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Read-only launch inputs (lengths, slots, block table) read through the
// constant address space so that wave-uniform reads are scalar loads.
__device__ inline int ldc(const int32_t *p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

// 16 bytes per lane from global memory (uniform base + per-lane offset) into
// LDS at dst + 16 * lane.
__device__ inline void dma16(const uint8_t *base, uint32_t off, uint8_t *dst_lds) {
    __builtin_amdgcn_global_load_lds(base + off, (lds_ptr)dst_lds, 16, 0, 0);
}
// The same copy with the non-temporal cache policy (the "nt" bit of the load's
// cache-policy operand), for data a launch reads exactly once: every load of the
// decode kernel (step subblocks, block-table entries, queries, appended rows).
// Streamed this way they stop displacing from L2 and the Infinity Cache what
// the step does reuse (the split-K pieces the combine reads next, the row table,
// the kernel's code and arguments); measured on MI355X the decode launch runs
// 11-14% faster on the Qwen3 batches and up to 10% on refill.
constexpr int kCachePolicyNonTemporal = 2;
__device__ inline void dma16_stream(const uint8_t *base, uint32_t off, uint8_t *dst_lds) {
    __builtin_amdgcn_global_load_lds(base + off, (lds_ptr)dst_lds, 16, 0, kCachePolicyNonTemporal);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define KVQ_VMCNT(n) (((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define KVQ_LGKM0 ((0xF) | (0x3 << 14) | (0x7 << 4))
// The waitcnt intrinsic does not order memory accesses at the IR level; the
// empty asm with a memory clobber keeps LDS reads of a stage below its wait.
#define KVQ_FENCE() __asm__ volatile("" ::: "memory")

__device__ inline void wait_vm_steps(int steps_after) {
    // outstanding DMA instructions allowed = kDmaPerStep * steps_after
    static_assert(kStages <= 4 && kDmaPerStep == 5, "wait table covers up to 4 stages x 5 loads");
    if (steps_after <= 0) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(0));
    else if (steps_after == 1 || kStages == 2) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(5));
    else if (steps_after == 2 || kStages == 3) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(10));
    else __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(15));
    KVQ_FENCE();
}

__device__ inline void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(KVQ_LGKM0);
    KVQ_FENCE();
}

__device__ inline uint32_t lds32(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

// score (log2 units / K1) of one token from its raw code dot product d
__device__ inline float tscore(float d, uint32_t kp, float Rh) {
    return fmaf(d, h_lo(kp), h_hi(kp) * Rh);
}

// ---- 2- and 3-bit main-cache codes as MFMA operands (decode and prefill) ----
// The step copies of both kernels put a 2- or 3-bit step in LDS the same way:
// lane (G, n) reads 8 bytes of low-plane key codes (token n, dims 32 G ..) and
// 8 of value codes, plus a high-plane dword each at 3 bits.
// 2-bit codes of one dword half-pair as the four f16 subnormal pairs the INT4
// nibble masks give: field f of bytes 0 and 2 (dims f and 4 + f of a chunk)
// scaled 1 for even f and 16 for odd f, so that the same query operand (and the
// same value tile scaling) serves both widths.
__device__ inline uint32_t int2_field(uint32_t x, int f) {
    switch (f) {
        case 0: return x & 0x00030003u;
        case 1: return (x << 2) & 0x00300030u;
        case 2: return (x >> 4) & 0x00030003u;
        default: return (x >> 2) & 0x00300030u;
    }
}
__device__ inline half8 int2_chunk(uint32_t x) {
    return pack8(int2_field(x, 0), int2_field(x, 1), int2_field(x, 2), int2_field(x, 3));
}
// The decode kernel's 2-bit operands leave each code at its field position:
// operand dword f holds field f of bytes 0 and 2 (dims f, 4 + f of the chunk)
// as (4^f c) 2^-24, one AND each; the query pairs carry the inverse scales.
__device__ inline half8 int2_chunk_pos(uint32_t x) {
    return pack8(x & 0x00030003u, x & 0x000C000Cu, x & 0x00300030u, x & 0x00C000C0u);
}
// INT8 key nibbles (INT4 order: dims (0, 4), (1, 5), (2, 6), (3, 7) of the
// chunk) at those scales: 1, 4, 16, 64 (15 * 64 < 1024 stays subnormal).
__device__ inline half8 nibble_chunk_pos(uint32_t x) {
    return pack8(x & 0x000F000Fu, (x >> 2) & 0x003C003Cu, (x >> 4) & 0x00F000F0u, (x >> 6) & 0x03C003C0u);
}
// 3-bit codes: a 2-bit field with its high bit ORed in at value 4 (bit 2 or 6
// of each half, next to the field's two bits).  h holds the high bits of the
// field's codes at bits 2 / 6 (+ 16) for the even / odd fields, or 8 above.
__device__ inline uint32_t int3_field(uint32_t x, uint32_t h, int f) {
    const uint32_t hs = f < 2 ? h : h >> 8;
    return int2_field(x, f) | (hs & ((f & 1) ? 0x00400040u : 0x00040004u));
}
// key chunk i: the high-plane dword shifted to its bytes (key plane layout in quant.h)
__device__ inline half8 int3_key_chunk(uint32_t x, uint32_t hh, int i) {
    const uint32_t h = i == 0 ? hh : (i == 1 ? hh >> 1 : (i == 2 ? hh << 2 : hh << 1));
    return pack8(int3_field(x, h, 0), int3_field(x, h, 1), int3_field(x, h, 2), int3_field(x, h, 3));
}
// value field f of low-plane dword cc, bytes (0, 2) (odd = false) or (1, 3): the
// high byte's bit for (cc, f) moved to bit 2 / 6 (value plane layout in quant.h)
__device__ inline uint32_t int3_value_field(uint32_t x, uint32_t hv, int cc, int f, bool odd) {
    const int g = cc == 0 ? (0x7362 >> (4 * f)) & 15 : (0x5140 >> (4 * f)) & 15;
    const int s = g + (odd ? 8 : 0) - ((f & 1) ? 6 : 2);
    const uint32_t h = s >= 0 ? hv >> s : hv << (-s);
    return int2_field(x, f) | (h & ((f & 1) ? 0x00400040u : 0x00040004u));
}

}  // namespace kvq
