// Split-K paged decode attention over the INT4 cache and the INT8 side cache.
//
// KV4-RL ("Key Contributions" item 4, "Methodology in Plain English"): the
// rotated query attends the INT4 region and the INT8 region as disjoint sets,
// packed codes are consumed directly, scale and offset are applied after the
// dot-product reduction, and the regions are merged through softmax
// statistics.  Here every worker's partial result (m, l, acc) is such a set of
// statistics, so the INT4/INT8 merge and the split-K merge are one log-sum-exp
// combine.
//
// Work: a (row, KV head) segment is a list of units of roughly equal bytes --
// INT4 steps of 32 positions and INT8 steps of 16 ring entries -- and the units
// of all segments are split evenly over the resident waves (one wave per
// workgroup), so a long-tailed length mix costs every wave the same.  A segment
// that one wave covers completely is finished by that wave; the others leave
// partial statistics for the combine kernel.
//
// Memory: each wave streams its steps through a ring of kStages LDS buffers
// with direct global->LDS loads (5 x 16 B per lane per step), so the bytes in
// flight cost no VGPRs.
//
// Compute per step, with 16x16x32 f16 MFMA:
//   scores[tok][col] = codes[tok][:] . Q[:][col]     (A = codes, B = query)
//   acc[row][dim]   += P[row][tok] * vcodes[tok][dim] (A = p, B = codes)
// The query and p*scale_v are split into f16 hi + lo parts so products keep
// fp32 accuracy.  With a query group g <= 8 the hi and lo parts share one MFMA:
// hi in columns (rows) [0, G), lo in [G, 2G) of the 16 the instruction has, and
// the two halves are added afterwards.  4-bit and 8-bit codes become f16 values
// exactly by masking them into the mantissa of a subnormal (code * 2^-24, or
// code * 2^-20 for the high nibble of a byte, compensated in the other operand
// or the accumulator).
#include <hip/hip_fp16.h>

#include "common.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

constexpr int kStages = 4;
constexpr int kStageBytes = 4352;       // 4 x 1 KB codes + 256 B params
constexpr int kDmaPerStep = 5;

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

// hi = f16(x), lo = f16(x - hi) for a pair: hi + lo carries ~21 bits of x.
__device__ inline void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = f16x2(a, b);
    const half2v h = __builtin_bit_cast(half2v, hi);
    lo = f16x2(a - (float)h[0], b - (float)h[1]);
}

__device__ inline float h_lo(uint32_t w) { return (float)__builtin_bit_cast(half2v, w)[0]; }
__device__ inline float h_hi(uint32_t w) { return (float)__builtin_bit_cast(half2v, w)[1]; }

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

// Cross-lane moves (VALU, no LDS): values of the lane 16 / 32 apart, and DPP
// shifts inside 16-lane rows.
__device__ inline float xor16(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
}
__device__ inline float xor32(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
}
__device__ inline float max_rows(float x) {      // max over lanes l, l^16, l^32, l^48
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_rows(float x) {      // sum over lanes l, l^16, l^32, l^48
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
template <int N>
__device__ inline float row_shl(float x) {        // lane i <- lane i + N (same row; 0 past the edge)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xF, 0xF, true));
}
template <int N>
__device__ inline uint32_t row_shr(uint32_t x) {  // lane i <- lane i - N
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x110 + N, 0xF, 0xF, true);
}

// 16 bytes per lane from global memory (uniform base + per-lane offset) into
// LDS at dst + 16 * lane.
__device__ inline void dma16(const uint8_t *base, uint32_t off, uint8_t *dst_lds) {
    __builtin_amdgcn_global_load_lds(base + off, (lds_ptr)dst_lds, 16, 0, 0);
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
    static_assert(kStages == 4 && kDmaPerStep == 5, "wait table assumes 4 stages x 5 loads");
    if (steps_after <= 0) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(0));
    else if (steps_after == 1) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(5));
    else if (steps_after == 2) __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(10));
    else __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(15));
    KVQ_FENCE();
}

__device__ inline void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(KVQ_LGKM0);
    KVQ_FENCE();
}

// ---------------------------------------------------------------------------
// Data of one step as read from its LDS stage.
struct StepRegs {
    u32x4 kA, kB;       // INT4: key codes of token l%16 (A/B), dims 32G..+32
                        // INT8: key bytes of entry l%16, dims 32G..+16 (kA) and +16..+32 (kB)
    u32x4 vA, vB;       // INT4: value codes, dims n + 32c / n + 16 + 32c, tokens 4G..4G+3
                        // INT8: value bytes, tiles 0..3 (vA) and 4..7 (vB), entries 4G..4G+3
    u32x4 kpA, kpB;     // key params of tokens 4G..4G+3 (INT8: kpA only)
    u32x4 vpA, vpB;     // value params
};

// GP: columns (rows) per hi/lo half -- 4 or 8 packs hi and lo into one MFMA,
// 16 uses separate MFMAs for hi and lo.
template <int GP>
struct SegCtx {
    static constexpr bool kPacked = GP <= 8;
    static constexpr int kQ = kPacked ? 1 : 2;     // query operand sets per chunk
    int lane, G, n, col;
    int g;
    half8 q4[kQ][4];    // query operands (INT4 nibble order; INT8 keys are split into nibbles)
    float K1;           // 2^(24 - e) * log2(e) / sqrt(128)
    float K2;           // sum(q~) * log2(e) / sqrt(128) of head col % GP
    float m, lsum, zsum;
    floatx4 O[8];       // acc[row 4G+i][16 t + n], odd tiles scaled by 16
};

// Wave-uniform position in the unit stream of one worker.
struct Cursor {
    int b, hk;          // segment (row, KV head)
    RowPlan rp;
    int r;              // unit index inside the segment
    int64_t u;          // global unit
};

__device__ inline void cursor_next(const DecodeArgs &a, Cursor &c) {
    ++c.u;
    if (++c.r < c.rp.cost) return;
    c.r = 0;
    if (++c.hk < a.H) return;
    c.hk = 0;
    for (++c.b; c.b < a.B; ++c.b) {
        c.rp = row_plan(ldc(a.ctx_len, c.b), a.s, a.w);
        if (c.rp.cost > 0) return;
    }
}

// Block table entries and slot the producer needs for the step at a cursor;
// looked up one step ahead so the scalar loads overlap the compute.
struct Lookup {
    int slot, pageA, pageB;
};

__device__ inline Lookup lookup(const DecodeArgs &a, const Cursor &c) {
    Lookup k;
    k.slot = ldc(a.slot, c.b);
    k.pageA = 0;
    k.pageB = 0;
    if (c.r < c.rp.n4) {
        const int pos0 = (c.rp.k0 + c.r) * 32;
        const int32_t *bt = a.block_table + (int64_t)k.slot * a.bt_stride;
        k.pageA = ldc(bt, pos0 >> a.logP);
        k.pageB = (pos0 + 16 < c.rp.hi4) ? ldc(bt, (pos0 + 16) >> a.logP) : k.pageA;
    }
    return k;
}

template <int GP>
__device__ inline void build_query(const DecodeArgs &a, int b, int hk, SegCtx<GP> &c) {
    // lane column col: head col % GP, part hi (col < GP) or lo (GP <= col < 2GP);
    // unpacked: every column < g carries its head in both operand sets.
    const int head = SegCtx<GP>::kPacked ? (c.col % GP) : c.col;
    const bool live = (SegCtx<GP>::kPacked ? c.col < 2 * GP : true) && head < c.g;
    float x[32];
    if (live) {
        const uint16_t *qp = a.q + ((int64_t)b * a.Hq + (int64_t)hk * c.g + head) * kHeadDim + 32 * c.G;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            u32x4 w = ldg<u32x4>(qp + 8 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * v + 2 * e] = bf16f(w[e] & 0xFFFFu);
                x[8 * v + 2 * e + 1] = bf16f(w[e] >> 16);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = 0.0f;
    }
    // block Hadamard (orthonormal) of the query; in-lane strides 1..16
#pragma unroll
    for (int len = 1; len < 32; len <<= 1) {
        if (len < a.h) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if ((i & len) == 0) {
                    float u = x[i], v = x[i + len];
                    x[i] = u + v;
                    x[i + len] = u - v;
                }
            }
        }
    }
    // strides 32 and 64 cross lanes (lane groups G differ in bit 0 / bit 1)
    if (32 < a.h) {
        const bool upper = (c.lane & 16) != 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float p = xor16(x[i], c.lane);
            x[i] = upper ? (p - x[i]) : (x[i] + p);
        }
    }
    if (64 < a.h) {
        const bool upper = (c.lane & 32) != 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const float p = xor32(x[i], c.lane);
            x[i] = upper ? (p - x[i]) : (x[i] + p);
        }
    }
    float sum = 0.0f, amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        x[i] *= a.inv_sqrt_h;
        sum += x[i];
        amax = fmaxf(amax, fabsf(x[i]));
    }
    sum = sum_rows(sum);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    int E = 0;
    (void)frexpf(amax, &E);
    const int e = amax > 0.0f ? 14 - E : 0;      // |q * 2^e| < 2^14
    const float sc = ldexpf(1.0f, e);
    const float c0 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
    c.K1 = ldexpf(c0, 24 - e);
    c.K2 = sum * c0;
    const bool lo_part = SegCtx<GP>::kPacked && c.col >= GP;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float *y = x + 8 * i;
        uint32_t h[4], l[4];
        // nibble order of a code dword: dims 0,4 | 1,5 (/16) | 2,6 | 3,7 (/16)
        split2(y[0] * sc, y[4] * sc, h[0], l[0]);
        split2(y[1] * sc * 0.0625f, y[5] * sc * 0.0625f, h[1], l[1]);
        split2(y[2] * sc, y[6] * sc, h[2], l[2]);
        split2(y[3] * sc * 0.0625f, y[7] * sc * 0.0625f, h[3], l[3]);
        if constexpr (SegCtx<GP>::kPacked) {
            c.q4[0][i] = lo_part ? pack8(l[0], l[1], l[2], l[3]) : pack8(h[0], h[1], h[2], h[3]);
        } else {
            c.q4[0][i] = pack8(h[0], h[1], h[2], h[3]);
            c.q4[1][i] = pack8(l[0], l[1], l[2], l[3]);
        }
    }
}

// Raw score sums of the 4 tokens of one subblock (packed mode: hi + lo columns).
template <int GP>
__device__ inline floatx4 combine_cols(floatx4 d) {
    if constexpr (GP <= 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] += row_shl<GP>(d[i]);
    }
    return d;
}

// Online-softmax update for this lane's 8 scores (tokens 4G+i of subblocks A,
// B) and the value MFMA A operands (rows = heads, k = [A0 A2 A1 A3 B0 B2 B1 B3]).
template <int GP, bool FULL>
__device__ inline void softmax_step(SegCtx<GP> &c, float sc[8], const u32x4 &vpA, const u32x4 &vpB,
                                    const bool valid[8], half8 pop[2]) {
    float mstep = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mstep = fmaxf(mstep, sc[i]);
    mstep = max_rows(mstep);
    const float mnew = fmaxf(c.m, mstep);
    const bool head_lane = (SegCtx<GP>::kPacked ? c.col < GP : true) && c.col < c.g;
    const bool grow = head_lane && mnew > c.m;
    if (__any(grow)) {
        const float alpha = grow ? (c.m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(c.m - mnew)) : 1.0f;
        c.lsum *= alpha;
        c.zsum *= alpha;
        const int rb = 4 * (c.lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rb + i;
            const float ar = __shfl(alpha, SegCtx<GP>::kPacked ? row % GP : row, 64);
#pragma unroll
            for (int t = 0; t < 8; ++t) c.O[t][i] *= ar;
        }
        if (grow) c.m = mnew;
    }
    const float m = c.m;
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t vp = i < 4 ? vpA[i] : vpB[i - 4];
        const float p = __builtin_amdgcn_exp2f(sc[i] - m);
        if (FULL) {
            c.lsum += p;
            c.zsum = fmaf(p, h_hi(vp), c.zsum);
            pv[i] = p * h_lo(vp);
        } else {
            // params of positions past the written context are arbitrary bytes
            // (possibly NaN as fp16): select, never multiply by zero
            c.lsum += valid[i] ? p : 0.0f;
            c.zsum = valid[i] ? fmaf(p, h_hi(vp), c.zsum) : c.zsum;
            pv[i] = valid[i] ? p * h_lo(vp) : 0.0f;
        }
    }
    uint32_t h[4], l[4];
    split2(pv[0], pv[2], h[0], l[0]);
    split2(pv[1], pv[3], h[1], l[1]);
    split2(pv[4], pv[6], h[2], l[2]);
    split2(pv[5], pv[7], h[3], l[3]);
    if constexpr (SegCtx<GP>::kPacked) {
        // rows [GP, 2GP) take the lo part of head row - GP
        const bool lo_row = c.col >= GP;
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t s = row_shr<GP>(l[k]);
            o[k] = lo_row ? s : h[k];
        }
        pop[0] = pack8(o[0], o[1], o[2], o[3]);
    } else {
        pop[0] = pack8(h[0], h[1], h[2], h[3]);
        pop[1] = pack8(l[0], l[1], l[2], l[3]);
    }
}

// ---------------------------------------------------------------------------
// Producer: issue the 5 direct-to-LDS loads of the step at cursor c into stage st.
__device__ inline void issue_step(const DecodeArgs &a, const Cursor &c, const Lookup &k, uint8_t *st,
                                  uint32_t offK4, uint32_t offV4, uint32_t offP4,
                                  uint32_t offK8, uint32_t offV8, uint32_t offP8, int lane) {
    if (c.r < c.rp.n4) {
        const int pos0 = (c.rp.k0 + c.r) * 32;
        const int subs = a.P >> 4;
        const uint8_t *baseA = a.int4_pool +
            ((size_t)((int64_t)k.pageA * a.H + c.hk) * subs + ((pos0 & (a.P - 1)) >> 4)) * kSub4Bytes;
        // subblock B past the INT4 region is never used; re-read A (valid memory)
        const uint8_t *baseB = (pos0 + 16 < c.rp.hi4)
            ? a.int4_pool + ((size_t)((int64_t)k.pageB * a.H + c.hk) * subs + (((pos0 + 16) & (a.P - 1)) >> 4)) * kSub4Bytes
            : baseA;
        dma16(baseA, offK4, st + 0);
        dma16(baseB, offK4, st + 1024);
        dma16(baseA, offV4, st + 2048);
        dma16(baseB, offV4, st + 3072);
        if (lane < 16) dma16((lane & 4) ? baseB : baseA, offP4, st + 4096);
    } else {
        const int sub = c.r - c.rp.n4;
        const uint8_t *base = a.int8_pool + ((size_t)((int64_t)k.slot * a.H + c.hk) * a.nr8 + sub) * kSub8Bytes;
        dma16(base, offK8, st + 0);
        dma16(base, offK8 + 16, st + 1024);
        dma16(base, offV8, st + 2048);
        dma16(base, offV8 + 16, st + 3072);
        if (lane < 8) dma16(base, offP8, st + 4096);
    }
}

__device__ inline StepRegs read_stage(const uint8_t *st, bool int4, int lane) {
    StepRegs r;
    const int G = lane >> 4;
    r.kA = *reinterpret_cast<const u32x4 *>(st + lane * 16);
    r.kB = *reinterpret_cast<const u32x4 *>(st + 1024 + lane * 16);
    r.vA = *reinterpret_cast<const u32x4 *>(st + 2048 + lane * 16);
    r.vB = *reinterpret_cast<const u32x4 *>(st + 3072 + lane * 16);
    r.kpA = *reinterpret_cast<const u32x4 *>(st + 4096 + G * 16);
    if (int4) {
        r.kpB = *reinterpret_cast<const u32x4 *>(st + 4160 + G * 16);
        r.vpA = *reinterpret_cast<const u32x4 *>(st + 4224 + G * 16);
        r.vpB = *reinterpret_cast<const u32x4 *>(st + 4288 + G * 16);
    } else {
        r.vpA = *reinterpret_cast<const u32x4 *>(st + 4160 + G * 16);
        const u32x4 z = {0u, 0u, 0u, 0u};
        r.kpB = z;
        r.vpB = z;
    }
    return r;
}

// score (log2 units) of one token from its raw code dot product d
__device__ inline float score(float d, uint32_t kp, float K1, float K2) {
    return fmaf(d, h_lo(kp) * K1, h_hi(kp) * K2);
}

template <int GP, bool FULL>
__device__ inline void compute_step4(SegCtx<GP> &c, const StepRegs &r, int pos0, int lo4, int hi4) {
    constexpr int kQ = SegCtx<GP>::kQ;
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    floatx4 dA[kQ], dB[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) dA[q] = dB[q] = zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = r.kA[i], x8 = x >> 8;
        const half8 ak = pack8(x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u);
        const uint32_t y = r.kB[i], y8 = y >> 8;
        const half8 bk = pack8(y & 0x000F000Fu, y & 0x00F000F0u, y8 & 0x000F000Fu, y8 & 0x00F000F0u);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            dA[q] = mfma16(ak, c.q4[q][i], dA[q]);
            dB[q] = mfma16(bk, c.q4[q][i], dB[q]);
        }
    }
    floatx4 sA = dA[0], sB = dB[0];
    if constexpr (kQ == 2) {
        sA += dA[1];
        sB += dB[1];
    }
    sA = combine_cols<GP>(sA);
    sB = combine_cols<GP>(sB);
    float sc[8];
    bool valid[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t kp = i < 4 ? r.kpA[i] : r.kpB[i - 4];
        const float s = score(i < 4 ? sA[i] : sB[i - 4], kp, c.K1, c.K2);
        if (FULL) {
            valid[i] = true;
            sc[i] = s;
        } else {
            const int p = pos0 + (i < 4 ? 0 : 16) + 4 * c.G + (i & 3);
            valid[i] = p >= lo4 && p < hi4;
            sc[i] = valid[i] ? s : kNegInf;
        }
    }
    half8 pop[2];
    softmax_step<GP, FULL>(c, sc, r.vpA, r.vpB, valid, pop);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        const uint32_t x = r.vA[cc], x8 = x >> 8, y = r.vB[cc], y8 = y >> 8;
        const half8 ve = pack8(x & 0x000F000Fu, x8 & 0x000F000Fu, y & 0x000F000Fu, y8 & 0x000F000Fu);
        const half8 vo = pack8(x & 0x00F000F0u, x8 & 0x00F000F0u, y & 0x00F000F0u, y8 & 0x00F000F0u);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            c.O[2 * cc] = mfma16(pop[q], ve, c.O[2 * cc]);
            c.O[2 * cc + 1] = mfma16(pop[q], vo, c.O[2 * cc + 1]);
        }
    }
}

// One INT8 subblock of 16 ring entries starting at e0 (the B half of the value
// MFMA is zero).
template <int GP>
__device__ inline void compute_step8(SegCtx<GP> &c, const StepRegs &r, int e0, int n8e) {
    constexpr int kQ = SegCtx<GP>::kQ;
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    floatx4 d[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) d[q] = zero4;
    floatx4 dh[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) dh[q] = zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // dims 32G + 8i .. +8: dwords 2i (even dims) and 2i+1 (odd dims); the
        // low and high nibbles of the 8 codes form two INT4-ordered dwords
        const uint32_t x0 = i < 2 ? r.kA[2 * i] : r.kB[2 * i - 4];
        const uint32_t x1 = i < 2 ? r.kA[2 * i + 1] : r.kB[2 * i - 3];
        const uint32_t xl = (x0 & 0x0F0F0F0Fu) | ((x1 & 0x0F0F0F0Fu) << 4);
        const uint32_t xh = ((x0 >> 4) & 0x0F0F0F0Fu) | (x1 & 0xF0F0F0F0u);
        const uint32_t l8 = xl >> 8, h8 = xh >> 8;
        const half8 al = pack8(xl & 0x000F000Fu, xl & 0x00F000F0u, l8 & 0x000F000Fu, l8 & 0x00F000F0u);
        const half8 ah = pack8(xh & 0x000F000Fu, xh & 0x00F000F0u, h8 & 0x000F000Fu, h8 & 0x00F000F0u);
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            d[q] = mfma16(al, c.q4[q][i], d[q]);
            dh[q] = mfma16(ah, c.q4[q][i], dh[q]);
        }
    }
    floatx4 s4 = d[0] + 16.0f * dh[0];
    if constexpr (kQ == 2) s4 += d[1] + 16.0f * dh[1];
    s4 = combine_cols<GP>(s4);
    float sc[8];
    bool valid[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i < 4) {
            const int e = e0 + 4 * c.G + i;
            valid[i] = e < n8e;
            const float s = score(s4[i], r.kpA[i], c.K1, c.K2);
            sc[i] = valid[i] ? s : kNegInf;
        } else {
            valid[i] = false;
            sc[i] = kNegInf;
        }
    }
    half8 pop[2];
    softmax_step<GP, false>(c, sc, r.vpA, r.vpB, valid, pop);
    const uint32_t M8 = 0x00FF00FFu;
    // odd value tiles accumulate 16x (matching the INT4 high-nibble scaling)
    const half8 sixteen = {16, 16, 16, 16, 16, 16, 16, 16};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t x = t < 4 ? r.vA[t] : r.vB[t - 4];
        const half8 vv = pack8(x & M8, (x >> 8) & M8, 0u, 0u);
#pragma unroll
        for (int q = 0; q < kQ; ++q) c.O[t] = mfma16((t & 1) ? pop[q] * sixteen : pop[q], vv, c.O[t]);
    }
}

// End of a segment: per-head l, z totals over the four lane rows, and in
// packed mode the hi and lo accumulator rows added (hi rows keep the sum).
template <int GP>
__device__ inline void reduce_segment(SegCtx<GP> &c) {
    c.lsum = sum_rows(c.lsum);
    c.zsum = sum_rows(c.zsum);
    if constexpr (GP == 4) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) c.O[t][i] += xor16(c.O[t][i], c.lane);
    } else if constexpr (GP == 8) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) c.O[t][i] += xor32(c.O[t][i], c.lane);
    }
}

// Head held by accumulator row 4G + i, or -1 (lo rows in packed mode, rows >= g).
template <int GP>
__device__ inline int row_head(const SegCtx<GP> &c, int i) {
    const int row = 4 * c.G + i;
    return (row < GP && row < c.g) ? row : -1;
}

// Output of a segment that one worker attended completely: straight from registers.
template <int GP>
__device__ inline void finalize_regs(const DecodeArgs &a, const SegCtx<GP> &c, int b, int hk) {
    float *ob = a.out + ((int64_t)b * a.Hq + (int64_t)hk * c.g) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = row_head(c, i);
        const float zr = __shfl(c.zsum, r < 0 ? 0 : r, 64);
        const float lr = __shfl(c.lsum, r < 0 ? 0 : r, 64);
        if (r >= 0) {
            const float inv = 1.0f / lr;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float sc = (t & 1) ? 1048576.0f : 16777216.0f;   // 2^20 / 2^24
                ob[r * kHeadDim + 16 * t + c.n] = (c.O[t][i] * sc + zr) * inv;
            }
        }
    }
    if (a.lse && c.lane < c.g && c.lane < GP)
        a.lse[(int64_t)b * a.Hq + (int64_t)hk * c.g + c.lane] = (c.m + __log2f(c.lsum)) / kLog2e;
}

// Partial statistics of a segment: per query head m, l and the unnormalised acc[128].
template <int GP>
__device__ inline void write_piece(const SegCtx<GP> &c, float *pp) {
    if (c.lane < c.g && c.lane < GP) {
        pp[c.lane * kPieceStride + 0] = c.m;
        pp[c.lane * kPieceStride + 1] = c.lsum;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = row_head(c, i);
        const float zr = __shfl(c.zsum, r < 0 ? 0 : r, 64);
        if (r >= 0) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float sc = (t & 1) ? 1048576.0f : 16777216.0f;
                pp[r * kPieceStride + 4 + 16 * t + c.n] = c.O[t][i] * sc + zr;
            }
        }
    }
}

// Units of all rows: each wave sums the per-row costs (all KV heads).
__device__ inline int64_t total_units(const DecodeArgs &a, int lane) {
    int64_t tot = 0;
    for (int b = lane; b < a.B; b += 64) tot += (int64_t)row_plan(a.ctx_len[b], a.s, a.w).cost * a.H;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o, 64);
    return uni64(tot);
}

template <int GP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];
    const int lane = threadIdx.x;
    const int64_t wid = blockIdx.x;
    const int64_t total = total_units(a, lane);
    const int64_t W = effective_workers(total, a.max_workers, a.min_units);
    if (wid == 0 && lane == 0) {
        a.ws_header[0] = total;
        a.ws_header[1] = W;
    }
    const int64_t u_begin = wid < W ? worker_begin(wid, total, W) : 0;
    const int64_t u_end = wid < W ? worker_begin(wid + 1, total, W) : 0;
    const bool active = wid < W && u_begin < u_end;
    if (!active && wid != 0) return;

    // Exclusive prefix of row costs; block 0 stores all of it for the combine
    // kernel, every active wave finds the row holding its first unit.
    int b0 = -1;
    int64_t pre0 = 0;
    int64_t base = 0;
    for (int cb = 0; cb < a.B; cb += 64) {
        const int b = cb + lane;
        const int64_t cost = b < a.B ? (int64_t)row_plan(a.ctx_len[b], a.s, a.w).cost * a.H : 0;
        int64_t incl = cost;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t t = __shfl_up(incl, o, 64);
            if (lane >= o) incl += t;
        }
        const int64_t excl = base + incl - cost;
        if (wid == 0 && b < a.B) a.ws_prefix[b] = excl;
        if (active && b0 < 0) {
            const uint64_t mk = __ballot(b < a.B && cost > 0 && excl <= u_begin && u_begin < excl + cost);
            if (mk) {
                const int src = uni(__ffsll((unsigned long long)mk) - 1);
                b0 = uni(cb + src);
                pre0 = uni64(__shfl(excl, src, 64));
                if (wid != 0) break;
            }
        }
        base = uni64(base + __shfl(incl, 63, 64));
    }
    if (!active) return;
    b0 = uni(b0);
    pre0 = uni64(pre0);

    Cursor start;
    start.b = b0;
    start.rp = row_plan(ldc(a.ctx_len, b0), a.s, a.w);
    start.hk = (int)((u_begin - pre0) / start.rp.cost);
    start.r = (int)(u_begin - pre0 - (int64_t)start.hk * start.rp.cost);
    start.u = u_begin;

    SegCtx<GP> c;
    c.lane = lane;
    c.G = lane >> 4;
    c.n = lane & 15;
    c.col = lane & 15;
    c.g = a.g;

    // per-lane source offsets of the direct-to-LDS loads (see issue_step)
    const uint32_t offK4 = kSub4K + c.n * 64 + c.G * 16;
    const uint32_t offV4 = kSub4V + lane * 16;
    const uint32_t offP4 = ((lane & 8) ? kSub4VP : kSub4KP) + (lane & 3) * 16;
    const uint32_t offK8 = kSub8K + c.n * 128 + c.G * 32;
    const uint32_t offV8 = kSub8V + lane * 32;
    const uint32_t offP8 = ((lane & 4) ? kSub8VP : kSub8KP) + (lane & 3) * 16;

    Cursor P = start, C = start;
    int issued = 0;
    Lookup look = lookup(a, P);
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
        if (P.u < u_end) {
            issue_step(a, P, look, smem + s * kStageBytes, offK4, offV4, offP4, offK8, offV8, offP8, lane);
            cursor_next(a, P);
            ++issued;
            if (P.u < u_end) look = lookup(a, P);
        }
    }
    bool open = false;
    for (int i = 0; C.u < u_end; ++i) {
        wait_vm_steps(issued - i - 1);
        uint8_t *st = smem + (i % kStages) * kStageBytes;
        const bool int4 = C.r < C.rp.n4;
        const StepRegs r = read_stage(st, int4, lane);
        wait_lgkm0();
        if (P.u < u_end) {
            issue_step(a, P, look, st, offK4, offV4, offP4, offK8, offV8, offP8, lane);
            cursor_next(a, P);
            ++issued;
            if (P.u < u_end) look = lookup(a, P);
        }
        if (!open) {
            build_query<GP>(a, C.b, C.hk, c);
            c.m = kNegInf;
            c.lsum = 0.0f;
            c.zsum = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) c.O[t] = floatx4{0.f, 0.f, 0.f, 0.f};
            open = true;
        }
        if (int4) {
            const int pos0 = (C.rp.k0 + C.r) * 32;
            if (pos0 >= C.rp.lo4 && pos0 + 32 <= C.rp.hi4)
                compute_step4<GP, true>(c, r, pos0, C.rp.lo4, C.rp.hi4);
            else
                compute_step4<GP, false>(c, r, pos0, C.rp.lo4, C.rp.hi4);
        } else {
            compute_step8<GP>(c, r, 16 * (C.r - C.rp.n4), C.rp.n8e);
        }
        if (C.r == C.rp.cost - 1 || C.u + 1 == u_end) {
            reduce_segment<GP>(c);
            const int64_t c0 = C.u - C.r;
            const bool whole = worker_of(c0, total, W) == worker_of(c0 + C.rp.cost - 1, total, W);
            if (whole)
                finalize_regs<GP>(a, c, C.b, C.hk);
            else
                write_piece<GP>(c, a.ws_piece + (wid + (int64_t)C.b * a.H + C.hk) * (int64_t)c.g * kPieceStride);
            open = false;
        }
        cursor_next(a, C);
    }
}

// Log-sum-exp combine of the pieces of one (row, KV head) segment that several
// workers share; one wave per segment, lane l handles query head 4k + l/16 and
// dims 8 (l % 16) .. +8.  Also writes the rows with no context.
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
    const int lane = threadIdx.x;
    const int64_t seg = blockIdx.x;
    const int b = (int)(seg / a.H), hk = (int)(seg % a.H);
    const RowPlan rp = row_plan(a.ctx_len[b], a.s, a.w);
    const int g = a.g;
    const int part = lane & 15;
    if (rp.cost == 0) {
        for (int i = lane; i < g * kHeadDim; i += 64) a.out[((int64_t)b * a.Hq + (int64_t)hk * g) * kHeadDim + i] = 0.0f;
        if (a.lse && lane < g) a.lse[(int64_t)b * a.Hq + (int64_t)hk * g + lane] = kNegInf;
        return;
    }
    const int64_t total = a.ws_header[0];
    const int64_t W = a.ws_header[1];
    const int64_t c0 = a.ws_prefix[b] + (int64_t)hk * rp.cost;
    const int64_t wf = worker_of(c0, total, W);
    const int64_t wl = worker_of(c0 + rp.cost - 1, total, W);
    if (wf == wl) return;           // finished by its only worker
    const float *basep = a.ws_piece + seg * (int64_t)g * kPieceStride;
    for (int hg = 0; hg < g; hg += 4) {
        const int j = hg + (lane >> 4);
        if (j >= g) continue;
        float M = kNegInf;
        for (int64_t w = wf; w <= wl; ++w) M = fmaxf(M, basep[(w * g + j) * kPieceStride]);
        float Ls = 0.0f;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
        for (int64_t w = wf; w <= wl; ++w) {
            const float *pp = basep + (w * g + j) * kPieceStride;
            const float m = pp[0];
            const float f = m == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m - M);
            Ls = fmaf(pp[1], f, Ls);
            const u32x4 v0 = ldg<u32x4>(pp + 4 + 8 * part);
            const u32x4 v1 = ldg<u32x4>(pp + 8 + 8 * part);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] = fmaf(__uint_as_float(v0[e]), f, acc[e]);
                acc[4 + e] = fmaf(__uint_as_float(v1[e]), f, acc[4 + e]);
            }
        }
        float *o = a.out + ((int64_t)b * a.Hq + (int64_t)hk * g + j) * kHeadDim + 8 * part;
        const float inv = 1.0f / Ls;
        u32x4 w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w0[e] = __float_as_uint(acc[e] * inv);
            w1[e] = __float_as_uint(acc[4 + e] * inv);
        }
        *reinterpret_cast<u32x4 *>(o) = w0;
        *reinterpret_cast<u32x4 *>(o + 4) = w1;
        if (a.lse && part == 0) a.lse[(int64_t)b * a.Hq + (int64_t)hk * g + j] = (M + __log2f(Ls)) / kLog2e;
    }
}

template <int GP>
static const void *split_fn() { return reinterpret_cast<const void *>(&decode_split_kernel<GP>); }

static int group_class(int g) { return g <= 4 ? 4 : (g <= 8 ? 8 : 16); }

hipError_t launch_decode(const DecodeArgs &a, int grid, hipStream_t stream) {
    switch (group_class(a.g)) {
        case 4: hipLaunchKernelGGL(decode_split_kernel<4>, dim3(grid), dim3(64), 0, stream, a); break;
        case 8: hipLaunchKernelGGL(decode_split_kernel<8>, dim3(grid), dim3(64), 0, stream, a); break;
        default: hipLaunchKernelGGL(decode_split_kernel<16>, dim3(grid), dim3(64), 0, stream, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.H), dim3(64), 0, stream, a);
    return hipGetLastError();
}

hipError_t decode_max_workers(int g, int *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    const void *fn = group_class(g) == 4 ? split_fn<4>() : (group_class(g) == 8 ? split_fn<8>() : split_fn<16>());
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    *out = cus * per_cu;
    return hipSuccess;
}

}  // namespace kvq
