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
// workgroup), so a long-tailed length mix costs every wave the same.
//
// Memory: each wave streams its steps through a ring of kStages LDS buffers
// with direct global->LDS loads (5 x 16 B per lane per step), kStages - 1 steps
// ahead of the step it computes, so the bytes in flight do not cost VGPRs.
//
// Compute per step, with 16x16x32 f16 MFMA:
//   scores[tok][head] = codes[tok][:] . q[head][:]    (A = codes, B = query)
//   acc[head][dim]   += p[head][tok] * vcodes[tok][dim] (A = p, B = codes)
// The query and p are split into f16 hi + lo parts so the products keep fp32
// accuracy; 4-bit and 8-bit codes become f16 values exactly by masking them
// into the mantissa of a subnormal (code * 2^-24, or code * 2^-20 for the high
// nibble of a byte, compensated in the other operand or the accumulator).
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

// f16 hi/lo split of a pair: hi = f16(x), lo = f16(x - hi).
__device__ inline void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    _Float16 ha = (_Float16)a, hb = (_Float16)b;
    half2v vh = {ha, hb};
    half2v vl = {(_Float16)(a - (float)ha), (_Float16)(b - (float)hb)};
    hi = __builtin_bit_cast(uint32_t, vh);
    lo = __builtin_bit_cast(uint32_t, vl);
}

__device__ inline float h_lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xFFFFu))); }
__device__ inline float h_hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }

__device__ inline float bf16f(uint32_t b) { return __uint_as_float(b << 16); }

template <typename T>
__device__ inline T ldg(const void *p) { return *reinterpret_cast<const T *>(p); }

typedef __attribute__((address_space(3))) void *lds_ptr;

// Values every lane holds the same copy of, made visibly wave-uniform so that
// the loads they index become scalar loads.
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read-only launch inputs (lengths, slots, block table) read through the
// constant address space so that wave-uniform reads are scalar loads.
__device__ inline int ldc(const int32_t *p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}
__device__ inline int64_t uni64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// 16 bytes per lane from global memory into LDS at dst + 16 * lane.
__device__ inline void dma16(const void *src, uint8_t *dst_lds) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr)dst_lds, 16, 0, 0);
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
    switch (steps_after) {
        case 0: __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(5)); break;
        case 2: __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(10)); break;
        default: __builtin_amdgcn_s_waitcnt(KVQ_VMCNT(15)); break;
    }
    KVQ_FENCE();
    static_assert(kStages == 4 && kDmaPerStep == 5, "wait table assumes 4 stages x 5 loads");
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

struct SegCtx {
    int lane, G, n;
    int g;
    half8 q4h[4], q4l[4], q8h[4], q8l[4];   // query operands, INT4 and INT8 element orders
    float K1;           // 2^(24 - e) * log2(e) / sqrt(128)
    float K2;           // sum(q~) * log2(e) / sqrt(128) for head l%16
    float m, lsum, zsum;
    floatx4 O[8];       // acc[head 4G+i][16 t + n], odd tiles scaled by 16
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

__device__ inline void build_query(const DecodeArgs &a, int b, int hk, SegCtx &c) {
    const int j = c.lane & 15;
    float x[32];
    if (j < c.g) {
        const uint16_t *qp = a.q + ((int64_t)b * a.Hq + (int64_t)hk * c.g + j) * kHeadDim + 32 * c.G;
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
#pragma unroll
    for (int ls = 16; ls <= 32; ls <<= 1) {
        if (2 * ls < a.h) {
            const bool upper = (c.lane & ls) != 0;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                float p = __shfl_xor(x[i], ls, 64);
                x[i] = upper ? (p - x[i]) : (x[i] + p);
            }
        }
    }
    float sum = 0.0f, amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        x[i] *= a.inv_sqrt_h;
        sum += x[i];
        amax = fmaxf(amax, fabsf(x[i]));
    }
    sum += __shfl_xor(sum, 16, 64);
    sum += __shfl_xor(sum, 32, 64);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    int E = 0;
    (void)frexpf(amax, &E);
    const int e = amax > 0.0f ? 14 - E : 0;      // |q * 2^e| < 2^14
    const float sc = ldexpf(1.0f, e);
    const float c0 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
    c.K1 = ldexpf(c0, 24 - e);
    c.K2 = sum * c0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float *y = x + 8 * i;
        uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
        // INT4 order: dims 0,4 | 1,5 (/16) | 2,6 | 3,7 (/16)
        split2(y[0] * sc, y[4] * sc, h0, l0);
        split2(y[1] * sc * 0.0625f, y[5] * sc * 0.0625f, h1, l1);
        split2(y[2] * sc, y[6] * sc, h2, l2);
        split2(y[3] * sc * 0.0625f, y[7] * sc * 0.0625f, h3, l3);
        c.q4h[i] = pack8(h0, h1, h2, h3);
        c.q4l[i] = pack8(l0, l1, l2, l3);
        // INT8 order: dims 0,2 | 1,3 | 4,6 | 5,7
        split2(y[0] * sc, y[2] * sc, h0, l0);
        split2(y[1] * sc, y[3] * sc, h1, l1);
        split2(y[4] * sc, y[6] * sc, h2, l2);
        split2(y[5] * sc, y[7] * sc, h3, l3);
        c.q8h[i] = pack8(h0, h1, h2, h3);
        c.q8l[i] = pack8(l0, l1, l2, l3);
    }
}

// Online-softmax update for 8 scores of this lane (tokens 4G+i of subblocks A,
// B) and the f16 hi/lo p*scale_v operands of the value MFMA (rows = heads,
// k = [A0 A2 A1 A3 B0 B2 B1 B3]).
__device__ inline void softmax_step(SegCtx &c, float sc[8], const u32x4 &vpA, const u32x4 &vpB,
                                    const bool valid[8], half8 &ph, half8 &pl) {
    float mstep = kNegInf;
#pragma unroll
    for (int i = 0; i < 8; ++i) mstep = fmaxf(mstep, sc[i]);
    mstep = fmaxf(mstep, __shfl_xor(mstep, 16, 64));
    mstep = fmaxf(mstep, __shfl_xor(mstep, 32, 64));
    const float mnew = fmaxf(c.m, mstep);
    const bool grow = mnew > c.m;
    if (__any(grow)) {
        const float alpha = (grow && c.m != kNegInf) ? __builtin_amdgcn_exp2f(c.m - mnew) : (grow ? 0.0f : 1.0f);
        c.lsum *= alpha;
        c.zsum *= alpha;
        const int rb = 4 * (c.lane >> 4);
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, rb + i, 64);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) c.O[t][i] *= ar[i];
        }
        c.m = mnew;
    }
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t vp = i < 4 ? vpA[i] : vpB[i - 4];
        const float p = valid[i] ? __builtin_amdgcn_exp2f(sc[i] - c.m) : 0.0f;
        c.lsum += p;
        c.zsum += valid[i] ? p * h_hi(vp) : 0.0f;
        pv[i] = valid[i] ? p * h_lo(vp) : 0.0f;
    }
    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
    split2(pv[0], pv[2], h0, l0);
    split2(pv[1], pv[3], h1, l1);
    split2(pv[4], pv[6], h2, l2);
    split2(pv[5], pv[7], h3, l3);
    ph = pack8(h0, h1, h2, h3);
    pl = pack8(l0, l1, l2, l3);
}

// ---------------------------------------------------------------------------
// Producer: issue the 5 direct-to-LDS loads of the step at cursor c into stage st.
__device__ inline void issue_step(const DecodeArgs &a, const Cursor &c, uint8_t *st, int lane) {
    const int G = lane >> 4, n = lane & 15;
    const int slot = ldc(a.slot, c.b);
    if (c.r < c.rp.n4) {
        const int pos0 = (c.rp.k0 + c.r) * 32;
        const int32_t *bt = a.block_table + (int64_t)slot * a.bt_stride;
        const int subs = a.P >> 4;
        const int pA = pos0, pB = pos0 + 16;
        const int pageA = ldc(bt, pA >> a.logP);
        const uint8_t *baseA = a.int4_pool +
            ((size_t)((int64_t)pageA * a.H + c.hk) * subs + ((pA & (a.P - 1)) >> 4)) * kSub4Bytes;
        const uint8_t *baseB = baseA;
        if (pB < c.rp.hi4) {
            const int pageB = ldc(bt, pB >> a.logP);
            baseB = a.int4_pool +
                ((size_t)((int64_t)pageB * a.H + c.hk) * subs + ((pB & (a.P - 1)) >> 4)) * kSub4Bytes;
        }
        dma16(baseA + kSub4K + n * 64 + G * 16, st + 0);
        dma16(baseB + kSub4K + n * 64 + G * 16, st + 1024);
        dma16(baseA + kSub4V + lane * 16, st + 2048);
        dma16(baseB + kSub4V + lane * 16, st + 3072);
        if (lane < 16) {
            const uint8_t *b = (lane & 4) ? baseB : baseA;
            dma16(b + ((lane & 8) ? kSub4VP : kSub4KP) + (lane & 3) * 16, st + 4096);
        }
    } else {
        const int sub = c.r - c.rp.n4;
        const uint8_t *base = a.int8_pool + ((size_t)((int64_t)slot * a.H + c.hk) * a.nr8 + sub) * kSub8Bytes;
        dma16(base + kSub8K + n * 128 + G * 32, st + 0);
        dma16(base + kSub8K + n * 128 + G * 32 + 16, st + 1024);
        dma16(base + kSub8V + lane * 32, st + 2048);
        dma16(base + kSub8V + lane * 32 + 16, st + 3072);
        if (lane < 8) {
            dma16(base + ((lane & 4) ? kSub8VP : kSub8KP) + (lane & 3) * 16, st + 4096);
        }
    }
}

__device__ inline StepRegs read_stage(const uint8_t *st, bool int4, int lane) {
    StepRegs r;
    const int G = lane >> 4;
    r.kA = *reinterpret_cast<const u32x4 *>(st + lane * 16);
    r.kB = *reinterpret_cast<const u32x4 *>(st + 1024 + lane * 16);
    r.vA = *reinterpret_cast<const u32x4 *>(st + 2048 + lane * 16);
    r.vB = *reinterpret_cast<const u32x4 *>(st + 3072 + lane * 16);
    if (int4) {
        r.kpA = *reinterpret_cast<const u32x4 *>(st + 4096 + G * 16);
        r.kpB = *reinterpret_cast<const u32x4 *>(st + 4160 + G * 16);
        r.vpA = *reinterpret_cast<const u32x4 *>(st + 4224 + G * 16);
        r.vpB = *reinterpret_cast<const u32x4 *>(st + 4288 + G * 16);
    } else {
        r.kpA = *reinterpret_cast<const u32x4 *>(st + 4096 + G * 16);
        r.vpA = *reinterpret_cast<const u32x4 *>(st + 4160 + G * 16);
        const u32x4 z = {0u, 0u, 0u, 0u};
        r.kpB = z;
        r.vpB = z;
    }
    return r;
}

__device__ inline void compute_step4(SegCtx &c, const StepRegs &r, int pos0, int lo4, int hi4) {
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    floatx4 dAh = zero4, dAl = zero4, dBh = zero4, dBl = zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = r.kA[i], x8 = x >> 8;
        const half8 ak = pack8(x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u);
        const uint32_t y = r.kB[i], y8 = y >> 8;
        const half8 bk = pack8(y & 0x000F000Fu, y & 0x00F000F0u, y8 & 0x000F000Fu, y8 & 0x00F000F0u);
        dAh = mfma16(ak, c.q4h[i], dAh);
        dBh = mfma16(bk, c.q4h[i], dBh);
        dAl = mfma16(ak, c.q4l[i], dAl);
        dBl = mfma16(bk, c.q4l[i], dBl);
    }
    float sc[8];
    bool valid[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t kp = i < 4 ? r.kpA[i] : r.kpB[i - 4];
        const float d = i < 4 ? dAh[i] + dAl[i] : dBh[i - 4] + dBl[i - 4];
        const int p = pos0 + (i < 4 ? 0 : 16) + 4 * c.G + (i & 3);
        valid[i] = p >= lo4 && p < hi4;
        const float s = d * (h_lo(kp) * c.K1) + h_hi(kp) * c.K2;
        sc[i] = valid[i] ? s : kNegInf;
    }
    half8 ph, pl;
    softmax_step(c, sc, r.vpA, r.vpB, valid, ph, pl);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
        const uint32_t x = r.vA[cc], x8 = x >> 8, y = r.vB[cc], y8 = y >> 8;
        const half8 ve = pack8(x & 0x000F000Fu, x8 & 0x000F000Fu, y & 0x000F000Fu, y8 & 0x000F000Fu);
        const half8 vo = pack8(x & 0x00F000F0u, x8 & 0x00F000F0u, y & 0x00F000F0u, y8 & 0x00F000F0u);
        c.O[2 * cc] = mfma16(ph, ve, c.O[2 * cc]);
        c.O[2 * cc + 1] = mfma16(ph, vo, c.O[2 * cc + 1]);
        c.O[2 * cc] = mfma16(pl, ve, c.O[2 * cc]);
        c.O[2 * cc + 1] = mfma16(pl, vo, c.O[2 * cc + 1]);
    }
}

// One INT8 subblock of 16 ring entries starting at e0 (the B half of the value
// MFMA is zero).
__device__ inline void compute_step8(SegCtx &c, const StepRegs &r, int e0, int n8e) {
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    floatx4 dh = zero4, dl = zero4;
    const uint32_t M8 = 0x00FF00FFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // dims 32G + 8i .. +8: dwords 2i, 2i+1 of the lane's 32 bytes
        const uint32_t x = i < 2 ? r.kA[2 * i] : r.kB[2 * i - 4];
        const uint32_t y = i < 2 ? r.kA[2 * i + 1] : r.kB[2 * i - 3];
        const half8 ak = pack8(x & M8, (x >> 8) & M8, y & M8, (y >> 8) & M8);
        dh = mfma16(ak, c.q8h[i], dh);
        dl = mfma16(ak, c.q8l[i], dl);
    }
    float sc[8];
    bool valid[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i < 4) {
            const uint32_t kp = r.kpA[i];
            const int e = e0 + 4 * c.G + i;
            valid[i] = e < n8e;
            const float s = (dh[i] + dl[i]) * (h_lo(kp) * c.K1) + h_hi(kp) * c.K2;
            sc[i] = valid[i] ? s : kNegInf;
        } else {
            valid[i] = false;
            sc[i] = kNegInf;
        }
    }
    half8 ph, pl;
    softmax_step(c, sc, r.vpA, r.vpB, valid, ph, pl);
    // odd value tiles accumulate 16x (matching the INT4 high-nibble scaling)
    const half8 sixteen = {16, 16, 16, 16, 16, 16, 16, 16};
    const half8 ph16 = ph * sixteen, pl16 = pl * sixteen;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t x = t < 4 ? r.vA[t] : r.vB[t - 4];
        const half8 vv = pack8(x & M8, (x >> 8) & M8, 0u, 0u);
        if (t & 1) {
            c.O[t] = mfma16(ph16, vv, c.O[t]);
            c.O[t] = mfma16(pl16, vv, c.O[t]);
        } else {
            c.O[t] = mfma16(ph, vv, c.O[t]);
            c.O[t] = mfma16(pl, vv, c.O[t]);
        }
    }
}

__device__ inline void write_piece(const DecodeArgs &a, SegCtx &c, int64_t piece) {
    float lsum = c.lsum, zsum = c.zsum;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    zsum += __shfl_xor(zsum, 16, 64);
    zsum += __shfl_xor(zsum, 32, 64);
    float *pp = a.ws_piece + piece * (int64_t)c.g * kPieceStride;
    if (c.lane < c.g) {
        pp[c.lane * kPieceStride + 0] = c.m;
        pp[c.lane * kPieceStride + 1] = lsum;
    }
    const int rb = 4 * (c.lane >> 4);
    float zr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) zr[i] = __shfl(zsum, rb + i, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rb + i;
        if (r < c.g) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float sc = (t & 1) ? 1048576.0f : 16777216.0f;   // 2^20 / 2^24
                pp[r * kPieceStride + 4 + 16 * t + c.n] = c.O[t][i] * sc + zr[i];
            }
        }
    }
}

// Units of all rows: each wave sums the per-row costs (all KV heads).
__device__ inline int64_t total_units(const DecodeArgs &a, int lane) {
    int64_t tot = 0;
    for (int b = lane; b < a.B; b += 64) {
        const int L = a.ctx_len[b];
        tot += (int64_t)row_plan(L, a.s, a.w).cost * a.H;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o, 64);
    return uni64(tot);
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_kernel(DecodeArgs a) {
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

    // Exclusive prefix of row costs; block 0 stores all of it, every active
    // wave finds the row holding its first unit.
    int b0 = -1;
    int64_t pre0 = 0;
    int64_t base = 0;
    for (int c0 = 0; c0 < a.B; c0 += 64) {
        const int b = c0 + lane;
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
            const uint64_t m = __ballot(b < a.B && cost > 0 && excl <= u_begin && u_begin < excl + cost);
            if (m) {
                const int src = uni(__ffsll((unsigned long long)m) - 1);
                b0 = uni(c0 + src);
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

    SegCtx c;
    c.lane = lane;
    c.G = lane >> 4;
    c.n = lane & 15;
    c.g = a.g;

    Cursor P = start, C = start;
    int issued = 0;
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
        if (P.u < u_end) {
            issue_step(a, P, smem + s * kStageBytes, lane);
            cursor_next(a, P);
            ++issued;
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
            issue_step(a, P, st, lane);
            cursor_next(a, P);
            ++issued;
        }
        if (!open) {
            build_query(a, C.b, C.hk, c);
            c.m = kNegInf;
            c.lsum = 0.0f;
            c.zsum = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) c.O[t] = floatx4{0.f, 0.f, 0.f, 0.f};
            open = true;
        }
        if (int4)
            compute_step4(c, r, (C.rp.k0 + C.r) * 32, C.rp.lo4, C.rp.hi4);
        else
            compute_step8(c, r, 16 * (C.r - C.rp.n4), C.rp.n8e);
        if (C.r == C.rp.cost - 1 || C.u + 1 == u_end) {
            write_piece(a, c, wid + (int64_t)C.b * a.H + C.hk);
            open = false;
        }
        cursor_next(a, C);
    }
}

// Log-sum-exp combine of all pieces of one (row, query head): one workgroup of
// 128 threads (one per output dim).
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
    const int d = threadIdx.x;
    const int row = blockIdx.x / a.Hq;
    const int jq = blockIdx.x % a.Hq;
    const int hk = jq / a.g;
    const int jr = jq % a.g;
    const RowPlan rp = row_plan(a.ctx_len[row], a.s, a.w);
    float *o = a.out + ((int64_t)row * a.Hq + jq) * kHeadDim;
    if (rp.cost == 0) {
        o[d] = 0.0f;
        if (a.lse && d == 0) a.lse[(int64_t)row * a.Hq + jq] = kNegInf;
        return;
    }
    const int64_t total = a.ws_header[0];
    const int64_t W = a.ws_header[1];
    const int64_t c0 = a.ws_prefix[row] + (int64_t)hk * rp.cost;
    const int64_t wf = worker_of(c0, total, W);
    const int64_t wl = worker_of(c0 + rp.cost - 1, total, W);
    const int64_t seg = (int64_t)row * a.H + hk;
    float M = kNegInf, Ls = 0.0f, acc = 0.0f;
    for (int64_t w = wf; w <= wl; ++w) {
        if (worker_begin(w, total, W) == worker_begin(w + 1, total, W)) continue;   // empty worker
        const float *pp = a.ws_piece + ((w + seg) * a.g + jr) * kPieceStride;
        const float m = pp[0];
        if (m == kNegInf) continue;
        const float l = pp[1];
        const float x = pp[4 + d];
        if (m > M) {
            const float f = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - m);
            Ls = Ls * f + l;
            acc = acc * f + x;
            M = m;
        } else {
            const float f = __builtin_amdgcn_exp2f(m - M);
            Ls += l * f;
            acc += x * f;
        }
    }
    o[d] = acc / Ls;
    if (a.lse && d == 0) a.lse[(int64_t)row * a.Hq + jq] = (M + __log2f(Ls)) / kLog2e;
}

hipError_t launch_decode(const DecodeArgs &a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(decode_split_kernel, dim3(grid), dim3(64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.Hq), dim3(128), 0, stream, a);
    return hipGetLastError();
}

hipError_t decode_max_workers(int *out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel, 64, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    *out = cus * per_cu;
    return hipSuccess;
}

}  // namespace kvq
