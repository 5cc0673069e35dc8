// Causal multi-row attention over the quantized cache: a chunk of query rows
// per sequence (chunked prefill, or the re-prefill of in-flight rollouts after
// a policy update that the KV4-RL page describes under "Future Directions").
//
// Reading of the method (KV4-RL, "Methodology in Plain English": attention
// reads the packed codes with the rotated query): the T rows of sequence b sit
// at positions L - T .. L - 1 (L = ctx_len[b], the chunk already appended) and
// row t attends positions [0, L - T + t], each key and value taken as the
// cache holds it at length L -- the INT8 side cache for the sinks and the last
// w positions, the INT4 pages elsewhere.  The last row is decode attention.
//
// Work: one wave per (sequence, KV head, prefill_tiles(bits) tiles of R rows), R =
// floor(16 / g), so that a tile's (row, query head) pairs fill the 16 columns
// of v_mfma_f32_16x16x32_f16.  The wave streams its rows' causal prefix
// through the same 3-stage LDS ring of 5-load steps as the decode kernel (INT4
// steps of 32 positions, INT8 steps of 16 ring entries) and per step computes,
// for each tile,
//   S[tok][col] = codes[tok][:] . Q[:][col]          A = codes, B = query
//   O[col][dim] += P[col][tok] * vcodes[tok][dim]    A = p * s_v, B = codes
// with the query and p * s_v each split into f16 hi + lo of the same scale
// (separate MFMAs into one fp32 accumulator, all 16 columns being in use).
// The code operands are unpacked once per step for all tiles.  The first
// product leaves lane (G, n) with column n's scores of tokens 4G..4G+3 of both
// 16-token halves of the step -- exactly the k slots the value layout gives
// that lane in the second product -- so p never crosses lanes.  Softmax
// statistics are per column, kept identical in the four lanes of a column.
#include <hip/hip_fp16.h>

#include "common.h"
#include "lanes.h"
#include "tiles.h"

namespace kvq {

namespace {

// Lazy running max: the max m of a column is raised only when a step's max
// exceeds it by more than kTau (log2 units), and the exponentials are taken
// against m + kTau, so p = 2^(s - m - kTau) <= 1 and p * s_v stays inside the
// f16 range (s_v itself is an fp16 value): the hi and lo parts of p * s_v can
// then both be at the unit scale and accumulate in one fp32 accumulator per
// tile, lo keeping absolute steps of 2^-24.  A raise rescales the tile's
// accumulator (32 products and the column's factor from its lanes), which
// with kTau = 0 most steps of a 32-column wave paid; a new maximum must now
// beat the running one by a factor of 16.  The price is lo's absolute step:
// 2^-24 against a largest p of 2^-kTau (measured on the parity cases: 2-bit
// errors 5.65e-4 -> 5.82e-4 from kTau = 2 to 4, far inside the 2e-3 bound).
constexpr float kTau = 4.0f;

// Mixed-precision helpers.  These are inline asm, and the compiler's hazard
// checks do not look inside inline asm: an operand written by an MFMA, a
// transcendental (exp) or a cross-lane move just before could be read stale.
// They are used only on operands that ordinary VALU instructions or LDS reads
// produce (params words, the query sum, f16 conversions and products), never
// on the MFMA scores or on exp results.

// a - (float)(low / high f16 half of h) in one mixed-precision fma (h * -1 + a
// with h read as f16), which the compiler otherwise emits as a conversion and
// a subtraction.  The difference is exact in fp32 when h holds a rounded to f16.
__device__ inline float sub_f16_lo(float a, uint32_t h) {
    float r;
    __asm__("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(a));
    return r;
}
__device__ inline float sub_f16_hi(float a, uint32_t h) {
    float r;
    __asm__("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(a));
    return r;
}

// hi(w) * x in one mixed-precision fma with a +0 addend (the compiler otherwise
// converts the half first); it rounds as the product does and differs only in
// giving +0 for a -0 product.
__device__ inline float mul_f16_hi(uint32_t w, float x) {
    float r;
    __asm__("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(x));
    return r;
}

// hi = f16(a, b), lo = f16(a - hi, b - hi): hi + lo carries ~22 bits of a, b.
__device__ inline void split_unit(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = f16x2(a, b);
    lo = f16x2(sub_f16_lo(a, hi), sub_f16_hi(b, hi));
}

// Position held by ring entry e at length L (e < min(L, s + w)): a sink, or the
// position of the recent window [max(s, L - w), L) that maps to e.
__device__ inline int ring_position(int e, int L, int s, int w) {
    if (e < s || w <= 0) return e;
    const int lo = max(s, L - w);
    return lo + ((e - s) - (lo - s) % w + w) % w;
}

// Block-table entries of the two 16-position subblocks of INT4 step r (the
// second is -1 past the INT4 region); loaded one step ahead of their use.
struct StepPages {
    int A, B;
};

__device__ inline StepPages step_pages(const PrefillArgs &a, const RowPlan &rp, int n4, int slot, int r) {
    StepPages p = {0, -1};
    if (r < n4) {
        const int pos0 = (rp.k0 + r) * 32;
        const int32_t *bt = a.block_table + (int64_t)slot * a.bt_stride;
        p.A = ldc(bt, pos0 >> a.logP);
        if (pos0 + 16 < rp.hi4) p.B = ldc(bt, (pos0 + 16) >> a.logP);
    }
    return p;
}

// 5 direct-to-LDS loads of step r of the tile into stage st (the decode kernel's
// step copy: key codes gathered by lane, value codes verbatim, params of both
// halves at kStKP / kStVP + 4 t).  BITS = 2 or 3: the main cache's low planes
// of subblocks A / B to 0 / 512 (keys) and 1024 / 1536 (values), at 3 bits the
// high planes to 2048 / 2304 (keys) and 2560 / 2816 (values), the params as
// for 4 bits -- still five loads.
template <int BITS>
__device__ inline void issue_prefill_step(const PrefillArgs &a, const RowPlan &rp, int n4, int slot, int hk, int r,
                                          StepPages pg, uint8_t *st, uint32_t offK, uint32_t offV, uint32_t offP4,
                                          uint32_t offP8, int lane) {
    if (r < n4) {
        constexpr size_t kSubBytes = (size_t)main_sub_bytes(BITS);
        const int pos0 = (rp.k0 + r) * 32;
        const int subs = a.P >> 4;
        const uint8_t *baseA = a.int4_pool +
            ((size_t)((int64_t)pg.A * a.H + hk) * subs + ((pos0 & (a.P - 1)) >> 4)) * kSubBytes;
        // subblock B past the INT4 region is never used; re-read A (valid memory)
        const uint8_t *baseB = baseA;
        if (pg.B >= 0) {
            baseB = a.int4_pool +
                ((size_t)((int64_t)pg.B * a.H + hk) * subs + (((pos0 + 16) & (a.P - 1)) >> 4)) * kSubBytes;
        }
        if constexpr (BITS == 2) {
            const uint32_t off = 16 * (uint32_t)lane;
            if (lane < 32) {
                dma16(baseA + kSub2K, off, st + 0);
                dma16(baseB + kSub2K, off, st + 512);
                dma16(baseA + kSub2V, off, st + 1024);
                dma16(baseB + kSub2V, off, st + 1536);
            }
            if (lane < 16) dma16((lane & 4) ? baseB : baseA, offP4 - kSub4KP + kSub2KP, st + 4096);
        } else if constexpr (BITS == 3) {
            const uint8_t *lo = lane < 32 ? baseA : baseB;
            const uint32_t off = 16 * (uint32_t)(lane & 31);
            dma16(lo + kSub3K, off, st + 0);
            dma16(lo + kSub3V, off, st + 1024);
            if (lane < 32) {
                const uint8_t *hi = lane < 16 ? baseA : baseB;
                const uint32_t offh = 16 * (uint32_t)(lane & 15);
                dma16(hi + kSub3KH, offh, st + 2048);
                dma16(hi + kSub3VH, offh, st + 2560);
            }
            if (lane < 16) dma16((lane & 4) ? baseB : baseA, offP4 - kSub4KP + kSub3KP, st + 4096);
        } else {
            dma16(baseA + kSub4K, offK, st + 0);
            dma16(baseB + kSub4K, offK, st + 1024);
            dma16(baseA + kSub4V, offV, st + 2048);
            dma16(baseB + kSub4V, offV, st + 3072);
            if (lane < 16) dma16((lane & 4) ? baseB : baseA, offP4, st + 4096);
        }
    } else {
        const uint8_t *base = a.int8_pool + ((size_t)((int64_t)slot * a.H + hk) * a.nr8 + (r - n4)) * kSub8Bytes;
        dma16(base + kSub8KLo, offK, st + 0);
        dma16(base + kSub8KHi, offK, st + 1024);
        dma16(base + kSub8VLo, offV, st + 2048);
        dma16(base + kSub8VHi, offV, st + 3072);
        if (lane < 16 && (lane & 4) == 0) dma16(base, offP8, st + 4096);
    }
}

}  // namespace

// Dispatch order of the waves (launches of at most 64 sequences): the
// workgroups are dispatched in linear index order and a wave's time grows with
// its causal prefix, so the waves are handed out longest prefix first over
// all sequences (heads of one block of rows together), which leaves the
// shortest waves for the end of the launch.  A wave of RW rows of sequence b
// ends at position pmax(b, v) = L_b - T_b + min((v + 1) RW, T_b) - 1.  Lane l
// holds sequence l; the wave finds the k-th largest pmax by a binary search on
// the count of waves at or above a bound, and among equal ones takes them in
// sequence order.  Simulated on the 8 x 1024-row Qwen3-8B chunks (waves of
// 8 rows, 2048 resident, time proportional to the prefix), the makespan goes
// from 7.5% to 3.9% above a perfect split.
struct PrefillTask {
    int b, hk, wv;          // b = -1: no work for this workgroup
};

__device__ inline int wave_sum_i(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return uni(x);
}
__device__ inline int wave_max_i(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
    return uni(x);
}

__device__ inline PrefillTask prefill_task(const PrefillArgs &a, int RW, int lane) {
    const int64_t i = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t k = i / a.H;
    PrefillTask tk;
    tk.b = -1;
    tk.hk = (int)(i - k * a.H);
    tk.wv = 0;
    const bool in = lane < a.B;
    const int T = in ? ldc(a.q_start, lane + 1) - ldc(a.q_start, lane) : 0;
    const int base = in ? ldc(a.ctx_len, lane) - T : 0;    // position of the chunk's first row
    const int nw = (T + RW - 1) / RW;
    // waves of this lane's sequence with pmax >= x
    auto count_ge = [&](int x) {
        const int y = x + 1 - base;
        const int c = T == 0 ? 0 : (y <= 1 ? nw : (y > T ? 0 : nw - (y + RW - 1) / RW + 1));
        return wave_sum_i(c);
    };
    if (k >= wave_sum_i(nw)) return tk;
    // the largest x with count_ge(x) > k (pmax >= 0 for every wave)
    int lo = 0, hi = wave_max_i(T > 0 ? base + T - 1 : 0);
    while (lo < hi) {
        const int mid = lo + (hi - lo + 1) / 2;
        if (count_ge(mid) > k) lo = mid;
        else hi = mid - 1;
    }
    // rank among the waves ending exactly at lo (at most one per sequence)
    const int j = (int)(k - count_ge(lo + 1));
    const int y = lo + 1 - base;
    const bool at = T > 0 && y >= 1 && y <= T && (y == T || y % RW == 0);
    uint64_t m = __ballot(at);
    for (int r = 0; r < j; ++r) m &= m - 1;
    const int src = __ffsll((unsigned long long)m) - 1;
    const int yb = __builtin_amdgcn_readlane(y, src), Tb = __builtin_amdgcn_readlane(T, src);
    const int nwb = __builtin_amdgcn_readlane(nw, src);
    tk.b = src;
    tk.wv = yb == Tb ? nwb - 1 : yb / RW - 1;
    return tk;
}

// Waves per SIMD: the two-tile 4-bit kernel needs ~250 registers (two waves);
// the one-tile 3- and 2-bit kernels fit 168 (three waves).
template <int BITS>
constexpr int kPrefillWaves = prefill_tiles(BITS) == 2 ? 2 : 3;

// BITS: width of the main cache's codes (4, 3 or 2; KV4-RL, "Future Directions").
template <int BITS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(kPrefillWaves<BITS>, kPrefillWaves<BITS>)))
void prefill_kernel(PrefillArgs a) {
    constexpr int NT = prefill_tiles(BITS);
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];
    const int lane = threadIdx.x;
    int b, hk, wv;
    if (a.B <= 64) {
        const PrefillTask tk = prefill_task(a, a.R * NT, lane);
        if (tk.b < 0) return;
        b = tk.b;
        hk = tk.hk;
        wv = tk.wv;
    } else {
        // waves in reverse order inside each sequence: its longest causal
        // prefixes are dispatched first
        b = blockIdx.z;
        hk = blockIdx.y;
        wv = (int)(gridDim.x - 1 - blockIdx.x);
    }
    const int row0 = ldc(a.q_start, b);
    const int T = ldc(a.q_start, b + 1) - row0;
    const int t0 = wv * a.R * NT;               // the wave's first row
    if (t0 >= T) return;
    const int L = ldc(a.ctx_len, b);
    const int slot = ldc(a.slot, b);
    const int nrow = min(a.R * NT, T - t0);
    const int pos0 = L - T + t0;                // position of the wave's first row
    const int pmax = pos0 + nrow - 1;           // and of its last

    // Tile k holds rows t0 + k R .. ; this lane's column n of tile k is (row
    // n / g, head n % g).  Columns past a tile's rows repeat the tile's column
    // 0 (a tile without rows: the wave's first column) and are never stored.
    const int G = lane >> 4, n = lane & 15;
    int ncol[NT], crow[NT], chead[NT], cpos[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const int nr = min(max(nrow - k * a.R, 0), a.R);
        ncol[k] = nr * a.g;
        const int cn = n < ncol[k] ? n : 0;
        crow[k] = nr > 0 ? k * a.R + cn / a.g : 0;     // row within the wave
        chead[k] = cn % a.g;
        cpos[k] = pos0 + crow[k];               // causal bound of the column
    }

    // ---- queries of the columns: dims 32 G .. 32 G + 31, rotated (SAW-INT4,
    // section 2, block-diagonal Hadamard; strides below 32 in the lane, 32 and
    // 64 across lanes G ^ 1, G ^ 2), scaled by one power of two 2^e for the
    // wave, split into f16 hi + lo of the same scale
    half8 qh[NT][4], ql[NT][4];
    float Rh[NT];
    float K1;
    {
        float x[NT][32];
        float sum[NT], amax = 0.0f;
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            const uint16_t *qp =
                a.q + ((int64_t)(row0 + t0 + crow[k]) * a.Hq + (int64_t)hk * a.g + chead[k]) * kHeadDim + 32 * G;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const u32x4 wq = ldg<u32x4>(qp + 8 * v);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[k][8 * v + 2 * e] = bf16f(wq[e] & 0xFFFFu);
                    x[k][8 * v + 2 * e + 1] = bf16f(wq[e] >> 16);
                }
            }
#pragma unroll
            for (int len = 1; len < 32; len <<= 1) {
                if (len < a.h) {
#pragma unroll
                    for (int i = 0; i < 32; ++i) {
                        if ((i & len) == 0) {
                            const float u = x[k][i], v = x[k][i + len];
                            x[k][i] = u + v;
                            x[k][i + len] = u - v;
                        }
                    }
                }
            }
            if (32 < a.h) {
#pragma unroll
                for (int i = 0; i < 32; ++i) x[k][i] = butterfly<16>(x[k][i], lane);
            }
            if (64 < a.h) {
#pragma unroll
                for (int i = 0; i < 32; ++i) x[k][i] = butterfly<32>(x[k][i], lane);
            }
            float sm = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                sm += x[k][i];
                amax = fmaxf(amax, fabsf(x[k][i]));
            }
            sum[k] = sum_rows(sm) * a.inv_sqrt_h;   // the column's four lanes
        }
        amax = wave_max(amax) * a.inv_sqrt_h;
        int E = 0;
        (void)frexpf(amax, &E);
        const int e = amax > 0.0f ? 14 - E : 0;      // |q * 2^e| < 2^14
        const float sc = a.inv_sqrt_h * ldexpf(1.0f, e);
        const float s16 = sc * 0.0625f;
        K1 = ldexpf(kLog2e * 0.08838834764831845f, 24 - e);   // log2(e) / sqrt(128), undoing 2^(e - 24)
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            Rh[k] = ldexpf(sum[k], e - 24);
            // chunks of 8 dims in the nibble order of a code dword: dims 0,4 | 1,5 (/16) | 2,6 | 3,7 (/16)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float *y = x[k] + 8 * c;
                uint32_t H[4], Lo[4];
                split2<1>(y[0] * sc, y[4] * sc, H[0], Lo[0]);
                split2<1>(y[1] * s16, y[5] * s16, H[1], Lo[1]);
                split2<1>(y[2] * sc, y[6] * sc, H[2], Lo[2]);
                split2<1>(y[3] * s16, y[7] * s16, H[3], Lo[3]);
                qh[k][c] = pack8(H[0], H[1], H[2], H[3]);
                ql[k][c] = pack8(Lo[0], Lo[1], Lo[2], Lo[3]);
            }
        }
    }

    // ---- the wave's steps: INT4 steps up to its last row, then INT8 subblocks
    const RowPlan rp = row_plan(L, a.s, a.w);
    const int lim4 = min(rp.hi4, pmax + 1);
    const int n4 = lim4 > rp.lo4 ? ((lim4 + 31) >> 5) - rp.k0 : 0;
    const int wlo = max(a.s, L - a.w);          // first position of the recent window
    const int n8 = pmax >= wlo ? rp.n8 : min(rp.n8, (min(a.s, rp.n8e) + 15) >> 4);
    const int nsteps = n4 + n8;

    const uint32_t offK = n * 64 + G * 16;
    const uint32_t offV = lane * 16;
    const uint32_t offP4 = ((lane & 8) ? kSub4VP : kSub4KP) + (lane & 3) * 16;
    const uint32_t offP8 = ((lane & 8) ? kSub8VP : kSub8KP) + (lane & 3) * 16;

    int issued = 0;
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
        if (s < nsteps) {
            issue_prefill_step<BITS>(a, rp, n4, slot, hk, s, step_pages(a, rp, n4, slot, s), smem + s * kStageBytes, offK,
                               offV, offP4, offP8, lane);
            ++issued;
        }
    }
    StepPages next = step_pages(a, rp, n4, slot, kStages);    // pages of the producer's next step

    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // O[k][t]: tile k, row 4 G + i = column 4 G + i, dims 16 t + n; the hi and lo
    // parts of p s_v accumulate together
    floatx4 O[NT][8];
#pragma unroll
    for (int k = 0; k < NT; ++k)
#pragma unroll
        for (int t = 0; t < 8; ++t) O[k][t] = zero4;
    float mK[NT], lsum[NT], zsum[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        mK[k] = kNegInf;
        lsum[k] = 0.0f;
        zsum[k] = 0.0f;
    }

    for (int i = 0; i < nsteps; ++i) {
        wait_vm_steps(issued - i - 1);
        uint8_t *st = smem + (i % kStages) * kStageBytes;
        // a 2- or 3-bit main-cache step: 8 bytes of low-plane codes per lane and
        // subblock in words 0-1, the lane's high-plane dword in word 2
        const bool main2 = BITS != 4 && i < n4;
        u32x4 kA, kB, vA, vB;
        if (main2) {
            const u32x2 ka = *reinterpret_cast<const u32x2 *>(st + lane * 8);
            const u32x2 kb = *reinterpret_cast<const u32x2 *>(st + 512 + lane * 8);
            const u32x2 va = *reinterpret_cast<const u32x2 *>(st + 1024 + lane * 8);
            const u32x2 vb = *reinterpret_cast<const u32x2 *>(st + 1536 + lane * 8);
            const uint32_t kha = BITS == 3 ? lds32(st + 2048 + 4 * lane) : 0u;
            const uint32_t khb = BITS == 3 ? lds32(st + 2304 + 4 * lane) : 0u;
            const uint32_t vha = BITS == 3 ? lds32(st + 2560 + 4 * lane) : 0u;
            const uint32_t vhb = BITS == 3 ? lds32(st + 2816 + 4 * lane) : 0u;
            kA = u32x4{ka[0], ka[1], kha, 0u};
            kB = u32x4{kb[0], kb[1], khb, 0u};
            vA = u32x4{va[0], va[1], vha, 0u};
            vB = u32x4{vb[0], vb[1], vhb, 0u};
        } else {
            kA = *reinterpret_cast<const u32x4 *>(st + lane * 16);
            kB = *reinterpret_cast<const u32x4 *>(st + 1024 + lane * 16);
            vA = *reinterpret_cast<const u32x4 *>(st + 2048 + lane * 16);
            vB = *reinterpret_cast<const u32x4 *>(st + 3072 + lane * 16);
        }
        const u32x4 kpA = *reinterpret_cast<const u32x4 *>(st + kStKP + 16 * G);
        const u32x4 kpB = *reinterpret_cast<const u32x4 *>(st + kStKP + 64 + 16 * G);
        const u32x4 vpA = *reinterpret_cast<const u32x4 *>(st + kStVP + 16 * G);
        const u32x4 vpB = *reinterpret_cast<const u32x4 *>(st + kStVP + 64 + 16 * G);
        wait_lgkm0();
        if (i + kStages < nsteps) {
            issue_prefill_step<BITS>(a, rp, n4, slot, hk, i + kStages, next, st, offK, offV, offP4, offP8, lane);
            ++issued;
            next = step_pages(a, rp, n4, slot, i + kStages + 1);
        }
        const bool int8 = i >= n4;

        // scores of tokens 4G + j (A half) and 16 + 4G + j (B half) for column n
        // of each tile; the key codes are unpacked once for both tiles
        floatx4 sA[NT], sB[NT];
#pragma unroll
        for (int k = 0; k < NT; ++k) sA[k] = sB[k] = zero4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            half8 ak, bk;
            if (main2) {
                // chunk c: dword c / 2 of the lane's 8 bytes, bytes (0, 2) or (1, 3)
                const uint32_t xa = kA[c >> 1] >> (8 * (c & 1)), xb = kB[c >> 1] >> (8 * (c & 1));
                ak = BITS == 3 ? int3_key_chunk(xa, kA[2], c) : int2_chunk(xa);
                bk = BITS == 3 ? int3_key_chunk(xb, kB[2], c) : int2_chunk(xb);
            } else {
                const uint32_t x = kA[c], x8 = x >> 8;
                ak = pack8(x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u);
                const uint32_t y = kB[c], y8 = y >> 8;
                bk = pack8(y & 0x000F000Fu, y & 0x00F000F0u, y8 & 0x000F000Fu, y8 & 0x00F000F0u);
            }
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                sA[k] = mfma16(ak, qh[k][c], sA[k]);
                sB[k] = mfma16(bk, qh[k][c], sB[k]);
                sA[k] = mfma16(ak, ql[k][c], sA[k]);
                sB[k] = mfma16(bk, ql[k][c], sB[k]);
            }
        }
        const int base = int8 ? 16 * (i - n4) : (rp.k0 + i) * 32;
        // an INT4 step inside the region and at or before the wave's first row
        // is valid for every column: no per-position tests
        const bool full = !int8 && base >= rp.lo4 && base + 32 <= min(rp.hi4, pos0 + 1);
        // value (scale, zero) of the step's tokens (shared by the columns)
        uint32_t vpr[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            vpr[j] = vpA[j];
            vpr[4 + j] = int8 ? 0u : vpB[j];
        }
        half8 ph[NT], pl[NT];
#pragma unroll
        for (int k = 0; k < NT; ++k) {
            float t[8];
            uint32_t vp[8];
            floatx4 a4 = sA[k];
            if (int8) {
#pragma unroll
                for (int j = 0; j < 4; ++j) a4[j] = fmaf(sB[k][j], 16.0f, a4[j]);   // high-nibble plane
            }
            if (full) {
                // the common step: one wave-uniform branch, no per-position selects
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    t[j] = fmaf(a4[j], h_lo(kpA[j]), mul_f16_hi(kpA[j], Rh[k]));
                    t[4 + j] = fmaf(sB[k][j], h_lo(kpB[j]), mul_f16_hi(kpB[j], Rh[k]));
                    vp[j] = vpr[j];
                    vp[4 + j] = vpr[4 + j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bool okA, okB;
                    if (int8) {
                        const int e = base + 4 * G + j;
                        okA = e < rp.n8e && ring_position(e, L, a.s, a.w) <= cpos[k];
                        okB = false;
                    } else {
                        const int pA = base + 4 * G + j, pB = pA + 16;
                        okA = pA >= rp.lo4 && pA < rp.hi4 && pA <= cpos[k];
                        okB = pB >= rp.lo4 && pB < rp.hi4 && pB <= cpos[k];
                    }
                    // params of positions outside the context may be arbitrary bytes
                    // (NaN as fp16): dropped by a select, never multiplied by zero
                    const float tA = fmaf(a4[j], h_lo(kpA[j]), mul_f16_hi(kpA[j], Rh[k]));
                    const float tB = fmaf(sB[k][j], h_lo(kpB[j]), mul_f16_hi(kpB[j], Rh[k]));
                    t[j] = okA ? tA : kNegInf;
                    t[4 + j] = okB ? tB : kNegInf;
                    vp[j] = okA ? vpr[j] : 0u;
                    vp[4 + j] = okB ? vpr[4 + j] : 0u;
                }
            }

            // online softmax of the column
            float ml = t[0];
#pragma unroll
            for (int j = 1; j < 8; ++j) ml = fmaxf(ml, t[j]);
            if (__any(ml * K1 > mK[k] + kTau)) {
                const float mt = max_rows(ml) * K1;
                const bool grow = mt > mK[k] + kTau;
                const float mnew = grow ? mt : mK[k];
                const float alpha = mK[k] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mK[k] - mnew);
                lsum[k] *= alpha;
                zsum[k] *= alpha;
                mK[k] = mnew;
                // accumulator row r of this lane is column 4 G + r
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ar = __shfl(alpha, 4 * G + r, 64);
#pragma unroll
                    for (int tt = 0; tt < 8; ++tt) O[k][tt][r] *= ar;
                }
            }
            // a column with no valid position yet keeps mK = -inf: its p are exp2(-inf) = 0
            const float nm = mK[k] == kNegInf ? 0.0f : -(mK[k] + kTau);
            float pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = __builtin_amdgcn_exp2f(fmaf(t[j], K1, nm));
                lsum[k] += p;
                zsum[k] = fmaf(p, h_hi(vp[j]), zsum[k]);
                pv[j] = p * h_lo(vp[j]);
            }
            if (int8) {
                // the B half of the step is the high-nibble plane of the same entries
#pragma unroll
                for (int j = 0; j < 4; ++j) pv[4 + j] = 16.0f * pv[j];
            }
            // A operand in the value layout's k order: A0 A2 A1 A3 | B0 B2 B1 B3
            uint32_t H0, H1, H2, H3, L0, L1, L2, L3;
            split_unit(pv[0], pv[2], H0, L0);
            split_unit(pv[1], pv[3], H1, L1);
            split_unit(pv[4], pv[6], H2, L2);
            split_unit(pv[5], pv[7], H3, L3);
            ph[k] = pack8(H0, H1, H2, H3);
            pl[k] = pack8(L0, L1, L2, L3);
        }
        // value tiles, unpacked once for both query tiles
        if (main2) {
            // dword cc, field f: dims 16 (4 cc + f) + n, tile 4 cc + f (odd tiles
            // scaled by 16 as the 4-bit ones)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint32_t x = vA[cc], x8 = x >> 8, y = vB[cc], y8 = y >> 8;
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const half8 vt = BITS == 3
                        ? pack8(int3_value_field(x, vA[2], cc, f, false), int3_value_field(x8, vA[2], cc, f, true),
                                int3_value_field(y, vB[2], cc, f, false), int3_value_field(y8, vB[2], cc, f, true))
                        : pack8(int2_field(x, f), int2_field(x8, f), int2_field(y, f), int2_field(y8, f));
#pragma unroll
                    for (int k = 0; k < NT; ++k) {
                        O[k][4 * cc + f] = mfma16(ph[k], vt, O[k][4 * cc + f]);
                        O[k][4 * cc + f] = mfma16(pl[k], vt, O[k][4 * cc + f]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t x = vA[c], x8 = x >> 8, y = vB[c], y8 = y >> 8;
                const half8 ve = pack8(x & 0x000F000Fu, x8 & 0x000F000Fu, y & 0x000F000Fu, y8 & 0x000F000Fu);
                const half8 vo = pack8(x & 0x00F000F0u, x8 & 0x00F000F0u, y & 0x00F000F0u, y8 & 0x00F000F0u);
#pragma unroll
                for (int k = 0; k < NT; ++k) {
                    O[k][2 * c] = mfma16(ph[k], ve, O[k][2 * c]);
                    O[k][2 * c] = mfma16(pl[k], ve, O[k][2 * c]);
                    O[k][2 * c + 1] = mfma16(ph[k], vo, O[k][2 * c + 1]);
                    O[k][2 * c + 1] = mfma16(pl[k], vo, O[k][2 * c + 1]);
                }
            }
        }
    }

    // ---- output: out = (sum p s_v c_v + sum p z_v) / sum p per column
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const float ls = sum_rows(lsum[k]);
        const float zs = sum_rows(zsum[k]);
        const float rl = 1.0f / ls;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int col = 4 * G + r;
            const float ir = __shfl(rl, col, 64);
            const float zr = __shfl(zs, col, 64);
            if (col < ncol[k]) {
                const int rr = k * a.R + col / a.g, hd = col % a.g;
                float *o = a.out + ((int64_t)(row0 + t0 + rr) * a.Hq + (int64_t)hk * a.g + hd) * kHeadDim;
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) {
                    const float sc = (tt & 1) ? 1048576.0f : 16777216.0f;   // 2^20 / 2^24 code scaling
                    o[16 * tt + n] = fmaf(O[k][tt][r], sc, zr) * ir;
                }
            }
        }
        if (a.lse && G == 0 && n < ncol[k])
            a.lse[(int64_t)(row0 + t0 + crow[k]) * a.Hq + (int64_t)hk * a.g + chead[k]] = (mK[k] + kTau + __log2f(ls)) / kLog2e;
    }
}

hipError_t launch_prefill(const PrefillArgs &a, int tiles, hipStream_t stream) {
    const dim3 grid((unsigned)tiles, (unsigned)a.H, (unsigned)a.B);
    if (a.bits == 2)
        hipLaunchKernelGGL(prefill_kernel<2>, grid, dim3(64), 0, stream, a);
    else if (a.bits == 3)
        hipLaunchKernelGGL(prefill_kernel<3>, grid, dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL(prefill_kernel<4>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
