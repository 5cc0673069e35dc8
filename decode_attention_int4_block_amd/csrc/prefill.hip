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
// Work: one wave per (sequence, KV head, tile of R rows), R = floor(16 / g), so
// that the tile's (row, query head) pairs fill the 16 columns of
// v_mfma_f32_16x16x32_f16.  The wave streams the tile's causal prefix through
// the same 3-stage LDS ring of 5-load steps as the decode kernel (INT4 steps of
// 32 positions, INT8 steps of 16 ring entries) and per step computes
//   S[tok][col] = codes[tok][:] . Q[:][col]          A = codes, B = query
//   O[col][dim] += P[col][tok] * vcodes[tok][dim]    A = p * s_v, B = codes
// with the query and p * s_v each split into f16 hi + lo (separate MFMAs, all
// 16 columns being in use).  The first product leaves lane (G, n) with column
// n's scores of tokens 4G..4G+3 of both 16-token halves of the step -- exactly
// the k slots the value layout gives that lane in the second product -- so p
// never crosses lanes.  Softmax statistics are per column, kept identical in
// the four lanes of a column.
#include <hip/hip_fp16.h>

#include "common.h"
#include "lanes.h"
#include "tiles.h"

namespace kvq {

namespace {

constexpr float kTau = 8.0f;            // lazy max: p <= 2^kTau
constexpr float kHiScale = 256.0f;      // hi part of p * s_v holds pv / 256

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
// halves at kStKP / kStVP + 4 t).
__device__ inline void issue_prefill_step(const PrefillArgs &a, const RowPlan &rp, int n4, int slot, int hk, int r,
                                          StepPages pg, uint8_t *st, uint32_t offK, uint32_t offV, uint32_t offP4,
                                          uint32_t offP8, int lane) {
    if (r < n4) {
        const int pos0 = (rp.k0 + r) * 32;
        const int subs = a.P >> 4;
        const uint8_t *baseA = a.int4_pool +
            ((size_t)((int64_t)pg.A * a.H + hk) * subs + ((pos0 & (a.P - 1)) >> 4)) * kSub4Bytes;
        // subblock B past the INT4 region is never used; re-read A (valid memory)
        const uint8_t *baseB = baseA;
        if (pg.B >= 0) {
            baseB = a.int4_pool +
                ((size_t)((int64_t)pg.B * a.H + hk) * subs + (((pos0 + 16) & (a.P - 1)) >> 4)) * kSub4Bytes;
        }
        dma16(baseA + kSub4K, offK, st + 0);
        dma16(baseB + kSub4K, offK, st + 1024);
        dma16(baseA + kSub4V, offV, st + 2048);
        dma16(baseB + kSub4V, offV, st + 3072);
        if (lane < 16) dma16((lane & 4) ? baseB : baseA, offP4, st + 4096);
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

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];
    const int lane = threadIdx.x;
    const int b = blockIdx.z, hk = blockIdx.y;
    const int row0 = ldc(a.q_start, b);
    const int T = ldc(a.q_start, b + 1) - row0;
    // tiles in reverse order: the longest causal prefixes are dispatched first
    const int tile = (int)(gridDim.x - 1 - blockIdx.x);
    const int t0 = tile * a.R;
    if (t0 >= T) return;
    const int L = ldc(a.ctx_len, b);
    const int slot = ldc(a.slot, b);
    const int nrow = min(a.R, T - t0);
    const int pos0 = L - T + t0;                // position of the tile's first row
    const int pmax = pos0 + nrow - 1;           // and of its last

    // This lane's column n = (row n / g, head n % g); columns past the tile's
    // rows repeat column 0 and are never stored.
    const int G = lane >> 4, n = lane & 15;
    const int ncol = nrow * a.g;
    const int cn = n < ncol ? n : 0;
    const int crow = cn / a.g, chead = cn % a.g;
    const int cpos = pos0 + crow;               // causal bound of the column

    // ---- query of the column: dims 32 G .. 32 G + 31, rotated (SAW-INT4,
    // section 2, block-diagonal Hadamard; strides below 32 in the lane, 32 and
    // 64 across lanes G ^ 1, G ^ 2), scaled by 2^e, split into f16 hi + lo
    half8 qh[4], ql[4];
    float K1, Rh;
    {
        const uint16_t *qp = a.q + ((int64_t)(row0 + t0 + crow) * a.Hq + (int64_t)hk * a.g + chead) * kHeadDim + 32 * G;
        float x[32];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const u32x4 wv = ldg<u32x4>(qp + 8 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * v + 2 * e] = bf16f(wv[e] & 0xFFFFu);
                x[8 * v + 2 * e + 1] = bf16f(wv[e] >> 16);
            }
        }
#pragma unroll
        for (int len = 1; len < 32; len <<= 1) {
            if (len < a.h) {
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    if ((i & len) == 0) {
                        const float u = x[i], v = x[i + len];
                        x[i] = u + v;
                        x[i + len] = u - v;
                    }
                }
            }
        }
        if (32 < a.h) {
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] = butterfly<16>(x[i], lane);
        }
        if (64 < a.h) {
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] = butterfly<32>(x[i], lane);
        }
        float sum = 0.0f, amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            sum += x[i];
            amax = fmaxf(amax, fabsf(x[i]));
        }
        sum = sum_rows(sum) * a.inv_sqrt_h;          // the column's four lanes
        amax = wave_max(amax) * a.inv_sqrt_h;
        int E = 0;
        (void)frexpf(amax, &E);
        const int e = amax > 0.0f ? 14 - E : 0;      // |q * 2^e| < 2^14
        const float sc = a.inv_sqrt_h * ldexpf(1.0f, e);
        const float s16 = sc * 0.0625f;
        K1 = ldexpf(kLog2e * 0.08838834764831845f, 24 - e);   // log2(e) / sqrt(128), undoing 2^(e - 24)
        Rh = ldexpf(sum, e - 24);
        // chunks of 8 dims in the nibble order of a code dword: dims 0,4 | 1,5 (/16) | 2,6 | 3,7 (/16)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float *y = x + 8 * k;
            uint32_t H[4], Lo[4];
            split2<1>(y[0] * sc, y[4] * sc, H[0], Lo[0]);
            split2<1>(y[1] * s16, y[5] * s16, H[1], Lo[1]);
            split2<1>(y[2] * sc, y[6] * sc, H[2], Lo[2]);
            split2<1>(y[3] * s16, y[7] * s16, H[3], Lo[3]);
            qh[k] = pack8(H[0], H[1], H[2], H[3]);
            ql[k] = pack8(Lo[0], Lo[1], Lo[2], Lo[3]);
        }
    }

    // ---- the tile's steps: INT4 steps up to its last row, then INT8 subblocks
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
            issue_prefill_step(a, rp, n4, slot, hk, s, step_pages(a, rp, n4, slot, s), smem + s * kStageBytes, offK,
                               offV, offP4, offP8, lane);
            ++issued;
        }
    }
    StepPages next = step_pages(a, rp, n4, slot, kStages);    // pages of the producer's next step

    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    floatx4 Oh[8], Ol[8];                       // O[col 4G + i][16 t + n], hi (x 256) and lo parts
#pragma unroll
    for (int t = 0; t < 8; ++t) Oh[t] = Ol[t] = zero4;
    float mK = kNegInf, lsum = 0.0f, zsum = 0.0f;

    for (int i = 0; i < nsteps; ++i) {
        wait_vm_steps(issued - i - 1);
        uint8_t *st = smem + (i % kStages) * kStageBytes;
        const u32x4 kA = *reinterpret_cast<const u32x4 *>(st + lane * 16);
        const u32x4 kB = *reinterpret_cast<const u32x4 *>(st + 1024 + lane * 16);
        const u32x4 vA = *reinterpret_cast<const u32x4 *>(st + 2048 + lane * 16);
        const u32x4 vB = *reinterpret_cast<const u32x4 *>(st + 3072 + lane * 16);
        const u32x4 kpA = *reinterpret_cast<const u32x4 *>(st + kStKP + 16 * G);
        const u32x4 kpB = *reinterpret_cast<const u32x4 *>(st + kStKP + 64 + 16 * G);
        const u32x4 vpA = *reinterpret_cast<const u32x4 *>(st + kStVP + 16 * G);
        const u32x4 vpB = *reinterpret_cast<const u32x4 *>(st + kStVP + 64 + 16 * G);
        wait_lgkm0();
        if (i + kStages < nsteps) {
            issue_prefill_step(a, rp, n4, slot, hk, i + kStages, next, st, offK, offV, offP4, offP8, lane);
            ++issued;
            next = step_pages(a, rp, n4, slot, i + kStages + 1);
        }
        const bool int8 = i >= n4;

        // scores of tokens 4G + j (A half) and 16 + 4G + j (B half) for column n
        floatx4 hA = zero4, lA = zero4, hB = zero4, lB = zero4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t x = kA[c], x8 = x >> 8;
            const half8 ak = pack8(x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u);
            const uint32_t y = kB[c], y8 = y >> 8;
            const half8 bk = pack8(y & 0x000F000Fu, y & 0x00F000F0u, y8 & 0x000F000Fu, y8 & 0x00F000F0u);
            hA = mfma16(ak, qh[c], hA);
            lA = mfma16(ak, ql[c], lA);
            hB = mfma16(bk, qh[c], hB);
            lB = mfma16(bk, ql[c], lB);
        }
        float t[8];
        uint32_t vp[8];
        {
            const floatx4 sB = hB + lB;
            floatx4 sA = hA + lA;
            if (int8) {
#pragma unroll
                for (int j = 0; j < 4; ++j) sA[j] = fmaf(sB[j], 16.0f, sA[j]);   // high-nibble plane
            }
            const int base = int8 ? 16 * (i - n4) : (rp.k0 + i) * 32;
            // an INT4 step inside the region and at or before the tile's first
            // row is valid for every column: no per-position tests
            const bool full = !int8 && base >= rp.lo4 && base + 32 <= min(rp.hi4, pos0 + 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bool okA, okB;
                if (full) {
                    okA = okB = true;
                } else if (int8) {
                    const int e = base + 4 * G + j;
                    okA = e < rp.n8e && ring_position(e, L, a.s, a.w) <= cpos;
                    okB = false;
                } else {
                    const int pA = base + 4 * G + j, pB = pA + 16;
                    okA = pA >= rp.lo4 && pA < rp.hi4 && pA <= cpos;
                    okB = pB >= rp.lo4 && pB < rp.hi4 && pB <= cpos;
                }
                // params of positions outside the context may be arbitrary bytes
                // (NaN as fp16): dropped by a select, never multiplied by zero
                const float tA = fmaf(sA[j], h_lo(kpA[j]), h_hi(kpA[j]) * Rh);
                const float tB = fmaf(sB[j], h_lo(kpB[j]), h_hi(kpB[j]) * Rh);
                t[j] = okA ? tA : kNegInf;
                t[4 + j] = okB ? tB : kNegInf;
                vp[j] = okA ? vpA[j] : 0u;
                vp[4 + j] = okB ? vpB[j] : 0u;
            }
        }

        // online softmax of the column (lazy max)
        float ml = t[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) ml = fmaxf(ml, t[j]);
        if (__any(ml * K1 > mK + kTau)) {
            const float mt = max_rows(ml) * K1;
            const bool grow = mt > mK + kTau;
            const float mnew = grow ? mt : mK;
            const float alpha = mK == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mK - mnew);
            lsum *= alpha;
            zsum *= alpha;
            mK = mnew;
            // accumulator row i of this lane is column 4 G + i
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * G + r, 64);
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) {
                    Oh[tt][r] *= ar;
                    Ol[tt][r] *= ar;
                }
            }
        }
        // a column with no valid position yet keeps mK = -inf: its p are exp2(-inf) = 0
        const float nm = mK == kNegInf ? 0.0f : -mK;
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float p = __builtin_amdgcn_exp2f(fmaf(t[j], K1, nm));
            lsum += p;
            zsum = fmaf(p, h_hi(vp[j]), zsum);
            pv[j] = p * h_lo(vp[j]);
        }
        if (int8) {
            // the B half of the step is the high-nibble plane of the same entries
#pragma unroll
            for (int j = 0; j < 4; ++j) pv[4 + j] = 16.0f * pv[j];
        }
        // A operand in the value layout's k order: A0 A2 A1 A3 | B0 B2 B1 B3
        uint32_t H0, H1, H2, H3, L0, L1, L2, L3;
        split2<256>(pv[0], pv[2], H0, L0);
        split2<256>(pv[1], pv[3], H1, L1);
        split2<256>(pv[4], pv[6], H2, L2);
        split2<256>(pv[5], pv[7], H3, L3);
        const half8 ph = pack8(H0, H1, H2, H3), pl = pack8(L0, L1, L2, L3);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t x = vA[c], x8 = x >> 8, y = vB[c], y8 = y >> 8;
            const half8 ve = pack8(x & 0x000F000Fu, x8 & 0x000F000Fu, y & 0x000F000Fu, y8 & 0x000F000Fu);
            const half8 vo = pack8(x & 0x00F000F0u, x8 & 0x00F000F0u, y & 0x00F000F0u, y8 & 0x00F000F0u);
            Oh[2 * c] = mfma16(ph, ve, Oh[2 * c]);
            Ol[2 * c] = mfma16(pl, ve, Ol[2 * c]);
            Oh[2 * c + 1] = mfma16(ph, vo, Oh[2 * c + 1]);
            Ol[2 * c + 1] = mfma16(pl, vo, Ol[2 * c + 1]);
        }
    }

    // ---- output: out = (sum p s_v c_v + sum p z_v) / sum p per column
    lsum = sum_rows(lsum);
    zsum = sum_rows(zsum);
    const float rl = 1.0f / lsum;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int col = 4 * G + r;
        const float ir = __shfl(rl, col, 64);
        const float zr = __shfl(zsum, col, 64);
        if (col < ncol) {
            const int rr = col / a.g, hd = col % a.g;
            float *o = a.out + ((int64_t)(row0 + t0 + rr) * a.Hq + (int64_t)hk * a.g + hd) * kHeadDim;
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const float sc = (tt & 1) ? 1048576.0f : 16777216.0f;   // 2^20 / 2^24 code scaling
                o[16 * tt + n] = fmaf(fmaf(Oh[tt][r], kHiScale, Ol[tt][r]), sc, zr) * ir;
            }
        }
    }
    if (a.lse && G == 0 && n < ncol)
        a.lse[(int64_t)(row0 + t0 + crow) * a.Hq + (int64_t)hk * a.g + chead] = (mK + __log2f(lsum)) / kLog2e;
}

hipError_t launch_prefill(const PrefillArgs &a, int tiles, hipStream_t stream) {
    hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)tiles, (unsigned)a.H, (unsigned)a.B), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
