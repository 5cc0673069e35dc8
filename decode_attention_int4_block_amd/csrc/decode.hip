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
// hi in columns (rows) [0, GP), lo in [GP, 2GP) of the 16 the instruction has.
// 4-bit and 8-bit codes become f16 values exactly by masking them into the
// mantissa of a subnormal (code * 2^-24, or code * 2^-20 for the high nibble of
// a byte, compensated in the other operand or the accumulator).
//
// The softmax runs on a dense layout: the GP x 32 scores of a step are spread
// over the 64 lanes (GP / 2 per lane) by DPP moves inside 16-lane rows, and the
// p * scale_v products are gathered back into the MFMA row layout the same way.
#include <hip/hip_fp16.h>

#include "common.h"
#include "lanes.h"
#include "quant.h"
#include "tiles.h"

namespace kvq {

// Per group class GP (query heads per hi/lo half of the MFMA columns).
template <int GP>
struct GC {
    static constexpr bool kPacked = GP <= 8;
    static constexpr int kQ = kPacked ? 1 : 2;      // query operand sets per chunk
    static constexpr int kNP = GP / 4;              // score pairs per lane and step
    static constexpr int kNE = 2 * kNP;             // scores per lane and step
    static constexpr int kParts = 16 / GP;          // lanes of a 16-lane row sharing a head
    static constexpr int kVPL = 2 * GP;             // query values per lane (GP x 128 / 64)
    // The running max used for exp2 is raised only when a step's max exceeds it
    // by more than kTau (log2 units), so p <= 2^kTau; the hi rows of p*s_v then
    // hold pv / kHiScale so that they stay inside the f16 range.
    static constexpr float kTau = kPacked ? 8.0f : 0.0f;
    static constexpr int kHiScale = kPacked ? 256 : 1;
};

// ---------------------------------------------------------------------------
// Max / sum over the lanes that hold the same query head in the dense layout
// (lanes l with equal l % GP: kParts per row, four rows).
template <int GP>
__device__ inline float head_max(float x) {
    if constexpr (GP <= 8) x = fmaxf(x, dppf<kRowRor + 8>(0.0f, x));
    if constexpr (GP == 4) x = fmaxf(x, dppf<kRowRor + 4>(0.0f, x));
    return max_rows(x);
}
template <int GP>
__device__ inline float head_sum(float x) {
    if constexpr (GP <= 8) x += dppf<kRowRor + 8>(0.0f, x);
    if constexpr (GP == 4) x += dppf<kRowRor + 4>(0.0f, x);
    return sum_rows(x);
}

// Slot J (0..3) of the packed MFMA rows: lanes with column c < GP take the hi
// word of head c, columns [GP, 2GP) the lo word of head c - GP, both from the
// dense lane of the same head holding slot J (part J / kNP of the row; the
// caller passes that lane's words of local slot J % kNP).
template <int GP, int J>
__device__ inline uint32_t gather_slot(uint32_t hi, uint32_t lo) {
    constexpr int NP = GC<GP>::kNP;
    constexpr int qs = J / NP;
    constexpr int BH = GP == 4 ? 0x1 : 0x3;
    constexpr int BL = GP == 4 ? 0x2 : 0xC;
    if constexpr (qs == 0) {
        return dpp<kRowShr + GP, BL>(hi, lo);
    } else if constexpr (qs == 1) {
        return dpp<kRowShl + GP, BH>(lo, hi);
    } else {
        const uint32_t r = dpp<kRowShl + GP * qs, BH>(0u, hi);
        return dpp<kRowShl + GP * (qs - 1), BL>(r, lo);
    }
}


// ---------------------------------------------------------------------------
// Dense layout.  Lane (G, c) of a step holds kNP pairs of scores of head
// c % GP: pair j = kNP (c / GP) + p (p < kNP) is tokens (j & 1) + 2 ee, ee in
// {0, 1}, of rows 4G.. of subblock j >> 1 -- the k order [A0 A2 | A1 A3 | B0 B2
// | B1 B3] of the value MFMA, one dword of f16 pairs per j.
template <int GP>
struct LaneCtx {
    int lane, G, n, part, head;
    uint32_t offKP;                             // stage byte offset of this lane's first key params
    int tok4[GC<GP>::kNE];                      // token (entry) of each dense score within the step
};

template <int GP>
__device__ inline LaneCtx<GP> lane_ctx(int lane) {
    constexpr int NP = GC<GP>::kNP;
    LaneCtx<GP> L;
    L.lane = lane;
    L.G = lane >> 4;
    L.n = lane & 15;
    L.part = L.n / GP;
    L.head = L.n % GP;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int j = NP * L.part + p;
#pragma unroll
        for (int ee = 0; ee < 2; ++ee) L.tok4[2 * p + ee] = 16 * (j >> 1) + 4 * L.G + (j & 1) + 2 * ee;
    }
    const int j0 = NP * L.part;
    L.offKP = kStKP + 4 * (16 * (j0 >> 1) + 4 * L.G + (j0 & 1));
    return L;
}

// Data of one step as read from its LDS stage.
template <int GP>
struct StepRegs {
    u32x4 kA, kB;       // INT4: key codes of token l%16 (A/B), dims 32G..+32
                        // INT8: key bytes of entry l%16, dims 32G..+16 (kA) and +16..+32 (kB)
    u32x4 vA, vB;       // INT4: value codes, dims n + 32c / n + 16 + 32c, tokens 4G..4G+3
                        // INT8: value bytes, tiles 0..3 (vA) and 4..7 (vB), entries 4G..4G+3
    uint32_t kp[GC<GP>::kNE], vp[GC<GP>::kNE];   // params of this lane's dense scores
};

template <int GP>
struct SegCtx {
    half8 q4[GC<GP>::kQ][4];   // query operands (INT4 nibble order; INT8 keys are split into nibbles)
    float K1;           // 2^(24 - e) * log2(e) / sqrt(128), wave-uniform
    float Rh;           // sum(q~ of this lane's head) * 2^(e - 24)
    float Ko;           // grouped keys: sum(o_d q~_d) * 2^(e - 24) over this lane's head (else 0)
    float mK;           // running max of this lane's head (log2 units)
    float lsum, zsum;   // sums of p and of p * zero_v over this lane's scores
    floatx4 O[8];       // acc[row 4G+i][16 t + n], tile t scaled by tile_scale
};

// Wave-uniform position in the unit stream of one worker.
struct Cursor {
    int b, hk;          // segment (row, KV head)
    RowPlan rp;
    int r;              // unit index inside the segment
    int64_t u;          // global unit
};

// ---------------------------------------------------------------------------
// Row table.  The lengths and slots of rows [0, kResRows) stay in VGPRs for the
// whole kernel (lane l holds rows l + 64 k), so the wave-uniform row walks read
// them with v_readlane instead of a memory round trip; rows beyond are read
// from memory.
constexpr int kResRows = 256;

struct RowRegs {
    int L[4], S[4];
};

__device__ inline RowRegs load_rows(const DecodeArgs &a, int lane) {
    // all eight loads issued back to back (rows past B read row 0, B >= 1)
    int Lr[4], Sr[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int b = lane + 64 * k < a.B ? lane + 64 * k : 0;
        Lr[k] = a.ctx_len[b];
        Sr[k] = a.slot[b];
    }
    RowRegs R;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const bool in = lane + 64 * k < a.B;
        R.L[k] = in ? Lr[k] : 0;
        R.S[k] = in ? Sr[k] : 0;
    }
    return R;
}

__device__ inline int pick4(const int (&v)[4], int k) {
    return k == 0 ? v[0] : (k == 1 ? v[1] : (k == 2 ? v[2] : v[3]));
}
// ctx_len and slot of the wave-uniform row b
__device__ inline int row_len(const DecodeArgs &a, const RowRegs &R, int b) {
    if (b < kResRows) return __builtin_amdgcn_readlane(pick4(R.L, b >> 6), b & 63);
    return ldc(a.ctx_len, b);
}
__device__ inline int row_slot(const DecodeArgs &a, const RowRegs &R, int b) {
    if (b < kResRows) return __builtin_amdgcn_readlane(pick4(R.S, b >> 6), b & 63);
    return ldc(a.slot, b);
}

// Units of the work split: a segment of `cost` steps counts as a.seg_wt
// weight-only units followed by its steps (unit index u is global over these).
// Weight units carry the segment's fixed cost into the split; no wave issues
// them.
__device__ inline int seg_units(const DecodeArgs &a, const RowPlan &rp) {
    return rp.cost > 0 ? rp.cost + a.seg_wt : 0;
}

__device__ inline void cursor_next(const DecodeArgs &a, const RowRegs &R, Cursor &c) {
    ++c.u;
    if (++c.r < c.rp.cost) return;
    c.r = 0;
    c.u += a.seg_wt;        // over the next segment's weight units
    if (++c.hk < a.H) return;
    c.hk = 0;
    for (++c.b; c.b < a.B; ++c.b) {
        c.rp = row_plan(row_len(a, R, c.b), a.s, a.w);
        if (c.rp.cost > 0) return;
    }
}

// Block-table entries of the producer's steps, gathered 16 units at a time
// a whole half-batch before they are used.  The gather goes straight into LDS
// (one dword per lane through the direct global->LDS path), so no VGPR holds a
// load in flight across steps; the in-order vector-memory counter the stage
// waits already use covers it.  pg[h][0][j] / pg[h][1][j] are the pages of
// subblocks A / B of unit hb + j (INT8 units: the slot in [0]).
constexpr int kPgHalf = 16;
constexpr int kPgBytes = 2 * 2 * kPgHalf * 4;

// Wave-uniform row walk of the half-batches: the row holding the next
// half-batch's first unit and that row's first unit.
struct BatchCursor {
    int b;
    int64_t pre;
};

__device__ inline void fetch_pages(const DecodeArgs &a, const RowRegs &R, int64_t hb, int64_t u_end,
                                   BatchCursor &bc, int lane, uint32_t *pg_half) {
    const int64_t u = hb + (lane & (kPgHalf - 1));
    const int64_t lim = min(hb + kPgHalf, u_end);
    int myL = 0, myslot = 0;
    int64_t mypre = 0;
    bool mine = false;
    int b = bc.b;
    int64_t pre = bc.pre;
    while (b < a.B) {
        const int L = row_len(a, R, b);
        const int64_t rowu = (int64_t)seg_units(a, row_plan(L, a.s, a.w)) * a.H;
        if (pre + rowu > hb && rowu > 0) {
            const int sl = row_slot(a, R, b);
            if (u >= pre && u < pre + rowu) {
                mine = true;
                mypre = pre;
                myL = L;
                myslot = sl;
            }
        }
        if (pre + rowu >= lim) break;
        pre += rowu;
        ++b;
    }
    bc.b = b;
    bc.pre = pre;
    const int32_t *src = nullptr;
    uint32_t val = 0;
    if (mine && u < u_end) {
        const RowPlan rp = row_plan(myL, a.s, a.w);
        const uint32_t off = (uint32_t)(u - mypre);
        const uint32_t vc = (uint32_t)seg_units(a, rp);
        const uint32_t hk = off / vc;
        const int r = (int)(off - hk * vc) - a.seg_wt;
        if (r < 0) {
            // a weight unit: no step, never read
        } else if (r < rp.n4) {
            const int pos0 = (rp.k0 + r) * 32;
            // lanes kPgHalf.. take subblock B (the producer ignores it past the INT4 region)
            const int pos = (lane >= kPgHalf && pos0 + 16 < rp.hi4) ? pos0 + 16 : pos0;
            src = a.block_table + (int64_t)myslot * a.bt_stride + (pos >> a.logP);
        } else {
            val = (uint32_t)myslot;
        }
    }
    // lanes [0, kPgHalf) fill pa, [kPgHalf, 2 kPgHalf) pb; the others write nothing
    if (lane < 2 * kPgHalf) {
        if (src != nullptr)
            __builtin_amdgcn_global_load_lds(src, (lds_ptr)pg_half, 4, 0, kCachePolicyNonTemporal);
        else
            pg_half[lane] = val;
    }
}

struct Lookup {
    int slot, pageA, pageB;
};

// ---------------------------------------------------------------------------
// Query of one segment: load, block Hadamard rotation (SAW-INT4, section 2),
// power-of-two scaling, hi/lo split, and the MFMA B operands.
//
// Lane (G, c) rotates head c % GP, dims 32 G + kVPL (c / GP) + e (e < kVPL):
// Hadamard strides below kVPL stay inside the lane, a stride s at or above it
// pairs lanes l and l ^ (s / 2).  The B operand of chunk i (dims 32 G + 8 i ..)
// for column c is then gathered from the lane of part i / (kVPL / 8).
// The bf16 query values of lane (G, c) -- head c % GP, dims 32 G + kVPL (c / GP)
// .. + kVPL -- are copied into LDS by the producer together with the first step
// of the segment (kVPL / 8 direct loads of 16 bytes per lane), so no load into
// registers is in flight across steps.  Lanes of heads past g copy head 0.
template <int GP>
struct QRing {
    static constexpr int kLoads = GC<GP>::kVPL / 8;     // 16-byte loads per lane
    static constexpr int kBytes = kLoads * 1024;        // bytes per slot
    u32x4 w[kLoads];
};

template <int GP>
__device__ inline void issue_query(const DecodeArgs &a, int b, int hk, const LaneCtx<GP> &L, uint8_t *slot) {
    constexpr int V = GC<GP>::kVPL;
    const int head = L.head < a.g ? L.head : 0;
    const uint16_t *qp = a.q + ((int64_t)b * a.Hq + (int64_t)hk * a.g + head) * kHeadDim + 32 * L.G + V * L.part;
#pragma unroll
    for (int v = 0; v < QRing<GP>::kLoads; ++v)
        __builtin_amdgcn_global_load_lds(qp + 8 * v, (lds_ptr)(slot + 1024 * v), 16, 0, kCachePolicyNonTemporal);
}

template <int GP>
__device__ inline QRing<GP> read_query(const uint8_t *slot, int lane) {
    QRing<GP> q;
#pragma unroll
    for (int v = 0; v < QRing<GP>::kLoads; ++v) q.w[v] = *reinterpret_cast<const u32x4 *>(slot + 1024 * v + 16 * lane);
    return q;
}

template <int GP, bool KG = false, int BITS = 4>
__device__ inline void build_query(const DecodeArgs &a, const QRing<GP> &qr, const LaneCtx<GP> &L, SegCtx<GP> &c) {
    constexpr int V = GC<GP>::kVPL;
    constexpr int CPL = V / 8;            // chunks of 8 dims per lane (= kNP)
    float x[V];
    if (L.head < a.g) {
#pragma unroll
        for (int v = 0; v < V / 8; ++v) {
            const u32x4 w = qr.w[v];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * v + 2 * e] = bf16f(w[e] & 0xFFFFu);
                x[8 * v + 2 * e + 1] = bf16f(w[e] >> 16);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) x[i] = 0.0f;
    }
#pragma unroll
    for (int len = 1; len < V; len <<= 1) {
        if (len < a.h) {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if ((i & len) == 0) {
                    const float u = x[i], v = x[i + len];
                    x[i] = u + v;
                    x[i + len] = u - v;
                }
            }
        }
    }
    if constexpr (V <= 8) {
        if (8 < a.h) {
#pragma unroll
            for (int i = 0; i < V; ++i) x[i] = butterfly<4>(x[i], L.lane);
        }
    }
    if constexpr (V <= 16) {
        if (16 < a.h) {
#pragma unroll
            for (int i = 0; i < V; ++i) x[i] = butterfly<8>(x[i], L.lane);
        }
    }
    if (32 < a.h) {
#pragma unroll
        for (int i = 0; i < V; ++i) x[i] = butterfly<16>(x[i], L.lane);
    }
    if (64 < a.h) {
#pragma unroll
        for (int i = 0; i < V; ++i) x[i] = butterfly<32>(x[i], L.lane);
    }
    float sum = 0.0f, amax = 0.0f, osum = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        sum += x[i];
        amax = fmaxf(amax, fabsf(x[i]));
    }
    if constexpr (KG) {
        // grouped keys: the levels of a width-b group sit o_b U = (2^(4-b) - 1) U / 2
        // above Z, a per-head constant of the score (dim 32 G + V part + i is in
        // group (V part + i) / 8)
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int jg = (V * L.part + i) >> 3;
            const int b = jg == 0 ? a.key_bits[0] : (jg == 1 ? a.key_bits[1] : (jg == 2 ? a.key_bits[2] : a.key_bits[3]));
            osum = fmaf((float)((1 << (4 - b)) - 1) * 0.5f, x[i], osum);
        }
        osum = head_sum<GP>(osum) * a.inv_sqrt_h;
    }
    sum = head_sum<GP>(sum) * a.inv_sqrt_h;
    amax = max_rows(amax);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    amax = __int_as_float(uni(__float_as_int(amax))) * a.inv_sqrt_h;
    int E = 0;
    (void)frexpf(amax, &E);
    const int e = amax > 0.0f ? 14 - E : 0;      // |q * 2^e| < 2^14
    const float sc = a.inv_sqrt_h * ldexpf(1.0f, e);
    const float s16 = sc * 0.0625f;
    const float c0 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)
    c.K1 = ldexpf(c0, 24 - e);
    c.Rh = ldexpf(sum, e - 24);
    c.Ko = KG ? ldexpf(osum, e - 24) : 0.0f;
    // chunks of 8 dims in the nibble order of a code dword:
    // dims 0,4 | 1,5 (/16) | 2,6 | 3,7 (/16); a 2-bit cache's key codes sit at
    // their field positions (x4^d in operand dword d), so its query pairs are
    // scaled by 1, 1/4, 1/16 and 1/64 instead
    constexpr bool kPos2 = BITS == 2 && !KG;
    const float sd[4] = {sc, kPos2 ? sc * 0.25f : s16, kPos2 ? s16 : sc, kPos2 ? sc * 0.015625f : s16};
    uint32_t H[CPL][4], Lo[CPL][4];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const float *y = x + 8 * k;
#pragma unroll
        for (int d = 0; d < 4; ++d) split2<1>(y[d] * sd[d], y[4 + d] * sd[d], H[k][d], Lo[k][d]);
    }
    if constexpr (GC<GP>::kPacked) {
        uint32_t w[4][4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            w[0][d] = gather_slot<GP, 0>(H[0][d], Lo[0][d]);
            w[1][d] = gather_slot<GP, 1>(H[1 % CPL][d], Lo[1 % CPL][d]);
            w[2][d] = gather_slot<GP, 2>(H[2 % CPL][d], Lo[2 % CPL][d]);
            w[3][d] = gather_slot<GP, 3>(H[3 % CPL][d], Lo[3 % CPL][d]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) c.q4[0][i] = pack8(w[i][0], w[i][1], w[i][2], w[i][3]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c.q4[0][i] = pack8(H[i][0], H[i][1], H[i][2], H[i][3]);
            c.q4[1][i] = pack8(Lo[i][0], Lo[i][1], Lo[i][2], Lo[i][3]);
        }
    }
}

// ---------------------------------------------------------------------------
// Score sums of the step in the MFMA layout -> dense layout.
// s[0..3]: tokens 4G + i of subblock A, s[4..7]: of subblock B, valid in the
// lanes of columns c < GP (hi + lo already added).
template <int GP>
__device__ inline void spread(const float s[8], float d[GC<GP>::kNE]) {
    constexpr int NP = GC<GP>::kNP;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int ee = 0; ee < 2; ++ee) {
            // part 0 lanes keep their own value of pair p
            float v = s[4 * (p >> 1) + (p & 1) + 2 * ee];
            if constexpr (GP == 4) {
                v = dppf<kRowShr + 4, 0x2>(v, s[1 + 2 * ee]);     // part 1: pair 1
                v = dppf<kRowShr + 8, 0x4>(v, s[4 + 2 * ee]);     // part 2: pair 2
                v = dppf<kRowShr + 12, 0x8>(v, s[5 + 2 * ee]);    // part 3: pair 3
            } else if constexpr (GP == 8) {
                v = dppf<kRowShr + 8, 0xC>(v, s[4 + p + 2 * ee]); // part 1: pair 2 + p
            }
            d[2 * p + ee] = v;
        }
    }
}


// Online-softmax update on the dense scores t (-inf where invalid, with the
// value params of invalid tokens zeroed); returns the value MFMA A operand(s):
// rows = query heads (packed: hi rows then lo rows), k = the step's 32 tokens
// in pair order.
template <int GP>
__device__ inline void softmax_dense(SegCtx<GP> &c, const LaneCtx<GP> &L, const float t[GC<GP>::kNE],
                                     const uint32_t vp[GC<GP>::kNE], half8 pop[GC<GP>::kQ]) {
    constexpr int NE = GC<GP>::kNE, NP = GC<GP>::kNP;
    constexpr int HS = GC<GP>::kHiScale;
    float ml = t[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) ml = fmaxf(ml, t[e]);
    // lanes of one head share mK, so a lane-local test finds every head whose
    // max must move; the head-wide max is taken only then
    if (__any(ml * c.K1 > c.mK + GC<GP>::kTau)) {
        const float mt = head_max<GP>(ml) * c.K1;
        const bool grow = mt > c.mK + GC<GP>::kTau;
        const float mnew = grow ? mt : c.mK;
        const float alpha = c.mK == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(c.mK - mnew);
        c.lsum *= alpha;
        c.zsum *= alpha;
        c.mK = mnew;
        // accumulator row 4G + i holds head (4G + i) % GP (unpacked: head 4G + i)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ar;
            if constexpr (GP == 4) {
                ar = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), i));
            } else if constexpr (GP == 8) {
                const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), i));
                const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 4 + i));
                ar = (L.G & 1) ? a1 : a0;
            } else {
                ar = __shfl(alpha, 4 * L.G + i, 64);
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) c.O[tt][i] *= ar;
        }
    }
    const float nm = -c.mK;
    float pv[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(t[e], c.K1, nm));
        c.lsum += p;
        c.zsum = fmaf(p, h_hi(vp[e]), c.zsum);
        pv[e] = p * h_lo(vp[e]);
    }
    uint32_t H[NP], Lw[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) split2<HS>(pv[2 * p], pv[2 * p + 1], H[p], Lw[p]);
    if constexpr (GC<GP>::kPacked) {
        pop[0] = pack8(gather_slot<GP, 0>(H[0], Lw[0]), gather_slot<GP, 1>(H[1 % NP], Lw[1 % NP]),
                       gather_slot<GP, 2>(H[2 % NP], Lw[2 % NP]), gather_slot<GP, 3>(H[3 % NP], Lw[3 % NP]));
    } else {
        pop[0] = pack8(H[0], H[1 % NP], H[2 % NP], H[3 % NP]);
        pop[1] = pack8(Lw[0], Lw[1 % NP], Lw[2 % NP], Lw[3 % NP]);
    }
}

// ---------------------------------------------------------------------------
// Producer: issue the 5 direct-to-LDS loads of the step at cursor c into stage
// st.  Both kinds of step leave key params at stage offset 4096 + 4 t and value
// params at 4224 + 4 t for token (entry) t.
//
// A 2-bit main-cache step copies its two subblocks' 512-byte code areas verbatim
// (32 lanes x 16 B; they are stored in lane order) to stage offsets 0 / 512
// (keys) and 1024 / 1536 (values), and its params like an INT4 step.  A 3-bit
// step copies its low planes the same way and its two 256-byte high planes to
// 2048 (keys) and 2560 (values).
template <int BITS, bool KG = false>
__device__ inline void issue_step(const DecodeArgs &a, const Cursor &c, const Lookup &k, uint8_t *st,
                                  uint32_t offK, uint32_t offV, uint32_t offP4, uint32_t offP8, int lane) {
    if (c.r < c.rp.n4) {
        const uint32_t kSubBytes = KG ? (uint32_t)a.sub_bytes : (uint32_t)main_sub_bytes(BITS);
        const int pos0 = (c.rp.k0 + c.r) * 32;
        // subblock indices fit 32 bits (the descriptor check bounds the pools);
        // a page holds 1 << (logP - 4) subblocks of a KV head
        const uint32_t sh = (uint32_t)a.logP - 4;
        const uint32_t idxA = (((uint32_t)k.pageA * (uint32_t)a.H + (uint32_t)c.hk) << sh) +
                              ((uint32_t)(pos0 & (a.P - 1)) >> 4);
        const uint8_t *baseA = a.int4_pool + (uint64_t)idxA * kSubBytes;
        // subblock B past the INT4 region is never used; re-read A (valid memory).
        // Pages of 32 or more positions hold both 16-position halves of a step.
        const uint8_t *baseB = pos0 + 16 >= c.rp.hi4 ? baseA
            : sh > 0 ? baseA + kSubBytes
            : a.int4_pool + (uint64_t)((uint32_t)k.pageB * (uint32_t)a.H + (uint32_t)c.hk) * kSubBytes;
        if constexpr (KG) {
            // grouped keys: the key areas of A and B verbatim to 0 / 1024 (4 sum(b)
            // lanes of 16 B each, at least 32), the value areas to 2048 (4 bits: A
            // 2048, B 3072; 2 and 3 bits: low planes A 2048, B 2560, high planes
            // A 3072, B 3328), the params as for INT4: five loads
            const uint32_t off = 16 * (uint32_t)lane;
            if ((int)off < a.key_area) {
                dma16_stream(baseA, off, st + 0);
                dma16_stream(baseB, off, st + 1024);
            }
            const uint8_t *va = baseA + a.key_area, *vb = baseB + a.key_area;
            if constexpr (BITS == 4) {
                dma16_stream(va, off, st + 2048);
                dma16_stream(vb, off, st + 3072);
            } else if constexpr (BITS == 2) {
                if (lane < 32) {
                    dma16_stream(va, off, st + 2048);
                    dma16_stream(vb, off, st + 2560);
                }
            } else {
                dma16_stream(lane < 32 ? va : vb, 16 * (uint32_t)(lane & 31), st + 2048);
                if (lane < 32) dma16_stream((lane < 16 ? va : vb) + 512, 16 * (uint32_t)(lane & 15), st + 3072);
            }
            const uint32_t offPg = (uint32_t)(a.key_area + value_area_bytes(BITS)) + ((lane & 8) ? 64u : 0u) +
                                   (uint32_t)(lane & 3) * 16u;
            if (lane < 16) dma16_stream((lane & 4) ? baseB : baseA, offPg, st + 4096);
            return;
        }
        if constexpr (BITS == 2) {
            const uint32_t off = 16 * (uint32_t)lane;
            if (lane < 32) {
                dma16_stream(baseA + kSub2K, off, st + 0);
                dma16_stream(baseB + kSub2K, off, st + 512);
                dma16_stream(baseA + kSub2V, off, st + 1024);
                dma16_stream(baseB + kSub2V, off, st + 1536);
            }
            // params: as for INT4, from the 2-bit subblock's param areas
            const uint32_t offP2 = offP4 - kSub4KP + kSub2KP;
            if (lane < 16) dma16_stream((lane & 4) ? baseB : baseA, offP2, st + 4096);
            return;
        }
        if constexpr (BITS == 3) {
            // low planes as the 2-bit step (lanes 0-31 subblock A, 32-63 B, one
            // load each for keys and values), high planes of A and B to stage
            // offsets 2048 (keys) and 2560 (values), params as for INT4: five loads
            const uint8_t *lo = lane < 32 ? baseA : baseB;
            const uint32_t off = 16 * (uint32_t)(lane & 31);
            dma16_stream(lo + kSub3K, off, st + 0);
            dma16_stream(lo + kSub3V, off, st + 1024);
            if (lane < 32) {
                const uint8_t *hi = lane < 16 ? baseA : baseB;
                const uint32_t offh = 16 * (uint32_t)(lane & 15);
                dma16_stream(hi + kSub3KH, offh, st + 2048);
                dma16_stream(hi + kSub3VH, offh, st + 2560);
            }
            const uint32_t offP3 = offP4 - kSub4KP + kSub3KP;
            if (lane < 16) dma16_stream((lane & 4) ? baseB : baseA, offP3, st + 4096);
            return;
        }
        dma16_stream(baseA + kSub4K, offK, st + 0);
        dma16_stream(baseB + kSub4K, offK, st + 1024);
        dma16_stream(baseA + kSub4V, offV, st + 2048);
        dma16_stream(baseB + kSub4V, offV, st + 3072);
        if (lane < 16) dma16_stream((lane & 4) ? baseB : baseA, offP4, st + 4096);
    } else {
        // the low-nibble planes take the place of subblock A, the high-nibble
        // planes that of subblock B
        const uint32_t sub = (uint32_t)(c.r - c.rp.n4);
        const uint32_t idx = ((uint32_t)k.slot * (uint32_t)a.H + (uint32_t)c.hk) * (uint32_t)a.nr8 + sub;
        const uint8_t *base = a.int8_pool + (uint64_t)idx * kSub8Bytes;
        dma16_stream(base + kSub8KLo, offK, st + 0);
        dma16_stream(base + kSub8KHi, offK, st + 1024);
        dma16_stream(base + kSub8VLo, offV, st + 2048);
        dma16_stream(base + kSub8VHi, offV, st + 3072);
        if (lane < 16 && (lane & 4) == 0) dma16_stream(base, offP8, st + 4096);
    }
}



// Paired 2-bit steps.  Two consecutive INT4-region steps of one segment
// (positions pos0 .. pos0 + 63, subblocks A, B, C, D) share a stage: five
// loads of 64 lanes copy the key codes of A | B and of C | D, the value codes
// of A | B and of C | D, and the params of all four (lanes 0-15 those of A and
// B, as for a single step, lanes 16-31 those of C and D).  Stage layout: the
// single step's at offset 0 (A, B) and again at 2048 (C, D), the params at
// 4096 and 4352.  A pair moves the bytes of one 4-bit step, and its producer
// work, stage wait and cursor advance are those of one step.
constexpr int kPairHalf = 2048;         // stage offset of the second step's codes
constexpr int kPairParams = 256;        // and of its params (relative to the first's)
constexpr int kStagePair = kStageBytes + kPairParams;

// Built where the second step's registers fit beside the first's: query
// groups up to 4, and up to 8 without the fused append (the 8-head fused
// kernel would spill).
template <int GP, bool APPEND, int BITS, bool KG>
constexpr bool kPair = BITS == 2 && !KG && (GP == 4 || (GP == 8 && !APPEND));

template <int GP, bool APPEND, int BITS, bool KG>
constexpr int kStageB = kPair<GP, APPEND, BITS, KG> ? kStagePair : kStageBytes;

// Whether the step at cursor c is paired with the next: both INT4-region steps
// of the segment inside the worker's range [.., u_end), and neither the unit of
// the appended token (the fused append patches that step's stage alone).
// Producer and consumer walk the same cursors, so they pair alike.
template <int GP, int BITS, bool KG, bool APPEND>
__device__ inline bool pairable(const Cursor &c, int64_t u_end) {
    if constexpr (!kPair<GP, APPEND, BITS, KG>) {
        return false;
    } else {
        bool ok = c.r + 1 < c.rp.n4 && c.u + 1 < u_end;
        if constexpr (APPEND) ok = ok && c.r != c.rp.rn && c.r + 1 != c.rp.rn;
        return ok;
    }
}

// Producer of a paired 2-bit step at cursor c (k0, k1: pages of its two units).
__device__ inline void issue_pair2(const DecodeArgs &a, const Cursor &c, const Lookup &k0, const Lookup &k1,
                                   uint8_t *st, uint32_t offP4, int lane) {
    const uint32_t sh = (uint32_t)a.logP - 4;
    const int pos0 = (c.rp.k0 + c.r) * 32;
    auto sub = [&](int page, int pos) {
        const uint32_t idx =
            (((uint32_t)page * (uint32_t)a.H + (uint32_t)c.hk) << sh) + ((uint32_t)(pos & (a.P - 1)) >> 4);
        return a.int4_pool + (uint64_t)idx * kSub2Bytes;
    };
    // B and C lie inside the INT4 region (the second step exists); D past it
    // is never used: re-read C (valid memory)
    const uint8_t *bA = sub(k0.pageA, pos0), *bB = sub(k0.pageB, pos0 + 16);
    const uint8_t *bC = sub(k1.pageA, pos0 + 32);
    const uint8_t *bD = pos0 + 48 < c.rp.hi4 ? sub(k1.pageB, pos0 + 48) : bC;
    const uint32_t o16 = 16u * (uint32_t)(lane & 31);
    const bool upper = lane >= 32;
    dma16_stream(upper ? bB : bA, kSub2K + o16, st + 0);
    dma16_stream(upper ? bD : bC, kSub2K + o16, st + kPairHalf);
    dma16_stream(upper ? bB : bA, kSub2V + o16, st + 1024);
    dma16_stream(upper ? bD : bC, kSub2V + o16, st + kPairHalf + 1024);
    if (lane < 32) {
        const uint8_t *pb = (lane & 16) ? ((lane & 4) ? bD : bC) : ((lane & 4) ? bB : bA);
        dma16_stream(pb, offP4 - kSub4KP + kSub2KP, st + kStKP);
    }
}

// main2: a 2- or 3-bit main-cache step (8 bytes of low-plane codes per lane and
// quarter; at 3 bits the lane's high-plane dword goes to word 2).
__device__ inline uint32_t lds16(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }

// KG: grouped keys.  A main-cache step then holds, per group i, this lane's
// slot of the group's key area in kA[i] / kB[i] (subblocks A / B): the nibble
// dword (width 4), the 16-bit field word (width 2), or the field word with the
// high-bit byte in bits 16-23 (width 3); values as the value width's step, at
// the stage offsets the grouped copy uses.
// pdelta: offset of the step's params from where a single step keeps them
// (the second step of a pair: kPairParams - kPairHalf).
template <int GP, int BITS, bool KG = false>
__device__ inline StepRegs<GP> read_stage(const DecodeArgs &a, const uint8_t *st, const LaneCtx<GP> &L, bool main2,
                                          int pdelta = 0) {
    StepRegs<GP> r;
    const int lane = L.lane;
    if (KG && main2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = a.key_bits[i];
            const uint8_t *g = st + a.kg_off[i];
            if (b == 4) {
                r.kA[i] = lds32(g + 4 * lane);
                r.kB[i] = lds32(g + 1024 + 4 * lane);
            } else {
                r.kA[i] = lds16(g + 2 * lane);
                r.kB[i] = lds16(g + 1024 + 2 * lane);
                if (b == 3) {
                    r.kA[i] |= (uint32_t)g[128 + lane] << 16;
                    r.kB[i] |= (uint32_t)g[1024 + 128 + lane] << 16;
                }
            }
        }
        if constexpr (BITS == 4) {
            r.vA = *reinterpret_cast<const u32x4 *>(st + 2048 + lane * 16);
            r.vB = *reinterpret_cast<const u32x4 *>(st + 3072 + lane * 16);
        } else {
            const u32x2 va = *reinterpret_cast<const u32x2 *>(st + 2048 + lane * 8);
            const u32x2 vb = *reinterpret_cast<const u32x2 *>(st + 2560 + lane * 8);
            const uint32_t vha = BITS == 3 ? lds32(st + 3072 + 4 * lane) : 0u;
            const uint32_t vhb = BITS == 3 ? lds32(st + 3328 + 4 * lane) : 0u;
            r.vA = u32x4{va[0], va[1], vha, 0u};
            r.vB = u32x4{vb[0], vb[1], vhb, 0u};
        }
    } else if ((BITS == 2 || BITS == 3) && main2) {
        const u32x2 ka = *reinterpret_cast<const u32x2 *>(st + lane * 8);
        const u32x2 kb = *reinterpret_cast<const u32x2 *>(st + 512 + lane * 8);
        const u32x2 va = *reinterpret_cast<const u32x2 *>(st + 1024 + lane * 8);
        const u32x2 vb = *reinterpret_cast<const u32x2 *>(st + 1536 + lane * 8);
        const uint32_t kha = BITS == 3 ? lds32(st + 2048 + 4 * lane) : 0u;
        const uint32_t khb = BITS == 3 ? lds32(st + 2304 + 4 * lane) : 0u;
        const uint32_t vha = BITS == 3 ? lds32(st + 2560 + 4 * lane) : 0u;
        const uint32_t vhb = BITS == 3 ? lds32(st + 2816 + 4 * lane) : 0u;
        r.kA = u32x4{ka[0], ka[1], kha, 0u};
        r.kB = u32x4{kb[0], kb[1], khb, 0u};
        r.vA = u32x4{va[0], va[1], vha, 0u};
        r.vB = u32x4{vb[0], vb[1], vhb, 0u};
    } else {
        r.kA = *reinterpret_cast<const u32x4 *>(st + lane * 16);
        r.kB = *reinterpret_cast<const u32x4 *>(st + 1024 + lane * 16);
        r.vA = *reinterpret_cast<const u32x4 *>(st + 2048 + lane * 16);
        r.vB = *reinterpret_cast<const u32x4 *>(st + 3072 + lane * 16);
    }
    const uint8_t *kp = st + pdelta + L.offKP;
    const uint8_t *vp = st + pdelta + L.offKP + (kStVP - kStKP);
    if constexpr (GP == 4) {
        // tokens t0, t0 + 2
        r.kp[0] = lds32(kp);
        r.kp[1] = lds32(kp + 8);
        r.vp[0] = lds32(vp);
        r.vp[1] = lds32(vp + 8);
    } else {
        // GP / 8 runs of 4 tokens (4G .. 4G + 3 of a subblock), pairs (0, 2), (1, 3)
#pragma unroll
        for (int s = 0; s < GP / 8; ++s) {
            const u32x4 wk = *reinterpret_cast<const u32x4 *>(kp + 64 * s);
            const u32x4 wv = *reinterpret_cast<const u32x4 *>(vp + 64 * s);
            r.kp[4 * s + 0] = wk[0]; r.kp[4 * s + 1] = wk[2];
            r.kp[4 * s + 2] = wk[1]; r.kp[4 * s + 3] = wk[3];
            r.vp[4 * s + 0] = wv[0]; r.vp[4 * s + 1] = wv[2];
            r.vp[4 * s + 2] = wv[1]; r.vp[4 * s + 3] = wv[3];
        }
    }
    return r;
}

// Hi + lo query columns of a score MFMA result.
template <int GP>
__device__ inline floatx4 combine_cols(floatx4 d) {
    if constexpr (GP <= 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] += dppf<kRowShl + GP>(0.0f, d[i]);
    }
    return d;
}

// One step: an INT4 step of 32 positions (subblocks A and B) or an INT8 step
// of the 16 ring entries of one subblock, whose low- and high-nibble planes
// stand in for A and B: the key dot products add as lo + 16 hi, and the value
// MFMA weighs the B half of k by 16 p.  Token t of the step is valid iff
// lo <= base + t < hi.
//
// The step is split so that the main loop can overlap consecutive steps of a
// segment: the key MFMAs of step i are issued, then the softmax and value MFMAs
// of step i - 1 run while they complete, then step i's scores are formed
// (kpart_mfma, vpart, kpart_tail).  KOut carries what vpart needs.
template <int GP>
struct KOut {
    float t[GC<GP>::kNE];       // scaled scores (log2 units / K1), -inf where invalid
    uint32_t vp[GC<GP>::kNE];   // value (scale, zero) of those positions, 0 where invalid
    u32x4 vA, vB;               // value codes
    bool int8;
};

// Key MFMAs of a step: raw accumulators of subblocks A and B.
template <int GP>
struct KAcc {
    floatx4 dA[GC<GP>::kQ], dB[GC<GP>::kQ];
};

// Grouped keys: the MFMA operand of one group's slot word x, each code c as the
// f16 subnormal (m c) 2^-24 (m = 2^(4 - b)) in the nibble order of the 4-bit
// operand -- dims (0, 4), (1, 5) x 16, (2, 6), (3, 7) x 16 of the group's 8 --
// so that the query operands serve every width.
__device__ inline half8 group_key_operand(uint32_t x, int b) {
    if (b == 4) {
        const uint32_t x8 = x >> 8;
        return pack8(x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u);
    }
    // bytes 0 and 1 (dims 0-3, 4-7 at bits 2f) to the two 16-bit halves
    const uint32_t y = (x & 0xFFu) | ((x & 0xFF00u) << 8);
    if (b == 2)
        return pack8((y << 2) & 0x000C000Cu, (y << 4) & 0x00C000C0u, (y >> 2) & 0x000C000Cu, y & 0x00C000C0u);
    // width 3: 2 c = 2 lo + 8 hi; the high bits of dims 0-3 / 4-7 to bits 0-3 / 16-19
    const uint32_t h = x >> 16;
    const uint32_t H = (h & 0x0Fu) | ((h & 0xF0u) << 12);
    return pack8(((y << 1) & 0x00060006u) | ((H << 3) & 0x00080008u),
                 ((y << 3) & 0x00600060u) | ((H << 6) & 0x00800080u),
                 ((y >> 3) & 0x00060006u) | ((H << 1) & 0x00080008u),
                 ((y >> 1) & 0x00600060u) | ((H << 4) & 0x00800080u));
}

template <int GP, int BITS, bool KG = false>
__device__ inline KAcc<GP> kpart_mfma(const DecodeArgs &a, const SegCtx<GP> &c, const StepRegs<GP> &r, bool main2) {
    constexpr int kQ = GC<GP>::kQ;
    // Operands of chunks 0-3 of subblocks A and B (an INT8 step: of its low- and
    // high-nibble planes), built by whichever kind of step this is; the MFMAs
    // below are shared, so the accumulators keep one register assignment.
    half8 ak[4], bk[4];
    if (KG && main2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = a.key_bits[i];
            ak[i] = group_key_operand(r.kA[i], b);
            bk[i] = group_key_operand(r.kB[i], b);
        }
    } else if ((BITS == 2 || BITS == 3) && main2) {
        // chunk i: dword i / 2 of the lane's 8 bytes, bytes (0, 2) or (1, 3)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t xa = r.kA[i >> 1] >> (8 * (i & 1)), xb = r.kB[i >> 1] >> (8 * (i & 1));
            ak[i] = BITS == 3 ? int3_key_chunk(xa, r.kA[2], i) : int2_chunk_pos(xa);
            bk[i] = BITS == 3 ? int3_key_chunk(xb, r.kB[2], i) : int2_chunk_pos(xb);
        }
    } else if (BITS == 2 && !KG) {
        // INT8 steps of a 2-bit cache: the nibbles at the 2-bit query scaling
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ak[i] = nibble_chunk_pos(r.kA[i]);
            bk[i] = nibble_chunk_pos(r.kB[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t x = r.kA[i], x8 = x >> 8;
            ak[i] = pack8(x & 0x000F000Fu, x & 0x00F000F0u, x8 & 0x000F000Fu, x8 & 0x00F000F0u);
            const uint32_t y = r.kB[i], y8 = y >> 8;
            bk[i] = pack8(y & 0x000F000Fu, y & 0x00F000F0u, y8 & 0x000F000Fu, y8 & 0x00F000F0u);
        }
    }
    const floatx4 zero4 = {0.f, 0.f, 0.f, 0.f};
    KAcc<GP> k;
#pragma unroll
    for (int q = 0; q < kQ; ++q) k.dA[q] = k.dB[q] = zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            k.dA[q] = mfma16(ak[i], c.q4[q][i], k.dA[q]);
            k.dB[q] = mfma16(bk[i], c.q4[q][i], k.dB[q]);
        }
    }
    return k;
}

// Scores of a step from its key accumulators: hi + lo columns, the dense
// layout, scale/offset, validity.
template <int GP, bool KG = false>
__device__ inline KOut<GP> kpart_tail(const SegCtx<GP> &c, const LaneCtx<GP> &L, const StepRegs<GP> &r,
                                      const KAcc<GP> &ka, bool int8, int base, int lo, int hi) {
    constexpr int kQ = GC<GP>::kQ, NE = GC<GP>::kNE;
    floatx4 sA = ka.dA[0], sB = ka.dB[0];
    if constexpr (kQ == 2) {
        sA += ka.dA[1];
        sB += ka.dB[1];
    }
    const float f8 = int8 ? 16.0f : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sA[i] = fmaf(sB[i], f8, sA[i]);
    sA = combine_cols<GP>(sA);
    sB = combine_cols<GP>(sB);
    const float s8[8] = {sA[0], sA[1], sA[2], sA[3], sB[0], sB[1], sB[2], sB[3]};
    float d[NE];
    spread<GP>(s8, d);
    KOut<GP> k;
    const uint32_t off = (uint32_t)(base - lo), span = (uint32_t)(hi - lo);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        // params of positions past the written context are arbitrary bytes
        // (possibly NaN as fp16): computed anyway, then dropped by a select
        // (never multiplied by zero)
        const bool ok = (uint32_t)L.tok4[e] + off < span;
        // grouped keys: the levels' offsets o_b U, a per-head constant (main-cache steps only)
        const float ts = tscore(KG && !int8 ? d[e] + c.Ko : d[e], r.kp[e], c.Rh);
        k.t[e] = ok ? ts : kNegInf;
        k.vp[e] = ok ? r.vp[e] : 0u;
    }
    k.vA = r.vA;
    k.vB = r.vB;
    k.int8 = int8;
    return k;
}

template <int GP, int BITS>
__device__ inline void vpart(SegCtx<GP> &c, const LaneCtx<GP> &L, const KOut<GP> &k) {
    constexpr int kQ = GC<GP>::kQ;
    half8 pop[kQ];
    softmax_dense<GP>(c, L, k.t, k.vp, pop);
    // INT8: k slots 2, 3 (the high-nibble plane) weigh 16 p of slots 0, 1; the
    // INT4 slots 2, 3 (subblock B) are kept by weight 1 and weight 0 on the
    // copy of slots 0, 1
    {
        const _Float16 wb = k.int8 ? (_Float16)0.0f : (_Float16)1.0f;
        const _Float16 wa = k.int8 ? (_Float16)16.0f : (_Float16)0.0f;
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
#pragma unroll
            for (int j = 0; j < 4; ++j) pop[q][4 + j] = pop[q][4 + j] * wb + pop[q][j] * wa;
        }
    }
    // B operand of accumulator tile t, built by whichever kind of step this is;
    // the MFMAs below are shared, so the accumulators keep one register
    // assignment across the branch.
    half8 vt[8];
    if ((BITS == 2 || BITS == 3) && !k.int8) {
        // 2-bit values: dword cc, field f = dims 16 (4 cc + f) + n, tile 4 cc + f,
        // the codes left at their field positions (x4^f); 3-bit: normalised
        // fields with the high bits of the lane's value-plane dword word 2
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const uint32_t x = k.vA[cc], x8 = x >> 8, y = k.vB[cc], y8 = y >> 8;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const uint32_t m = 0x00030003u << (2 * f);
                vt[4 * cc + f] = BITS == 3
                    ? pack8(int3_value_field(x, k.vA[2], cc, f, false), int3_value_field(x8, k.vA[2], cc, f, true),
                            int3_value_field(y, k.vB[2], cc, f, false), int3_value_field(y8, k.vB[2], cc, f, true))
                    : pack8(x & m, x8 & m, y & m, y8 & m);
            }
        }
    } else if (BITS == 2) {
        // INT8 steps of a 2-bit cache: each nibble moved to its tile's scaling
        // 4^(t % 4) (tiles 2 cc and 2 cc + 1)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const uint32_t x = k.vA[cc], x8 = x >> 8, y = k.vB[cc], y8 = y >> 8;
            if (cc & 1) {
                vt[2 * cc] = pack8((x << 4) & 0x00F000F0u, (x8 << 4) & 0x00F000F0u, (y << 4) & 0x00F000F0u,
                                   (y8 << 4) & 0x00F000F0u);
                vt[2 * cc + 1] = pack8((x << 2) & 0x03C003C0u, (x8 << 2) & 0x03C003C0u, (y << 2) & 0x03C003C0u,
                                       (y8 << 2) & 0x03C003C0u);
            } else {
                vt[2 * cc] = pack8(x & 0x000F000Fu, x8 & 0x000F000Fu, y & 0x000F000Fu, y8 & 0x000F000Fu);
                vt[2 * cc + 1] = pack8((x >> 2) & 0x003C003Cu, (x8 >> 2) & 0x003C003Cu, (y >> 2) & 0x003C003Cu,
                                       (y8 >> 2) & 0x003C003Cu);
            }
        }
    } else {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const uint32_t x = k.vA[cc], x8 = x >> 8, y = k.vB[cc], y8 = y >> 8;
            vt[2 * cc] = pack8(x & 0x000F000Fu, x8 & 0x000F000Fu, y & 0x000F000Fu, y8 & 0x000F000Fu);
            vt[2 * cc + 1] = pack8(x & 0x00F000F0u, x8 & 0x00F000F0u, y & 0x00F000F0u, y8 & 0x00F000F0u);
        }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) c.O[t] = mfma16(pop[q], vt[t], c.O[t]);
    }
}

// ---------------------------------------------------------------------------
// End of a segment.  Per-head l, z totals, and the accumulator rows of each
// head brought together: R[t][k] is dims 16 t + n of head seg_head(k).
template <int GP>
struct SegOut {
    static constexpr int kK = GC<GP>::kPacked ? 2 : 4;
    float R[8][kK];
    int head[kK];       // query head of R[.][k] in this lane, or -1
};

template <int GP>
__device__ inline SegOut<GP> reduce_segment(SegCtx<GP> &c, const LaneCtx<GP> &L, int g) {
    constexpr float HS = (float)GC<GP>::kHiScale;
    c.lsum = head_sum<GP>(c.lsum);
    c.zsum = head_sum<GP>(c.zsum);
    SegOut<GP> s;
    if constexpr (GP == 4) {
        // rows 0-3 (G = 0) hi, 4-7 (G = 1) lo of heads 0-3: row 0 gets heads
        // k, row 1 heads k + 2
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                float r0, r1;
                swap16(c.O[t][k], c.O[t][k + 2], r0, r1);
                s.R[t][k] = fmaf(r0, HS, r1);
            }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int hd = k + 2 * L.G;
            s.head[k] = (L.G < 2 && hd < g) ? hd : -1;
        }
    } else if constexpr (GP == 8) {
        // rows 0-7 (G = 0, 1) hi, 8-15 (G = 2, 3) lo of heads 0-7
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                float r0, r1;
                swap32(c.O[t][k], c.O[t][k + 2], r0, r1);
                s.R[t][k] = fmaf(r0, HS, r1);
            }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int hd = k + 4 * (L.G & 1) + 2 * (L.G >> 1);
            s.head[k] = hd < g ? hd : -1;
        }
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int k = 0; k < 4; ++k) s.R[t][k] = c.O[t][k];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int hd = 4 * L.G + k;
            s.head[k] = hd < g ? hd : -1;
        }
    }
    return s;
}

// Factor from accumulator tile t to the value codes' units times 2^24 (the
// codes enter the MFMAs as f16 subnormals c 2^-24): odd tiles hold 16 c, and a
// 2-bit cache's tiles 4^(t % 4) c.
template <int BITS>
__device__ inline float tile_scale(int t) {
    if constexpr (BITS == 2) return ldexpf(1.0f, 24 - 2 * (t & 3));
    return (t & 1) ? 1048576.0f : 16777216.0f;      // 2^20 / 2^24
}

// Output of a segment that one worker attended completely: straight from registers.
template <int GP, int BITS>
__device__ inline void finalize_regs(const DecodeArgs &a, const SegCtx<GP> &c, const LaneCtx<GP> &L,
                                     const SegOut<GP> &s, int b, int hk) {
    float *ob = a.out + ((int64_t)b * a.Hq + (int64_t)hk * a.g) * kHeadDim;
    const float rl = 1.0f / c.lsum;
#pragma unroll
    for (int k = 0; k < SegOut<GP>::kK; ++k) {
        const int hd = s.head[k];
        const float zr = __shfl(c.zsum, hd < 0 ? 0 : hd, 64);
        const float ir = __shfl(rl, hd < 0 ? 0 : hd, 64);
        if (hd >= 0) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                ob[hd * kHeadDim + 16 * t + L.n] = fmaf(s.R[t][k], tile_scale<BITS>(t), zr) * ir;
            }
        }
    }
    if (a.lse && L.lane < a.g && L.lane < GP)
        a.lse[(int64_t)b * a.Hq + (int64_t)hk * a.g + L.lane] = (c.mK + __log2f(c.lsum)) / kLog2e;
}

// Partial statistics of a segment: per query head m, l and the unnormalised acc[128].
template <int GP, int BITS>
__device__ inline void write_piece(const DecodeArgs &a, const SegCtx<GP> &c, const LaneCtx<GP> &L,
                                   const SegOut<GP> &s, float *pp) {
    if (L.lane < a.g && L.lane < GP) {
        pp[L.lane * kPieceStride + 0] = c.mK;
        pp[L.lane * kPieceStride + 1] = c.lsum;
    }
#pragma unroll
    for (int k = 0; k < SegOut<GP>::kK; ++k) {
        const int hd = s.head[k];
        const float zr = __shfl(c.zsum, hd < 0 ? 0 : hd, 64);
        if (hd >= 0) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                pp[hd * kPieceStride + 4 + 16 * t + L.n] = fmaf(s.R[t][k], tile_scale<BITS>(t), zr);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Fused append.  Each row appends one token at position L - 1 before it is
// attended (KV4-RL, "Methodology in Plain English": the new K/V is quantized on
// the fly as it enters the cache).  The worker whose range holds the unit that
// attends position L - 1 (RowPlan::rn) quantizes the token, stores it into the
// INT4 cache and, for a sink or recent position, the INT8 side cache, exactly
// as the quantize-append kernel does, and patches the copy of the step already
// in its LDS stage.  No other worker reads those bytes in this launch: the
// unit is the only one covering that INT8 subblock (or, without a recent
// window, that INT4 subblock); an INT4 step whose range ends before L - 1 may
// copy the subblock holding it, but masks that position.
//
// The token's bf16 key and value (lanes 0-15 and 16-31, 16 bytes each) and the
// block-table entry of its page come into an LDS slot with the step's own
// copies, so the stage wait covers them.
constexpr int kKvBytes = 528;           // 256 B key, 256 B value, page entry, pad
constexpr int kKvPage = 512;

__device__ inline void issue_new_token(const DecodeArgs &a, const RowRegs &R, const Cursor &c, uint8_t *slot,
                                       int lane) {
    const int64_t row = (int64_t)c.b * a.H + c.hk;
    const uint16_t *src = (lane < 16 ? a.k_new : a.v_new) + row * kHeadDim + 8 * (lane & 15);
    if (lane < 32) __builtin_amdgcn_global_load_lds(src, (lds_ptr)slot, 16, 0, kCachePolicyNonTemporal);
    const int p = row_len(a, R, c.b) - 1;
    const int32_t *pe = a.block_table + (int64_t)row_slot(a, R, c.b) * a.bt_stride + (p >> a.logP);
    if (lane == 0) __builtin_amdgcn_global_load_lds(pe, (lds_ptr)(slot + kKvPage), 4, 0, kCachePolicyNonTemporal);
}

template <int BITS>
__device__ inline void append_new_token(const DecodeArgs &a, const RowRegs &R, const Cursor &c,
                                        const uint8_t *kv, uint8_t *st, int lane) {
    const int vd0 = 32 * (lane >> 4) + (lane & 15);
    const uint32_t kw = lds32(kv + 4 * lane);
    const uint32_t vlo = *reinterpret_cast<const uint16_t *>(kv + 256 + 2 * vd0);
    const uint32_t vhi = *reinterpret_cast<const uint16_t *>(kv + 256 + 2 * (vd0 + 16));
    const int page = uni((int)lds32(kv + kKvPage));
    const TokenCodes tc = quantize_token(kw, vlo, vhi, a.h, a.inv_sqrt_h, lane, (float)((1 << BITS) - 1));
    const int p = row_len(a, R, c.b) - 1;
    uint8_t *base4 = a.int4_pool +
        ((size_t)((int64_t)page * a.H + c.hk) * (a.P >> 4) + ((p & (a.P - 1)) >> 4)) * main_sub_bytes(BITS);
    const bool int8 = c.rp.rn >= c.rp.n4;
    const int e = ((c.rp.rn - c.rp.n4) << 4) + c.rp.tn;
    uint8_t *base8 = int8
        ? a.int8_pool + ((size_t)((int64_t)row_slot(a, R, c.b) * a.H + c.hk) * a.nr8 + (e >> 4)) * kSub8Bytes
        : nullptr;
    Sub2Token s2 = {0u, 0u, 0u, 0u};
    if constexpr (BITS == 4) {
        store_token(tc, base4, p & 15, base8, e & 15, int8, lane);
    } else {
        s2 = sub2_token<BITS>(tc, lane);
        put_sub2_token<BITS>(s2, tc, base4 + kSub2K, base4 + (BITS == 3 ? kSub3V : kSub2V), base4 + kSub3KH,
                             base4 + kSub3VH, base4 + (BITS == 3 ? kSub3KP : kSub2KP),
                             base4 + (BITS == 3 ? kSub3VP : kSub2VP), p & 15, lane);
        if (int8) store_token_int8(tc, base8, e & 15, lane);
    }
    // the stage holds the step as the cache was before this token.  Key bytes
    // sit by lane (stage byte 256 (l / 16) + 16 t + l % 16 is subblock byte
    // 64 t + l), value bytes as in the subblock, params at kStKP / kStVP + 4 t.
    const int t = c.rp.tn;
    if (int8) {
        const int kq = 256 * (lane >> 4) + 16 * t + (lane & 15);
        const int vq = 2048 + sub_v_byte(t, lane);
        st[kq] = tc.k8lo;
        st[kq + 1024] = tc.k8hi;
        st[vq] = tc.v8lo;
        st[vq + 1024] = tc.v8hi;
        if (lane == 0) {
            *reinterpret_cast<uint32_t *>(st + kStKP + 4 * t) = tc.kp8;
            *reinterpret_cast<uint32_t *>(st + kStVP + 4 * t) = tc.vp8;
        }
    } else if constexpr (BITS != 4) {
        // a 2- / 3-bit step holds each area of subblocks A and B verbatim:
        // low planes at 512 sb (keys) and 1024 + 512 sb (values), high planes
        // at 2048 + 256 sb and 2560 + 256 sb, params as above
        const int sb = t >> 4;
        put_sub2_token<BITS>(s2, tc, st + 512 * sb, st + 1024 + 512 * sb, st + 2048 + 256 * sb, st + 2560 + 256 * sb,
                             st + kStKP + 64 * sb, st + kStVP + 64 * sb, t & 15, lane);
    } else {
        const int sb = t >> 4, tt = t & 15;
        st[1024 * sb + 256 * (lane >> 4) + 16 * tt + (lane & 15)] = tc.k4;
        st[2048 + 1024 * sb + sub_v_byte(tt, lane)] = tc.v4;
        if (lane == 0) {
            *reinterpret_cast<uint32_t *>(st + kStKP + 4 * t) = tc.kp4;
            *reinterpret_cast<uint32_t *>(st + kStVP + 4 * t) = tc.vp4;
        }
    }
}

// LDS of one wave: the stage ring, the page half-batches and the query ring
// (one slot per stage).  The request is padded to 1/kWavesPerCU of a CU's
// 160 KB: random 2 KB reads from more waves per CU lose HBM efficiency
// (measured on MI355X: 8 waves per CU stream random 2176-byte subblocks ~25%
// faster than 12).
constexpr int kWavesPerCU = 8;

template <int GP, bool APPEND, int SB = kStageBytes>
struct SmemLayout {
    static constexpr int kPages = kStages * SB;
    static constexpr int kQ = kPages + kPgBytes;
    static constexpr int kKv = kQ + kStages * QRing<GP>::kBytes;
    static constexpr int kNeed = kKv + (APPEND ? kStages * kKvBytes : 0);
    static constexpr int kPad = 160 * 1024 / kWavesPerCU;
    static constexpr int kRequest = kNeed > kPad ? kNeed : kPad;
};

// Inclusive prefix sum over the 64 lanes.
__device__ inline int64_t wave_scan(int64_t x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t t = __shfl_up(x, o, 64);
        if (lane >= o) x += t;
    }
    return x;
}

// Inclusive prefix sum over the 64 lanes in 32 bits with DPP moves: shifts by
// 1, 2, 4, 8 inside each 16-lane row, then the total of row 0 (2) is added to
// row 1 (3) and that of rows 0-1 to rows 2-3.
__device__ inline uint32_t wave_scan32(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 1, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 2, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 4, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr + 8, 0xF, 0xF, true);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return x;
}

__device__ inline int64_t readlane64(int64_t x, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)x, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)x >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// MEM = true builds the kernel's memory skeleton: the same prologue, work
// split, page gathers, DMA ring, waits and stage reads, without the arithmetic
// and without outputs -- the bandwidth this access pattern reaches on the
// device, as a measured ceiling for the full kernel.
// KG = true: the main cache holds keys with a width per RoPE-block group
// (a.key_bits) and values of width BITS.
//
// Two waves per SIMD (at most 256 registers each), except the 16-head group
// kernels with the fused append or a 2- / 3-bit cache: those need more than
// 256, and at one wave per SIMD the compiler keeps the rest in the
// accumulation registers instead of spilling to scratch memory.
template <int GP, bool APPEND, int BITS>
constexpr int kSplitMinWaves = (GP == 16 && (APPEND || BITS != 4)) ? 1 : 2;

// Workers per workgroup of one instantiation: kSplitWaves when a wave's LDS fits
// its 1/8 share of the CU (two workgroups per CU), else 1 (the 8-head fused and
// 16-head kernels need 21-27 KB per wave: a workgroup of four would leave room
// for one per CU, i.e. one wave per SIMD).
template <int GP, bool APPEND, int BITS, bool KG = false>
using SplitSmem = SmemLayout<GP, APPEND, kStageB<GP, APPEND, BITS, KG>>;

template <int GP, bool APPEND, int BITS = 4, bool KG = false>
constexpr int kSplitWG =
    SplitSmem<GP, APPEND, BITS, KG>::kNeed <= SplitSmem<GP, APPEND, BITS, KG>::kPad ? kSplitWaves : 1;

template <int GP, bool APPEND, int BITS, bool MEM = false, bool KG = false>
__global__ __launch_bounds__((64 * kSplitWG<GP, APPEND, BITS, KG>))
__attribute__((amdgpu_waves_per_eu(kSplitMinWaves<GP, APPEND, BITS>, 2)))
void decode_split_kernel(DecodeArgs a) {
    using SL = SplitSmem<GP, APPEND, BITS, KG>;
    constexpr int NW = kSplitWG<GP, APPEND, BITS, KG>;
    constexpr int SB = kStageB<GP, APPEND, BITS, KG>;       // bytes of a stage slot
    constexpr bool PAIR = kPair<GP, APPEND, BITS, KG>;
    // NW independent workers per workgroup (no barriers), each with its own
    // slice of the workgroup's LDS
    __shared__ __attribute__((aligned(16))) uint8_t smem_wg[NW * SL::kRequest];
    const int lane = threadIdx.x & 63;
    const int wave = NW > 1 ? uni((int)(threadIdx.x >> 6)) : 0;
    const int64_t wid = (int64_t)blockIdx.x * NW + wave;
    uint8_t *const smem = smem_wg + wave * SL::kRequest;

    // Exclusive prefix of the row costs (units of all KV heads of a row).  The
    // rows of the register table take one load round trip and four
    // independent lane scans; rows beyond it are summed from memory.
    const RowRegs R = load_rows(a, lane);
    // The kernel arguments of the prologue, in one scalar round trip under the
    // row table's loads (left to itself the compiler loads them where first
    // used, each load waited on the prologue's critical path).
    __asm__ volatile("" ::"s"(a.ws_header), "s"(a.ws_wseg), "s"(a.block_table), "s"(a.bt_stride), "s"(a.H),
                     "s"(a.P), "s"(a.logP), "s"(a.s), "s"(a.w), "s"(a.nr8), "s"(a.max_workers), "s"(a.min_units),
                     "s"(a.simds), "s"(a.part_wt[0]), "s"(a.part_wt[1]), "s"(a.part_wt[2]), "s"(a.part_wt[3]), "s"(a.seg_wt),
                     "s"(a.int4_pool), "s"(a.int8_pool), "s"(a.q), "s"(a.Hq), "s"(a.g), "s"(a.ws_piece),
                     "s"(a.out), "s"(a.lse));
    int64_t cost[4], excl[4];
    int64_t res_total = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        cost[k] = lane + 64 * k < a.B ? (int64_t)seg_units(a, row_plan(R.L[k], a.s, a.w)) * a.H : 0;
    // 32-bit DPP scans when 256 row costs cannot reach 2^31 (every realistic
    // batch), 64-bit shuffle scans otherwise
    const bool small = !__any(cost[0] >= (1 << 22) || cost[1] >= (1 << 22) || cost[2] >= (1 << 22) ||
                              cost[3] >= (1 << 22));
    if (small) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t inc = wave_scan32((uint32_t)cost[k]);
            excl[k] = res_total + (int64_t)(inc - (uint32_t)cost[k]);
            res_total += (int64_t)(uint32_t)__builtin_amdgcn_readlane(inc, 63);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t inc = wave_scan(cost[k], lane);
            excl[k] = res_total + inc - cost[k];
            res_total += readlane64(inc, 63);
        }
    }
    int64_t total = res_total;
    if (a.B > kResRows) {
        int64_t rest = 0;
        for (int b = kResRows + lane; b < a.B; b += 64)
            rest += (int64_t)seg_units(a, row_plan(a.ctx_len[b], a.s, a.w)) * a.H;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) rest += __shfl_xor(rest, o, 64);
        total += uni64(rest);
    }
    const Partition part = make_partition(total, a.max_workers, a.part_wt, a.min_units, NW, a.simds);
    const int64_t W = part.W;
    const int64_t u_begin = wid < W ? part_begin(part, wid) : 0;
    const int64_t u_end = wid < W ? part_begin(part, wid + 1) : 0;
    const bool active = wid < W && u_begin < u_end;
    if (lane == 0) {
        if (wid == 0) a.ws_header[0] = (int32_t)W;
        if (wid < W && !active) {                   // a worker without units leaves no pieces
            a.ws_wseg[2 * wid] = -1;
            a.ws_wseg[2 * wid + 1] = -1;
        }
    }
    if (!active) return;

    // The row holding this wave's first unit.
    int b0 = -1;
    int64_t pre0 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint64_t mk = __ballot(active && cost[k] > 0 && excl[k] <= u_begin && u_begin < excl[k] + cost[k]);
        if (mk) {
            const int src = uni(__ffsll((unsigned long long)mk) - 1);
            b0 = 64 * k + src;
            pre0 = readlane64(excl[k], src);
        }
    }
    if (a.B > kResRows && b0 < 0) {
        int64_t base = res_total;
        for (int cb = kResRows; cb < a.B; cb += 64) {
            const int b = cb + lane;
            const int64_t c = b < a.B ? (int64_t)seg_units(a, row_plan(a.ctx_len[b], a.s, a.w)) * a.H : 0;
            const int64_t incl = wave_scan(c, lane);
            const int64_t ex = base + incl - c;
            const uint64_t mk = __ballot(b < a.B && c > 0 && ex <= u_begin && u_begin < ex + c);
            if (mk) {
                const int src = uni(__ffsll((unsigned long long)mk) - 1);
                b0 = uni(cb + src);
                pre0 = readlane64(ex, src);
                break;
            }
            base = uni64(base + readlane64(incl, 63));
        }
    }
    b0 = uni(b0);
    pre0 = uni64(pre0);

    Cursor start;
    start.b = b0;
    start.rp = row_plan(row_len(a, R, b0), a.s, a.w);
    {
        const int vc = seg_units(a, start.rp);
        start.hk = (int)div_nonneg(u_begin - pre0, vc);
        const int v = (int)(u_begin - pre0 - (int64_t)start.hk * vc);
        // a range that opens on weight units starts at the segment's first step
        start.r = v < a.seg_wt ? 0 : v - a.seg_wt;
        start.u = u_begin + (v < a.seg_wt ? a.seg_wt - v : 0);
    }
    if (start.u >= u_end) {                     // weight units only: no steps, no pieces
        if (lane == 0) {
            a.ws_wseg[2 * wid] = -1;
            a.ws_wseg[2 * wid + 1] = -1;
        }
        return;
    }

    const LaneCtx<GP> L = lane_ctx<GP>(lane);
    SegCtx<GP> c;
    c.lsum = 0.0f;
    c.zsum = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) c.O[t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // per-lane source offsets of the direct-to-LDS loads (see issue_step)
    const uint32_t offK = L.n * 64 + L.G * 16;
    const uint32_t offV = lane * 16;
    const uint32_t offP4 = ((lane & 8) ? kSub4VP : kSub4KP) + (lane & 3) * 16;
    const uint32_t offP8 = ((lane & 8) ? kSub8VP : kSub8KP) + (lane & 3) * 16;

    Cursor P = start, C = start;
    int issued = 0;
    // page half-batches in LDS: the half of unit hb + j is (hb / 32) & 1
    uint32_t *pg = reinterpret_cast<uint32_t *>(smem + SL::kPages);
    uint8_t *qring = smem + SL::kQ;
    uint8_t *kvring = smem + SL::kKv;        // fused append: one slot per stage
    BatchCursor bc = {b0, pre0};
    int64_t hb = u_begin;                     // first unit of the producer's current half
    int hcur = 0;                             // its half index
    fetch_pages(a, R, hb, u_end, bc, lane, pg);
    if (hb + kPgHalf < u_end) fetch_pages(a, R, hb + kPgHalf, u_end, bc, lane, pg + 2 * kPgHalf);
    // Both halves landed (nothing else is in flight yet).  A gather whose lanes
    // all hold INT8, weight or past-the-range units issues no load at all, so
    // a partial count here could leave the first half in flight.
    __builtin_amdgcn_s_waitcnt(0);
    KVQ_FENCE();
    // pages of the producer's next step (LDS reads; waited with the stage reads)
    auto read_pages = [&](const Cursor &c, int d) {
        int j = (int)(c.u + d - hb);
        int h = hcur;
        if (j >= kPgHalf) {
            j -= kPgHalf;
            h ^= 1;
        }
        Lookup k;
        k.pageA = (int)pg[(2 * h) * kPgHalf + j];
        k.pageB = (int)pg[(2 * h + 1) * kPgHalf + j];
        return k;
    };
    // after the producer leaves the current half, refill it with the units 64 ahead
    auto advance_half = [&](const Cursor &c) {
        if (c.u - hb >= kPgHalf) {
            hb += kPgHalf;
            if (hb + kPgHalf < u_end) fetch_pages(a, R, hb + kPgHalf, u_end, bc, lane, pg + 2 * hcur * kPgHalf);
            hcur ^= 1;
        }
    };
    auto uniform = [](const Lookup &k) {
        Lookup u;
        u.pageA = uni(k.pageA);
        u.pageB = uni(k.pageB);
        u.slot = u.pageA;
        return u;
    };
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
        if (P.u < u_end) {
            const bool pp = pairable<GP, BITS, KG, APPEND>(P, u_end);
            const Lookup look = uniform(read_pages(P, 0));
            if (P.r == 0 || P.u == start.u) issue_query<GP>(a, P.b, P.hk, L, qring + s * QRing<GP>::kBytes);
            if constexpr (APPEND) {
                if (P.r == P.rp.rn) issue_new_token(a, R, P, kvring + s * kKvBytes, lane);
            }
            if (PAIR && pp) {
                issue_pair2(a, P, look, uniform(read_pages(P, 1)), smem + s * SB, offP4, lane);
                ++P.u;          // the pair's second step (same segment)
                ++P.r;
            } else {
                issue_step<BITS, KG>(a, P, look, smem + s * SB, offK, offV, offP4, offP8, lane);
            }
            cursor_next(a, R, P);
            ++issued;
            advance_half(P);
        }
    }
    int32_t wseg0 = -1, wseg1 = -1;     // segments of this wave's first / last piece
    // End of the segment of the step at cursor E, once its value part is done.
    auto end_segment = [&](const Cursor &E) {
        const SegOut<GP> so = reduce_segment<GP>(c, L, a.g);
        // this wave covers [u_begin, u_end) in order: it did the segment's
        // first unit iff that lies in its range, its last iff r is the last
        // index; with both it holds the whole segment.  The combine kernel
        // finds a split segment's workers from the two records.
        const bool first = E.u - E.r >= u_begin, last = E.r == E.rp.cost - 1;
        const int64_t seg = (int64_t)E.b * a.H + E.hk;
        if (lane == 0) {
            if (first) a.ws_first[seg] = (int32_t)wid;
            if (last) a.ws_last[seg] = (int32_t)wid;
        }
        if (!first) wseg0 = (int32_t)seg;            // only the wave's first segment can start earlier
        if (!last) wseg1 = (int32_t)seg;             // only its last one can go on after it
        if (first && last)
            finalize_regs<GP, BITS>(a, c, L, so, E.b, E.hk);
        else
            write_piece<GP, BITS>(a, c, L, so, a.ws_piece + (wid + seg) * (int64_t)a.g * kPieceStride);
    };
    bool open = false;          // the next step continues the current segment
    bool pend = false;          // a step of the current segment awaits its value part
    KOut<GP> kp;                // that step's scores and value codes
    Cursor E = C;               // its cursor
    // Each iteration reads the next step's stage (and query, and the pages of
    // the producer's step after next) from LDS first, then issues the
    // producer's step into the slot the current step freed, and only then
    // waits for the reads: their latency runs under the producer's work.
    // (A query copy issued with a later step only makes the stage waits
    // stricter.)
    Lookup look = {0, 0, 0};    // pages of the producer's step P
    Lookup look1 = {0, 0, 0};   // and of its second step when it is a pair
    bool ppair = false;         // the producer's step P is a pair
    if (P.u < u_end) {
        ppair = pairable<GP, BITS, KG, APPEND>(P, u_end);
        look = read_pages(P, 0);
        if (PAIR && ppair) look1 = read_pages(P, 1);
    }
    wait_vm_steps(issued - 1);
    if constexpr (APPEND) {
        if (C.r == C.rp.rn) append_new_token<BITS>(a, R, C, kvring, smem, lane);
    }
    bool cpair = pairable<GP, BITS, KG, APPEND>(C, u_end);      // the step at C is a pair
    StepRegs<GP> r = read_stage<GP, BITS, KG>(a, smem, L, C.r < C.rp.n4);
    StepRegs<GP> r1 = r;        // its second step
    if (PAIR && cpair) r1 = read_stage<GP, BITS, KG>(a, smem + kPairHalf, L, true, kPairParams - kPairHalf);
    QRing<GP> qr = read_query<GP>(qring, lane);     // the first step opens a segment
    wait_lgkm0();
    look = uniform(look);
    look1 = uniform(look1);
    uint32_t sink = 0;          // MEM: what the stage reads returned, kept live
    for (int i = 0; C.u < u_end; ++i) {
        const int scur = i % kStages, snxt = (i + 1) % kStages;
        const bool int4 = C.r < C.rp.n4;
        if constexpr (MEM) {
            sink ^= r.kA[0] ^ r.kB[1] ^ r.vA[2] ^ r.vB[3] ^ r.kp[0] ^ r.vp[0] ^ qr.w[0][0];
            if (PAIR && cpair) {
                sink ^= r1.kA[0] ^ r1.kB[1] ^ r1.vA[0] ^ r1.vB[1] ^ r1.kp[0] ^ r1.vp[0];
                ++C.u;
                ++C.r;
            }
            if (C.r == C.rp.cost - 1 || C.u + 1 == u_end) open = false;
            cursor_next(a, R, C);
        } else {
        if (!open) {
            // this step starts a segment: finish the previous one first
            if (pend) {
                vpart<GP, BITS>(c, L, kp);
                end_segment(E);
                pend = false;
            }
            // a segment's first step finds mK = -inf and scales O, lsum and
            // zsum (finite leftovers of the previous segment) by 0
            build_query<GP, KG, BITS>(a, qr, L, c);
            c.mK = kNegInf;
            open = true;
        }
        const int e0 = 16 * (C.r - C.rp.n4);
        const int sbase = int4 ? (C.rp.k0 + C.r) * 32 : e0;
        const int slo = int4 ? C.rp.lo4 : 0;
        const int shi = int4 ? C.rp.hi4 : min(C.rp.n8e, e0 + 16);
        const KAcc<GP> ka = kpart_mfma<GP, BITS, KG>(a, c, r, int4);
        if (pend) vpart<GP, BITS>(c, L, kp);    // previous step, same segment
        kp = kpart_tail<GP, KG>(c, L, r, ka, !int4, sbase, slo, shi);
        pend = true;
        E = C;
        if (PAIR && cpair) {
            // the pair's second step: the same sequence, 32 positions on
            const KAcc<GP> ka1 = kpart_mfma<GP, BITS, KG>(a, c, r1, true);
            vpart<GP, BITS>(c, L, kp);
            kp = kpart_tail<GP, KG>(c, L, r1, ka1, false, sbase + 32, slo, shi);
            ++C.u;
            ++C.r;
            E = C;
        }
        if (C.r == C.rp.cost - 1 || C.u + 1 == u_end) open = false;
        cursor_next(a, R, C);
        }
        // the next step's stage (its DMA is i + 1's, issued three steps ago)
        if (C.u < u_end) {
            wait_vm_steps(issued - i - 2);
            if constexpr (APPEND) {
                if (C.r == C.rp.rn)
                    append_new_token<BITS>(a, R, C, kvring + snxt * kKvBytes, smem + snxt * SB, lane);
            }
            cpair = pairable<GP, BITS, KG, APPEND>(C, u_end);
            r = read_stage<GP, BITS, KG>(a, smem + snxt * SB, L, C.r < C.rp.n4);
            if (PAIR && cpair)
                r1 = read_stage<GP, BITS, KG>(a, smem + snxt * SB + kPairHalf, L, true, kPairParams - kPairHalf);
            if (!open) qr = read_query<GP>(qring + snxt * QRing<GP>::kBytes, lane);
        }
        // producer: step P into the slot this iteration's step was read from
        if (P.u < u_end) {
            uint8_t *qs = qring + scur * QRing<GP>::kBytes;
            if (P.r == 0 || P.u == start.u) issue_query<GP>(a, P.b, P.hk, L, qs);
            if constexpr (APPEND) {
                if (P.r == P.rp.rn) issue_new_token(a, R, P, kvring + scur * kKvBytes, lane);
            }
            if (PAIR && ppair) {
                issue_pair2(a, P, look, look1, smem + scur * SB, offP4, lane);
                ++P.u;
                ++P.r;
            } else {
                issue_step<BITS, KG>(a, P, look, smem + scur * SB, offK, offV, offP4, offP8, lane);
            }
            cursor_next(a, R, P);
            ++issued;
            advance_half(P);
            if (P.u < u_end) {
                ppair = pairable<GP, BITS, KG, APPEND>(P, u_end);
                look = read_pages(P, 0);
                if (PAIR && ppair) look1 = read_pages(P, 1);
            }
        }
        wait_lgkm0();
        look = uniform(look);
        if (PAIR) look1 = uniform(look1);
    }
    if constexpr (MEM) {
        // practically never true, but not provably so: the reads stay
        if (sink == 0x9E3779B9u + (uint32_t)a.B) a.ws_header[1] = (int32_t)sink;
        return;
    }
    if (pend) {
        vpart<GP, BITS>(c, L, kp);
        end_segment(E);
    }
    if (lane == 0) {
        a.ws_wseg[2 * wid] = wseg0;
        a.ws_wseg[2 * wid + 1] = wseg1;
    }
}

// Log-sum-exp combine of the pieces of the (row, KV head) segments that several
// workers share; also writes the rows with no context.
//
// Workgroups [0, B*H) take one segment each: rows without context, and
// segments of at most kChunkPieces pieces, merged directly in worker order by
// the kCombWaves waves of the workgroup (block_fold_heads).  A longer segment
// (a long row split over many workers) is folded by the helper workgroups
// B*H + h, kLongHelpers per chunk of kChunkPieces workers: the helpers whose
// chunks hold pieces of the segment split its (query head, dim slice) tasks
// among themselves, and each task reads all of the segment's pieces for its
// slice in one pass (fold_long_task): a segment of up to 512 pieces costs a
// task one round trip of piece loads.
//
// Lane l handles query heads l / 16 (g <= 4), or 8 k + l / 16 and 8 k + 4 +
// l / 16, and dims 8 (l % 16) .. + 8 of a piece laid out as
// [head][m, l, 0, 0, acc[128]].
constexpr int kCombBatch = 8;

struct MergeAcc {
    float M, Ls, acc[8];
};

__device__ inline void merge_init(MergeAcc &r) {
    r.M = kNegInf;
    r.Ls = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.acc[e] = 0.0f;
}

// Folds pieces ptr(0), ..., ptr(cnt - 1) (wave-uniform bases) for the NH
// heads jj[h] of this lane, kCombBatch / NH pieces per round trip.
template <int NH, typename PtrFn>
__device__ inline void fold_pieces(MergeAcc (&r)[NH], PtrFn ptr, int cnt, const int (&jj)[NH], int part) {
    constexpr int NB = kCombBatch / NH;
    for (int k0 = 0; k0 < cnt; k0 += NB) {
        float m[NH][NB], l[NH][NB];
        u32x4 v0[NH][NB], v1[NH][NB];
        // branch-free: a batch past the last piece re-reads it and drops it,
        // so all of a batch's loads issue before the first wait
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const float *pt = ptr(min(k0 + t, cnt - 1));
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const float *pp = pt + jj[h] * kPieceStride;
                const float2 ml = *reinterpret_cast<const float2 *>(pp);
                m[h][t] = k0 + t < cnt ? ml.x : kNegInf;
                l[h][t] = ml.y;
                v0[h][t] = ldg<u32x4>(pp + 4 + 8 * part);
                v1[h][t] = ldg<u32x4>(pp + 8 + 8 * part);
            }
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float Mn = r[h].M;
#pragma unroll
            for (int t = 0; t < NB; ++t) Mn = fmaxf(Mn, m[h][t]);
            const float fr = r[h].M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(r[h].M - Mn);
            r[h].Ls *= fr;
#pragma unroll
            for (int e = 0; e < 8; ++e) r[h].acc[e] *= fr;
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                const float f = m[h][t] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m[h][t] - Mn);
                r[h].Ls = fmaf(l[h][t], f, r[h].Ls);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    r[h].acc[e] = fmaf(__uint_as_float(v0[h][t][e]), f, r[h].acc[e]);
                    r[h].acc[4 + e] = fmaf(__uint_as_float(v1[h][t][e]), f, r[h].acc[4 + e]);
                }
            }
            r[h].M = Mn;
        }
    }
}

// Normalized output (and lse) of head j from a fold.
__device__ inline void merge_write(const DecodeArgs &a, const MergeAcc &r, int b, int hk, int j, int part) {
    float *o = a.out + ((int64_t)b * a.Hq + (int64_t)hk * a.g + j) * kHeadDim + 8 * part;
    const float inv = 1.0f / r.Ls;
    u32x4 w0, w1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        w0[e] = __float_as_uint(r.acc[e] * inv);
        w1[e] = __float_as_uint(r.acc[4 + e] * inv);
    }
    *reinterpret_cast<u32x4 *>(o) = w0;
    *reinterpret_cast<u32x4 *>(o + 4) = w1;
    if (a.lse && part == 0) a.lse[(int64_t)b * a.Hq + (int64_t)hk * a.g + j] = (r.M + __log2f(r.Ls)) / kLog2e;
}

__device__ inline int wave_min(int x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
    return uni(x);
}

// A combine workgroup is kCombWaves waves.  A fold of more pieces than one
// round trip of one wave carries is split into kCombWaves contiguous ranges,
// one per wave; wave 0 then merges the waves' partials in wave order, so the
// result does not depend on timing.
constexpr int kCombWaves = 4;

struct CombShared {
    MergeAcc part[kCombWaves][2][64];   // per wave, per head slot, per lane
    int before;                         // the helper's count before its add
};

// r <- fold of (r, o): both rescaled to the larger running max.
__device__ inline void merge_acc(MergeAcc &r, const MergeAcc &o) {
    const float Mn = fmaxf(r.M, o.M);
    if (Mn == kNegInf) return;
    const float fr = r.M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(r.M - Mn);
    const float fo = o.M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(o.M - Mn);
    r.Ls = fmaf(r.Ls, fr, o.Ls * fo);
#pragma unroll
    for (int e = 0; e < 8; ++e) r.acc[e] = fmaf(r.acc[e], fr, o.acc[e] * fo);
    r.M = Mn;
}

// Folds pieces ptr(0) .. ptr(cnt - 1) for every head of the group with the
// whole workgroup and hands each head's result to out(r, j) in wave 0: one
// pass of single heads for g <= 4, else passes over pairs of head quartets
// (lane l takes heads hg + l / 16 and hg + 4 + l / 16).  Every wave of the
// workgroup must call it with the same cnt (it holds workgroup barriers).
template <typename PtrFn, typename OutFn>
__device__ inline void block_fold_heads(int g, int wave, int lane, int part, int cnt, PtrFn ptr, OutFn out,
                                        CombShared &sh) {
    const int per_trip = g <= 4 ? kCombBatch : kCombBatch / 2;
    const int nw = cnt <= per_trip ? 1 : kCombWaves;
    const int lo = wave < nw ? wave * cnt / nw : 0;
    const int hi = wave < nw ? (wave + 1) * cnt / nw : 0;
    auto sub = [&](int k) { return ptr(lo + k); };
    if (g <= 4) {
        const int j = lane >> 4;
        MergeAcc r[1];
        merge_init(r[0]);
        const int jj[1] = {j < g ? j : 0};
        if (hi > lo) fold_pieces<1>(r, sub, hi - lo, jj, part);
        if (nw > 1) {
            sh.part[wave][0][lane] = r[0];
            __syncthreads();
            if (wave == 0)
                for (int k = 1; k < nw; ++k) merge_acc(r[0], sh.part[k][0][lane]);
            __syncthreads();
        }
        if (wave == 0 && j < g) out(r[0], j);
        return;
    }
    for (int hg = 0; hg < g; hg += 8) {
        const int j[2] = {hg + (lane >> 4), hg + 4 + (lane >> 4)};
        const int jj[2] = {j[0] < g ? j[0] : 0, j[1] < g ? j[1] : 0};
        MergeAcc r[2];
        merge_init(r[0]);
        merge_init(r[1]);
        if (hi > lo) fold_pieces<2>(r, sub, hi - lo, jj, part);
        if (nw > 1) {
            sh.part[wave][0][lane] = r[0];
            sh.part[wave][1][lane] = r[1];
            __syncthreads();
            if (wave == 0) {
                for (int k = 1; k < nw; ++k) {
                    merge_acc(r[0], sh.part[k][0][lane]);
                    merge_acc(r[1], sh.part[k][1][lane]);
                }
            }
            __syncthreads();
        }
        if (wave == 0) {
            if (j[0] < g) out(r[0], j[0]);
            if (j[1] < g) out(r[1], j[1]);
        }
    }
}

// Long segments.  A helper task is one query head j and one slice of the
// output's dims; the workgroup's lanes are nq dim quads (4 dims each) times
// 64 kCombWaves / nq piece slots, and each lane folds every slot-count-th
// piece of the segment, kLongBatch pieces per round trip (their loads issue
// together).  The lanes of a quad then merge in a fixed tree inside each wave
// and the waves' partials in wave order through LDS, so the result does not
// depend on timing.  Every piece of the segment is read once per slice, all
// of a slice's round trips by one workgroup.
constexpr int kLongBatch = 8;
constexpr int kLongHelpers = 4;         // helper workgroups per chunk of kChunkPieces workers
constexpr int kLongSlices = 8;          // dim slices per query head at most (16 dims each)

struct Fold4 {
    float M, Ls, acc[4];
};

struct LongShared {
    Fold4 part[kCombWaves][32];         // per wave, per dim quad
};

__device__ inline void fold4_merge(Fold4 &r, const Fold4 &o) {
    const float Mn = fmaxf(r.M, o.M);
    if (Mn == kNegInf) return;
    const float fr = r.M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(r.M - Mn);
    const float fo = o.M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(o.M - Mn);
    r.Ls = fmaf(r.Ls, fr, o.Ls * fo);
#pragma unroll
    for (int e = 0; e < 4; ++e) r.acc[e] = fmaf(r.acc[e], fr, o.acc[e] * fo);
    r.M = Mn;
}

// Folds head j, dims [d0, d0 + 4 nq) of the n pieces at basep, basep +
// piece_elems, ... and writes the normalized output (and lse).  Every wave of
// the workgroup calls it with the same arguments (it holds barriers).
__device__ inline void fold_long_task(const DecodeArgs &a, const float *basep, int64_t piece_elems, int n, int j,
                                      int d0, int nq, int b, int hk, LongShared &sh) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int q = lane & (nq - 1);
    const int nslots = 64 * kCombWaves / nq;
    const int slot = (int)(threadIdx.x / nq);
    const float *ph = basep + j * kPieceStride;
    Fold4 r;
    r.M = kNegInf;
    r.Ls = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) r.acc[e] = 0.0f;
    for (int k0 = slot; k0 < n; k0 += nslots * kLongBatch) {
        float m[kLongBatch], l[kLongBatch];
        u32x4 v[kLongBatch];
        // branch-free: slots past the last piece re-read it and drop it
#pragma unroll
        for (int t = 0; t < kLongBatch; ++t) {
            const int k = k0 + t * nslots;
            const float *pp = ph + (int64_t)min(k, n - 1) * piece_elems;
            const float2 ml = *reinterpret_cast<const float2 *>(pp);
            m[t] = k < n ? ml.x : kNegInf;
            l[t] = ml.y;
            v[t] = ldg<u32x4>(pp + 4 + d0 + 4 * q);
        }
        float Mn = r.M;
#pragma unroll
        for (int t = 0; t < kLongBatch; ++t) Mn = fmaxf(Mn, m[t]);
        if (Mn == kNegInf) continue;
        const float fr = r.M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(r.M - Mn);
        r.Ls *= fr;
#pragma unroll
        for (int e = 0; e < 4; ++e) r.acc[e] *= fr;
#pragma unroll
        for (int t = 0; t < kLongBatch; ++t) {
            const float f = m[t] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m[t] - Mn);
            r.Ls = fmaf(l[t], f, r.Ls);
#pragma unroll
            for (int e = 0; e < 4; ++e) r.acc[e] = fmaf(__uint_as_float(v[t][e]), f, r.acc[e]);
        }
        r.M = Mn;
    }
    // the slots of one quad inside the wave: lanes q, q + nq, ...
    for (int o = nq; o < 64; o <<= 1) {
        Fold4 x;
        x.M = __shfl_xor(r.M, o, 64);
        x.Ls = __shfl_xor(r.Ls, o, 64);
#pragma unroll
        for (int e = 0; e < 4; ++e) x.acc[e] = __shfl_xor(r.acc[e], o, 64);
        fold4_merge(r, x);
    }
    if (lane < nq) sh.part[wave][lane] = r;
    __syncthreads();
    if (wave == 0 && lane < nq) {
        for (int w = 1; w < kCombWaves; ++w) fold4_merge(r, sh.part[w][lane]);
        const int64_t hq = (int64_t)b * a.Hq + (int64_t)hk * a.g + j;
        const float inv = 1.0f / r.Ls;
        u32x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = __float_as_uint(r.acc[e] * inv);
        *reinterpret_cast<u32x4 *>(a.out + hq * kHeadDim + d0 + 4 * q) = o4;
        if (a.lse && d0 == 0 && lane == 0) a.lse[hq] = (r.M + __log2f(r.Ls)) / kLog2e;
    }
    __syncthreads();
}

__global__ __launch_bounds__(64 * kCombWaves) void decode_combine_kernel(DecodeArgs a) {
    constexpr int T = kChunkPieces;
    __shared__ CombShared sh;
    __shared__ LongShared lsh;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = a.g;
    const int part = lane & 15;
    const int64_t nseg = (int64_t)a.B * a.H;
    const int64_t piece_elems = (int64_t)g * kPieceStride;
    if ((int64_t)blockIdx.x < nseg) {
        const int64_t seg = blockIdx.x;
        const int b = (int)(seg / a.H), hk = (int)(seg % a.H);
        // independent scalar loads, one round trip
        const int Lb = ldc(a.ctx_len, b);
        const int64_t wf = ldc(a.ws_first, seg), wl = ldc(a.ws_last, seg);
        const RowPlan rp = row_plan(Lb, a.s, a.w);
        if (rp.cost == 0) {
            if (wave == 0) {
                for (int i = lane; i < g * kHeadDim; i += 64)
                    a.out[((int64_t)b * a.Hq + (int64_t)hk * g) * kHeadDim + i] = 0.0f;
                if (a.lse && lane < g) a.lse[(int64_t)b * a.Hq + (int64_t)hk * g + lane] = kNegInf;
            }
            return;
        }
        const int n = (int)(wl - wf + 1);
        if (n == 1 || n > T) return;            // finished by its only worker / folded by the helpers
        const float *basep = a.ws_piece + (wf + seg) * piece_elems;
        block_fold_heads(g, wave, lane, part, n, [&](int k) { return basep + k * piece_elems; },
                         [&](const MergeAcc &r, int j) { merge_write(a, r, b, hk, j, part); }, sh);
        return;
    }
    // helper h of the chunk of workers [w0, w0 + T): the worker count and the
    // workers' segment records load in one round trip (the records array holds
    // the whole grid's; those of workers >= W are dropped afterwards), the
    // records' segment bounds in a second.
    const int64_t hix = (int64_t)blockIdx.x - nseg;
    const int64_t jc = hix / kLongHelpers;
    const int hm = (int)(hix - jc * kLongHelpers);
    const int64_t w0 = jc * T;
    const bool mine = lane < 2 * T && w0 + lane / 2 < a.max_workers;
    int v = mine ? a.ws_wseg[2 * w0 + lane] : -1;
    const int64_t W = ldc(a.ws_header, 0);
    if (w0 >= W) return;
    if (w0 + lane / 2 >= W || v >= nseg) v = -1;
    // keep the long segments among them
    int vf = 0, vl = 0;
    if (v >= 0) {
        vf = a.ws_first[v];
        vl = a.ws_last[v];
        if (vl - vf + 1 <= T) v = -1;
    }
    int prev = -1;
    for (;;) {
        // the long segments of these workers' pieces, in increasing order (the
        // same in every wave: each wave reads the same records)
        const int s = wave_min(v > prev ? v : 0x7fffffff);
        if (s == 0x7fffffff) break;
        prev = s;
        // its bounds, from a lane that holds it
        const int src = __ffsll((unsigned long long)__ballot(v == s)) - 1;
        const int64_t wf = __builtin_amdgcn_readlane(vf, src), wl = __builtin_amdgcn_readlane(vl, src);
        const int n = (int)(wl - wf + 1);
        const int b = s / a.H, hk = s % a.H;
        // every helper of the chunks [wf / T, wl / T] finds this segment; they
        // share its tasks (query head, dim slice) round robin, with slices as
        // narrow as the helper count allows
        const int64_t jf = wf / T, jl = wl / T;
        const int nh = (int)((jl - jf + 1) * kLongHelpers);
        const int rank = (int)((jc - jf) * kLongHelpers + hm);
        int nc = kLongSlices;
        while (nc > 1 && g * nc > nh) nc >>= 1;
        const float *basep = a.ws_piece + (wf + s) * piece_elems;
        for (int t = rank; t < g * nc; t += nh)
            fold_long_task(a, basep, piece_elems, n, t / nc, (t % nc) * (kHeadDim / nc), 32 / nc, b, hk, lsh);
    }
}

template <int GP, bool APPEND, int BITS, bool MEM = false, bool KG = false>
static void launch_split(const DecodeArgs &a, int grid, hipStream_t stream) {
    constexpr int NW = kSplitWG<GP, APPEND, BITS, KG>;
    hipLaunchKernelGGL((decode_split_kernel<GP, APPEND, BITS, MEM, KG>), dim3(grid / NW), dim3(64 * NW), 0, stream, a);
}

struct SplitFn {
    const void *fn;
    int wg;         // workers per workgroup
};

template <int GP, bool APPEND, int BITS, bool KG = false>
static SplitFn split_fn() {
    return {reinterpret_cast<const void *>(&decode_split_kernel<GP, APPEND, BITS, false, KG>), kSplitWG<GP, APPEND, BITS, KG>};
}

static int group_class(int g) { return g <= 4 ? 4 : (g <= 8 ? 8 : 16); }

hipError_t launch_decode(const DecodeArgs &a, int grid, hipStream_t stream, bool grouped) {
    const bool fused = a.k_new != nullptr;
    if (grouped) {
        // grouped keys: attention only, query groups up to 8 (checked by the caller)
        const bool g4 = group_class(a.g) == 4;
        if (a.bits == 2) {
            if (g4) launch_split<4, false, 2, false, true>(a, grid, stream);
            else launch_split<8, false, 2, false, true>(a, grid, stream);
        } else if (a.bits == 3) {
            if (g4) launch_split<4, false, 3, false, true>(a, grid, stream);
            else launch_split<8, false, 3, false, true>(a, grid, stream);
        } else {
            if (g4) launch_split<4, false, 4, false, true>(a, grid, stream);
            else launch_split<8, false, 4, false, true>(a, grid, stream);
        }
    } else if (a.bits == 2) {
        switch (group_class(a.g) + (fused ? 1 : 0)) {
            case 4: launch_split<4, false, 2>(a, grid, stream); break;
            case 5: launch_split<4, true, 2>(a, grid, stream); break;
            case 8: launch_split<8, false, 2>(a, grid, stream); break;
            case 9: launch_split<8, true, 2>(a, grid, stream); break;
            case 16: launch_split<16, false, 2>(a, grid, stream); break;
            default: launch_split<16, true, 2>(a, grid, stream); break;
        }
    } else if (a.bits == 3) {
        switch (group_class(a.g) + (fused ? 1 : 0)) {
            case 4: launch_split<4, false, 3>(a, grid, stream); break;
            case 5: launch_split<4, true, 3>(a, grid, stream); break;
            case 8: launch_split<8, false, 3>(a, grid, stream); break;
            case 9: launch_split<8, true, 3>(a, grid, stream); break;
            case 16: launch_split<16, false, 3>(a, grid, stream); break;
            default: launch_split<16, true, 3>(a, grid, stream); break;
        }
    } else {
        switch (group_class(a.g) + (fused ? 1 : 0)) {
            case 4: launch_split<4, false, 4>(a, grid, stream); break;
            case 5: launch_split<4, true, 4>(a, grid, stream); break;
            case 8: launch_split<8, false, 4>(a, grid, stream); break;
            case 9: launch_split<8, true, 4>(a, grid, stream); break;
            case 16: launch_split<16, false, 4>(a, grid, stream); break;
            default: launch_split<16, true, 4>(a, grid, stream); break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int helpers = (grid + kChunkPieces - 1) / kChunkPieces * kLongHelpers;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.B * a.H + helpers), dim3(64 * kCombWaves), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_read_ceiling(const DecodeArgs &a, int grid, hipStream_t stream) {
    const int cls = group_class(a.g);
    if (cls == 16) return hipErrorNotSupported;
    if (a.bits == 2) {
        if (cls == 4) launch_split<4, false, 2, true>(a, grid, stream);
        else launch_split<8, false, 2, true>(a, grid, stream);
    } else if (a.bits == 3) {
        if (cls == 4) launch_split<4, false, 3, true>(a, grid, stream);
        else launch_split<8, false, 3, true>(a, grid, stream);
    } else {
        if (cls == 4) launch_split<4, false, 4, true>(a, grid, stream);
        else launch_split<8, false, 4, true>(a, grid, stream);
    }
    return hipGetLastError();
}

hipError_t decode_max_workers(int g, bool fused, int bits, int *out, bool grouped, int *out_wg) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int per_cu = 0;
    const int cls = group_class(g);
    SplitFn fn;
    if (grouped)
        fn = bits == 2 ? (cls == 4 ? split_fn<4, false, 2, true>() : split_fn<8, false, 2, true>())
           : bits == 3 ? (cls == 4 ? split_fn<4, false, 3, true>() : split_fn<8, false, 3, true>())
                       : (cls == 4 ? split_fn<4, false, 4, true>() : split_fn<8, false, 4, true>());
    else if (bits == 2 && fused)
        fn = cls == 4 ? split_fn<4, true, 2>() : (cls == 8 ? split_fn<8, true, 2>() : split_fn<16, true, 2>());
    else if (bits == 2)
        fn = cls == 4 ? split_fn<4, false, 2>() : (cls == 8 ? split_fn<8, false, 2>() : split_fn<16, false, 2>());
    else if (bits == 3 && fused)
        fn = cls == 4 ? split_fn<4, true, 3>() : (cls == 8 ? split_fn<8, true, 3>() : split_fn<16, true, 3>());
    else if (bits == 3)
        fn = cls == 4 ? split_fn<4, false, 3>() : (cls == 8 ? split_fn<8, false, 3>() : split_fn<16, false, 3>());
    else if (fused)
        fn = cls == 4 ? split_fn<4, true, 4>() : (cls == 8 ? split_fn<8, true, 4>() : split_fn<16, true, 4>());
    else
        fn = cls == 4 ? split_fn<4, false, 4>() : (cls == 8 ? split_fn<8, false, 4>() : split_fn<16, false, 4>());
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn.fn, 64 * fn.wg, 0);
    if (e != hipSuccess) return e;
    // The split kernel relies on every worker being resident at once (a worker
    // that starts late finishes late).  Measured on MI355X, a workgroup's LDS
    // is handed out in blocks larger than the occupancy query assumes (13.3 KB
    // per workgroup admits 11, not 12, per CU), so bound the count by 160 KB of
    // LDS per CU in 2 KB blocks as well.
    hipFuncAttributes attr;
    e = hipFuncGetAttributes(&attr, fn.fn);
    if (e != hipSuccess) return e;
    const size_t lds = (attr.sharedSizeBytes + 2047) & ~(size_t)2047;
    if (lds > 0) {
        const int by_lds = (int)((160u * 1024u) / lds);
        if (by_lds < per_cu) per_cu = by_lds;
    }
    if (per_cu < 1) per_cu = 1;
    *out = cus * per_cu * fn.wg;            // workers (waves)
    if (out_wg) *out_wg = fn.wg;
    return hipSuccess;
}

}  // namespace kvq
