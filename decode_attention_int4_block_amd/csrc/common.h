// Shared device-side definitions of the INT4 / INT8 cache layouts (see include/kvq.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kSub = 16;                    // tokens (or ring entries) per subblock

// INT4 subblock: 16 tokens x (64 B key codes + 64 B value codes + 4 + 4 B params)
constexpr int kSub4Bytes = 2176;
constexpr int kSub4K = 0;
constexpr int kSub4V = 1024;
constexpr int kSub4KP = 2048;
constexpr int kSub4VP = 2112;

// INT8 subblock: 16 entries x (128 B key codes + 128 B value codes + 4 + 4 B params),
// the codes as a low-nibble and a high-nibble plane in the INT4 code layouts
constexpr int kSub8Bytes = 4224;
constexpr int kSub8KLo = 0;
constexpr int kSub8KHi = 1024;
constexpr int kSub8VLo = 2048;
constexpr int kSub8VHi = 3072;
constexpr int kSub8KP = 4096;
constexpr int kSub8VP = 4160;

// 2-bit subblock (main cache at code_bits = 2): 16 tokens x (32 B key codes +
// 32 B value codes + 4 + 4 B params); layouts in quant.h (store_token_int2).
constexpr int kSub2Bytes = 1152;
constexpr int kSub2K = 0;
constexpr int kSub2V = 512;
constexpr int kSub2KP = 1024;
constexpr int kSub2VP = 1088;

// 3-bit subblock (code_bits = 3): the low two bits of every code in the 2-bit
// layouts (512 B keys, 512 B values), the high bits as a key plane and a value
// plane of 256 B each, then the params; layouts in quant.h (store_token_int3).
constexpr int kSub3Bytes = 1664;
constexpr int kSub3K = 0;
constexpr int kSub3V = 512;
constexpr int kSub3KH = 1024;
constexpr int kSub3VH = 1280;
constexpr int kSub3KP = 1536;
constexpr int kSub3VP = 1600;

__host__ __device__ constexpr int main_sub_bytes(int bits) {
    return bits == 2 ? kSub2Bytes : (bits == 3 ? kSub3Bytes : kSub4Bytes);
}

// Main cache with keys of a width per RoPE-block group (key_bits): group j
// of the keys is the dims d with (d mod 32) / 8 == j.  A subblock holds the
// group key areas (64 key_bits[j] bytes each, in group order), the value area
// of the value width, then the key and value params (layout in include/kvq.h).
__host__ __device__ constexpr int value_area_bytes(int bits) {
    return bits == 2 ? 512 : (bits == 3 ? 768 : 1024);
}

// Workspace of the decode attention: header, per-row cost prefix, partial pieces.
constexpr int kPieceStride = 132;           // floats per (piece, query head): m, l, 0, 0, acc[128]
constexpr size_t kWsHeaderBytes = 256;
constexpr int kChunkPieces = 32;            // a segment with more pieces is folded by the combine's helpers

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Work of one row, in units of roughly equal bytes: INT4 steps of 32 positions
// aligned to multiples of 32 (2 x 2176 B) and INT8 steps of one 16-entry
// subblock (4224 B).
struct RowPlan {
    int lo4, hi4;   // INT4 region [lo4, hi4)
    int k0, n4;     // first 32-position step index and number of INT4 steps
    int n8e, n8;    // valid ring entries and INT8 steps
    int cost;       // n4 + n8 units
    int rn, tn;     // the newest position L - 1: its unit, and its token (INT4 step)
                    // or ring entry (INT8 step) inside that unit; rn = -1 when L = 0
};

__host__ __device__ inline RowPlan row_plan(int L, int s, int w) {
    RowPlan r;
    r.lo4 = s;
    r.hi4 = L - w;
    if (r.hi4 > r.lo4) {
        r.k0 = r.lo4 >> 5;
        r.n4 = ((r.hi4 + 31) >> 5) - r.k0;
    } else {
        r.k0 = 0;
        r.n4 = 0;
    }
    int cap = s + w;
    r.n8e = L < cap ? L : cap;
    if (r.n8e < 0) r.n8e = 0;
    r.n8 = (r.n8e + 15) >> 4;
    r.cost = r.n4 + r.n8;
    const int p = L - 1;
    if (L <= 0) {
        r.rn = -1;
        r.tn = 0;
    } else if (p < s || w > 0) {
        // a sink, or the recent window (which always holds the newest
        // position): ring entry p for a sink, else s + (p - s) mod w
        const int e = p < s ? p : s + (p - s) % w;
        r.rn = r.n4 + (e >> 4);
        r.tn = e & 15;
    } else {
        r.rn = (p >> 5) - r.k0;
        r.tn = p & 31;
    }
    return r;
}

// q = n / d for the split's non-negative operands (d > 0).  A wave-uniform
// 64-bit division costs about a hundred scalar instructions on the prologue's
// critical path; operands that fit 32 bits take the 32-bit divide, and
// numerators below 2^53 a double-precision quotient corrected to the exact one
// (the rounded quotient is within 1 of it).
__host__ __device__ inline int64_t div_nonneg(int64_t n, int64_t d) {
    if ((uint64_t)(n | d) < ((uint64_t)1 << 32)) return (int64_t)((uint32_t)n / (uint32_t)d);
    if (n < ((int64_t)1 << 53) && d < ((int64_t)1 << 32)) {
        int64_t q = (int64_t)((double)n / (double)d);
        if (q * d > n)
            --q;
        else if ((q + 1) * d <= n)
            ++q;
        return q;
    }
    return n / d;
}

// Workers of a launch: min_units per worker, capped at max_workers.  A launch
// with fewer units than 512 workers of min_units each (a few short rows) takes
// half that per worker: its time is one worker's chain of steps, not the
// combine of the extra pieces (measured: a 1024-token row, 20 -> 17 us).
// Between one worker per SIMD (simds, when given) and max_workers, the count
// is rounded down to one per SIMD: a few workers past it would put a second
// wave on a few SIMDs, and those pairs end the launch (measured on one 128K
// row: split 20.6 -> 18.4 us, and half the pieces for the combine).
__host__ __device__ inline int64_t effective_workers(int64_t total, int64_t max_workers, int64_t min_units,
                                                     int64_t simds = 0) {
    if (total < 512 * min_units && min_units > 1) min_units = (min_units + 1) / 2;
    int64_t w = div_nonneg(total + min_units - 1, min_units);
    if (w < 1) w = 1;
    if (simds > 0 && w > simds && w < max_workers) w = simds;
    return w < max_workers ? w : max_workers;
}

// Workers (one wave each) per workgroup of the split kernel.  A workgroup's
// waves are placed on different SIMDs of one CU, so with two workgroups per CU
// every SIMD runs one wave of each, and the wave of the workgroup dispatched
// first is the older one on every SIMD.  (With one-wave workgroups the SIMD of
// each wave varies from launch to launch, and some SIMDs receive two waves of
// the first-dispatched set, which then share its issue slots.)
constexpr int kSplitWaves = 4;

// Weighted split of the units over W workers: worker w takes a share in
// proportion to wt[2 r + o], where r = (w >= W / 2) and o = the parity of its
// workgroup w / wg (wg = 1 or kSplitWaves workers per workgroup), so that
// waves of different measured speed (dispatch order, XCD) finish together.
// With fewer units than W full workers need, an even split over the workers
// needed.
struct Partition {
    int64_t total, W, half;
    int64_t wt[4];
    int64_t csum;           // cumulative weight of all W workers
    int32_t wg_log2;        // log2 of the workers per workgroup
};

// Workers of [0, n) in even-numbered workgroups of 2^l workers.
__host__ __device__ inline int64_t even_wg_workers(int64_t n, int l) {
    const int64_t S = (int64_t)1 << l;
    const int64_t rem = n & (2 * S - 1);
    return (n >> (l + 1)) * S + (rem < S ? rem : S);
}

__host__ __device__ inline int64_t count_even(const Partition &p, int64_t a, int64_t b) {
    return even_wg_workers(b, p.wg_log2) - even_wg_workers(a, p.wg_log2);
}

// Cumulative weight of the workers [0, w).
__host__ __device__ inline int64_t part_cum(const Partition &p, int64_t w) {
    const int64_t w0 = w < p.half ? w : p.half;
    const int64_t e0 = count_even(p, 0, w0);
    int64_t c = e0 * p.wt[0] + (w0 - e0) * p.wt[1];
    if (w > p.half) {
        const int64_t e1 = count_even(p, p.half, w);
        c += e1 * p.wt[2] + (w - p.half - e1) * p.wt[3];
    }
    return c;
}

// wg: workers per workgroup of the launch (1 or kSplitWaves); simds: SIMDs of
// the device, or 0 for no rounding of the worker count.
__host__ __device__ inline Partition make_partition(int64_t total, int64_t max_workers, const int32_t *wt,
                                                    int64_t min_units, int wg = kSplitWaves, int64_t simds = 0) {
    Partition p;
    p.wg_log2 = wg >= 4 ? 2 : (wg >= 2 ? 1 : 0);
    p.total = total;
    p.W = effective_workers(total, max_workers, min_units, simds);
    p.half = p.W / 2;
    const bool weighted = p.W == max_workers && p.W >= 2;
    for (int i = 0; i < 4; ++i) p.wt[i] = weighted ? wt[i] : 1;
    p.csum = part_cum(p, p.W);
    return p;
}

// First unit of worker w (w <= W).
__host__ __device__ inline int64_t part_begin(const Partition &p, int64_t w) {
    return div_nonneg(p.total * part_cum(p, w), p.csum);
}

// The worker whose unit range contains unit u (u < total); workers with empty
// ranges are never returned.  (The inverse of part_begin, for checking it.)
__host__ __device__ inline int64_t part_of(const Partition &p, int64_t u) {
    // invert the cumulative weight, then correct the rounding
    const int64_t c = div_nonneg(u * p.csum, p.total);
    const int64_t ch = part_cum(p, p.half);
    int64_t w = c < ch ? div_nonneg(2 * c, p.wt[0] + p.wt[1]) : p.half + div_nonneg(2 * (c - ch), p.wt[2] + p.wt[3]);
    if (w > p.W - 1) w = p.W - 1;
    if (w < 0) w = 0;
    while (w > 0 && part_begin(p, w) > u) --w;
    while (w < p.W - 1 && part_begin(p, w + 1) <= u) ++w;
    return w;
}

struct AppendArgs {
    const uint16_t *k;
    const uint16_t *v;
    const int32_t *slot;
    const int32_t *pos;
    int32_t T;
    const int32_t *block_table;
    int32_t bt_stride;
    const int32_t *len_after;
    uint8_t *int4_pool;
    uint8_t *int8_pool;
    int32_t H, P, h, s, w, nr8;
    int32_t bits;       // main cache code width: 4, 3 or 2 (the values' with grouped keys)
    float inv_sqrt_h;   // fp32 value nearest to 1/sqrt(h)
    int32_t key_bits[4];    // grouped keys: width of each RoPE-block group (KG launches)
    int32_t kg_off[4];      // grouped keys: byte offset of each group's key area
    int32_t key_area;       // grouped keys: bytes of the key area
    int32_t sub_bytes;      // grouped keys: bytes of a main-cache subblock
};

struct DecodeArgs {
    const uint16_t *q;
    int32_t Hq, g;
    const int32_t *slot;
    const int32_t *block_table;
    int32_t bt_stride;
    const int32_t *ctx_len;
    int32_t B;
    uint8_t *int4_pool;     // written only by the fused append
    uint8_t *int8_pool;
    const uint16_t *k_new;  // [B][H][128] bf16 key / value each row appends at
    const uint16_t *v_new;  //   position ctx_len - 1 (fused append), or nullptr
    int32_t H, P, logP, h, s, w, nr8;
    int32_t bits;                       // main cache code width: 4, 3 or 2
    float inv_sqrt_h;
    int32_t max_workers, min_units;
    int32_t simds;                      // SIMDs of the device (4 per CU)
    int32_t part_wt[4];                 // worker weights (Partition)
    int32_t seg_wt;                     // weight-only units counted before each segment
    int32_t key_bits[4];    // grouped keys: width of each RoPE-block group (KG launches)
    int32_t kg_off[4];      // grouped keys: byte offset of each group's key area
    int32_t key_area;       // grouped keys: bytes of the key area
    int32_t sub_bytes;      // grouped keys: bytes of a main-cache subblock
    int32_t *ws_header;     // [0] workers of this launch
    int32_t *ws_first;      // [B*H] worker that attended the segment's first unit
    int32_t *ws_last;       // [B*H] worker that attended the segment's last unit
    int32_t *ws_wseg;       // [2*workers] segment of each worker's first / last piece, or -1
    float *ws_piece;        // [max_workers + B*H][g][kPieceStride] per-worker pieces
    float *out;
    float *lse;
};

// Query tiles of 16 columns per prefill wave: two share each step's unpacked
// codes for the 4-bit cache; the 3- and 2-bit operand builders leave no
// registers for a second tile (it spilled 156-176 B per lane).
__host__ __device__ constexpr int prefill_tiles(int bits) { return bits == 4 ? 2 : 1; }

// Causal multi-row attention over the quantized cache (prefill).
struct PrefillArgs {
    const uint16_t *q;          // [N][Hq][128] bf16 query rows
    int32_t Hq, g, R;           // query heads, group size, rows per 16-column tile (R g <= 16)
    const int32_t *q_start;     // [B + 1] first query row of each sequence
    const int32_t *slot;
    const int32_t *block_table;
    int32_t bt_stride;
    const int32_t *ctx_len;
    int32_t B;
    const uint8_t *int4_pool;
    const uint8_t *int8_pool;
    int32_t H, P, logP, h, s, w, nr8;
    int32_t bits;               // main cache code width: 4, 3 or 2
    float inv_sqrt_h;
    float *out;                 // [N][Hq][128]
    float *lse;                 // [N][Hq] or nullptr
};

hipError_t launch_quant_append(const AppendArgs &a, hipStream_t stream, bool grouped = false);
hipError_t launch_prefill(const PrefillArgs &a, int tiles, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int grid, hipStream_t stream, bool grouped = false);
hipError_t launch_decode_read_ceiling(const DecodeArgs &a, int grid, hipStream_t stream);
hipError_t decode_max_workers(int g, bool fused, int bits, int *out, bool grouped = false, int *out_wg = nullptr);

}  // namespace kvq
