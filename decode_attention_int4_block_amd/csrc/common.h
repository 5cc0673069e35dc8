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

// Workspace of the decode attention: header, per-row cost prefix, partial pieces.
constexpr int kPieceStride = 132;           // floats per (piece, query head): m, l, 0, 0, acc[128]
constexpr size_t kWsHeaderBytes = 256;

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Work of one row, in units of roughly equal bytes: INT4 steps of 32 positions
// aligned to multiples of 32 (2 x 2176 B) and INT8 steps of one 16-entry
// subblock (4224 B).
struct RowPlan {
    int lo4, hi4;   // INT4 region [lo4, hi4)
    int k0, n4;     // first 32-position step index and number of INT4 steps
    int n8e, n8;    // valid ring entries and INT8 steps
    int cost;       // n4 + n8 units
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
    return r;
}

// Start unit of worker w when `total` units are split over `workers` workers.
__host__ __device__ inline int64_t worker_begin(int64_t w, int64_t total, int64_t workers) {
    return (w * total) / workers;
}

// The worker whose unit range contains unit u.
__host__ __device__ inline int64_t worker_of(int64_t u, int64_t total, int64_t workers) {
    return ((u + 1) * workers - 1) / total;
}

__host__ __device__ inline int64_t effective_workers(int64_t total, int64_t max_workers, int64_t min_units) {
    int64_t w = (total + min_units - 1) / min_units;
    if (w < 1) w = 1;
    return w < max_workers ? w : max_workers;
}

// Two-phase split of the units: workers [0, w1) share units [0, u1) evenly and
// workers [w1, w1 + w2) share [u1, total).  With fewer units than all
// w1max + w2max workers can take, one even split over the workers needed.
struct Partition {
    int64_t total, u1, w1, w2;
};

__host__ __device__ inline Partition make_partition(int64_t total, int64_t w1max, int64_t w2max, int64_t share_q16,
                                                    int64_t min_units) {
    Partition p;
    p.total = total;
    p.w1 = effective_workers(total, w1max + w2max, min_units);
    p.u1 = total;
    p.w2 = 0;
    if (w1max > 0 && w2max > 0 && p.w1 == w1max + w2max) {
        p.w1 = w1max;
        p.u1 = (total * share_q16) >> 16;
        p.w2 = w2max;
    }
    return p;
}

__host__ __device__ inline int64_t part_begin(const Partition &p, int64_t w) {
    if (w <= p.w1) return worker_begin(w, p.u1, p.w1);
    return p.u1 + worker_begin(w - p.w1, p.total - p.u1, p.w2);
}

__host__ __device__ inline int64_t part_of(const Partition &p, int64_t u) {
    if (u < p.u1) return worker_of(u, p.u1, p.w1);
    return p.w1 + worker_of(u - p.u1, p.total - p.u1, p.w2);
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
    float inv_sqrt_h;   // fp32 value nearest to 1/sqrt(h)
};

struct DecodeArgs {
    const uint16_t *q;
    int32_t Hq, g;
    const int32_t *slot;
    const int32_t *block_table;
    int32_t bt_stride;
    const int32_t *ctx_len;
    int32_t B;
    const uint8_t *int4_pool;
    const uint8_t *int8_pool;
    int32_t H, P, logP, h, s, w, nr8;
    float inv_sqrt_h;
    int32_t max_workers, min_units;     // first-phase workers
    int32_t extra_workers;              // second-phase workers
    int32_t share_q16;                  // fraction of the units in the first phase, x 2^16
    int64_t *ws_header;     // [0] total units, [1] u1, [2] w1, [3] w2 (the Partition)
    int64_t *ws_prefix;     // [B] exclusive prefix of per-row units (all KV heads)
    float *ws_piece;        // [max_workers + B*H][g][kPieceStride] per-worker pieces
    float *out;
    float *lse;
};

hipError_t launch_quant_append(const AppendArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, int grid, hipStream_t stream);
hipError_t decode_max_workers(int g, int *out);

}  // namespace kvq
