// C ABI of the INT4 KV-cache library: argument checks, buffer sizes, launches.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/kvq.h"
#include <stdarg.h>

#include "common.h"

namespace {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
kvq_status fail(kvq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kvq_status ok() {
    g_err[0] = '\0';
    return KVQ_OK;
}

constexpr int kMinUnitsPerWorker = 8;
// Work split over the resident waves (two per SIMD), weighted by their measured
// speed on MI355X (per-wave timestamps over the Qwen3-8B batch): the SIMD's
// issue arbitration favours the older of its two waves -- that of the
// workgroup dispatched first to the CU, workers [0, W/2) -- by ~35% per step,
// the second workgroup starts its first step ~3 us later, and workgroups are
// dispatched round-robin over the 8 XCDs, of which the odd-numbered ones (odd
// workgroup index) stream ~3% slower.  Weights (units per worker, relative):
// {first half, even workgroup}, {first, odd}, {second, even}, {second, odd}.
constexpr int32_t kPartWeights[4] = {139, 135, 99, 96};
// A segment's start (query build) and end (reduction, piece or output stores)
// take about as long as two steps of one wave (regression of the per-wave
// durations on units and segments, Qwen3-8B batch), so the split counts each
// segment as this many units more than it streams.
constexpr int32_t kSegWeight = 2;
constexpr int kMaxDevices = 64;
// per device, group class (g <= 4, <= 8, <= 16), main-cache width (4, 2, 3 bits)
// and kernel (attention only, fused append); then the grouped-key kernels
// (attention only, g <= 4 or <= 8, value width)
std::atomic<int> g_max_workers[kMaxDevices][24];
std::atomic<int> g_cus[kMaxDevices];     // compute units per device

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

kvq_status check_cache(const kvq_cache *c) {
    if (!c) return fail(KVQ_ERR_NULL, "cache descriptor is NULL");
    if (c->head_dim != kvq::kHeadDim)
        return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d: only 128 is supported", c->head_dim);
    if (c->num_kv_heads < 1) return fail(KVQ_ERR_SHAPE, "num_kv_heads %d < 1", c->num_kv_heads);
    if (c->page_size < 16 || !is_pow2(c->page_size))
        return fail(KVQ_ERR_SHAPE, "page_size %d is not a power of two >= 16", c->page_size);
    if (c->num_pages < 0 || c->num_slots < 0) return fail(KVQ_ERR_SHAPE, "negative num_pages/num_slots");
    if (!is_pow2(c->had_block) || c->had_block > 128)
        return fail(KVQ_ERR_SHAPE, "had_block %d is not a power of two in [1, 128]", c->had_block);
    if (c->sink < 0 || c->recent < 0) return fail(KVQ_ERR_SHAPE, "negative sink/recent");
    if ((int64_t)c->sink + c->recent > (1 << 20)) return fail(KVQ_ERR_SHAPE, "sink + recent too large");
    if (c->code_bits != 0 && c->code_bits != 2 && c->code_bits != 3 && c->code_bits != 4)
        return fail(KVQ_ERR_UNSUPPORTED, "code_bits %d: the main cache holds 4-, 3- or 2-bit codes", c->code_bits);
    if (c->key_bits[0] != 0 || c->key_bits[1] != 0 || c->key_bits[2] != 0 || c->key_bits[3] != 0) {
        for (int j = 0; j < 4; ++j)
            if (c->key_bits[j] < 2 || c->key_bits[j] > 4)
                return fail(KVQ_ERR_UNSUPPORTED, "key_bits[%d] = %d: group widths are 2, 3 or 4", j, c->key_bits[j]);
        const bool equal = c->key_bits[0] == c->key_bits[1] && c->key_bits[1] == c->key_bits[2] &&
                           c->key_bits[2] == c->key_bits[3];
        if (!equal && c->had_block > 8)
            return fail(KVQ_ERR_UNSUPPORTED, "had_block %d > 8 with different group widths: a rotation block "
                        "would span two RoPE-block groups", c->had_block);
    }
    // the kernels index subblocks with 32-bit integers
    const uint64_t subs4 = (uint64_t)c->num_pages * (uint64_t)c->num_kv_heads * (uint64_t)(c->page_size / kvq::kSub);
    const uint64_t subs8 = (uint64_t)c->num_slots * (uint64_t)c->num_kv_heads *
                           (uint64_t)kvq::ceil_div(c->sink + c->recent, kvq::kSub);
    if (subs4 >= ((uint64_t)1 << 32) || subs8 >= ((uint64_t)1 << 32))
        return fail(KVQ_ERR_SHAPE, "a pool of 2^32 or more subblocks (%llu main, %llu ring)",
                    (unsigned long long)subs4, (unsigned long long)subs8);
    return KVQ_OK;
}

int bits_of(const kvq_cache *c) { return c->code_bits == 2 || c->code_bits == 3 ? c->code_bits : 4; }

bool grouped_of(const kvq_cache *c) { return c->key_bits[0] != 0; }

// Grouped keys: the key area offsets and the subblock bytes (include/kvq.h).
struct GroupLayout {
    int32_t off[4], key_area, sub_bytes;
};

GroupLayout group_layout(const kvq_cache *c) {
    GroupLayout g;
    int o = 0;
    for (int j = 0; j < 4; ++j) {
        g.off[j] = o;
        o += 64 * c->key_bits[j];
    }
    g.key_area = o;
    g.sub_bytes = o + kvq::value_area_bytes(bits_of(c)) + 128;
    return g;
}

size_t main_sub_bytes_of(const kvq_cache *c) {
    return grouped_of(c) ? (size_t)group_layout(c).sub_bytes : (size_t)kvq::main_sub_bytes(bits_of(c));
}

int nr8_of(const kvq_cache *c) { return kvq::ceil_div(c->sink + c->recent, kvq::kSub); }

float inv_sqrt(int h) { return (float)(1.0 / sqrt((double)h)); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

kvq_status max_workers(int g, bool fused, int bits, int *out, bool grouped = false, int *out_wg = nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "device index %d", dev);
    const int bi = bits == 2 ? 1 : (bits == 3 ? 2 : 0);
    const int cls = grouped ? 18 + (g <= 4 ? 0 : 3) + bi
                            : (g <= 4 ? 0 : (g <= 8 ? 1 : 2)) + 6 * bi + (fused ? 3 : 0);
    int v = g_max_workers[dev][cls].load(std::memory_order_relaxed);
    if (v <= 0) {
        int wg = 1;
        hipError_t e = kvq::decode_max_workers(g, fused, bits, &v, grouped, &wg);
        if (e != hipSuccess) return fail(KVQ_ERR_HIP, "occupancy query failed: %s", hipGetErrorString(e));
        // workers and workers per workgroup in one word (workers < 2^24)
        v = (v << 4) | wg;
        g_max_workers[dev][cls].store(v, std::memory_order_relaxed);
    }
    *out = v >> 4;
    if (out_wg) *out_wg = v & 15;
    return KVQ_OK;
}

kvq_status cu_count(int *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "device index %d", dev);
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
            return fail(KVQ_ERR_HIP, "compute unit count query failed");
        g_cus[dev].store(v, std::memory_order_relaxed);
    }
    *out = v;
    return KVQ_OK;
}

struct WsLayout {
    size_t first_off, last_off, wseg_off, piece_off, total;
};

WsLayout ws_layout(const kvq_cache *c, int B, int g, int workers) {
    WsLayout l;
    const size_t segs = (size_t)B * c->num_kv_heads;
    l.first_off = kvq::kWsHeaderBytes;
    l.last_off = align256(l.first_off + segs * sizeof(int32_t));
    l.wseg_off = align256(l.last_off + segs * sizeof(int32_t));
    l.piece_off = align256(l.wseg_off + 2 * (size_t)workers * sizeof(int32_t));
    const size_t pieces = (size_t)workers + (size_t)B * c->num_kv_heads;
    l.total = align256(l.piece_off + pieces * (size_t)g * kvq::kPieceStride * sizeof(float));
    return l;
}

}  // namespace

extern "C" {

size_t kvq_int4_pool_bytes(const kvq_cache *c) {
    if (check_cache(c) != KVQ_OK) return 0;
    return (size_t)c->num_pages * c->num_kv_heads * (c->page_size / kvq::kSub) * main_sub_bytes_of(c);
}

size_t kvq_int8_pool_bytes(const kvq_cache *c) {
    if (check_cache(c) != KVQ_OK) return 0;
    return (size_t)c->num_slots * c->num_kv_heads * nr8_of(c) * kvq::kSub8Bytes;
}

kvq_status kv_quant_append(const kvq_cache *c, const uint16_t *k, const uint16_t *v,
                           const int32_t *slot, const int32_t *pos, int32_t T,
                           const int32_t *block_table, int32_t bt_stride,
                           const int32_t *len_after, void *stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (T < 0) return fail(KVQ_ERR_SHAPE, "T = %d < 0", T);
    if (T == 0) return ok();
    if ((int64_t)T * c->num_kv_heads > ((int64_t)1 << 31) - 4)
        return fail(KVQ_ERR_SHAPE, "T * num_kv_heads too large for one call");
    if (!k || !v || !slot || !pos || !block_table || !len_after)
        return fail(KVQ_ERR_NULL, "a required device pointer is NULL");
    if (!c->int4_pool) return fail(KVQ_ERR_NULL, "int4_pool is NULL");
    if (c->sink + c->recent > 0 && !c->int8_pool) return fail(KVQ_ERR_NULL, "int8_pool is NULL");
    if (bt_stride < 1) return fail(KVQ_ERR_SHAPE, "bt_stride %d < 1", bt_stride);
    kvq::AppendArgs a;
    a.k = k;
    a.v = v;
    a.slot = slot;
    a.pos = pos;
    a.T = T;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.len_after = len_after;
    a.int4_pool = static_cast<uint8_t *>(c->int4_pool);
    a.int8_pool = static_cast<uint8_t *>(c->int8_pool);
    a.H = c->num_kv_heads;
    a.P = c->page_size;
    a.h = c->had_block;
    a.s = c->sink;
    a.w = c->recent;
    a.nr8 = nr8_of(c);
    a.bits = bits_of(c);
    a.inv_sqrt_h = inv_sqrt(c->had_block);
    const GroupLayout gl = group_layout(c);
    for (int j = 0; j < 4; ++j) {
        a.key_bits[j] = c->key_bits[j];
        a.kg_off[j] = gl.off[j];
    }
    a.key_area = gl.key_area;
    a.sub_bytes = gl.sub_bytes;
    hipError_t e = kvq::launch_quant_append(a, static_cast<hipStream_t>(stream), grouped_of(c));
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "quant-append launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t kv_decode_attn_workspace_bytes(const kvq_cache *c, int32_t B, int32_t num_q_heads) {
    if (check_cache(c) != KVQ_OK || B < 0 || num_q_heads < 1 || num_q_heads % c->num_kv_heads) return 0;
    const int g = num_q_heads / c->num_kv_heads;
    if (g > 16) return 0;
    // large enough for both kernels (attention only and fused append)
    int workers = 0, workers_fused = 0;
    const int bits = bits_of(c);
    if (grouped_of(c) && g > 8) return 0;
    if (max_workers(g, false, bits, &workers, grouped_of(c)) != KVQ_OK) return 0;
    if (max_workers(g, true, bits, &workers_fused) != KVQ_OK) return 0;
    const size_t a = ws_layout(c, B, g, workers).total, b = ws_layout(c, B, g, workers_fused).total;
    return a > b ? a : b;
}

}  // extern "C"

namespace {

// Attention of a batch, or (fused) the append of each row's token followed by
// the attention, in one split-kernel launch.
kvq_status decode_launch(const kvq_cache *c, bool fused, const uint16_t *k_new, const uint16_t *v_new,
                         const uint16_t *q, int32_t num_q_heads, const int32_t *slot, const int32_t *block_table,
                         int32_t bt_stride, const int32_t *ctx_len, int32_t B, float *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream, bool ceiling = false) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (B < 0) return fail(KVQ_ERR_SHAPE, "B = %d < 0", B);
    if (num_q_heads < 1 || num_q_heads % c->num_kv_heads)
        return fail(KVQ_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    num_q_heads, c->num_kv_heads);
    const int g = num_q_heads / c->num_kv_heads;
    if (g > 16) return fail(KVQ_ERR_UNSUPPORTED, "query group %d > 16", g);
    if (B == 0) return ok();
    if ((int64_t)B * num_q_heads > ((int64_t)1 << 31) - 1) return fail(KVQ_ERR_SHAPE, "B * num_q_heads too large");
    if (!q || !slot || !block_table || !ctx_len || (!out && !ceiling) || (fused && (!k_new || !v_new)))
        return fail(KVQ_ERR_NULL, "a required device pointer is NULL");
    if (ceiling && g > 8) return fail(KVQ_ERR_UNSUPPORTED, "the read ceiling covers query groups up to 8");
    const bool grouped = grouped_of(c);
    if (grouped && (fused || ceiling))
        return fail(KVQ_ERR_UNSUPPORTED, "grouped key widths are served by kv_quant_append + kv_decode_attn");
    if (grouped && g > 8) return fail(KVQ_ERR_UNSUPPORTED, "grouped key widths: query group %d > 8", g);
    if (!c->int4_pool) return fail(KVQ_ERR_NULL, "int4_pool is NULL");
    if (c->sink + c->recent > 0 && !c->int8_pool) return fail(KVQ_ERR_NULL, "int8_pool is NULL");
    if (bt_stride < 1) return fail(KVQ_ERR_SHAPE, "bt_stride %d < 1", bt_stride);
    if (!workspace) return fail(KVQ_ERR_WORKSPACE, "workspace is NULL");
    int workers = 0, wg = 1;
    st = max_workers(g, fused, bits_of(c), &workers, grouped, &wg);
    if (st != KVQ_OK) return st;
    const WsLayout l = ws_layout(c, B, g, workers);
    if (workspace_bytes < l.total)
        return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, l.total);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    kvq::DecodeArgs a;
    a.q = q;
    a.Hq = num_q_heads;
    a.g = g;
    a.slot = slot;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.ctx_len = ctx_len;
    a.B = B;
    a.int4_pool = static_cast<uint8_t *>(c->int4_pool);
    a.int8_pool = static_cast<uint8_t *>(c->int8_pool);
    a.k_new = fused ? k_new : nullptr;
    a.v_new = fused ? v_new : nullptr;
    a.H = c->num_kv_heads;
    a.P = c->page_size;
    a.logP = __builtin_ctz((unsigned)c->page_size);
    a.h = c->had_block;
    a.s = c->sink;
    a.w = c->recent;
    a.nr8 = nr8_of(c);
    a.bits = bits_of(c);
    a.inv_sqrt_h = inv_sqrt(c->had_block);
    const GroupLayout gl = group_layout(c);
    for (int j = 0; j < 4; ++j) {
        a.key_bits[j] = c->key_bits[j];
        a.kg_off[j] = gl.off[j];
    }
    a.key_area = gl.key_area;
    a.sub_bytes = gl.sub_bytes;
    a.max_workers = workers;
    a.min_units = kMinUnitsPerWorker;
    // the weights describe two split workgroups per CU (an older and a younger
    // wave on every SIMD); with one per CU every wave runs alone on its SIMD
    int cus = 0;
    st = cu_count(&cus);
    if (st != KVQ_OK) return st;
    a.simds = 4 * cus;
    const bool paired = wg == kvq::kSplitWaves && (int64_t)workers >= 2LL * kvq::kSplitWaves * cus;
    for (int i = 0; i < 4; ++i) a.part_wt[i] = paired ? kPartWeights[i] : 1;
    a.seg_wt = kSegWeight;
    a.ws_header = reinterpret_cast<int32_t *>(ws);
    a.ws_first = reinterpret_cast<int32_t *>(ws + l.first_off);
    a.ws_wseg = reinterpret_cast<int32_t *>(ws + l.wseg_off);
    a.ws_last = reinterpret_cast<int32_t *>(ws + l.last_off);
    a.ws_piece = reinterpret_cast<float *>(ws + l.piece_off);
    a.out = out;
    a.lse = lse;
    hipError_t e = ceiling ? kvq::launch_decode_read_ceiling(a, workers, static_cast<hipStream_t>(stream))
                           : kvq::launch_decode(a, workers, static_cast<hipStream_t>(stream), grouped);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

kvq_status kv_decode_attn(const kvq_cache *c, const uint16_t *q, int32_t num_q_heads,
                          const int32_t *slot, const int32_t *block_table, int32_t bt_stride,
                          const int32_t *ctx_len, int32_t B, float *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return decode_launch(c, false, nullptr, nullptr, q, num_q_heads, slot, block_table, bt_stride, ctx_len, B, out, lse,
                         workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of kv_decode_attn_noalloc: the decode workspace (worker records,
// chunk partials, pieces) in a device array that the code object brings along,
// so that the call allocates nothing.  Each device holds its own copy at its
// own address; host code must use that address (hipGetSymbolAddress), never
// the array's name, which on the host is only a stand-in for the symbol.
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];
std::atomic<uintptr_t> g_scratch[kMaxDevices];

// Address of `scratch` on the current device, looked up once per device.
kvq_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_UNSUPPORTED, "device index %d", dev);
    uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == 0) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        p = reinterpret_cast<uintptr_t>(ptr);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = reinterpret_cast<void *>(p);
    return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kv_decode_attn_noalloc(const kvq_cache *c, const uint16_t *q, int32_t num_q_heads, const int32_t *slot,
                                  const int32_t *block_table, int32_t bt_stride, const int32_t *ctx_len, int32_t B,
                                  float *out, float *lse, void *stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (B < 0 || num_q_heads < 1 || num_q_heads % c->num_kv_heads || num_q_heads / c->num_kv_heads > 16)
        return decode_launch(c, false, nullptr, nullptr, q, num_q_heads, slot, block_table, bt_stride, ctx_len, B,
                             out, lse, nullptr, 0, stream);       // reports the argument error
    if (B == 0) return ok();
    if (!q || !slot || !block_table || !ctx_len || !out)
        return fail(KVQ_ERR_NULL, "a required device pointer is NULL");
    const size_t need = kv_decode_attn_workspace_bytes(c, B, num_q_heads);
    if (need == 0) return fail(KVQ_ERR_HIP, "workspace size query failed");
    if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES)
        return fail(KVQ_ERR_WORKSPACE, "B = %d rows of %d query heads need %zu bytes of scratch; the static scratch "
                    "holds %zu (use kv_decode_attn with a workspace)", B, num_q_heads, need,
                    (size_t)KVQ_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != KVQ_OK) return st;
    return decode_launch(c, false, nullptr, nullptr, q, num_q_heads, slot, block_table, bt_stride, ctx_len, B, out,
                         lse, ws, (size_t)KVQ_NOALLOC_SCRATCH_BYTES, stream);
}

kvq_status kv_decode_read_ceiling(const kvq_cache *c, const uint16_t *q, int32_t num_q_heads, const int32_t *slot,
                                  const int32_t *block_table, int32_t bt_stride, const int32_t *ctx_len, int32_t B,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    return decode_launch(c, false, nullptr, nullptr, q, num_q_heads, slot, block_table, bt_stride, ctx_len, B, nullptr,
                         nullptr, workspace, workspace_bytes, stream, true);
}

kvq_status kv_append_decode_attn(const kvq_cache *c, const uint16_t *k, const uint16_t *v, const uint16_t *q,
                                 int32_t num_q_heads, const int32_t *slot, const int32_t *block_table,
                                 int32_t bt_stride, const int32_t *ctx_len, int32_t B, float *out, float *lse,
                                 void *workspace, size_t workspace_bytes, void *stream) {
    return decode_launch(c, true, k, v, q, num_q_heads, slot, block_table, bt_stride, ctx_len, B, out, lse, workspace,
                         workspace_bytes, stream);
}

kvq_status kv_prefill_attn(const kvq_cache *c, const uint16_t *q, int32_t num_q_heads, const int32_t *q_start,
                           int32_t max_rows, const int32_t *slot, const int32_t *block_table, int32_t bt_stride,
                           const int32_t *ctx_len, int32_t B, float *out, float *lse, void *stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (B < 0 || max_rows < 0) return fail(KVQ_ERR_SHAPE, "B = %d, max_rows = %d: negative", B, max_rows);
    if (num_q_heads < 1 || num_q_heads % c->num_kv_heads)
        return fail(KVQ_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    num_q_heads, c->num_kv_heads);
    const int g = num_q_heads / c->num_kv_heads;
    if (g > 16) return fail(KVQ_ERR_UNSUPPORTED, "query group %d > 16", g);
    if (B == 0 || max_rows == 0) return ok();
    if (B > 65535 || c->num_kv_heads > 65535) return fail(KVQ_ERR_SHAPE, "B or num_kv_heads above 65535");
    if (!q || !q_start || !slot || !block_table || !ctx_len || !out)
        return fail(KVQ_ERR_NULL, "a required device pointer is NULL");
    if (!c->int4_pool) return fail(KVQ_ERR_NULL, "int4_pool is NULL");
    if (c->sink + c->recent > 0 && !c->int8_pool) return fail(KVQ_ERR_NULL, "int8_pool is NULL");
    if (bt_stride < 1) return fail(KVQ_ERR_SHAPE, "bt_stride %d < 1", bt_stride);
    if (grouped_of(c))
        return fail(KVQ_ERR_UNSUPPORTED, "prefill attention does not read grouped key widths");
    kvq::PrefillArgs a;
    a.q = q;
    a.Hq = num_q_heads;
    a.g = g;
    a.R = 16 / g;
    a.q_start = q_start;
    a.slot = slot;
    a.block_table = block_table;
    a.bt_stride = bt_stride;
    a.ctx_len = ctx_len;
    a.B = B;
    a.int4_pool = static_cast<const uint8_t *>(c->int4_pool);
    a.int8_pool = static_cast<const uint8_t *>(c->int8_pool);
    a.H = c->num_kv_heads;
    a.P = c->page_size;
    a.logP = __builtin_ctz((unsigned)c->page_size);
    a.h = c->had_block;
    a.s = c->sink;
    a.w = c->recent;
    a.nr8 = nr8_of(c);
    a.bits = bits_of(c);
    a.inv_sqrt_h = inv_sqrt(c->had_block);
    a.out = out;
    a.lse = lse;
    const int64_t rows_per_wave = (int64_t)a.R * kvq::prefill_tiles(a.bits);
    const int64_t tiles = ((int64_t)max_rows + rows_per_wave - 1) / rows_per_wave;
    if (tiles > 0x7FFFFFFF) return fail(KVQ_ERR_SHAPE, "max_rows too large");
    hipError_t e = kvq::launch_prefill(a, (int)tiles, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

const char *kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_NULL: return "null pointer";
        case KVQ_ERR_SHAPE: return "bad shape or size";
        case KVQ_ERR_UNSUPPORTED: return "unsupported";
        case KVQ_ERR_WORKSPACE: return "workspace too small";
        case KVQ_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *kvq_last_error(void) { return g_err; }

}  // extern "C"
