/*
 * kvq.h -- C ABI of the INT4 KV-cache library for AMD Instinct MI355X (gfx950).
 *
 * Two operations make up one decode step of calibration-free 4-bit KV-cache
 * quantization with a bounded INT8 side cache:
 *
 *   kv_quant_append -- quantize new key/value vectors on the fly and write them
 *                      into a paged INT4 cache (plus the INT8 side cache for
 *                      sink and recent positions);
 *   kv_decode_attn  -- decode attention that reads the packed codes directly,
 *                      attends the INT4 region and the INT8 region as disjoint
 *                      sets and merges them by log-sum-exp.
 *
 * kv_append_decode_attn does both for one new token per row in a single pass;
 * kv_prefill_attn attends a chunk of causal query rows per sequence.
 *
 * The method: KV4-RL ("Unlocking Faster Asynchronous Rollouts for RLVR with
 * INT4 KV Cache Quantization"), sections "Key Contributions" item 4 and
 * "Methodology in Plain English"; the block-diagonal Hadamard rotation of keys
 * is SAW-INT4 ("System-Aware 4-Bit KV-Cache Quantization for Real-World LLM
 * Serving"), section 2.
 *
 * General rules
 *   - Every pointer argument except `cache` is DEVICE memory owned by the caller
 *     (`cache` itself is a host struct that holds device pointers).  The library
 *     never allocates, frees or synchronizes, keeps no mutable global state
 *     except a per-device cache of device properties, and may be called from
 *     several host threads.  Buffers must stay valid until the stream has
 *     passed the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Host-side argument checks run before anything is enqueued; on failure a
 *     status is returned and nothing is enqueued.  A failed kernel launch is
 *     reported as KVQ_ERR_HIP.  Device-side data (positions in range, valid
 *     block-table entries, slots in range) is a precondition and is NOT
 *     checked; violating it is undefined behaviour.
 *   - bf16 and fp16 values are passed as uint16_t bit patterns.
 *   - No C++ exception crosses this interface.
 *
 * Parameters of the method (kvq_cache):
 *   head_dim   = 128 (one quantization group per 128-dim token-head vector);
 *   had_block  = h, the Hadamard block size: a power of two in [1, 128];
 *   sink       = s, recent = w: positions [0, s) and the last w positions of a
 *                sequence are attended from the INT8 side cache, the rest from
 *                INT4.  s + w may be 0 (INT4 only).
 *
 * ---------------------------------------------------------------------------
 * Quantization (both caches).  For a 128-dim vector y (keys: the fp32
 * block-Hadamard rotation of the bf16 key, butterfly strides 1, 2, ..., h/2 in
 * that order, then one multiply by the fp32 value nearest 1/sqrt(h); values:
 * the bf16 value itself):
 *   mn = min y, mx = max y, scale_f = fp32((mx - mn) / qmax), qmax = 15 or 255;
 *   scale = fp16(scale_f), zero = fp16(mn)         (round to nearest even);
 *   code_i = 0 if scale == 0, else clamp(rint(fp32(y_i - zero) / scale), 0, qmax)
 *   dequantized y_i = scale * code_i + zero.
 *
 * Regions.  For a sequence of length L: INT8 region = [0, min(s, L)) U
 * [max(s, L - w), L); INT4 region = [s, L - w) when non-empty.  Every position
 * is stored in INT4; INT8 copies live in a ring of s + w entries: position
 * p < s -> entry p, other positions -> entry s + (p - s) mod w.  An append of
 * position p writes its INT8 copy iff p < s or p >= len_after - w.
 *
 * ---------------------------------------------------------------------------
 * INT4 pool layout (int4_pool, kvq_int4_pool_bytes bytes, 256-byte aligned).
 *   A page of P tokens (P a power of two >= 16) and one KV head is P/16 "subblocks" of 16
 *   tokens; subblock j of (page, kv_head) starts at byte
 *       ((page * num_kv_heads + kv_head) * (P / 16) + j) * 2176
 *   and holds token rows t = 0..15 (position = page_row_base + 16 j + t):
 *     [   0, 1024) key codes, token-major: byte 64 t + i holds the codes of
 *                  rotated dims 2i (low nibble) and 2i + 1 (high nibble);
 *     [1024, 2048) value codes, token-fastest: with G = t / 4 and r = t % 4,
 *                  byte 4 * ((G * 16 + n) * 4 + c) + r holds value dim
 *                  32 c + n (low nibble) and 32 c + 16 + n (high nibble),
 *                  for n = 0..15, c = 0..3;
 *     [2048, 2112) key   (scale, zero) fp16 pairs, 4 bytes per token;
 *     [2112, 2176) value (scale, zero) fp16 pairs, 4 bytes per token.
 *   2176 bytes / (16 tokens * 256 elements) = 4.25 bits per element.
 *
 * INT8 side-cache layout (int8_pool, kvq_int8_pool_bytes bytes).
 *   Each (slot, kv_head) owns NR = ceil((s + w) / 16) subblocks of 16 ring
 *   entries; subblock j starts at byte
 *       ((slot * num_kv_heads + kv_head) * NR + j) * 4224
 *   and holds entries e = 0..15 (ring entry 16 j + e).  Each 8-bit code c is
 *   split into its low nibble c & 15 and high nibble c >> 4, and each nibble
 *   plane is laid out like the codes of an INT4 subblock:
 *     [   0, 1024) key low nibbles:  byte 64 e + i holds rotated dims 2i (low
 *                  nibble of the byte) and 2i + 1 (high nibble of the byte);
 *     [1024, 2048) key high nibbles, same arrangement;
 *     [2048, 3072) value low nibbles: with G = e / 4 and r = e % 4, byte
 *                  4 * ((G * 16 + n) * 4 + c) + r holds value dims 32 c + n
 *                  (low nibble of the byte) and 32 c + 16 + n (high nibble);
 *     [3072, 4096) value high nibbles, same arrangement;
 *     [4096, 4160) key   (scale, zero) fp16 pairs, 4 bytes per entry;
 *     [4160, 4224) value (scale, zero) fp16 pairs, 4 bytes per entry.
 *
 * 2-bit main cache (code_bits = 2; KV4-RL, "Future Directions": caches below
 * 4 bits under the same sink / recent protection).  Same quantization with
 * qmax = 3; same pages, subblocks of 16 tokens and INT8 side cache.  Subblock j
 * of (page, kv_head) starts at byte ((page * num_kv_heads + kv_head) * (P/16) + j) * 1152:
 *     [   0,  512) key codes: the 8 bytes at (G * 16 + t) * 8 hold token t's
 *                  rotated dims 32 G .. 32 G + 31 (G = 0..3); within dword w
 *                  (dims 32 G + 16 w + i, i = 0..15) byte {0, 2, 1, 3}[i / 4]
 *                  holds dim i in bits 2 (i % 4) .. 2 (i % 4) + 1;
 *     [ 512, 1024) value codes: dword (G * 16 + n) * 2 + cc (G = t / 4),
 *                  byte r = token 4 G + r, bits 2 f .. 2 f + 1 = value dim
 *                  n + 16 f + 64 cc (n = 0..15, cc = 0..1, f = 0..3);
 *     [1024, 1088) key   (scale, zero) fp16 pairs, 4 bytes per token;
 *     [1088, 1152) value (scale, zero) fp16 pairs, 4 bytes per token.
 *   1152 bytes / (16 tokens * 256 elements) = 2.25 bits per element.
 *
 * 3-bit main cache (code_bits = 3; the same "Future Directions" item).  qmax = 7;
 * subblock j starts at byte ((page * num_kv_heads + kv_head) * (P/16) + j) * 1664:
 *     [   0,  512) the low two bits of every key code, in the 2-bit key layout;
 *     [ 512, 1024) the low two bits of every value code, in the 2-bit value layout;
 *     [1024, 1280) key high bits: dword G * 16 + t holds token t's dims
 *                  32 G .. 32 G + 31; the dim in 2-bit dword w, byte b, bits
 *                  2 f .. 2 f + 1 has its bit 2 at bit
 *                  16 (b / 2) + 4 f + (w == 0 ? 2 : 0) + (b % 2);
 *     [1280, 1536) value high bits: dword G * 16 + n, byte r = token 4 G + r;
 *                  dim n + 16 f + 64 cc has its bit 2 at bit {2, 6, 3, 7}[f]
 *                  (cc = 0) or {0, 4, 1, 5}[f] (cc = 1) of the byte;
 *     [1536, 1600) key   (scale, zero) fp16 pairs, 4 bytes per token;
 *     [1600, 1664) value (scale, zero) fp16 pairs, 4 bytes per token.
 *   1664 bytes / (16 tokens * 256 elements) = 3.25 bits per element.
 *
 *   kv_quant_append, kv_decode_attn, kv_append_decode_attn and kv_prefill_attn
 *   serve all three widths.
 *
 * Keys with a bit width per RoPE-block group (key_bits; RoPE-Aware Bit
 * Allocation for KV-Cache Quantization, Abstract: integer bit widths per RoPE
 * frequency block, served from a packed cache; the allocation is the caller's).
 *   Groups: rotated key dim d belongs to group (d mod 32) / 8, so group j holds
 *   the rotate-half RoPE blocks (f, f + 64) with f in 8 j .. 8 j + 7 and
 *   32 + 8 j .. 32 + 8 j + 7; key_bits[j] in {2, 3, 4}.  Unless all four widths
 *   are equal, had_block must be at most 8 so that each Hadamard block stays
 *   inside one group.
 *   Quantization of the main-cache keys: the per-token U = fp16(fp32(mx - mn) /
 *   15) and Z = fp16(mn) of the 4-bit cache; a dim of width b has m = 2^(4 - b),
 *   o = (m - 1) / 2, Z_b = fp32(Z + o U), code = 0 if U == 0, else
 *   clamp(rint(fp32(fp32(y - Z_b) / (m U))), 0, 2^b - 1); dequantized
 *   y = Z + U (o + m code).  Widths (4, 4, 4, 4) give the 4-bit codes exactly.
 *   Values keep code_bits; the INT8 side cache does not change.
 *   Subblock of 16 tokens (KA = 64 (key_bits[0] + .. + key_bits[3]); VA = 1024,
 *   768 or 512 for 4-, 3- or 2-bit values; subblock bytes KA + VA + 128):
 *     [0, KA) key codes, group j at O_j = 64 (key_bits[0] + .. + key_bits[j-1]);
 *       slot s = 16 G + t (G = 0..3, token t) holds dims 32 G + 8 j + e, e = 0..7:
 *       width 4: bytes O_j + 4 s + k hold dims 2k (low nibble), 2k + 1 (high);
 *       width 2: bytes O_j + 2 s + k hold dims 4k + f at bits 2f .. 2f + 1;
 *       width 3: the low two bits as width 2, then byte O_j + 128 + s holds
 *                bit 2 of dim e's code at bit e;
 *     [KA, KA + VA) value codes in the code_bits value layout above (3 bits:
 *       the 2-bit value layout of the low bits, then the value high plane);
 *     [KA + VA, + 64) key (U, Z) fp16 pairs, [KA + VA + 64, + 64) value
 *       (scale, zero) fp16 pairs, 4 bytes per token.
 *   kv_quant_append and kv_decode_attn serve grouped keys for query groups up
 *   to 8; kv_append_decode_attn and kv_prefill_attn return KVQ_ERR_UNSUPPORTED.
 *
 * Block table: int32 [num_slots][bt_stride], row = slot; entry i is the page
 * holding positions [i P, (i + 1) P) of that slot's sequence.  Only entries
 * i < ceil(L / P) are read.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_NULL = 1,        /* a required pointer is NULL                        */
    KVQ_ERR_SHAPE = 2,       /* sizes are inconsistent or out of range            */
    KVQ_ERR_UNSUPPORTED = 3, /* valid request outside what is implemented         */
    KVQ_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required           */
    KVQ_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed        */
} kvq_status;

typedef struct {
    int32_t num_kv_heads;    /* >= 1                                              */
    int32_t head_dim;        /* must be 128                                       */
    int32_t page_size;       /* tokens per page: a power of two >= 16             */
    int32_t num_pages;       /* pages in int4_pool; num_pages * num_kv_heads *
                                page_size / 16 < 2^32 (subblocks of the pool)     */
    int32_t num_slots;       /* sequence slots (rows of the block table / INT8);
                                num_slots * num_kv_heads * ceil((sink + recent)
                                / 16) < 2^32                                      */
    int32_t had_block;       /* Hadamard block size h: power of two in [1, 128]   */
    int32_t sink;            /* s >= 0                                            */
    int32_t recent;          /* w >= 0                                            */
    void *int4_pool;         /* device, kvq_int4_pool_bytes(cache) bytes          */
    void *int8_pool;         /* device, kvq_int8_pool_bytes(cache) bytes; may be
                                NULL only when sink + recent == 0                 */
    int32_t code_bits;       /* width of the main (paged) cache's codes: 4, or 3
                                or 2 for the sub-4-bit caches (0 means 4).  The
                                INT8 side cache is the same for all.              */
    int32_t key_bits[4];     /* all 0: keys take code_bits.  Otherwise the width
                                of each RoPE-block group of the main-cache keys,
                                each in {2, 3, 4} (values keep code_bits)         */
} kvq_cache;

/* Bytes of the INT4 pool / INT8 side cache for this descriptor (0 on bad input). */
size_t kvq_int4_pool_bytes(const kvq_cache *cache);
size_t kvq_int8_pool_bytes(const kvq_cache *cache);

/*
 * kv_quant_append -- quantize T new (token, all KV heads) key/value vectors and
 * append them (KV4-RL, "Methodology in Plain English": every new K/V vector is
 * quantized on the fly; SAW-INT4 section 2: rotation and quantization fused).
 *
 *   k, v        bf16 [T][num_kv_heads][128], row-major (device).
 *   slot        int32 [T]: slot of each token's sequence (device).
 *   pos         int32 [T]: position of each token in its sequence (device).
 *   T           number of tokens; T == 0 is a no-op returning KVQ_OK.
 *   block_table int32 [num_slots][bt_stride] (device).
 *   len_after   int32 [num_slots]: sequence length of each slot after this call
 *               (device); only entries of slots named in `slot` are read.
 *
 * Positions within one call must be distinct per slot.  Each (token, head)
 * has exactly one writer; tokens of different calls on one stream are
 * ordered by the stream.
 *
 * Input domain: the stored scale and offset are fp16, so every quantized
 * vector y (the rotated key, the value) must have |min y| <= 65504 and
 * (max y - min y) / qmax <= 65504 (qmax = 15, 7 or 3 for the main cache, 255
 * for the INT8 copy); with the rotation |y_i| <= sqrt(h) * max |k|, so keys
 * with |k_i| <= 65504 / sqrt(h) are always inside.  Outside the domain the
 * offset or scale is stored as +-inf and the token's dequantized values are
 * not finite (no error is reported: device data is not checked).  NaN or Inf
 * inputs are outside the domain as well.
 */
kvq_status kv_quant_append(const kvq_cache *cache,
                           const uint16_t *k, const uint16_t *v,
                           const int32_t *slot, const int32_t *pos, int32_t T,
                           const int32_t *block_table, int32_t bt_stride,
                           const int32_t *len_after, void *stream);

/* Workspace bytes kv_decode_attn and kv_append_decode_attn need for B rows and
 * num_q_heads query heads on the current HIP device (0 on bad input). */
size_t kv_decode_attn_workspace_bytes(const kvq_cache *cache, int32_t B, int32_t num_q_heads);

/*
 * kv_decode_attn -- one decode step of attention for B rows (KV4-RL, "Key
 * Contributions" item 4: disjoint INT4 and INT8 regions combined through
 * regional softmax statistics; "Methodology in Plain English": queries are
 * rotated to match the rotated keys, packed codes are consumed directly and
 * scale/offset are applied after the dot-product reduction).
 *
 *   q            bf16 [B][num_q_heads][128] (device), unrotated.
 *   num_q_heads  multiple of num_kv_heads, group g = num_q_heads / num_kv_heads
 *                with 1 <= g <= 16; query head j uses KV head j / g.
 *   slot         int32 [B] (device): slot of each row.
 *   block_table  int32 [num_slots][bt_stride] (device).
 *   ctx_len      int32 [B] (device): context length L of each row, counting any
 *                token appended this step; 0 <= L <= bt_stride * page_size.
 *   out          fp32 [B][num_q_heads][128] (device): softmax(q.k / sqrt(128)) v.
 *                Rows with L == 0 get 0.
 *   lse          fp32 [B][num_q_heads] (device) or NULL: natural-log
 *                log-sum-exp of the scaled scores; -inf when L == 0.
 *   workspace    device scratch of at least kv_decode_attn_workspace_bytes();
 *                contents need no initialization and are overwritten.  Calls
 *                sharing one workspace must be ordered (same stream).
 */
kvq_status kv_decode_attn(const kvq_cache *cache,
                          const uint16_t *q, int32_t num_q_heads,
                          const int32_t *slot, const int32_t *block_table, int32_t bt_stride,
                          const int32_t *ctx_len, int32_t B,
                          float *out, float *lse,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_decode_read_ceiling -- a measurement, not part of the method: the memory
 * traffic of kv_decode_attn without its arithmetic.  Same arguments as
 * kv_decode_attn minus out and lse; the same work split over the same number
 * of waves, the same block-table gathers, direct-to-LDS step copies, waits
 * and LDS reads, so it reads every byte kv_decode_attn reads, in the same
 * order, and computes and writes nothing (the workspace header may be
 * touched).  Its duration is the bandwidth this access pattern reaches on the
 * device: a ceiling to put kv_decode_attn's own against.  Query groups up to 8
 * (KVQ_ERR_UNSUPPORTED above).
 */
kvq_status kv_decode_read_ceiling(const kvq_cache *cache,
                                  const uint16_t *q, int32_t num_q_heads,
                                  const int32_t *slot,
                                  const int32_t *block_table, int32_t bt_stride,
                                  const int32_t *ctx_len, int32_t B,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_decode_attn_noalloc -- kv_decode_attn without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * kernels and results as kv_decode_attn; the workspace is a static device
 * array of KVQ_NOALLOC_SCRATCH_BYTES that the library's code object holds on
 * every device it runs on until the process ends.  The call allocates and frees
 * nothing.
 *
 *   Limit: B rows of num_q_heads heads fit when kv_decode_attn_workspace_bytes
 *   (cache, B, num_q_heads) <= KVQ_NOALLOC_SCRATCH_BYTES (e.g. 256 rows of 32
 *   query heads over 8 KV heads need about 9 MB, 512 such rows about 13 MB);
 *   larger requests return KVQ_ERR_WORKSPACE and enqueue nothing.
 *   Every call on one device shares that device's array: calls that can run
 *   at the same time on one device (different streams, or host threads with
 *   no ordering between their streams) race and give wrong results; calls on
 *   one stream are ordered and safe.  Nothing in the array needs clearing
 *   between calls (each launch writes what it later reads).
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
kvq_status kv_decode_attn_noalloc(const kvq_cache *cache,
                                  const uint16_t *q, int32_t num_q_heads,
                                  const int32_t *slot,
                                  const int32_t *block_table, int32_t bt_stride,
                                  const int32_t *ctx_len, int32_t B,
                                  float *out, float *lse, void *stream);

/*
 * kv_append_decode_attn -- one decode step with the append fused in: every
 * row b with ctx_len[b] >= 1 first appends its new token (key k[b], value
 * v[b]) at position ctx_len[b] - 1 of slot[b], quantized exactly as
 * kv_quant_append does, then attends q[b] over positions [0, ctx_len[b]), in
 * one pass over the cache (KV4-RL, "Methodology in Plain English": new K/V
 * vectors are quantized on the fly inside the decode pipeline; "Key
 * Contributions" item 4 for the attention).
 *
 * The cache bytes written and out / lse are the same as those of
 * kv_quant_append(k, v, slot, pos = ctx_len - 1, T = B, len_after[slot[b]] =
 * ctx_len[b]) followed by kv_decode_attn on the same stream (out / lse within
 * float rounding of the split order; bit-identical when both kernels use the
 * same number of workers).
 *
 *   k, v         bf16 [B][num_kv_heads][128] (device): the token each row
 *                appends; rows with ctx_len == 0 append nothing.
 *   slot         int32 [B] (device): distinct slots (each row owns its slot).
 *   block_table  must map position ctx_len[b] - 1 of each row to its page.
 *   the other arguments are those of kv_decode_attn; the workspace size is
 *   kv_decode_attn_workspace_bytes(), which covers both entry points.
 */
kvq_status kv_append_decode_attn(const kvq_cache *cache,
                                 const uint16_t *k, const uint16_t *v,
                                 const uint16_t *q, int32_t num_q_heads,
                                 const int32_t *slot, const int32_t *block_table, int32_t bt_stride,
                                 const int32_t *ctx_len, int32_t B,
                                 float *out, float *lse,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * kv_prefill_attn -- causal attention of a chunk of query rows per sequence
 * over the quantized cache: chunked prefill, or the re-prefill of in-flight
 * rollouts after a policy update (KV4-RL, "Future Directions"), reading the
 * packed codes with the rotated query as decode attention does (KV4-RL,
 * "Methodology in Plain English").
 *
 *   q            bf16 [N][num_q_heads][128] (device), unrotated; rows of
 *                sequence b are q_start[b] .. q_start[b + 1] - 1.
 *   q_start      int32 [B + 1] (device), non-decreasing, q_start[0] = 0,
 *                q_start[B] = N.  T_b = q_start[b + 1] - q_start[b] must satisfy
 *                T_b <= max_rows and T_b <= ctx_len[b].
 *   max_rows     host int: an upper bound on every T_b (sizes the launch).
 *   slot, block_table, bt_stride, ctx_len, B: as for kv_decode_attn.  ctx_len
 *                counts the chunk, whose keys/values must already be in the
 *                cache (kv_quant_append with len_after = ctx_len).
 *   out          fp32 [N][num_q_heads][128] (device): row t of sequence b sits
 *                at position p = ctx_len[b] - T_b + t and gets
 *                softmax(q.k / sqrt(128)) v over positions [0, p], each key and
 *                value as the cache holds it at length ctx_len[b] (the INT8
 *                copy for the sinks and the last `recent` positions, the main
 *                cache of code_bits 4, 3 or 2 elsewhere).  Its last row equals
 *                kv_decode_attn's output.
 *   lse          fp32 [N][num_q_heads] (device) or NULL.
 *
 * No workspace.  Returns KVQ_OK without launching when B == 0 or max_rows == 0.
 * B and num_kv_heads must not exceed 65535.  A cache with grouped key widths
 * (key_bits) returns KVQ_ERR_UNSUPPORTED.
 */
kvq_status kv_prefill_attn(const kvq_cache *cache,
                           const uint16_t *q, int32_t num_q_heads,
                           const int32_t *q_start, int32_t max_rows,
                           const int32_t *slot, const int32_t *block_table, int32_t bt_stride,
                           const int32_t *ctx_len, int32_t B,
                           float *out, float *lse, void *stream);

/* Static description of a status code. */
const char *kvq_status_string(kvq_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
