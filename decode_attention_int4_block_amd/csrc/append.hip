// Quantize-append kernel: block-diagonal Hadamard rotation of keys, per-token
// asymmetric INT4 quantization of keys and values, packed into the paged INT4
// cache, plus the INT8 side-cache copy of sink and recent positions.
//
// KV4-RL, "Methodology in Plain English": each new K/V vector is quantized on
// the fly into one affine group per 128-dim token-head vector with FP16 scale
// and offset; keys are stored Hadamard-rotated.  SAW-INT4, section 2: the
// rotation is block-diagonal with block size h and is fused with quantization
// in one kernel.  The side cache holds sinks and the recent window (KV4-RL,
// "Key Contributions" item 4).  One wave64 per (token, KV head); the
// arithmetic is quantize_token in quant.h.
#include "quant.h"

namespace kvq {

// BITS: width of the main cache's codes, 4, 3 or 2 (the sub-4-bit caches of
// KV4-RL, "Future Directions", with the same INT8 sink / recent copies).
// KG: keys with a width per RoPE-block group (a.key_bits; RoPE-Aware Bit
// Allocation for KV-Cache Quantization, Abstract), values at BITS.
template <int BITS, bool KG = false>
__global__ __launch_bounds__(256) void quant_append_kernel(AppendArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)a.T * a.H) return;
    const int t = (int)(item / a.H);
    const int hk = (int)(item % a.H);

    const int slot = a.slot[t];
    const int p = a.pos[t];
    const int page = a.block_table[(int64_t)slot * a.bt_stride + p / a.P];
    const int row = p % a.P;
    const size_t sub_bytes = KG ? (size_t)a.sub_bytes : (size_t)main_sub_bytes(BITS);
    uint8_t *base4 = a.int4_pool + ((size_t)((int64_t)page * a.H + hk) * (a.P / kSub) + (row >> 4)) * sub_bytes;

    const uint16_t *krow = a.k + item * kHeadDim;
    const uint16_t *vrow = a.v + item * kHeadDim;
    const int vd0 = 32 * (lane >> 4) + (lane & 15);
    int kbits = 0;
    if constexpr (KG) {
        const int j = key_group_of_lane(lane);
        kbits = j == 0 ? a.key_bits[0] : (j == 1 ? a.key_bits[1] : (j == 2 ? a.key_bits[2] : a.key_bits[3]));
    }
    const TokenCodes tc = quantize_token(reinterpret_cast<const uint32_t *>(krow)[lane], vrow[vd0], vrow[vd0 + 16],
                                         a.h, a.inv_sqrt_h, lane, (float)((1 << BITS) - 1), kbits);

    // INT8 side cache: sinks and the final recent window
    const int L_after = a.len_after[slot];
    const bool write8 = ((p < a.s) || (p >= L_after - a.w)) && (a.s + a.w) > 0;
    const int e = p < a.s ? p : (a.w > 0 ? a.s + (p - a.s) % a.w : 0);
    uint8_t *base8 = write8 ? a.int8_pool + ((size_t)((int64_t)slot * a.H + hk) * a.nr8 + (e >> 4)) * kSub8Bytes
                            : nullptr;
    if constexpr (KG) {
        store_token_grouped<BITS>(tc, base4, row & 15, lane, a.key_bits, a.kg_off, a.key_area);
        if (write8) store_token_int8(tc, base8, e & 15, lane);
    } else if constexpr (BITS == 2) {
        store_token_int2(tc, base4, row & 15, lane);
        if (write8) store_token_int8(tc, base8, e & 15, lane);
    } else if constexpr (BITS == 3) {
        store_token_int3(tc, base4, row & 15, lane);
        if (write8) store_token_int8(tc, base8, e & 15, lane);
    } else {
        store_token(tc, base4, row & 15, base8, e & 15, write8, lane);
    }
}

hipError_t launch_quant_append(const AppendArgs &a, hipStream_t stream, bool grouped) {
    const int64_t items = (int64_t)a.T * a.H;
    const int64_t blocks = (items + 3) / 4;
    if (grouped) {
        if (a.bits == 2)
            hipLaunchKernelGGL((quant_append_kernel<2, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
        else if (a.bits == 3)
            hipLaunchKernelGGL((quant_append_kernel<3, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((quant_append_kernel<4, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    } else if (a.bits == 2)
        hipLaunchKernelGGL(quant_append_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else if (a.bits == 3)
        hipLaunchKernelGGL(quant_append_kernel<3>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(quant_append_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
