// Per-token quantizer shared by the quantize-append kernel and the fused
// append + decode path, so both produce the same codes bit for bit.
//
// KV4-RL, "Methodology in Plain English": one affine group per 128-dim
// token-head vector with FP16 scale and offset; keys are stored rotated.
// SAW-INT4, section 2: block-diagonal Hadamard rotation with block size h.
//
// One wave64 handles one (token, KV head).  Lane l holds key dims 2l, 2l+1 (the
// natural order for the butterflies) and value dims n + 32c and n + 16 + 32c
// (n = l % 16, c = l / 16), which is the byte the value layout wants.
#pragma once

#include <hip/hip_fp16.h>

#include "common.h"
#include "lanes.h"

namespace kvq {

__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Scale / zero of a vector with extrema mn, mx for qmax levels (fp32 decisions,
// IEEE division, round-to-nearest-even to fp16).
struct QParams {
    __half sh, zh;
    float sf, zf;
};

__device__ inline QParams qparams(float mn, float mx, float qmax) {
#pragma clang fp contract(off)
    QParams p;
    float range = mx - mn;
    float scale_f = __fdiv_rn(range, qmax);
    p.sh = __float2half_rn(scale_f);
    p.zh = __float2half_rn(mn);
    p.sf = __half2float(p.sh);
    p.zf = __half2float(p.zh);
    return p;
}

__device__ inline uint32_t qcode(float y, const QParams &p, float qmax) {
#pragma clang fp contract(off)
    if (p.sf == 0.0f) return 0u;
    float t = __fdiv_rn(y - p.zf, p.sf);
    float r = rintf(t);
    r = fminf(fmaxf(r, 0.0f), qmax);
    return (uint32_t)r;
}

__device__ inline uint32_t qparam_word(const QParams &p) {
    return (uint32_t)__half_as_ushort(p.sh) | ((uint32_t)__half_as_ushort(p.zh) << 16);
}

// Codes and params of one (token, KV head) in both caches.
struct TokenCodes {
    uint8_t k4, v4;             // this lane's INT4 bytes (key dims 2l, 2l+1; value dims n+32c, n+16+32c)
    uint8_t k8lo, k8hi;         // INT8 key codes split into nibble planes
    uint8_t v8lo, v8hi;
    uint32_t kp4, vp4, kp8, vp8; // (scale, zero) fp16 pairs, wave-uniform
};

// kw: this lane's bf16 pair of key dims 2l, 2l+1; vlo, vhi: its value dims
// n + 32c and n + 16 + 32c (bf16 bits).
__device__ inline TokenCodes quantize_token(uint32_t kw, uint32_t vlo, uint32_t vhi, int h, float inv_sqrt_h,
                                            int lane) {
#pragma clang fp contract(off)
    // ---- keys: fp32 block Hadamard, strides 1, 2, ..., h/2 ascending --------
    float x0 = bf16_to_f32(kw & 0xFFFFu);
    float x1 = bf16_to_f32(kw >> 16);
    if (h >= 2) {
        float s0 = x0 + x1;
        float d0 = x0 - x1;
        x0 = s0;
        x1 = d0;
    }
    // element distance len = 2, 4, ..., 64 is lane distance len / 2
    if (h > 2) { x0 = butterfly<1>(x0, lane); x1 = butterfly<1>(x1, lane); }
    if (h > 4) { x0 = butterfly<2>(x0, lane); x1 = butterfly<2>(x1, lane); }
    if (h > 8) { x0 = butterfly<4>(x0, lane); x1 = butterfly<4>(x1, lane); }
    if (h > 16) { x0 = butterfly<8>(x0, lane); x1 = butterfly<8>(x1, lane); }
    if (h > 32) { x0 = butterfly<16>(x0, lane); x1 = butterfly<16>(x1, lane); }
    if (h > 64) { x0 = butterfly<32>(x0, lane); x1 = butterfly<32>(x1, lane); }
    x0 = x0 * inv_sqrt_h;
    x1 = x1 * inv_sqrt_h;
    const float kmn = wave_min(fminf(x0, x1));
    const float kmx = wave_max(fmaxf(x0, x1));
    // ---- values (not rotated) ------------------------------------------------
    const float v0 = bf16_to_f32(vlo);
    const float v1 = bf16_to_f32(vhi);
    const float vmn = wave_min(fminf(v0, v1));
    const float vmx = wave_max(fmaxf(v0, v1));
    TokenCodes t;
    {
        const QParams kp = qparams(kmn, kmx, 15.0f);
        const QParams vp = qparams(vmn, vmx, 15.0f);
        t.k4 = (uint8_t)(qcode(x0, kp, 15.0f) | (qcode(x1, kp, 15.0f) << 4));
        t.v4 = (uint8_t)(qcode(v0, vp, 15.0f) | (qcode(v1, vp, 15.0f) << 4));
        t.kp4 = qparam_word(kp);
        t.vp4 = qparam_word(vp);
    }
    {
        const QParams kp = qparams(kmn, kmx, 255.0f);
        const QParams vp = qparams(vmn, vmx, 255.0f);
        const uint32_t k0 = qcode(x0, kp, 255.0f), k1 = qcode(x1, kp, 255.0f);
        t.k8lo = (uint8_t)((k0 & 15u) | ((k1 & 15u) << 4));
        t.k8hi = (uint8_t)((k0 >> 4) | ((k1 >> 4) << 4));
        const uint32_t c0 = qcode(v0, vp, 255.0f), c1 = qcode(v1, vp, 255.0f);
        t.v8lo = (uint8_t)((c0 & 15u) | ((c1 & 15u) << 4));
        t.v8hi = (uint8_t)((c0 >> 4) | ((c1 >> 4) << 4));
        t.kp8 = qparam_word(kp);
        t.vp8 = qparam_word(vp);
    }
    return t;
}

// Byte offsets inside an INT4 subblock / INT8 ring subblock of token (entry)
// tok's data held by this lane.
__device__ inline int sub_k_byte(int tok, int lane) { return tok * 64 + lane; }
__device__ inline int sub_v_byte(int tok, int lane) {
    const int G = tok >> 2, r = tok & 3, vn = lane & 15, vc = lane >> 4;
    return 4 * ((G * 16 + vn) * 4 + vc) + r;
}

// Stores of one token into an INT4 subblock and (when write8) an INT8 ring subblock.
__device__ inline void store_token(const TokenCodes &t, uint8_t *base4, int tok, uint8_t *base8, int ee, bool write8,
                                   int lane) {
    base4[kSub4K + sub_k_byte(tok, lane)] = t.k4;
    base4[kSub4V + sub_v_byte(tok, lane)] = t.v4;
    if (lane == 0) {
        *reinterpret_cast<uint32_t *>(base4 + kSub4KP + 4 * tok) = t.kp4;
        *reinterpret_cast<uint32_t *>(base4 + kSub4VP + 4 * tok) = t.vp4;
    }
    if (write8) {
        // low / high nibble planes, each in the INT4 subblock layout
        base8[kSub8KLo + sub_k_byte(ee, lane)] = t.k8lo;
        base8[kSub8KHi + sub_k_byte(ee, lane)] = t.k8hi;
        base8[kSub8VLo + sub_v_byte(ee, lane)] = t.v8lo;
        base8[kSub8VHi + sub_v_byte(ee, lane)] = t.v8hi;
        if (lane == 0) {
            *reinterpret_cast<uint32_t *>(base8 + kSub8KP + 4 * ee) = t.kp8;
            *reinterpret_cast<uint32_t *>(base8 + kSub8VP + 4 * ee) = t.vp8;
        }
    }
}

}  // namespace kvq
