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

// Code of a key dim whose RoPE-block group has width b (grouped keys): the
// step is 2^(4 - b) U and the levels are centred in the 4-bit span, so Z_b =
// Z + (2^(4 - b) - 1) U / 2 (p holds U and Z, the 4-bit params).
__device__ inline uint32_t gcode(float y, const QParams &p, int b) {
#pragma clang fp contract(off)
    if (p.sf == 0.0f) return 0u;
    const float m = (float)(1 << (4 - b));
    const float o = (m - 1.0f) * 0.5f;
    const float zb = p.zf + o * p.sf;
    float t = __fdiv_rn(y - zb, m * p.sf);
    float r = rintf(t);
    r = fminf(fmaxf(r, 0.0f), (float)((1 << b) - 1));
    return (uint32_t)r;
}

__device__ inline uint32_t qparam_word(const QParams &p) {
    return (uint32_t)__half_as_ushort(p.sh) | ((uint32_t)__half_as_ushort(p.zh) << 16);
}

// Codes and params of one (token, KV head) in both caches.
struct TokenCodes {
    uint8_t k4, v4;             // this lane's main-cache codes as a nibble pair (key dims 2l, 2l+1;
                                // value dims n+32c, n+16+32c): the INT4 byte, or two 3- / 2-bit codes
    uint8_t k8lo, k8hi;         // INT8 key codes split into nibble planes
    uint8_t v8lo, v8hi;
    uint32_t kp4, vp4, kp8, vp8; // (scale, zero) fp16 pairs, wave-uniform
};

// kw: this lane's bf16 pair of key dims 2l, 2l+1; vlo, vhi: its value dims
// n + 32c and n + 16 + 32c (bf16 bits).  qmain: levels - 1 of the main cache
// (15, or 7 / 3 for the 3- / 2-bit caches).
//
// kbits != 0: grouped keys, this lane's key dims having width kbits; the key
// params are then the 4-bit ones (U, Z) and the codes come from gcode.
__device__ inline TokenCodes quantize_token(uint32_t kw, uint32_t vlo, uint32_t vhi, int h, float inv_sqrt_h,
                                            int lane, float qmain = 15.0f, int kbits = 0) {
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
        const QParams kp = qparams(kmn, kmx, kbits ? 15.0f : qmain);
        const QParams vp = qparams(vmn, vmx, qmain);
        if (kbits)
            t.k4 = (uint8_t)(gcode(x0, kp, kbits) | (gcode(x1, kp, kbits) << 4));
        else
            t.k4 = (uint8_t)(qcode(x0, kp, qmain) | (qcode(x1, kp, qmain) << 4));
        t.v4 = (uint8_t)(qcode(v0, vp, qmain) | (qcode(v1, vp, qmain) << 4));
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

// 2-bit main cache.  Key codes of token t: 8 bytes at (G 16 + t) 8 for dims
// 32 G .. 32 G + 31; within dword w (dims 32 G + 16 w + j, j < 16) byte
// {0, 2, 1, 3}[j / 4] holds dim j in bits 2 (j % 4).  Value codes: dword
// (G 16 + n) 2 + cc of the value area, byte r = token 4 G + r, bits 2 f =
// dim n + 16 f + 64 cc.  A byte holds four codes, two from each of two lanes:
// the key byte of lanes l and l ^ 1, the value byte of lanes l and l ^ 16.
__device__ inline int sub2_k_byte(int tok, int lane) {
    const int q = ((2 * lane) & 15) >> 2;        // dims 2l, 2l+1 sit at 4 q + (0, 1) or (2, 3) of their dword
    return ((lane >> 4) * 16 + tok) * 8 + (((lane & 15) >> 3) << 2) + (((q & 1) << 1) | (q >> 1));
}
__device__ inline int sub2_v_byte(int tok, int lane) {
    const int G = tok >> 2, r = tok & 3, n = lane & 15, c = lane >> 4;
    return ((G * 16 + n) * 2 + (c >> 1)) * 4 + r;
}
// The byte this lane's pair of codes completes (valid in the lanes that store it).
__device__ inline uint32_t int2_key_byte(uint8_t nib2, int lane) {
    const uint32_t mine = ((nib2 & 3u) | (((uint32_t)nib2 >> 4) << 2)) << (4 * (lane & 1));
    return mine | (uint32_t)__shfl_xor((int)mine, 1, 64);
}
__device__ inline uint32_t int2_value_byte(uint8_t nib2, int lane) {
    const uint32_t mine = ((nib2 & 3u) | (((uint32_t)nib2 >> 4) << 2)) << (4 * ((lane >> 4) & 1));
    return mine | (uint32_t)__shfl_xor((int)mine, 16, 64);
}

// 3-bit main cache: the low two bits of each code go to the 2-bit layouts
// above; the high bits form two planes laid out for the decode kernel's
// 2-bit unpacking, each byte (key: each dword) holding a single token so that
// a token's stores touch no other token's bits.
//
// Key high plane: dword G 16 + t holds token t's dims 32 G .. 32 G + 31.  The
// dim in 2-bit dword w, byte b, field f (dims 32 G + 16 w + j, b = {0, 2, 1,
// 3}[j / 4], f = j % 4) sits at bit 16 (b / 2) + 4 f + (w ? 0 : 2) + (b % 2).
__device__ inline int int3_key_hibit(int within) {
    const int w = within >> 4, j = within & 15;
    const int b = (0x3120 >> (4 * (j >> 2))) & 3;       // {0, 2, 1, 3}[j / 4]
    return 16 * (b >> 1) + 4 * (j & 3) + (w ? 0 : 2) + (b & 1);
}
// Value high plane: dword G 16 + n, byte r = token 4 G + r; dim n + 16 f + 64 cc
// sits at bit {2, 6, 3, 7}[f] (cc = 0) or {0, 4, 1, 5}[f] (cc = 1) of the byte.
__device__ inline int int3_value_hibit(int cc, int f) {
    return cc == 0 ? (0x7362 >> (4 * f)) & 15 : (0x5140 >> (4 * f)) & 15;
}
// This lane's high bits (codes of nibble pair k4 / v4) placed in the key dword of
// its 32-dim group, and in the value byte of its value lane n.
__device__ inline uint32_t int3_key_hibits(uint8_t k4, int lane) {
    const int within = 2 * (lane & 15);
    return (((uint32_t)k4 >> 2) & 1u) << int3_key_hibit(within) |
           (((uint32_t)k4 >> 6) & 1u) << int3_key_hibit(within + 1);
}
__device__ inline uint32_t int3_value_hibits(uint8_t v4, int lane) {
    const int c = lane >> 4, cc = c >> 1;
    return (((uint32_t)v4 >> 2) & 1u) << int3_value_hibit(cc, (2 * c) & 3) |
           (((uint32_t)v4 >> 6) & 1u) << int3_value_hibit(cc, (2 * c + 1) & 3);
}

// One token's bytes in the 2- / 3-bit layouts, as this lane holds them: the
// 2-bit key byte (valid in even lanes) and value byte (lanes with bit 4
// clear), and at 3 bits the key high-plane dword (valid in lanes 16 G) and the
// value high-plane byte (lanes 0-15).  Call with the whole wave.
struct Sub2Token {
    uint32_t kb, vb, kh, vh;
};

template <int BITS>
__device__ inline Sub2Token sub2_token(const TokenCodes &t, int lane) {
    const uint8_t lo2 = BITS == 3 ? 0x33u : 0xFFu;     // at 3 bits the low planes take bits 0-1
    Sub2Token s;
    s.kb = int2_key_byte((uint8_t)(t.k4 & lo2), lane);
    s.vb = int2_value_byte((uint8_t)(t.v4 & lo2), lane);
    s.kh = s.vh = 0u;
    if constexpr (BITS == 3) {
        uint32_t kh = int3_key_hibits(t.k4, lane);
        kh |= (uint32_t)__shfl_xor((int)kh, 1, 64);
        kh |= (uint32_t)__shfl_xor((int)kh, 2, 64);
        kh |= (uint32_t)__shfl_xor((int)kh, 4, 64);
        kh |= (uint32_t)__shfl_xor((int)kh, 8, 64);
        uint32_t vh = int3_value_hibits(t.v4, lane);
        vh |= (uint32_t)__shfl_xor((int)vh, 16, 64);
        vh |= (uint32_t)__shfl_xor((int)vh, 32, 64);
        s.kh = kh;
        s.vh = vh;
    }
    return s;
}

// Places token tok (0-15) of a 2- / 3-bit subblock whose areas start at the
// given addresses: key and value low planes, (3 bits) key and value high
// planes, key and value params.  The same bytes go to the cache and to a
// stage copy of the subblock, whose areas sit elsewhere.
template <int BITS>
__device__ inline void put_sub2_token(const Sub2Token &s, const TokenCodes &t, uint8_t *k, uint8_t *v, uint8_t *kh,
                                      uint8_t *vh, uint8_t *kp, uint8_t *vp, int tok, int lane) {
    if ((lane & 1) == 0) k[sub2_k_byte(tok, lane)] = (uint8_t)s.kb;
    if (((lane >> 4) & 1) == 0) v[sub2_v_byte(tok, lane)] = (uint8_t)s.vb;
    if constexpr (BITS == 3) {
        if ((lane & 15) == 0) *reinterpret_cast<uint32_t *>(kh + 4 * ((lane >> 4) * 16 + tok)) = s.kh;
        if (lane < 16) vh[4 * ((tok >> 2) * 16 + lane) + (tok & 3)] = (uint8_t)s.vh;
    }
    if (lane == 0) {
        *reinterpret_cast<uint32_t *>(kp + 4 * tok) = t.kp4;
        *reinterpret_cast<uint32_t *>(vp + 4 * tok) = t.vp4;
    }
}

// Stores of one token into a 3-bit subblock.  Call with the whole wave.
__device__ inline void store_token_int3(const TokenCodes &t, uint8_t *base3, int tok, int lane) {
    put_sub2_token<3>(sub2_token<3>(t, lane), t, base3 + kSub3K, base3 + kSub3V, base3 + kSub3KH, base3 + kSub3VH,
                      base3 + kSub3KP, base3 + kSub3VP, tok, lane);
}

// Stores of one token into a 2-bit subblock.  Call with the whole wave.
__device__ inline void store_token_int2(const TokenCodes &t, uint8_t *base2, int tok, int lane) {
    put_sub2_token<2>(sub2_token<2>(t, lane), t, base2 + kSub2K, base2 + kSub2V, nullptr, nullptr, base2 + kSub2KP,
                      base2 + kSub2VP, tok, lane);
}

// Grouped keys: the RoPE-block group of this lane's key dims 2l, 2l + 1.
__device__ inline int key_group_of_lane(int lane) { return (lane & 15) >> 2; }

// Stores of one token into a grouped-key subblock (layout in include/kvq.h):
// this lane's key codes (dims e, e + 1 of slot 16 G + tok, e = 2 (l % 4)) at
// their group's width, the value codes at BITS (the value area starts at
// a.key_area), the params.  The key bytes of width 2 and 3 join the codes of
// two or four lanes by shuffles, so every lane must call it.
template <int BITS>
__device__ inline void store_token_grouped(const TokenCodes &t, uint8_t *base, int tok, int lane,
                                           const int32_t (&key_bits)[4], const int32_t (&kg_off)[4],
                                           int key_area) {
    const int j = key_group_of_lane(lane);
    const int b = j == 0 ? key_bits[0] : (j == 1 ? key_bits[1] : (j == 2 ? key_bits[2] : key_bits[3]));
    const int off = j == 0 ? kg_off[0] : (j == 1 ? kg_off[1] : (j == 2 ? kg_off[2] : kg_off[3]));
    const int s = 16 * (lane >> 4) + tok;
    const int k = lane & 3;
    const uint32_t c0 = t.k4 & 15u, c1 = (uint32_t)t.k4 >> 4;
    // two-bit fields of dims e, e + 1 in their byte (width 2 codes, or the low
    // bits of width 3), joined with the other lane of the byte
    uint32_t lo = (((c0 & 3u) | ((c1 & 3u) << 2)) << (4 * (k & 1)));
    lo |= (uint32_t)__shfl_xor((int)lo, 1, 64);
    // bit 2 of dims e, e + 1 at bits e, e + 1 of the slot's high byte
    uint32_t hi = (((c0 >> 2) & 1u) | (((c1 >> 2) & 1u) << 1)) << (2 * k);
    hi |= (uint32_t)__shfl_xor((int)hi, 1, 64);
    hi |= (uint32_t)__shfl_xor((int)hi, 2, 64);
    uint8_t *kg = base + off;
    if (b == 4) {
        kg[4 * s + k] = t.k4;
    } else {
        if ((k & 1) == 0) kg[2 * s + (k >> 1)] = (uint8_t)lo;
        if (b == 3 && k == 0) kg[128 + s] = (uint8_t)hi;
    }
    uint8_t *va = base + key_area;
    if constexpr (BITS == 4) {
        va[sub_v_byte(tok, lane)] = t.v4;
    } else {
        const Sub2Token s2 = sub2_token<BITS>(t, lane);
        if (((lane >> 4) & 1) == 0) va[sub2_v_byte(tok, lane)] = (uint8_t)s2.vb;
        if constexpr (BITS == 3) {
            if (lane < 16) va[512 + 4 * ((tok >> 2) * 16 + lane) + (tok & 3)] = (uint8_t)s2.vh;
        }
    }
    if (lane == 0) {
        uint8_t *pp = va + value_area_bytes(BITS);
        *reinterpret_cast<uint32_t *>(pp + 4 * tok) = t.kp4;
        *reinterpret_cast<uint32_t *>(pp + 64 + 4 * tok) = t.vp4;
    }
}

// INT8 ring copy of one token (when write8).
__device__ inline void store_token_int8(const TokenCodes &t, uint8_t *base8, int ee, int lane) {
    base8[kSub8KLo + sub_k_byte(ee, lane)] = t.k8lo;
    base8[kSub8KHi + sub_k_byte(ee, lane)] = t.k8hi;
    base8[kSub8VLo + sub_v_byte(ee, lane)] = t.v8lo;
    base8[kSub8VHi + sub_v_byte(ee, lane)] = t.v8hi;
    if (lane == 0) {
        *reinterpret_cast<uint32_t *>(base8 + kSub8KP + 4 * ee) = t.kp8;
        *reinterpret_cast<uint32_t *>(base8 + kSub8VP + 4 * ee) = t.vp8;
    }
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
