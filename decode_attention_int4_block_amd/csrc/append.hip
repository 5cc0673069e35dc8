// Quantize-append kernel: block-diagonal Hadamard rotation of keys, per-token
// asymmetric INT4 quantization of keys and values, packed into the paged INT4
// cache, plus the INT8 side-cache copy of sink and recent positions.
//
// KV4-RL, "Methodology in Plain English": each new K/V vector is quantized on
// the fly into one affine group per 128-dim token-head vector with FP16 scale
// and offset; keys are stored Hadamard-rotated.  SAW-INT4, section 2: the
// rotation is block-diagonal with block size h and is fused with quantization
// in one kernel.  The side cache holds sinks and the recent window (KV4-RL,
// "Key Contributions" item 4).
//
// One wave64 handles one (token, KV head).  Lane l holds key dims 2l, 2l+1 (the
// natural order for the butterflies) and value dims n + 32c and n + 16 + 32c
// (n = l % 16, c = l / 16), which is the byte the value layout wants.
#include <hip/hip_fp16.h>

#include "common.h"

namespace kvq {


__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ inline float wave_min(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

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

__global__ __launch_bounds__(256) void quant_append_kernel(AppendArgs a) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)a.T * a.H) return;
    const int t = (int)(item / a.H);
    const int hk = (int)(item % a.H);

    const int slot = a.slot[t];
    const int p = a.pos[t];
    const int page = a.block_table[(int64_t)slot * a.bt_stride + p / a.P];
    const int row = p % a.P;
    const int sub = row >> 4;
    const int tok = row & 15;
    uint8_t *base4 = a.int4_pool +
        ((size_t)((int64_t)page * a.H + hk) * (a.P / kSub) + sub) * kSub4Bytes;

    const uint16_t *krow = a.k + item * kHeadDim;
    const uint16_t *vrow = a.v + item * kHeadDim;

    // ---- keys: fp32 block Hadamard, strides 1, 2, ..., h/2 ascending --------
    const uint32_t kw = reinterpret_cast<const uint32_t *>(krow)[lane];
    float x0 = bf16_to_f32(kw & 0xFFFFu);
    float x1 = bf16_to_f32(kw >> 16);
    if (a.h >= 2) {
        float s0 = x0 + x1;
        float d0 = x0 - x1;
        x0 = s0;
        x1 = d0;
    }
    for (int len = 2; len < a.h; len <<= 1) {
        const int ls = len >> 1;                 // lane distance of elements len apart
        const float p0 = __shfl_xor(x0, ls, 64);
        const float p1 = __shfl_xor(x1, ls, 64);
        const bool upper = (lane & ls) != 0;
        x0 = upper ? (p0 - x0) : (x0 + p0);
        x1 = upper ? (p1 - x1) : (x1 + p1);
    }
    x0 = x0 * a.inv_sqrt_h;
    x1 = x1 * a.inv_sqrt_h;

    const float kmn = wave_min(fminf(x0, x1));
    const float kmx = wave_max(fmaxf(x0, x1));

    // ---- values (not rotated) ------------------------------------------------
    const int vn = lane & 15, vc = lane >> 4;
    const int vd0 = 32 * vc + vn;
    const float v0 = bf16_to_f32(vrow[vd0]);
    const float v1 = bf16_to_f32(vrow[vd0 + 16]);
    const float vmn = wave_min(fminf(v0, v1));
    const float vmx = wave_max(fmaxf(v0, v1));

    // ---- INT4 main cache -----------------------------------------------------
    {
        const QParams kp = qparams(kmn, kmx, 15.0f);
        const QParams vp = qparams(vmn, vmx, 15.0f);
        const uint32_t kb = qcode(x0, kp, 15.0f) | (qcode(x1, kp, 15.0f) << 4);
        const uint32_t vb = qcode(v0, vp, 15.0f) | (qcode(v1, vp, 15.0f) << 4);
        base4[kSub4K + tok * 64 + lane] = (uint8_t)kb;
        const int G = tok >> 2, r = tok & 3;
        base4[kSub4V + 4 * ((G * 16 + vn) * 4 + vc) + r] = (uint8_t)vb;
        if (lane == 0) {
            *reinterpret_cast<uint32_t *>(base4 + kSub4KP + 4 * tok) = qparam_word(kp);
            *reinterpret_cast<uint32_t *>(base4 + kSub4VP + 4 * tok) = qparam_word(vp);
        }
    }

    // ---- INT8 side cache: sinks and the final recent window ------------------
    const int L_after = a.len_after[slot];
    const bool write8 = (p < a.s) || (p >= L_after - a.w);
    if (write8 && (a.s + a.w) > 0) {
        const int e = p < a.s ? p : a.s + (p - a.s) % a.w;
        const int esub = e >> 4, ee = e & 15;
        uint8_t *base8 = a.int8_pool +
            ((size_t)((int64_t)slot * a.H + hk) * a.nr8 + esub) * kSub8Bytes;
        const QParams kp = qparams(kmn, kmx, 255.0f);
        const QParams vp = qparams(vmn, vmx, 255.0f);
        // low / high nibble planes, each in the INT4 subblock layout
        const uint32_t k0 = qcode(x0, kp, 255.0f), k1 = qcode(x1, kp, 255.0f);
        base8[kSub8KLo + ee * 64 + lane] = (uint8_t)((k0 & 15u) | ((k1 & 15u) << 4));
        base8[kSub8KHi + ee * 64 + lane] = (uint8_t)((k0 >> 4) | ((k1 >> 4) << 4));
        const uint32_t c0 = qcode(v0, vp, 255.0f), c1 = qcode(v1, vp, 255.0f);
        const int G = ee >> 2, r = ee & 3;
        const int vo = 4 * ((G * 16 + vn) * 4 + vc) + r;
        base8[kSub8VLo + vo] = (uint8_t)((c0 & 15u) | ((c1 & 15u) << 4));
        base8[kSub8VHi + vo] = (uint8_t)((c0 >> 4) | ((c1 >> 4) << 4));
        if (lane == 0) {
            *reinterpret_cast<uint32_t *>(base8 + kSub8KP + 4 * ee) = qparam_word(kp);
            *reinterpret_cast<uint32_t *>(base8 + kSub8VP + 4 * ee) = qparam_word(vp);
        }
    }
}

hipError_t launch_quant_append(const AppendArgs &a, hipStream_t stream) {
    const int64_t items = (int64_t)a.T * a.H;
    const int64_t blocks = (items + 3) / 4;
    hipLaunchKernelGGL(quant_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
