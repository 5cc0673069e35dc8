// Cross-lane helpers of one wave64 on gfx950: DPP moves inside 16-lane rows,
// permlane swaps across rows, butterflies and reductions built from them.
// No LDS traffic: every move is a VALU operation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// Cross-lane moves (VALU, no LDS).  DPP controls inside 16-lane rows:
// row_shl:n (lane i <- i + n), row_shr:n (lane i <- i - n), row_ror:n
// (lane i <- (i - n) mod 16); the bank mask selects which groups of 4 lanes of
// each row are written, the others keep `old`.
constexpr int kRowShl = 0x100, kRowShr = 0x110, kRowRor = 0x120;
// quad_perm controls: lane i of each group of 4 reads lane i ^ 1 / i ^ 2
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;

template <int CTRL, int BANKS = 0xF>
__device__ inline uint32_t dpp(uint32_t old, uint32_t src) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, 0xF, BANKS, false);
}
template <int CTRL, int BANKS = 0xF>
__device__ inline float dppf(float old, float src) {
    return __uint_as_float(dpp<CTRL, BANKS>(__float_as_uint(old), __float_as_uint(src)));
}

// (r0, r1) of permlane16_swap(a, b): rows [a0 b0 a2 b2] and [a1 b1 a3 b3].
__device__ inline void swap16(float a, float b, float &r0, float &r1) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    r0 = __uint_as_float(r[0]);
    r1 = __uint_as_float(r[1]);
}
// (r0, r1) of permlane32_swap(a, b): rows [a0 a1 b0 b1] and [a2 a3 b2 b3].
__device__ inline void swap32(float a, float b, float &r0, float &r1) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    r0 = __uint_as_float(r[0]);
    r1 = __uint_as_float(r[1]);
}

__device__ inline float max_rows(float x) {      // max over lanes l, l^16, l^32, l^48
    float r0, r1;
    swap32(x, x, r0, r1);
    x = fmaxf(r0, r1);
    swap16(x, x, r0, r1);
    return fmaxf(r0, r1);
}
__device__ inline float sum_rows(float x) {      // sum over lanes l, l^16, l^32, l^48
    float r0, r1;
    swap32(x, x, r0, r1);
    x = r0 + r1;
    swap16(x, x, r0, r1);
    return r0 + r1;
}

// Hadamard butterfly between lanes l and l ^ X: the lower lane ends with
// (its value) + (partner's), the upper with (partner's) - (its value).  Each
// result is one rounded add or subtract (the fma multiplies by +-1 exactly).
template <int X>
__device__ inline float butterfly(float x, int lane) {
    static_assert(X == 1 || X == 2 || X == 4 || X == 8 || X == 16 || X == 32, "lane distance");
    const float sgn = (lane & X) ? -1.0f : 1.0f;
    if constexpr (X == 16 || X == 32) {
        float r0, r1;
        if constexpr (X == 16) swap16(x, x, r0, r1);
        else swap32(x, x, r0, r1);
        // lower rows: r0 = own, r1 = partner; upper rows: r0 = partner, r1 = own
        return fmaf(r1, sgn, r0);
    } else {
        float p;
        if constexpr (X == 1) {
            p = dppf<kQuadXor1>(0.0f, x);
        } else if constexpr (X == 2) {
            p = dppf<kQuadXor2>(0.0f, x);
        } else if constexpr (X == 8) {
            p = dppf<kRowRor + 8>(0.0f, x);
        } else {
            p = dppf<kRowShl + X, 0x5>(x, x);        // banks 0, 2 read lane + 4
            p = dppf<kRowShr + X, 0xA>(p, x);        // banks 1, 3 read lane - 4
        }
        return fmaf(x, sgn, p);
    }
}

// Minimum / maximum over all 64 lanes: rotations by 8, 4, 2, 1 inside each
// 16-lane row, then across the four rows.  Every lane ends with the result.
__device__ inline float min_rows(float x) {      // min over lanes l, l^16, l^32, l^48
    float r0, r1;
    swap32(x, x, r0, r1);
    x = fminf(r0, r1);
    swap16(x, x, r0, r1);
    return fminf(r0, r1);
}
__device__ inline float wave_min(float x) {
    x = fminf(x, dppf<kRowRor + 8>(0.0f, x));
    x = fminf(x, dppf<kRowRor + 4>(0.0f, x));
    x = fminf(x, dppf<kRowRor + 2>(0.0f, x));
    x = fminf(x, dppf<kRowRor + 1>(0.0f, x));
    return min_rows(x);
}
__device__ inline float wave_max(float x) {
    x = fmaxf(x, dppf<kRowRor + 8>(0.0f, x));
    x = fmaxf(x, dppf<kRowRor + 4>(0.0f, x));
    x = fmaxf(x, dppf<kRowRor + 2>(0.0f, x));
    x = fmaxf(x, dppf<kRowRor + 1>(0.0f, x));
    return max_rows(x);
}

}  // namespace kvq
