// Quantizers of a cache row, shared by the kernels that store a quantized
// row (the cache write, and the matrix-core decode's new-token append), so
// that a stored row has the same bytes whichever kernel stored it.  A row of
// D elements is spread over LPR = D / 8 consecutive lanes, 8 elements each.
#pragma once
#include "pkv_device.h"

namespace pkv {

// Quantize 8 elements of a row (spread over LPR lanes); returns the packed
// codes and the row's scale.  INT8: s = amax / 127, codes
// clamp(rne(x / s), -127, 127).  FP8 e4m3: s = amax / 448, codes
// e4m3(clamp(x / s, -448, 448)) with the hardware's round-to-nearest-even
// convert.  Divisions are IEEE single precision.
template <Elem CE, int LPR>
__device__ __forceinline__ uint2 quantize8(const float (&x)[8], float& scale_out) {
    constexpr float kQmax = CE == Elem::F8 ? 448.0f : 127.0f;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = group_max<LPR>(amax);
    uint32_t packed[2] = {0u, 0u};
    float s = 0.f;
    if (amax > 0.f) {
        s = amax / kQmax;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                r[j] = x[4 * i + j] / s;
                if constexpr (CE == Elem::I8) r[j] = __builtin_rintf(r[j]);
                r[j] = fminf(fmaxf(r[j], -kQmax), kQmax);
            }
            if constexpr (CE == Elem::F8) {
                packed[i] = f32x4_to_f8(r[0], r[1], r[2], r[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    packed[i] |= ((uint32_t)(int32_t)r[j] & 0xffu) << (8 * j);
            }
        }
    }
    scale_out = s;
    return make_uint2(packed[0], packed[1]);
}

// 4-bit codes of 8 elements of a row (spread over LPR lanes) by the linear
// b-bit formula with b = 4 over the row's min and max: code = rne((x - min)
// / range * 15) clamped to [0, 15], range = max - min, each step in IEEE
// single precision; element 2i goes to the low nibble of byte i.
template <int LPR>
__device__ __forceinline__ uint32_t quantize8_u4(const float (&x)[8], float& lo_out,
                                                 float& range_out) {
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        lo = fminf(lo, x[i]);
        hi = fmaxf(hi, x[i]);
    }
    lo = -group_max<LPR>(-lo);
    hi = group_max<LPR>(hi);
    const float range = hi - lo;
    uint32_t w = 0u;
    if (range != 0.f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float r = __builtin_rintf((x[i] - lo) / range * 15.0f);
            r = fminf(fmaxf(r, 0.0f), 15.0f);
            w |= (uint32_t)r << (4 * i);
        }
    }
    lo_out = lo;
    range_out = range;
    return w;
}

}  // namespace pkv
