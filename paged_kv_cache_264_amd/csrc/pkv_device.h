// Device-side building blocks for gfx950 (CDNA4, wave64): element types,
// 16-byte vector access, DPP lane reductions.  Internal to libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// F8: 8-bit floating point e4m3 (OCP "E4M3FN", largest finite value 448),
// the format of gfx950's fp8 convert instructions.
// U4: 4-bit codes 0..15, two per byte (element 2i in the low nibble of byte
// i), with two fp32 values (x_min, x_max - x_min) per (slot, kv head) row.
enum class Elem : int { F32 = 0, F16 = 1, BF16 = 2, I8 = 3, F8 = 4, U4 = 5 };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

template <Elem E> struct ElemInfo;
template <> struct ElemInfo<Elem::F32> { static constexpr int bytes = 4, bits = 32; };
template <> struct ElemInfo<Elem::F16> { static constexpr int bytes = 2, bits = 16; };
template <> struct ElemInfo<Elem::BF16> { static constexpr int bytes = 2, bits = 16; };
template <> struct ElemInfo<Elem::I8> { static constexpr int bytes = 1, bits = 8; };
template <> struct ElemInfo<Elem::F8> { static constexpr int bytes = 1, bits = 8; };
template <> struct ElemInfo<Elem::U4> { static constexpr int bytes = 1, bits = 4; };  // bytes: rounded up

// caches of 1-byte codes with one fp32 scale per (slot, kv head)
constexpr bool is_scaled(Elem e) { return e == Elem::I8 || e == Elem::F8; }

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
}
__device__ __forceinline__ float bf2f(uint16_t bits) {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
}
// low / high 16-bit halves of a packed dword
__device__ __forceinline__ float lo_h(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float hi_h(uint32_t w) { return h2f((uint16_t)(w >> 16)); }
__device__ __forceinline__ float lo_bf(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// four e4m3 codes of a dword -> fp32 (exact), bytes 0..3 in order
__device__ __forceinline__ void f8x4_to_f32(uint32_t w, float& x0, float& x1, float& x2,
                                            float& x3) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    x0 = lo[0];
    x1 = lo[1];
    x2 = hi[0];
    x3 = hi[1];
}
// four fp32 values (|x| <= 448) -> e4m3 codes, round to nearest even, bytes 0..3
__device__ __forceinline__ uint32_t f32x4_to_f8(float x0, float x1, float x2, float x3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
    return (uint32_t)w;
}

// float -> storage with round-to-nearest-even
template <Elem E> __device__ __forceinline__ void store_elem(void* base, size_t i, float x);
template <> __device__ __forceinline__ void store_elem<Elem::F32>(void* base, size_t i, float x) {
    static_cast<float*>(base)[i] = x;
}
template <> __device__ __forceinline__ void store_elem<Elem::F16>(void* base, size_t i, float x) {
    static_cast<_Float16*>(base)[i] = (_Float16)x;
}
template <> __device__ __forceinline__ void store_elem<Elem::BF16>(void* base, size_t i, float x) {
    static_cast<__bf16*>(base)[i] = (__bf16)x;
}

template <Elem E> __device__ __forceinline__ float load_elem(const void* base, size_t i);
template <> __device__ __forceinline__ float load_elem<Elem::F32>(const void* base, size_t i) {
    return static_cast<const float*>(base)[i];
}
template <> __device__ __forceinline__ float load_elem<Elem::F16>(const void* base, size_t i) {
    return h2f(static_cast<const uint16_t*>(base)[i]);
}
template <> __device__ __forceinline__ float load_elem<Elem::BF16>(const void* base, size_t i) {
    return bf2f(static_cast<const uint16_t*>(base)[i]);
}

// ---------------------------------------------------------------------------
// DPP lane exchange (gfx9 encodings of the data-parallel-primitive control)
// ---------------------------------------------------------------------------
enum : int {
    kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]
    kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]
    kDppRowHalfMirror = 0x141, // lane i <-> 7-i inside each group of 8
    kDppRowMirror = 0x140,     // lane i <-> 15-i inside each row of 16
    kDppRowXor8 = 0x128,       // row_ror:8, i.e. lane i <-> i ^ 8 inside each row of 16
    kDppRowBcast = 0x150,      // + n: row_newbcast:n, lane n of each row of 16 to the whole row
};

// Every pattern used here gives each lane a source inside its own row, so
// the bound control (a lane without a source reads 0) never acts; it lets the
// compiler fold the lane move into the add that consumes it (one
// v_add_f32_dpp instead of a v_mov_b32_dpp and a v_add_f32).
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N a power of two, 1..64); every lane of
// the group receives the sum.  Inside a row of 16 the exchange uses DPP
// (quad xor 1 and 2, then half-row and row mirrors, which pair whole quads and
// whole half-rows once those hold uniform partial sums); wider groups use a
// cross-row xor shuffle.
template <int N> __device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

template <int N> __device__ __forceinline__ float group_max(float x) {
    if constexpr (N >= 2) x = fmaxf(x, dpp<kDppQuadXor1>(x));
    if constexpr (N >= 4) x = fmaxf(x, dpp<kDppQuadXor2>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp<kDppRowMirror>(x));
    if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16));
    if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
