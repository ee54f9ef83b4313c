// Split-context single-query decode attention over a paged KV cache, for
// gfx950 (CDNA4, wave64).
//
// What is computed: for every sequence b and q head h,
//     out[b][h] = softmax(scale * q[b][h] . K^T) V
// over the sequence's cached tokens, which are fetched through its block table
// from 16-token blocks anywhere in the pool (docs.lazyllm.ai lesson 4,
// section 4.2: page table, global block pool, unchanged attention equation;
// "Efficient AI Lecture 13" notes, "PagedAttention" steps 1-4).  The context is
// cut into partitions of P tokens; each work-group reduces one partition with
// an online softmax (running max m, running sum l: caojiahao2.github.io
// section 3.2) and the partials are merged exactly afterwards.
//
// Mapping onto the hardware (decode streams every K/V byte exactly once, so
// the kernel is HBM bound; the design goal is many outstanding 16-byte loads
// per lane and little ALU work per byte):
//   * grid: one work-group of 4 waves per (partition, q-head tile, sequence);
//     a q-head tile is GT q heads that read the same kv head, so each K/V
//     byte loaded feeds GT heads (GQA / MQA sharing).
//   * cache tile layout [block][kv_head][16][D]: the 16 token rows of one
//     (block, kv head) are contiguous, so a wave load of 16 bytes per lane
//     reads 1 KiB of consecutive bytes (whole 128-byte lines).
//   * a token row (D * elem bytes) is owned by L = row_bytes / 16 consecutive
//     lanes; q.k is a per-lane partial dot (packed dot2 instructions for
//     fp16 / bf16) finished by a DPP butterfly inside the row; tiles of 2 or 4
//     heads with 16-bit caches at D = 128 use a reduce-scatter butterfly that
//     leaves one complete score (and one exponential) per lane (Scatter).
//   * every row of lanes keeps its own online-softmax state (m, l, acc) for
//     the tokens it sees, so the loop has no cross-row traffic; rows and waves
//     are merged once at the end (shuffles, then LDS).
//   * the exponential is exp2 with log2(e) folded into the scale.
//   * tokens past the context are masked with selects (never a multiply), and
//     the K/V rows past it are outside the tile's buffer window, so they load
//     as zeros: whatever bytes sit in unused slots (NaN included) cannot leak.
//   * a sequence whose context fits in one partition gets its final output
//     here (when an output pointer is given); longer ones leave a partial
//     (m, l, o) per partition for the merge kernel.  The merge runs as a
//     second launch: merging inside this kernel would need device-scope
//     release/acquire fences per work-group, which on gfx950 write back and
//     invalidate the per-XCD L2 and cost far more than the extra launch.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegBig = -3.0e38f;  // finite stand-in for -inf in running maxima

template <Elem CE, int D> struct Geom {
    static constexpr int BITS = ElemInfo<CE>::bits;
    static constexpr int ROW = D * BITS / 8;     // bytes per token row
    static constexpr int L = ROW / 16;           // lanes per token row
    static constexpr int E = 128 / BITS;         // cache elements per lane (16 bytes)
    static constexpr int R = kWave / L;          // token rows per wave load
    static constexpr int LPB = kBlockSize / R;   // wave loads per 16-token block
    static constexpr int U = LPB < 4 ? LPB : 4;  // wave loads per step
    static constexpr int STEPS = LPB / U;
    static_assert(L >= 1 && L <= kWave && (L & (L - 1)) == 0, "row must map to 2^k lanes");
    static_assert(R * LPB == kBlockSize, "block must split into whole wave loads");
};

// ---- q slice held by a lane, and its dot product with one 16-byte K chunk --

template <Elem QE, Elem CE, int E> struct QSlice;

// fp32 / fp16 / bf16 cache: q kept in the cache's own packed format
template <Elem T, int E> struct QSlice<T, T, E> {
    uint4 v;
    __device__ __forceinline__ void load(const void* q, size_t elem_off) {
        v = *reinterpret_cast<const uint4*>(static_cast<const char*>(q) +
                                            elem_off * ElemInfo<T>::bytes);
    }
    __device__ __forceinline__ float dot(const uint4& k) const {
        if constexpr (T == Elem::F16) {
            float d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.x),
                                             __builtin_bit_cast(half2_t, k.x), 0.0f, false);
            d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.y),
                                       __builtin_bit_cast(half2_t, k.y), d, false);
            d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.z),
                                       __builtin_bit_cast(half2_t, k.z), d, false);
            d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.w),
                                       __builtin_bit_cast(half2_t, k.w), d, false);
            return d;
        } else if constexpr (T == Elem::BF16) {
            float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, v.x),
                                                      __builtin_bit_cast(bf162_t, k.x), 0.0f,
                                                      false);
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, v.y),
                                                __builtin_bit_cast(bf162_t, k.y), d, false);
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, v.z),
                                                __builtin_bit_cast(bf162_t, k.z), d, false);
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, v.w),
                                                __builtin_bit_cast(bf162_t, k.w), d, false);
            return d;
        } else {
            float d = __builtin_bit_cast(float, v.x) * __builtin_bit_cast(float, k.x);
            d = fmaf(__builtin_bit_cast(float, v.y), __builtin_bit_cast(float, k.y), d);
            d = fmaf(__builtin_bit_cast(float, v.z), __builtin_bit_cast(float, k.z), d);
            d = fmaf(__builtin_bit_cast(float, v.w), __builtin_bit_cast(float, k.w), d);
            return d;
        }
    }
};

__device__ __forceinline__ float i8_at(uint32_t w, int k) {
    return (float)(int8_t)(w >> (8 * k));
}

// INT8 / FP8 cache: q widened to fp32 once; the codes are widened in the dot
template <Elem QE, Elem CE> struct QSliceScaled {
    float v[16];
    __device__ __forceinline__ void load(const void* q, size_t elem_off) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + elem_off);
        uint4 a = p[0], b = p[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (QE == Elem::F16) {
                v[2 * i] = lo_h(w[i]);
                v[2 * i + 1] = hi_h(w[i]);
            } else {
                v[2 * i] = lo_bf(w[i]);
                v[2 * i + 1] = hi_bf(w[i]);
            }
        }
    }
    __device__ __forceinline__ float dot(const uint4& k) const {
        const uint32_t w[4] = {k.x, k.y, k.z, k.w};
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x0, x1, x2, x3;
            if constexpr (CE == Elem::F8) {
                f8x4_to_f32(w[i], x0, x1, x2, x3);
            } else {
                x0 = i8_at(w[i], 0);
                x1 = i8_at(w[i], 1);
                x2 = i8_at(w[i], 2);
                x3 = i8_at(w[i], 3);
            }
            d0 = fmaf(v[4 * i + 0], x0, d0);
            d1 = fmaf(v[4 * i + 1], x1, d1);
            d0 = fmaf(v[4 * i + 2], x2, d0);
            d1 = fmaf(v[4 * i + 3], x3, d1);
        }
        return d0 + d1;
    }
};
template <Elem QE> struct QSlice<QE, Elem::I8, 16> : QSliceScaled<QE, Elem::I8> {};
template <Elem QE> struct QSlice<QE, Elem::F8, 16> : QSliceScaled<QE, Elem::F8> {};

// 4-bit cache: q kept packed in its own 16-bit format, paired as the codes
// come out of a 32-bit word: pair k of word i is (q[8i+k], q[8i+k+4]),
// matching (nibble k, nibble k+4), so one v_dot2 takes two codes and
// q . (x_min + step c) = step * sum q c + x_min * sum q.  For fp16 q a code
// pair is a pair of fp16 subnormals (masking only, below); bf16 subnormal
// products would fall under fp32's normal range, so for bf16 q a pair becomes
// two bf16 values 16 + code by OR-ing the nibbles, shifted into the mantissa,
// with the bits of 16.0, and the 16 sum q is taken off again.
template <Elem QE> struct QSlice<QE, Elem::U4, 32> {
    uint32_t v[16];  // [word i][pair k] -> v[4 i + k]
    float sum;
    __device__ __forceinline__ void load(const void* q, size_t elem_off) {
        const uint16_t* p = static_cast<const uint16_t*>(q) + elem_off;
        uint16_t x[32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 a = reinterpret_cast<const uint4*>(p)[c];
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[8 * c + 2 * t] = (uint16_t)(w[t] & 0xffffu);
                x[8 * c + 2 * t + 1] = (uint16_t)(w[t] >> 16);
            }
        }
        sum = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) sum += QE == Elem::F16 ? h2f(x[i]) : bf2f(x[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[4 * i + k] = (uint32_t)x[8 * i + k] | ((uint32_t)x[8 * i + k + 4] << 16);
    }
    // bf16 q: sum over the chunk's 32 codes of q * (16 + code); bf16 16.0 is
    // 0x4180 and the mantissa step at that exponent is 1/8, so code << 3
    __device__ __forceinline__ float dot16(const uint4& k) const {
        const uint32_t w[4] = {k.x, k.y, k.z, k.w};
        constexpr uint32_t kMagic = 0x41804180u;
        constexpr int kSh = 3;
        constexpr uint32_t kMask = 0x000F000Fu << kSh;
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                const int sh = kSh - 4 * kq;   // nibble kq (and kq + 4) to the mantissa
                const uint32_t bits = ((sh >= 0 ? (w[i] << sh) : (w[i] >> -sh)) & kMask) | kMagic;
                float& d = (kq & 1) ? d1 : d0;
                d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, v[4 * i + kq]),
                                                    __builtin_bit_cast(bf162_t, bits), d, false);
            }
        }
        return d0 + d1;
    }
    // fp16 q: a nibble masked into the low mantissa bits of a half whose
    // exponent bits are zero is the subnormal code * 2^-24 (code * 2^-20 at
    // bits 4..7), exact, so a mask alone makes the v_dot2 operand: nibbles 0
    // and 2 of each half land at bits 0..3, nibbles 1 and 3 at bits 4..7.
    // Returns the sums over pairs 0, 2 and over pairs 1, 3 of q * code * 2^-24
    // and q * code * 2^-20.
    __device__ __forceinline__ void dot_sub(const uint4& k, float& d0, float& d1) const {
        const uint32_t w[4] = {k.x, k.y, k.z, k.w};
        d0 = 0.f;
        d1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w8 = w[i] >> 8;
            const uint32_t b[4] = {w[i] & 0x000F000Fu, w[i] & 0x00F000F0u, w8 & 0x000F000Fu,
                                   w8 & 0x00F000F0u};
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                float& d = (kq & 1) ? d1 : d0;
                d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v[4 * i + kq]),
                                           __builtin_bit_cast(half2_t, b[kq]), d, false);
            }
        }
    }
    // this lane's share of q . dequantized K row
    __device__ __forceinline__ float score(const uint4& k, float step, float zmin) const {
        if constexpr (QE == Elem::F16) {
            float d0, d1;
            dot_sub(k, d0, d1);
            return fmaf(fmaf(d1, 0x1p20f, d0 * 0x1p24f), step, zmin * sum);
        } else {
            return fmaf(dot16(k), step, fmaf(-16.0f, step, zmin) * sum);
        }
    }
};

// Codes of one row of the new token: this lane's 16 elements, whose row spans
// L lanes.  Same arithmetic as the quantizing cache write: exact absolute
// maximum, s = amax / qmax (IEEE division; qmax 127 for INT8, 448 for FP8
// e4m3), then x / s rounded half to even and clamped (INT8), or clamped to
// +-448 and converted to e4m3 with round-to-nearest-even (FP8).
template <Elem CE, int L>
__device__ __forceinline__ uint4 quantize16(const float (&x)[16], float& scale_out) {
    constexpr float kQmax = CE == Elem::F8 ? 448.0f : 127.0f;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = group_max<L>(amax);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    float s = 0.f;
    if (amax > 0.f) {
        s = amax / kQmax;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                r[j] = x[4 * i + j] / s;
                if constexpr (CE == Elem::I8) r[j] = __builtin_rintf(r[j]);
                r[j] = fminf(fmaxf(r[j], -kQmax), kQmax);
            }
            if constexpr (CE == Elem::F8) {
                w[i] = f32x4_to_f8(r[0], r[1], r[2], r[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[i] |= ((uint32_t)(int32_t)r[j] & 0xffu) << (8 * j);
            }
        }
    }
    scale_out = s;
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 4-bit codes of one row of the new token: this lane's 32 elements, whose
// row spans L lanes.  Same arithmetic as the quantizing cache write: the
// row's exact min and max, range = max - min, code = rne((x - min) / range
// * 15) clamped to [0, 15], each step in IEEE single precision.
template <int L>
__device__ __forceinline__ uint4 quantize32_u4(const float (&x)[32], float& lo_out,
                                               float& range_out) {
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
        lo = fminf(lo, x[i]);
        hi = fmaxf(hi, x[i]);
    }
    lo = -group_max<L>(-lo);
    hi = group_max<L>(hi);
    const float range = hi - lo;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (range != 0.f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            float r = __builtin_rintf((x[i] - lo) / range * 15.0f);
            r = fminf(fmaxf(r, 0.0f), 15.0f);
            w[i / 8] |= (uint32_t)r << (4 * (i % 8));
        }
    }
    lo_out = lo;
    range_out = range;
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// widen one 16-byte V chunk to E floats
template <Elem CE, int E> __device__ __forceinline__ void widen(const uint4& c, float (&x)[E]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (CE == Elem::F32) {
            x[i] = __builtin_bit_cast(float, w[i]);
        } else if constexpr (CE == Elem::F16) {
            x[2 * i] = lo_h(w[i]);
            x[2 * i + 1] = hi_h(w[i]);
        } else if constexpr (CE == Elem::BF16) {
            x[2 * i] = lo_bf(w[i]);
            x[2 * i + 1] = hi_bf(w[i]);
        } else if constexpr (CE == Elem::F8) {
            f8x4_to_f32(w[i], x[4 * i + 0], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
        } else if constexpr (CE == Elem::U4) {
            // low nibbles are elements 8i, 8i+2, 8i+4, 8i+6, high ones the odd
            // elements.  A byte c <= 15 read as an e4m3 code is exactly
            // c * 2^-9 (codes 1..7 are the subnormals m * 2^-9, 8..15 the
            // normals (8 + m) * 2^-9), so one packed fp8 convert widens two
            // codes; the values come out scaled by 2^-9 (kU4Widen undoes it)
            const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
            float l[4], h[4];
            f8x4_to_f32(lo, l[0], l[1], l[2], l[3]);
            f8x4_to_f32(hi, h[0], h[1], h[2], h[3]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[8 * i + 2 * j] = l[j];
                x[8 * i + 2 * j + 1] = h[j];
            }
        } else {
            x[4 * i + 0] = i8_at(w[i], 0);
            x[4 * i + 1] = i8_at(w[i], 1);
            x[4 * i + 2] = i8_at(w[i], 2);
            x[4 * i + 3] = i8_at(w[i], 3);
        }
    }
}

// 4-bit V codes are widened to code * 2^-9 (see widen); their weights carry
// the 2^9 back (a power of two: the products are the same as with the codes)
constexpr float kU4Widen = 512.0f;

// K/V tiles are read through raw buffer loads.  A buffer resource covers one
// (block, kv head) tile; a load whose offset lies outside the resource returns
// zeros without touching memory, so a block that does not exist (past the end
// of a wave's run, or an invalid id) is "loaded" from a zero-sized resource.
// Every load is then issued without a branch and the compiler waits for
// exactly the block being consumed.  The loads carry the non-temporal hint:
// each K/V byte is used once per call.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;  // gfx9 family: 32-bit data format, raw access
constexpr int kNonTemporal = 2;           // cache-policy bit "nt" of the load

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                             kBufferWord3);
}

__device__ __forceinline__ uint4 ld16_stream(__amdgpu_buffer_rsrc_t r, int offset) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, kNonTemporal);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float ld_f32(__amdgpu_buffer_rsrc_t r, int offset) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, offset, 0, 0));
}

// The K and V bytes (and INT8 scales) of one 16-token block of one kv head as
// held by one wave: STEPS x U wave loads of 16 bytes per lane each.
template <Elem CE, int D> struct BlockRegs {
    using G = Geom<CE, D>;
    uint4 k[G::STEPS][G::U], v[G::STEPS][G::U];
    float ks[G::STEPS][G::U], vs[G::STEPS][G::U];  // INT8 / FP8 scale, 4-bit range
    float kz[G::STEPS][G::U], vz[G::STEPS][G::U];  // 4-bit x_min
    int jb;   // logical block index in the sequence
    bool ok;  // the block exists and its id was inside the pool
};

// Blocks in flight per wave.  Measured on MI355X: a third block in flight
// helps the single-head 4-bit tile only (its blocks are a quarter of an fp16
// block's bytes for a similar amount of work: 134.3 -> 131.3 us on a 64 x
// U[512, 4096] batch) and no other tile; the depths stay selectable.
#ifndef PKV_LAZY_RESCALE
#define PKV_LAZY_RESCALE 1
#endif
#ifndef PKV_DEPTH_SMALL_TILE
#define PKV_DEPTH_SMALL_TILE 2
#endif
#ifndef PKV_DEPTH_LARGE_TILE
#define PKV_DEPTH_LARGE_TILE 2
#endif
#ifndef PKV_DEPTH_U4_SINGLE
#define PKV_DEPTH_U4_SINGLE 3
#endif
template <Elem CE, int GT>
constexpr int kPipelineDepth =
    (CE == Elem::U4 && GT == 1)             ? PKV_DEPTH_U4_SINGLE
    : (GT == 4 && ElemInfo<CE>::bits <= 16) ? PKV_DEPTH_LARGE_TILE
                                            : PKV_DEPTH_SMALL_TILE;

// ---- scores by a transposed (reduce-scatter) butterfly -------------------
// When a token row spans exactly one 16-lane DPP row and a block is four wave
// loads (16-bit caches at D = 128: token group g = 0..3 holds rows 4g..4g+3),
// every lane has GT x 4 partial dot products (GT heads x 4 groups) that must
// be summed over its row.  Summing each one over all 16 lanes costs 4 DPP adds
// per value and leaves 16 copies of every score, each of which then takes its
// own exponential.  Here each exchange step instead hands half of the
// remaining values to the partner lane and keeps the other half (partners
// lane ^ 8, ^ 7, ^ 2, ^ 1: row_ror:8, row_half_mirror and quad_perm), so
// after four steps a lane holds the complete score of one (head, group)
// pair: GT x 4 - 1 adds in all for GT = 4, and one exponential per lane.
// The half a lane keeps is the same slot index in every lane because lanes
// take their q heads and their K token groups in a lane-dependent order
// (slot s holds head s ^ head_xor(lane), slot u holds group u ^ 2 b3, b3 =
// bit 3 of the lane's place in the row); one split of the groups is done by a
// per-lane select instead, since a K group that depends on lane bits below 3
// would break the 128-byte lines a wave load reads.  The scores then go back
// to all lanes of the row by DPP row broadcasts, one per (head, group).
#ifndef PKV_WAVES_16BIT
#define PKV_WAVES_16BIT 1
#endif
#ifndef PKV_SCATTER_MIN_GT
#define PKV_SCATTER_MIN_GT 2
#endif
template <int GT> struct Scatter;
template <> struct Scatter<4> {
    // lane bits b3 b2 b1 b0 = place in the row; head 2 b2 + (b1 ^ b2),
    // group 2 b3 + (b0 ^ b2)
    static constexpr int kPartnerA = kDppQuadXor1, kPartnerB = kDppRowXor8;  // same head
    __device__ static int head_xor(int s) { return (s & 4) >> 1 | (((s >> 1) ^ (s >> 2)) & 1); }
    __device__ static bool sel(int s) { return ((s ^ (s >> 2)) & 1) != 0; }
    static constexpr int src(int h, int g) {
        return 8 * (g >> 1) + 4 * (h >> 1) + 2 * ((h & 1) ^ (h >> 1)) + ((g & 1) ^ (h >> 1));
    }
    __device__ static float reduce(const float (&x)[4][4], bool sl) {
        float y[4][2], z[2][2], w[2];
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int u = 0; u < 2; ++u) y[h][u] = x[h][u] + dpp<kDppRowXor8>(x[h][u + 2]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int u = 0; u < 2; ++u) z[h][u] = y[h][u] + dpp<kDppRowHalfMirror>(y[h + 2][u]);
#pragma unroll
        for (int u = 0; u < 2; ++u) w[u] = z[0][u] + dpp<kDppQuadXor2>(z[1][u]);
        const float keep = sl ? w[1] : w[0], send = sl ? w[0] : w[1];
        return keep + dpp<kDppQuadXor1>(send);
    }
};
template <> struct Scatter<2> {
    // head b2, group 2 b3 + (b1 ^ b2); lanes i and i ^ 1 hold the same score
    static constexpr int kPartnerA = kDppQuadXor2, kPartnerB = kDppRowXor8;
    __device__ static int head_xor(int s) { return (s >> 2) & 1; }
    __device__ static bool sel(int s) { return (((s >> 1) ^ (s >> 2)) & 1) != 0; }
    static constexpr int src(int h, int g) { return 8 * (g >> 1) + 4 * h + 2 * ((g & 1) ^ h); }
    __device__ static float reduce(const float (&x)[2][4], bool sl) {
        float y[2][2], z[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int u = 0; u < 2; ++u) y[h][u] = x[h][u] + dpp<kDppRowXor8>(x[h][u + 2]);
#pragma unroll
        for (int u = 0; u < 2; ++u) z[u] = y[0][u] + dpp<kDppRowHalfMirror>(y[1][u]);
        const float keep = sl ? z[1] : z[0], send = sl ? z[0] : z[1];
        const float w = keep + dpp<kDppQuadXor2>(send);
        return w + dpp<kDppQuadXor1>(w);
    }
};
template <> struct Scatter<1> {
    // group 2 b3 + b2; lanes i, i ^ 1, i ^ 2, i ^ 3 hold the same score
    [[maybe_unused]] static constexpr int kPartnerA = kDppRowHalfMirror;
    [[maybe_unused]] static constexpr int kPartnerB = kDppRowXor8;
    __device__ static int head_xor(int) { return 0; }
    __device__ static bool sel(int s) { return ((s >> 2) & 1) != 0; }
    static constexpr int src(int, int g) { return 8 * (g >> 1) + 4 * (g & 1); }
    __device__ static float reduce(const float (&x)[1][4], bool sl) {
        float y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) y[u] = x[0][u] + dpp<kDppRowXor8>(x[0][u + 2]);
        const float keep = sl ? y[1] : y[0], send = sl ? y[0] : y[1];
        float w = keep + dpp<kDppRowHalfMirror>(send);
        w += dpp<kDppQuadXor2>(w);
        return w + dpp<kDppQuadXor1>(w);
    }
};
// lane `src` of each row of 16 to the whole row; `src` is a constant once the
// loops around the call are unrolled, so the switch folds away
__device__ __forceinline__ float row_bcast(float x, int src) {
    switch (src & 15) {
    case 0: return dpp<kDppRowBcast + 0>(x);
    case 1: return dpp<kDppRowBcast + 1>(x);
    case 2: return dpp<kDppRowBcast + 2>(x);
    case 3: return dpp<kDppRowBcast + 3>(x);
    case 4: return dpp<kDppRowBcast + 4>(x);
    case 5: return dpp<kDppRowBcast + 5>(x);
    case 6: return dpp<kDppRowBcast + 6>(x);
    case 7: return dpp<kDppRowBcast + 7>(x);
    case 8: return dpp<kDppRowBcast + 8>(x);
    case 9: return dpp<kDppRowBcast + 9>(x);
    case 10: return dpp<kDppRowBcast + 10>(x);
    case 11: return dpp<kDppRowBcast + 11>(x);
    case 12: return dpp<kDppRowBcast + 12>(x);
    case 13: return dpp<kDppRowBcast + 13>(x);
    case 14: return dpp<kDppRowBcast + 14>(x);
    default: return dpp<kDppRowBcast + 15>(x);
    }
}

// Waves per SIMD asked of the register allocator where the default falls
// just short of a step: 4-bit single-head tiles at D = 128 (4).  16-bit
// single-head tiles at D = 128 take 100 VGPRs (4 waves); asking for 5 gives
// 96 with one spill reloaded in the block loop, measured slower on MI355X
// (LLaMA-7B batch 404 -> 412 us, 16 x 32k 1407 -> 1434 us), so it is off.
template <Elem CE, int D, int GT>
constexpr int kMinWavesPerEU = (GT == 1 && D == 128 && CE == Elem::U4) ? 4
                               : (GT == 1 && D == 128 && (CE == Elem::F16 || CE == Elem::BF16))
                                   ? PKV_WAVES_16BIT
                                   : 1;

// Waves per work-group; each streams its share of the item's blocks.
// Measured on MI355X (same-box A/B, steps of the fused decode): eight waves
// against four, LLaMA-7B-shaped fp16 batch 392.5 vs 393.1 us, INT8 184.2 vs
// 186.4, FP8 179.8 vs 180.8, GQA 32/8 bf16 364.3 vs 369.9, 16 x 32k
// 1342.6 vs 1353.9; the 4-bit tiles measured slower with eight (123.5 vs
// 117.7 us) and keep four, as do the tiles whose registers pass 256 per lane
// (head_dim 256, and 8 fp32 heads): with eight waves (two per SIMD) those
// would spill to memory instead of to accumulation registers.
template <Elem CE, int D, int GT>
constexpr int kDecodeWaves =
    (CE == Elem::U4 || D > 128 || (CE == Elem::F32 && GT == 8)) ? 4 : 8;

template <Elem QE, Elem CE, int D, int GT>
__global__ __launch_bounds__((kDecodeWaves<CE, D, GT> * 64))
__attribute__((amdgpu_waves_per_eu(kMinWavesPerEU<CE, D, GT>)))
void paged_decode_kernel(DecodeArgs a) {
    using G = Geom<CE, D>;
    constexpr int L = G::L, E = G::E, R = G::R, U = G::U, STEPS = G::STEPS;
    constexpr int NW = kDecodeWaves<CE, D, GT>;
    constexpr int kDecodeThreads = NW * 64;
    static_assert(kDecodeThreads >= kScheduleMaxSeqs, "one thread per ranked sequence");
    constexpr bool kInt8 = is_scaled(CE);  // 1-byte codes with a per-row scale
    constexpr bool kU4 = CE == Elem::U4;    // 4-bit codes with a per-row (x_min, range)
    constexpr float kInv15 = 1.0f / 15.0f;
    // scores by the reduce-scatter butterfly (16-bit caches, one DPP row per
    // token row, four wave loads per block)
    constexpr bool kScatter = (CE == Elem::F16 || CE == Elem::BF16) && QE == CE && L == 16 &&
                              U == 4 && STEPS == 1 && GT >= PKV_SCATTER_MIN_GT && GT <= 4;
    using SC = Scatter<(GT <= 4 ? GT : 1)>;

    __shared__ float s_m[NW][GT];
    __shared__ float s_l[NW][GT];
    // rows of a wave kept apart for the final LDS merge (the rest are added
    // by lane shuffles first): as many as 4, within 32 KiB of LDS
    constexpr int kKeepCap = 32768 / (NW * GT * D * 4);
    constexpr int RK = kKeepCap >= 4 ? (R < 4 ? R : 4) : kKeepCap >= 2 ? (R < 2 ? R : 2) : 1;
    __shared__ float s_acc[NW][RK][GT][D];
    // (rank key, item count) per sequence, read two sequences per 16-byte LDS load
    __shared__ __align__(16) int2 s_key[kScheduleMaxSeqs];
    __shared__ int s_pick[3];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = lane / L;   // token row inside a wave load
    const int slice = lane % L; // which E elements of the row this lane holds

    const int NP = a.num_partitions;
    const int P = a.partition_size;
    const int n_cap = a.max_blocks_per_seq * kBlockSize;
    auto clamp_len = [&](int v) { return v < 0 ? 0 : (v > n_cap ? n_cap : v); };

    // ---- which (sequence, partition, q-head tile) this work-group takes ----
    // Natural order: partitions fastest, then tiles, then sequences.
    // Longest-first order: work items (partition x tile) of all sequences
    // sorted by partition length, longest first, so that the work dispatched
    // last is the shortest and the ragged tail of a batch is small.  Every
    // work-group ranks the sequences itself (one per thread, in LDS), on the
    // path from kernel start to its first K/V load, so the ranking is kept
    // branch-free: a sequence's key packs its partition span (in blocks) above
    // 255 - index (longer first, then lower index), and a rank is the sum of
    // the item counts of the larger keys, two keys per LDS load.
    int b, part, tile, n;
    if (a.longest_first) {
        const int item = blockIdx.x / a.n_tiles;
        tile = blockIdx.x % a.n_tiles;
        // Work-groups go to the 8 XCDs round-robin, so with a multiple of 16
        // tiles XCD x would get tiles x, x + 8, ... of every sequence.  Taken
        // through this bijection (per 16 tiles: bit 3 of t to bit 0, bits
        // 0-2 to bits 1-3), XCD x reads tiles 2 x and 2 x + 1, whose K (and
        // V) rows of a block lie next to each other in the pool.  Measured
        // (same box, bit-identical output): LLaMA-7B-shaped batch 391.7
        // against 398.0 us per launch, INT8 cache 194.5 against 197.3; maps
        // in which no XCD reads two adjacent tiles (tiles 2, 4 or 8 apart)
        // stayed at 396-398 us.
        if ((a.n_tiles & 15) == 0) {
            const int t = tile;
            tile = (t & ~15) | ((t >> 3) & 1) | ((t & 7) << 1);
        }
        int my_key = -1, cnt = 0, my_n = 0;
        if (tid < a.num_seqs) {
            my_n = clamp_len(a.context_lens[tid]);
            const int nn =
                my_n - attend_begin(my_n, a.window, a.seq_start, tid) / kBlockSize * kBlockSize;
            const int c = partition_count(nn, P);
            const int span_blocks = c > 0 ? partition_span(nn, c) / kBlockSize : 0;
            static_assert(kScheduleMaxSeqs <= 256, "sequence index must fit 8 key bits");
            my_key = span_blocks << 8 | (255 - tid);
            cnt = c > 0 ? c : 1;  // an empty sequence still takes one item: it writes zeros
        }
        // every one of the kScheduleMaxSeqs entries is written; those
        // past the batch hold count 0 and so add nothing to a rank
        if (tid < kScheduleMaxSeqs) s_key[tid] = make_int2(my_key, cnt);
        if (tid == 0) s_pick[0] = -1;
        __syncthreads();
        if (tid < a.num_seqs) {
            int start = 0;
            const int nj = (a.num_seqs + 1) & ~1;  // <= kScheduleMaxSeqs
#pragma unroll 4
            for (int j = 0; j < nj; j += 2) {
                const int4 kk = *reinterpret_cast<const int4*>(&s_key[j]);
                start += kk.x > my_key ? kk.y : 0;
                start += kk.z > my_key ? kk.w : 0;
            }
            if (item >= start && item < start + cnt) {
                s_pick[0] = tid;
                s_pick[1] = item - start;
                s_pick[2] = my_n;
            }
        }
        __syncthreads();
        b = s_pick[0];
        part = s_pick[1];
        n = s_pick[2];
        if (b < 0) return;  // beyond the last item (uniform)
    } else {
        part = blockIdx.x % NP;
        const int rest = blockIdx.x / NP;
        tile = rest % a.n_tiles;
        b = rest / a.n_tiles;
        n = clamp_len(a.context_lens[b]);
    }

    // sliding window or per-sequence start: positions below `lo` are not
    // attended to; the partitions split the positions from the block-aligned
    // `base` on
    const int lo = attend_begin(n, a.window, a.seq_start, b);
    const int base = lo / kBlockSize * kBlockSize;
    const int n_parts = partition_count(n - base, P);
    const int span = n_parts > 0 ? partition_span(n - base, n_parts) : 0;
    const int Hq = a.num_q_heads;
    const int h0 = tile * GT;
    const int g = Hq / a.num_kv_heads;
    const int kvh = h0 / g;

    const bool direct_out = a.out != nullptr;
    // The output of a sequence whose earlier positions were attended to
    // elsewhere (a shared prefix, partials pre_*): this work-group's result
    // (max M in log2 units, sum L, unnormalized O) merged with those partials
    // by the running-max / running-sum rule; nothing attended at all gives 0.
    const bool pre = a.pre_m != nullptr && a.seq_start != nullptr && direct_out;
    auto merge_pre = [&](int h, int d, float M2, float L, float O) -> float {
        const size_t pb = ((size_t)b * Hq + h0 + h) * a.pre_np;
        const int n0 = min(max(a.seq_start[b], 0), n_cap);
        const int np = min(max(partition_count(n0, a.pre_partition_size), 1), a.pre_np);
        float Mx = M2;
        for (int p = 0; p < np; ++p) Mx = fmaxf(Mx, a.pre_m[pb + p] * kLog2e);
        const float f = fast_exp2(M2 - Mx);
        float LL = L * f, OO = O * f;
        for (int p = 0; p < np; ++p) {
            const float w = a.pre_l[pb + p] * fast_exp2(fmaf(a.pre_m[pb + p], kLog2e, -Mx));
            LL += w;
            OO = fmaf(w, a.pre_o[(pb + p) * D + d], OO);
        }
        return LL > 0.f ? OO / LL : 0.f;
    };
    if (part >= n_parts) {
        if (part == 0 && n_parts == 0) {  // no position to attend to
            if (pre) {  // the prefix alone
                for (int i = tid; i < GT * D; i += kDecodeThreads)
                    store_elem<QE>(a.out, ((size_t)b * Hq + h0 + i / D) * D + i % D,
                                   merge_pre(i / D, i % D, kNegBig, 0.f, 0.f));
            } else if (direct_out) {  // the output is zero
                for (int i = tid; i < GT * D; i += kDecodeThreads)
                    store_elem<QE>(a.out, ((size_t)b * Hq + h0 + i / D) * D + i % D, 0.0f);
            } else if (a.seq_start != nullptr) {
                // an empty partial (weight 0) for the merge with the positions
                // attended to elsewhere
                for (int i = tid; i < GT * D; i += kDecodeThreads) {
                    const size_t pi = ((size_t)b * Hq + h0 + i / D) * NP;
                    a.o_part[pi * D + i % D] = 0.f;
                    if (i % D == 0) {
                        a.m_part[pi] = kNegBig;
                        a.l_part[pi] = 0.f;
                    }
                }
            }
        }
        return;
    }

    // q slices of the GT heads, and the running state of this lane's row
    QSlice<QE, CE, E> qs[GT];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        const int hq = kScatter ? (h ^ SC::head_xor(slice)) : h;
        qs[h].load(a.q, ((size_t)b * Hq + h0 + hq) * D + slice * E);
    }
    // scatter mode: K slot u of this lane holds token group u ^ kflip
    const int kflip = kScatter ? (slice & 8) >> 2 : 0;
    const bool ssel = kScatter && SC::sel(slice);
    const int sgroup = 2 * (kflip >> 1) + (ssel ? 1 : 0);  // group of the lane's score
    float ms = kNegBig, ls = 0.f;  // running max / this lane's share of the sum

    float m[GT], l[GT], acc[GT][E];
    float zacc[GT];  // 4-bit caches: sum of p * x_min, added to every channel at the end
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        m[h] = kNegBig;
        l[h] = 0.f;
        zacc[h] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }

    const int t_begin = base + part * span;
    const int t_end = min(n, t_begin + span);
    const int blk_begin = t_begin / kBlockSize;
    const int blk_end = (t_end + kBlockSize - 1) / kBlockSize;
    const int32_t* table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
    const float c = a.scale_log2;

    // ---- append of the step's new token (position n-1), when given --------
    // The work-group owning the last partition leaves the new token's slot
    // out of the block loop and folds the token in afterwards from the input
    // row (quantized like the cache write for an INT8 cache), which it also
    // stores into the slot.  Nothing of it is live during the loop.
    const bool has_new = a.k_new != nullptr && n > 0 && t_end == n;
    const int n_loop = has_new ? n - 1 : n;  // tokens the block loop attends to

    // Each wave takes a contiguous run of the partition's blocks.  Block ids
    // are wave-uniform scalar loads, issued one block ahead of their use; they
    // are counted apart from the vector K/V loads (lgkmcnt vs vmcnt), so
    // waiting for an id never drains the K/V loads in flight.
    const int nblk = blk_end - blk_begin;
    const int per_wave = (nblk + NW - 1) / NW;
    const int my0 = blk_begin + wave * per_wave;
    const int n_my = max(0, min(per_wave, blk_end - my0));
    const int32_t* my_ids = table + my0;
    const int last = max(n_my - 1, 0);
    constexpr int kTileBytes = kBlockSize * G::ROW;

    // block i of this wave's run; i >= n_my (or a bad id) gives an empty tile
    auto load_block = [&](BlockRegs<CE, D>& r, int phys, int i) {
        r.jb = my0 + i;
        r.ok = i < n_my && phys >= 0 && (int64_t)phys < a.num_blocks;
        const size_t tile_idx = (size_t)(r.ok ? phys : 0) * a.num_kv_heads + kvh;
        // the window ends at the last token the loop attends to: rows past it
        // (the unused tail of a last block, the new token's slot) load as zeros
        // (uniform in the work-group; said so, or the loads get per-lane descriptors)
        const int rows = __builtin_amdgcn_readfirstlane(
            r.ok ? min(max(n_loop - r.jb * kBlockSize, 0), kBlockSize) : 0);
        const int bytes = rows * G::ROW;
        const __amdgpu_buffer_rsrc_t kr =
            tile_rsrc(static_cast<const char*>(a.k_cache) + tile_idx * kTileBytes, bytes);
        const __amdgpu_buffer_rsrc_t vr =
            tile_rsrc(static_cast<const char*>(a.v_cache) + tile_idx * kTileBytes, bytes);
        __amdgpu_buffer_rsrc_t ksr, vsr;
        if constexpr (kInt8) {
            ksr = tile_rsrc(a.k_scale + tile_idx * kBlockSize, rows * 4);
            vsr = tile_rsrc(a.v_scale + tile_idx * kBlockSize, rows * 4);
        }
        // 4-bit rows: one 8-byte (x_min, range) pair per row, read in place
        // from the row's slot (every slot of the tile exists; values of rows
        // outside the window may be anything and every use selects them away)
        const float2* kzs = nullptr;
        const float2* vzs = nullptr;
        if constexpr (kU4) {
            kzs = reinterpret_cast<const float2*>(a.k_scale) + tile_idx * kBlockSize;
            vzs = reinterpret_cast<const float2*>(a.v_scale) + tile_idx * kBlockSize;
        }
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int tok = (st * U + u) * R;  // first token of this wave load
                r.k[st][u] = ld16_stream(kr, (st * U + (u ^ kflip)) * R * G::ROW + lane * 16);
                r.v[st][u] = ld16_stream(vr, tok * G::ROW + lane * 16);
                if constexpr (kInt8) {
                    r.ks[st][u] = ld_f32(ksr, (tok + row) * 4);
                    r.vs[st][u] = ld_f32(vsr, (tok + row) * 4);
                }
                if constexpr (kU4) {
                    const float2 kp = kzs[tok + row];
                    const float2 vp = vzs[tok + row];
                    r.kz[st][u] = kp.x;
                    r.ks[st][u] = kp.y;
                    r.vz[st][u] = vp.x;
                    r.vs[st][u] = vp.y;
                }
            }
        }
    };

    auto compute_block = [&](const BlockRegs<CE, D>& r) {
        const int jb = r.jb;
        const bool full = r.ok && jb * kBlockSize >= lo && (jb + 1) * kBlockSize <= n_loop;
        // V rows past the loop's last token arrive as zeros (buffer window);
        // only a block that starts before the first attended position (a
        // sliding window or a per-sequence start) must zero rows itself
        const bool below_lo = r.ok && jb * kBlockSize < lo;
        if constexpr (kScatter) {
            // one score per lane: head h0 + head_xor(slice), token group sgroup
            float x[GT][U];
#pragma unroll
            for (int h = 0; h < GT; ++h)
#pragma unroll
                for (int u = 0; u < U; ++u) x[h][u] = qs[h].dot(r.k[0][u]);
            const float sc = SC::reduce(x, ssel);
            const int t_own = jb * kBlockSize + sgroup * R + row;
            const bool v_own = full || (r.ok && t_own >= lo && t_own < n_loop);
            const float s = v_own ? sc * c : -INFINITY;
            // the running max of the lane's head over the row's four groups
            float mx = fmaxf(s, dpp<SC::kPartnerA>(s));
            mx = fmaxf(mx, dpp<SC::kPartnerB>(mx));
            mx = fmaxf(mx, ms);
            const float p = fast_exp2(s - mx);
            if (__builtin_amdgcn_ballot_w64(mx > ms) != 0) {
                const float alpha = fast_exp2(ms - mx);
                ls *= alpha;
                float ah[GT];
#pragma unroll
                for (int h = 0; h < GT; ++h) ah[h] = row_bcast(alpha, SC::src(h, 0));
#pragma unroll
                for (int h = 0; h < GT; ++h)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[h][e] *= ah[h];
                ms = mx;
            }
            ls += p;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vx[E];
                widen<CE, E>(r.v[0][u], vx);
                if (below_lo) {  // rows before the first attended position
                    const bool ok_u = jb * kBlockSize + u * R + row >= lo;
#pragma unroll
                    for (int e = 0; e < E; ++e) vx[e] = ok_u ? vx[e] : 0.f;
                }
#pragma unroll
                for (int h = 0; h < GT; ++h) {
                    const float pv = row_bcast(p, SC::src(h, u));
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pv, vx[e], acc[h][e]);
                }
            }
            return;
        }
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            bool valid[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = jb * kBlockSize + (st * U + u) * R + row;
                valid[u] = full || (r.ok && t >= lo && t < n_loop);
            }

            // scores of the U tokens this row sees, for every head of the tile,
            // then the online-softmax update of (m, l) and the rescale of acc
            float p[GT][U];
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                float s[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float d;
                    if constexpr (kU4)
                        d = group_sum<L>(qs[h].score(r.k[st][u], r.ks[st][u] * kInv15,
                                                     r.kz[st][u]));
                    else
                        d = group_sum<L>(qs[h].dot(r.k[st][u]));
                    if constexpr (kInt8) d *= r.ks[st][u];
                    s[u] = valid[u] ? d * c : -INFINITY;
                }
                float mx = m[h];
#pragma unroll
                for (int u = 0; u < U; ++u) mx = fmaxf(mx, s[u]);
                float psum = 0.f;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    p[h][u] = fast_exp2(s[u] - mx);
                    psum += p[h][u];
                }
                // Tiles of several heads rescale only when some row's running
                // max grew (rare after the first blocks; otherwise the factor
                // is exactly 1).  Measured: a win for GQA tiles, a loss for
                // 16-bit single-head tiles (8 accumulators per lane), which
                // rescale unconditionally; 4-bit tiles hold 32 per lane and
                // rescale lazily too.
                if (!(PKV_LAZY_RESCALE && (GT > 1 || kU4)) ||
                    __builtin_amdgcn_ballot_w64(mx > m[h]) != 0) {
                    const float alpha = fast_exp2(m[h] - mx);
                    l[h] *= alpha;
                    if constexpr (kU4) zacc[h] *= alpha;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
                    m[h] = mx;
                }
                l[h] += psum;
            }
            // V: one wave load at a time, widened once and shared by the heads
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vx[E];
                widen<CE, E>(r.v[st][u], vx);
                if constexpr (kU4) {
                    // p (x_min + step c) = (p step) c + p x_min: the codes take
                    // one FMA each, p x_min a running scalar.  Masked rows get
                    // step = x_min = 0 (their values may be anything, NaN too).
                } else if constexpr (!kInt8 || CE == Elem::F8) {
                    // rows before the first attended position are selected
                    // away: their bytes may be anything (an e4m3 NaN code too),
                    // and a zero weight times NaN would still be NaN.  INT8
                    // codes always widen to finite values, which the zero
                    // weight of an invalid row cancels.
                    if (below_lo) {
#pragma unroll
                        for (int e = 0; e < E; ++e) vx[e] = valid[u] ? vx[e] : 0.f;
                    }
                }
                float vstep = 0.f, vmin = 0.f;
                if constexpr (kU4) {
                    vstep = valid[u] ? r.vs[st][u] * kInv15 * kU4Widen : 0.f;
                    vmin = valid[u] ? r.vz[st][u] : 0.f;
                }
#pragma unroll
                for (int h = 0; h < GT; ++h) {
                    float pv = p[h][u];
                    if constexpr (kInt8) pv = valid[u] ? pv * r.vs[st][u] : 0.f;
                    if constexpr (kU4) {
                        zacc[h] = fmaf(pv, vmin, zacc[h]);
                        pv *= vstep;
                    }
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pv, vx[e], acc[h][e]);
                }
            }
        }
    };

    // kDepth blocks in flight per wave: the loads of the next blocks are
    // issued before block i is consumed, and the next id is requested
    // meanwhile.  Loads past the run are empty, so only the consumption of the
    // blocks of the last round sits behind a branch.
    constexpr int kDepth = kPipelineDepth<CE, GT>;
    if (n_my > 0 && kDepth == 2) {
        BlockRegs<CE, D> ra, rb;
        load_block(ra, my_ids[0], 0);
        int next_id = my_ids[min(1, last)];
        for (int i = 0; i < n_my; i += 2) {
            load_block(rb, next_id, i + 1);
            next_id = my_ids[min(i + 2, last)];
            compute_block(ra);
            load_block(ra, next_id, i + 2);
            next_id = my_ids[min(i + 3, last)];
            if (i + 1 < n_my) compute_block(rb);
        }
    } else if (n_my > 0) {  // three blocks in flight
        BlockRegs<CE, D> ra, rb, rc;
        load_block(ra, my_ids[0], 0);
        load_block(rb, my_ids[min(1, last)], 1);
        int next_id = my_ids[min(2, last)];
        for (int i = 0; i < n_my; i += 3) {
            load_block(rc, next_id, i + 2);
            next_id = my_ids[min(i + 3, last)];
            compute_block(ra);
            load_block(ra, next_id, i + 3);
            next_id = my_ids[min(i + 4, last)];
            if (i + 1 < n_my) compute_block(rb);
            load_block(rb, next_id, i + 4);
            next_id = my_ids[min(i + 5, last)];
            if (i + 2 < n_my) compute_block(rc);
        }
    }

    if constexpr (kScatter) {
        // back to one (m, l) per head in every lane of the row: the head's sum
        // is spread over the lanes of its four groups
        float lh = ls + dpp<SC::kPartnerA>(ls);
        lh += dpp<SC::kPartnerB>(lh);
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            m[h] = row_bcast(ms, SC::src(h, 0));
            l[h] = row_bcast(lh, SC::src(h, 0));
        }
    }

    if (has_new && wave == 0) {
        // the new row: every lane loads its slice; row 0 of wave 0 folds it in
        const size_t src = ((size_t)b * a.num_kv_heads + kvh) * D + (size_t)slice * E;
        uint4 kc, vc;
        float ks = 1.f, vs = 1.f;
        float kz = 0.f, vz = 0.f;
        if constexpr (kU4) {
            float xk[32], xv[32];
            const uint4* pk = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_new) + src);
            const uint4* pv = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_new) + src);
#pragma unroll
            for (int cix = 0; cix < 4; ++cix) {
                const uint4 k4 = pk[cix], v4 = pv[cix];
                const uint32_t wk[4] = {k4.x, k4.y, k4.z, k4.w};
                const uint32_t wv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xk[8 * cix + 2 * i] = QE == Elem::F16 ? lo_h(wk[i]) : lo_bf(wk[i]);
                    xk[8 * cix + 2 * i + 1] = QE == Elem::F16 ? hi_h(wk[i]) : hi_bf(wk[i]);
                    xv[8 * cix + 2 * i] = QE == Elem::F16 ? lo_h(wv[i]) : lo_bf(wv[i]);
                    xv[8 * cix + 2 * i + 1] = QE == Elem::F16 ? hi_h(wv[i]) : hi_bf(wv[i]);
                }
            }
            kc = quantize32_u4<L>(xk, kz, ks);
            vc = quantize32_u4<L>(xv, vz, vs);
        } else if constexpr (!kInt8) {
            kc = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + src * G::BITS / 8);
            vc = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + src * G::BITS / 8);
        } else {
            float xk[16], xv[16];
            const uint4* pk = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_new) + src);
            const uint4* pv = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_new) + src);
            const uint4 k0 = pk[0], k1 = pk[1], v0 = pv[0], v1 = pv[1];
            const uint32_t wk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
            const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xk[2 * i] = QE == Elem::F16 ? lo_h(wk[i]) : lo_bf(wk[i]);
                xk[2 * i + 1] = QE == Elem::F16 ? hi_h(wk[i]) : hi_bf(wk[i]);
                xv[2 * i] = QE == Elem::F16 ? lo_h(wv[i]) : lo_bf(wv[i]);
                xv[2 * i + 1] = QE == Elem::F16 ? hi_h(wv[i]) : hi_bf(wv[i]);
            }
            kc = quantize16<CE, L>(xk, ks);
            vc = quantize16<CE, L>(xv, vs);
        }
        const int new_jb = (n - 1) / kBlockSize, new_off = (n - 1) % kBlockSize;
        const int phys = table[new_jb];
        if (h0 % g == 0 && row == 0 && phys >= 0 && (int64_t)phys < a.num_blocks) {
            // one writer per kv head: the first q-head tile's row 0 of wave 0
            const size_t trow = ((size_t)phys * a.num_kv_heads + kvh) * kBlockSize + new_off;
            const size_t dst = trow * D + (size_t)slice * E;  // elements of the cache type
            *reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.k_cache)) + dst * G::BITS / 8) = kc;
            *reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.v_cache)) + dst * G::BITS / 8) = vc;
            if constexpr (kInt8) {
                if (slice == 0) {
                    const_cast<float*>(a.k_scale)[trow] = ks;
                    const_cast<float*>(a.v_scale)[trow] = vs;
                }
            }
            if constexpr (kU4) {
                if (slice == 0) {
                    const_cast<float*>(a.k_scale)[2 * trow] = kz;
                    const_cast<float*>(a.k_scale)[2 * trow + 1] = ks;
                    const_cast<float*>(a.v_scale)[2 * trow] = vz;
                    const_cast<float*>(a.v_scale)[2 * trow + 1] = vs;
                }
            }
        }
        float vx[E];
        widen<CE, E>(vc, vx);
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            float d;
            if constexpr (kU4)
                d = group_sum<L>(qs[h].score(kc, ks * kInv15, kz));
            else if constexpr (kScatter) {
                // this lane holds head h in slot h ^ head_xor(slice)
                const int want = h ^ SC::head_xor(slice);
                float mine = qs[0].dot(kc);
#pragma unroll
                for (int s2 = 1; s2 < GT; ++s2) {
                    const float t2 = qs[s2].dot(kc);
                    mine = want == s2 ? t2 : mine;
                }
                d = group_sum<L>(mine);
            } else
                d = group_sum<L>(qs[h].dot(kc));
            if constexpr (kInt8) d *= ks;
            const float sn = d * c;
            if (row == 0) {  // one row takes the token
                const float mx = fmaxf(m[h], sn);
                const float alpha = fast_exp2(m[h] - mx);
                const float pn = fast_exp2(sn - mx);
                l[h] = fmaf(l[h], alpha, pn);
                float pv = kInt8 ? pn * vs : pn;
                if constexpr (kU4) {
                    zacc[h] = fmaf(pn, vz, zacc[h] * alpha);
                    pv = pn * (vs * kInv15 * kU4Widen);
                }
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] = fmaf(pv, vx[e], acc[h][e] * alpha);
                m[h] = mx;
            }
        }
    }

    if constexpr (kU4) {
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] += zacc[h];
    }

    // ---- merge the R rows of each wave (lanes with equal `slice`) ----------
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        float M = m[h];
#pragma unroll
        for (int off = L; off < kWave; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float f = fast_exp2(m[h] - M);
        float lh = l[h] * f;
#pragma unroll
        for (int off = L; off < kWave; off <<= 1) lh += __shfl_xor(lh, off);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float x = acc[h][e] * f;
#pragma unroll
            for (int off = L * RK; off < kWave; off <<= 1) x += __shfl_xor(x, off);
            acc[h][e] = x;
        }
        if (lane == 0) {
            s_m[wave][h] = M;
            s_l[wave][h] = lh;
        }
        if (row < RK) {
#pragma unroll
            for (int e = 0; e < E; ++e) s_acc[wave][row][h][slice * E + e] = acc[h][e];
        }
    }
    __syncthreads();

    // ---- merge the waves; write out (single partition) or the partial -----
    const bool single = direct_out && (n_parts == 1);
    for (int i = tid; i < GT * D; i += kDecodeThreads) {
        const int h = i / D, d = i % D;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(s_m[w][h] - M);
            lsum = fmaf(s_l[w][h], f, lsum);
            float ow = s_acc[w][0][h][d];
#pragma unroll
            for (int rk = 1; rk < RK; ++rk) ow += s_acc[w][rk][h][d];
            o = fmaf(ow, f, o);
        }
        const size_t bh = (size_t)b * Hq + h0 + h;
        if (single) {
            store_elem<QE>(a.out, bh * D + d, pre ? merge_pre(h, d, M, lsum, o) : o / lsum);
        } else {
            const size_t pi = bh * NP + part;
            a.o_part[pi * D + d] = o / lsum;
            if (d == 0) {
                a.m_part[pi] = M * kLn2;  // natural-log units
                a.l_part[pi] = lsum;
            }
        }
    }
}

template <Elem QE, Elem CE, int D, int GT>
hipError_t launch4(const DecodeArgs& a, hipStream_t stream) {
    const int64_t n_wg = (int64_t)a.num_partitions * a.n_tiles * a.num_seqs;
    if (n_wg <= 0) return hipSuccess;
    if (n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((paged_decode_kernel<QE, CE, D, GT>), dim3((unsigned)n_wg),
                       dim3(kDecodeWaves<CE, D, GT> * 64), 0, stream, a);
    return hipGetLastError();
}

template <Elem QE, Elem CE, int D>
hipError_t launch3(const DecodeArgs& a, int gt, hipStream_t s) {
    switch (gt) {
    case 1: return launch4<QE, CE, D, 1>(a, s);
    case 2: return launch4<QE, CE, D, 2>(a, s);
    case 4:
        // 4-bit tiles stop at 2 heads (32 fp32 q and accumulator values per head)
        if constexpr (CE != Elem::U4) return launch4<QE, CE, D, 4>(a, s);
        return hipErrorInvalidValue;
    case 8:
        // 1-byte-code tiles stop at 4 heads: 8 would hold 8 x 16 fp32
        // accumulators per lane and spill
        if constexpr (!is_scaled(CE) && CE != Elem::U4) return launch4<QE, CE, D, 8>(a, s);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <Elem QE, Elem CE>
hipError_t launch2(const DecodeArgs& a, int d, int gt, hipStream_t s) {
    switch (d) {
    case 64:
        // a 32-byte 4-bit row would put two blocks in one wave load
        if constexpr (CE != Elem::U4) return launch3<QE, CE, 64>(a, gt, s);
        return hipErrorInvalidValue;
    case 128: return launch3<QE, CE, 128>(a, gt, s);
    case 256: return launch3<QE, CE, 256>(a, gt, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, int q_dtype, int cache_dtype, int head_dim,
                               int heads_per_tile, hipStream_t stream) {
    const Elem qe = static_cast<Elem>(q_dtype), ce = static_cast<Elem>(cache_dtype);
    if (qe == Elem::F32 && ce == Elem::F32)
        return launch2<Elem::F32, Elem::F32>(a, head_dim, heads_per_tile, stream);
    if (qe == Elem::F16 && ce == Elem::F16)
        return launch2<Elem::F16, Elem::F16>(a, head_dim, heads_per_tile, stream);
    if (qe == Elem::BF16 && ce == Elem::BF16)
        return launch2<Elem::BF16, Elem::BF16>(a, head_dim, heads_per_tile, stream);
    if (qe == Elem::F16 && ce == Elem::I8)
        return launch2<Elem::F16, Elem::I8>(a, head_dim, heads_per_tile, stream);
    if (qe == Elem::BF16 && ce == Elem::I8)
        return launch2<Elem::BF16, Elem::I8>(a, head_dim, heads_per_tile, stream);
    if (qe == Elem::F16 && ce == Elem::F8)
        return launch2<Elem::F16, Elem::F8>(a, head_dim, heads_per_tile, stream);
    if (qe == Elem::BF16 && ce == Elem::F8)
        return launch2<Elem::BF16, Elem::F8>(a, head_dim, heads_per_tile, stream);
    if (qe == Elem::F16 && ce == Elem::U4)
        return launch2<Elem::F16, Elem::U4>(a, head_dim, heads_per_tile, stream);
    if (qe == Elem::BF16 && ce == Elem::U4)
        return launch2<Elem::BF16, Elem::U4>(a, head_dim, heads_per_tile, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
