// Slot-mapped cache append with optional INT8 / FP8 / 4-bit quantize-on-write.
//
// Each new token's K and V rows are written into the pool at the slot the
// block manager assigned (block = slot / 16, offset = slot % 16), for every kv
// head; only the new token's keys and values are written (juejin "LLM
// Engineer's Handbook", section "KV cache").  In INT8 mode every (token, kv
// head) row gets one fp32 scale s = max|x| / 127 and codes
// clamp(round_half_even(x / s), -127, 127) (docs.lazyllm.ai lesson 4,
// section 5.3; the juejin absmax passage and its half-to-even rounding).
//
// Layout on gfx950: a row of D elements is handled by D/8 consecutive lanes,
// 8 elements each (one 16-byte load for 16-bit sources); the INT8 absolute
// maximum is a DPP max inside the row.  The division is IEEE single precision
// (correctly rounded) and rounding uses v_rndne, so codes are bit-exact.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_quant.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

template <Elem SE> struct Src8 {
    float x[8];
    uint4 raw[ElemInfo<SE>::bytes == 4 ? 2 : 1];
    __device__ __forceinline__ void load(const void* base, size_t elem_off) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const char*>(base) +
                                                        elem_off * ElemInfo<SE>::bytes);
        raw[0] = p[0];
        if constexpr (ElemInfo<SE>::bytes == 4) raw[1] = p[1];
    }
    __device__ __forceinline__ void widen() {
        if constexpr (SE == Elem::F32) {
            const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w,
                                   raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = __builtin_bit_cast(float, w[i]);
        } else {
            const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = SE == Elem::F16 ? lo_h(w[i]) : lo_bf(w[i]);
                x[2 * i + 1] = SE == Elem::F16 ? hi_h(w[i]) : hi_bf(w[i]);
            }
        }
    }
};

template <Elem SE, Elem CE, int D>
__global__ __launch_bounds__(kThreads) void kv_cache_write_kernel(CacheWriteArgs a) {
    constexpr int LPR = D / 8;  // lanes per row
    constexpr int RPB = kThreads / LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int j = threadIdx.x % LPR;
    const int64_t n_rows = a.num_tokens * a.num_kv_heads;
    if (row >= n_rows) return;  // whole rows leave together (rows are lane-aligned)
    const int64_t tok = row / a.num_kv_heads;
    const int h = (int)(row % a.num_kv_heads);
    int64_t slot = -1;
    if (a.slot_mapping) {
        slot = a.slot_mapping[tok];
    } else {
        const int n_cap = a.max_blocks_per_seq * kBlockSize;
        const int n = min(a.context_lens[tok], n_cap);
        if (n >= 1) {
            const int phys = a.block_tables[tok * a.max_blocks_per_seq + (n - 1) / kBlockSize];
            slot = phys < 0 ? -1 : (int64_t)phys * kBlockSize + (n - 1) % kBlockSize;
        }
    }
    if (slot < 0 || slot >= a.num_blocks * kBlockSize) return;
    const int64_t blk = slot / kBlockSize, off = slot % kBlockSize;
    const size_t src = (size_t)row * D + (size_t)j * 8;
    const size_t dst_row = ((size_t)blk * a.num_kv_heads + h) * kBlockSize + (size_t)off;
    const size_t dst = dst_row * D + (size_t)j * 8;

    if constexpr (CE == Elem::U4) {
        Src8<SE> k, v;
        k.load(a.k, src);
        v.load(a.v, src);
        k.widen();
        v.widen();
        float klo, kr, vlo, vr;
        const uint32_t kc = quantize8_u4<LPR>(k.x, klo, kr);
        const uint32_t vc = quantize8_u4<LPR>(v.x, vlo, vr);
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.k_cache) + dst / 2) = kc;
        *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.v_cache) + dst / 2) = vc;
        if (j == 0) {
            *reinterpret_cast<float2*>(a.k_scale + 2 * dst_row) = make_float2(klo, kr);
            *reinterpret_cast<float2*>(a.v_scale + 2 * dst_row) = make_float2(vlo, vr);
        }
    } else if constexpr (is_scaled(CE)) {
        Src8<SE> k, v;
        k.load(a.k, src);
        v.load(a.v, src);
        k.widen();
        v.widen();
        float ks, vs;
        const uint2 kc = quantize8<CE, LPR>(k.x, ks);
        const uint2 vc = quantize8<CE, LPR>(v.x, vs);
        *reinterpret_cast<uint2*>(static_cast<int8_t*>(a.k_cache) + dst) = kc;
        *reinterpret_cast<uint2*>(static_cast<int8_t*>(a.v_cache) + dst) = vc;
        if (j == 0) {
            a.k_scale[dst_row] = ks;
            a.v_scale[dst_row] = vs;
        }
    } else {
        // plain copy of this lane's 8 elements (16 or 32 bytes)
        constexpr int kChunks = ElemInfo<SE>::bytes * 8 / 16;
        constexpr size_t EB = ElemInfo<SE>::bytes;
        const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(a.k) + src * EB);
        const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(a.v) + src * EB);
        uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(a.k_cache) + dst * EB);
        uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(a.v_cache) + dst * EB);
        uint4 kx[kChunks], vx[kChunks];
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            kx[i] = ks[i];
            vx[i] = vs[i];
        }
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            kd[i] = kx[i];
            vd[i] = vx[i];
        }
    }
}

template <Elem SE, Elem CE>
hipError_t launch_d(const CacheWriteArgs& a, int d, hipStream_t s) {
    const int64_t n_rows = a.num_tokens * a.num_kv_heads;
    if (n_rows == 0) return hipSuccess;
    const int rpb = kThreads / (d / 8);
    const int64_t n_wg = (n_rows + rpb - 1) / rpb;
    if (n_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)n_wg), block(kThreads);
    switch (d) {
    case 64: hipLaunchKernelGGL((kv_cache_write_kernel<SE, CE, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((kv_cache_write_kernel<SE, CE, 128>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((kv_cache_write_kernel<SE, CE, 256>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_cache_write(const CacheWriteArgs& a, int src_dtype, int cache_dtype,
                                 int head_dim, hipStream_t stream) {
    const Elem se = static_cast<Elem>(src_dtype), ce = static_cast<Elem>(cache_dtype);
    if (ce == se) {
        switch (se) {
        case Elem::F32: return launch_d<Elem::F32, Elem::F32>(a, head_dim, stream);
        case Elem::F16: return launch_d<Elem::F16, Elem::F16>(a, head_dim, stream);
        case Elem::BF16: return launch_d<Elem::BF16, Elem::BF16>(a, head_dim, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (ce == Elem::I8) {
        switch (se) {
        case Elem::F32: return launch_d<Elem::F32, Elem::I8>(a, head_dim, stream);
        case Elem::F16: return launch_d<Elem::F16, Elem::I8>(a, head_dim, stream);
        case Elem::BF16: return launch_d<Elem::BF16, Elem::I8>(a, head_dim, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (ce == Elem::U4) {
        switch (se) {
        case Elem::F32: return launch_d<Elem::F32, Elem::U4>(a, head_dim, stream);
        case Elem::F16: return launch_d<Elem::F16, Elem::U4>(a, head_dim, stream);
        case Elem::BF16: return launch_d<Elem::BF16, Elem::U4>(a, head_dim, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (ce == Elem::F8) {
        switch (se) {
        case Elem::F32: return launch_d<Elem::F32, Elem::F8>(a, head_dim, stream);
        case Elem::F16: return launch_d<Elem::F16, Elem::F8>(a, head_dim, stream);
        case Elem::BF16: return launch_d<Elem::BF16, Elem::F8>(a, head_dim, stream);
        default: return hipErrorInvalidValue;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
