// Whole-block copies inside the pool: the copy-on-write step of prefix
// sharing.  When a sequence writes into a partly filled block that other
// sequences of the same prompt still share, it continues in a private copy of
// that block (the sharing of prompt blocks between parallel samples or beams
// that the "Efficient AI Lecture 13" notes list among the advantages of
// PagedAttention).
//
// Layout: block b of the pool is one contiguous run of
// num_kv_heads * 16 * head_dim elements in k_cache and another in v_cache
// (plus num_kv_heads * 16 fp32 scales each for an INT8 cache), so a copy is a
// flat memcpy of that run.  One work-group moves one 16 KiB chunk of one run
// with four 16-byte loads per lane in flight, then four stores; the launch is
// pairs x chunks work-groups, a single extra work-group per pair moving the
// scale rows.  Pure streaming: HBM bound.  Loads and stores are non-temporal
// (measured on MI355X for 1024 LLaMA-7B block pairs: 6.27 TB/s moved vs 5.59
// with ordinary accesses, 5.37 for a device-to-device memcpy of the same
// bytes); more than four 16-byte accesses per lane, or a loop per work-group,
// measured slower.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kChunk = (int64_t)kThreads * 16 * kUnroll;   // bytes per work-group

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void copy_run(const char* src, char* dst, int64_t begin, int64_t end) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t off = begin + ((int64_t)u * kThreads + threadIdx.x) * 16;
        if (off < end) r[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + off));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t off = begin + ((int64_t)u * kThreads + threadIdx.x) * 16;
        if (off < end) __builtin_nontemporal_store(r[u], reinterpret_cast<u32x4*>(dst + off));
    }
}

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyBlocksArgs a, int chunks,
                                                               int per_pair) {
    const int64_t item = blockIdx.x;
    const int64_t pair = item / per_pair;
    const int r = (int)(item - pair * per_pair);
    const int32_t src = a.pairs[2 * pair];
    const int32_t dst = a.pairs[2 * pair + 1];
    if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks || src == dst) return;
    if (r < 2 * chunks) {
        const bool is_v = r >= chunks;
        const int64_t c = is_v ? r - chunks : r;
        const char* base = static_cast<const char*>(is_v ? a.v_cache : a.k_cache);
        char* out = static_cast<char*>(is_v ? a.v_cache : a.k_cache);
        const int64_t begin = c * kChunk;
        const int64_t end = begin + kChunk < a.block_bytes ? begin + kChunk : a.block_bytes;
        copy_run(base + src * a.block_bytes, out + dst * a.block_bytes, begin, end);
    } else {
        // both scale rows (INT8 cache only), 16 bytes per lane
        for (int64_t off = (int64_t)threadIdx.x * 16; off < 2 * a.scale_bytes;
             off += (int64_t)kThreads * 16) {
            const bool is_v = off >= a.scale_bytes;
            const int64_t o = is_v ? off - a.scale_bytes : off;
            char* s = reinterpret_cast<char*>(is_v ? a.v_scale : a.k_scale);
            *reinterpret_cast<uint4*>(s + dst * a.scale_bytes + o) =
                *reinterpret_cast<const uint4*>(s + src * a.scale_bytes + o);
        }
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
    if (a.num_pairs <= 0) return hipSuccess;
    const int64_t chunks = (a.block_bytes + kChunk - 1) / kChunk;
    const int64_t per_pair = 2 * chunks + (a.scale_bytes > 0 ? 1 : 0);
    const int64_t grid = a.num_pairs * per_pair;
    if (chunks > INT32_MAX / 4 || grid > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a,
                       (int)chunks, (int)per_pair);
    return hipGetLastError();
}

}  // namespace pkv
