// Kernels that measure the rates this GPU reaches on the resources the
// attention kernels are bound by, as context for their roofline fractions:
// no attention arithmetic, no output beyond a word that keeps the work alive.
//   * stream_read_kernel: a plain streaming read of one contiguous buffer,
//     each work-group a contiguous chunk, four 16-byte non-temporal loads
//     per lane in flight.
//   * tile_read_kernel: the decode's own access pattern: one work-group per
//     (sequence, kv head) item, items in the order the caller lists them,
//     eight waves (as the decode's single-head tiles) each walking a
//     contiguous run of the sequence's blocks
//     through its block table with two blocks in flight, each block one
//     (block, kv head) tile of K and one of V, read up to the context's last
//     token (buffer windows, as in the decode).
//   * mfma_rate_kernel: back-to-back independent 16x16x32 fp16 MFMAs, eight
//     accumulators per wave, no memory traffic: the sustained matrix-core
//     rate (clock included) under a load like the prefill kernel's.
//   * lds_rate_kernel: the prefill kernel's LDS operand reads (the 16-byte K
//     reads and the V^T transpose reads) on either of its two tile layouts.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;           // the streaming read
constexpr int kTileWaves = 8;           // the tile read (measured: 8 waves 6.63 TB/s, 4 waves
                                        // 6.48, 8 waves over 2/4/8 adjacent kv heads 6.44/6.19/5.87
                                        // on the LLaMA-7B-shaped batch)
constexpr unsigned kMagic = 0x9e3779b9u;   // a fold value that real data never produces in practice

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2 /* non-temporal */);
}

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* src, int64_t bytes,
                                                               int64_t chunk, unsigned* sink) {
    const int64_t begin = (int64_t)blockIdx.x * chunk;
    const int64_t end = begin + chunk < bytes ? begin + chunk : bytes;
    u32x4 acc = {0u, 0u, 0u, 0u};
    constexpr int kStep = kThreads * 16 * 4;
    for (int64_t off = begin; off < end; off += kStep) {
        const int64_t left = end - off;
        const __amdgpu_buffer_rsrc_t r = window(src + off, (int)(left < kStep ? left : kStep));
        u32x4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = ld16(r, (u * kThreads + (int)threadIdx.x) * 16);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= x[u];
    }
    const unsigned f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == kMagic) sink[0] = f;
}

__global__ __launch_bounds__(kTileWaves * 64) void tile_read_kernel(TileReadArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int2 it = a.items[blockIdx.x];
    const int b = it.x, kvh = it.y;
    if (b < 0 || b >= a.num_seqs || kvh < 0 || kvh >= a.num_kv_heads) return;  // bad item: skipped
    int n = a.context_lens[b];
    const int n_cap = a.max_blocks_per_seq * kBlockSize;
    n = n < 0 ? 0 : (n > n_cap ? n_cap : n);
    const int nblk = (n + kBlockSize - 1) / kBlockSize;
    const int per = (nblk + kTileWaves - 1) / kTileWaves;
    const int j0 = wave * per, j1 = min(nblk, j0 + per);
    const int32_t* table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
    const int row = a.tile_bytes / kBlockSize;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int j = j0; j < j1; j += 2) {
        u32x4 x[2][2][4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int jj = j + q;
            const int id = table[jj < j1 ? jj : j0];
            const bool ok = jj < j1 && id >= 0 && (int64_t)id < a.num_blocks;
            const int rows = __builtin_amdgcn_readfirstlane(
                ok ? min(max(n - jj * kBlockSize, 0), kBlockSize) : 0);
            const size_t tile = ((size_t)(ok ? id : 0) * a.num_kv_heads + kvh) * a.tile_bytes;
            const __amdgpu_buffer_rsrc_t rk = window(static_cast<const char*>(a.k_cache) + tile, rows * row);
            const __amdgpu_buffer_rsrc_t rv = window(static_cast<const char*>(a.v_cache) + tile, rows * row);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[q][0][u] = ld16(rk, (u * 64 + lane) * 16);
                x[q][1][u] = ld16(rv, (u * 64 + lane) * 16);
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u) acc ^= x[q][0][u] ^ x[q][1][u];
    }
    const unsigned f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == kMagic) a.sink[0] = f;
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// The MFMAs are written as instructions, so that the eight accumulators stay
// in place from round to round (the compiler moves builtin accumulators
// between register files here, three moves per MFMA).  No memory access; the
// drain before the accumulators are read covers the MFMA result latency.
__global__ __launch_bounds__(256) void mfma_rate_kernel(int rounds, unsigned* sink) {
    const int lane = threadIdx.x & 63;
    f16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(lane * 0.01f + i);
        b[i] = (_Float16)(i * 0.02f - lane * 0.001f);
    }
    f32x4_t c0 = {0.f, 0.5f, 0.25f, 0.125f}, c1 = c0 + 1.f, c2 = c0 + 2.f, c3 = c0 + 3.f,
            c4 = c0 + 4.f, c5 = c0 + 5.f, c6 = c0 + 6.f, c7 = c0 + 7.f;
#pragma unroll 1
    for (int r = 0; r < rounds; ++r) {
        asm volatile(
            "v_mfma_f32_16x16x32_f16 %0, %8, %9, %0\n"
            "v_mfma_f32_16x16x32_f16 %1, %8, %9, %1\n"
            "v_mfma_f32_16x16x32_f16 %2, %8, %9, %2\n"
            "v_mfma_f32_16x16x32_f16 %3, %8, %9, %3\n"
            "v_mfma_f32_16x16x32_f16 %4, %8, %9, %4\n"
            "v_mfma_f32_16x16x32_f16 %5, %8, %9, %5\n"
            "v_mfma_f32_16x16x32_f16 %6, %8, %9, %6\n"
            "v_mfma_f32_16x16x32_f16 %7, %8, %9, %7"
            : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
            : "v"(a), "v"(b));
    }
    asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
    const f32x4_t s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
    const unsigned f = __float_as_uint(s[0] + s[1] + s[2] + s[3]);
    if (f == kMagic) sink[0] = f;
}

// 512 threads over 32 KiB of LDS: eight 4 KiB tiles of 16 rows x 256 bytes
// (the prefill kernel's fp16 tile at head_dim 128).  Each wave reads 8 KiB
// per round, at its own tile offset.  Patterns: 0 the K operand read on the K
// layout (16-byte chunk c of row t at slot c ^ t), 1 the same read on the V
// layout (slot c ^ (2 (t & 7) + (((t & 7) >> 2) ^ (t >> 3)))), 2 the V^T
// transpose read on the V layout, 3 the transpose read on the K layout.
template <bool TR>
__global__ __launch_bounds__(512) void lds_rate_kernel(int rounds, int k_layout, unsigned* sink) {
    __shared__ __attribute__((aligned(16))) char lds[32768];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 32768 / 4; i += 512) reinterpret_cast<unsigned*>(lds)[i] = i * 2654435761u;
    __syncthreads();
    auto swz = [&](int t) {
        return k_layout ? (t & 15) : 2 * (t & 7) + (((t & 7) >> 2) ^ (t >> 3));
    };
    int off[8];
    if (!TR) {  // lane: token col, chunks 4 kk + grp; two tiles, kk = 0..3
        const int col = lane & 15, grp = lane >> 4;
#pragma unroll
        for (int j = 0; j < 8; ++j) off[j] = (j >> 2) * 4096 + col * 256 + 16 * (((j & 3) * 4 + grp) ^ swz(col));
    } else {    // lane: token 4 grp + (lane / 4) % 4, 8 bytes of chunks 2 nn, 2 nn + 1
        const int g = lane >> 4, t = 4 * g + ((lane >> 2) & 3), qa = lane & 3;
#pragma unroll
        for (int j = 0; j < 8; ++j) off[j] = t * 256 + 16 * ((2 * j + (qa >> 1)) ^ swz(t)) + 8 * (qa & 1);
    }
    unsigned acc = 0u;
#pragma unroll 1
    for (int r = 0; r < rounds; ++r) {
        const int base = ((r + wave) & 3) * 8192;  // <= 24576; offsets < 8192
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (!TR) {
                const uint4 x = *reinterpret_cast<const uint4*>(lds + base + off[j]);
                acc ^= x.x ^ x.y ^ x.z ^ x.w;
            } else {
                typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
                const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + base + off[j]));
                const s16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + base + 4096 + off[j]));
                acc ^= __builtin_bit_cast(uint2, x).x ^ __builtin_bit_cast(uint2, x).y ^
                       __builtin_bit_cast(uint2, y).x ^ __builtin_bit_cast(uint2, y).y;
            }
        }
    }
    if (acc == kMagic) sink[0] = acc;
}

}  // namespace

hipError_t launch_mfma_rate(int groups, int rounds, unsigned* sink, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)groups), dim3(256), 0, stream, rounds, sink);
    return hipGetLastError();
}

hipError_t launch_lds_rate(int pattern, int groups, int rounds, unsigned* sink, hipStream_t stream) {
    const int k_layout = pattern == 0 || pattern == 3;
    if (pattern < 2)
        hipLaunchKernelGGL(lds_rate_kernel<false>, dim3((unsigned)groups), dim3(512), 0, stream, rounds, k_layout, sink);
    else
        hipLaunchKernelGGL(lds_rate_kernel<true>, dim3((unsigned)groups), dim3(512), 0, stream, rounds, k_layout, sink);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, unsigned* sink, hipStream_t stream) {
    if (bytes <= 0) return hipSuccess;
    constexpr int64_t kWgs = 2048;
    int64_t chunk = (bytes + kWgs - 1) / kWgs;
    chunk = (chunk + 4095) / 4096 * 4096;
    const int64_t grid = (bytes + chunk - 1) / chunk;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       static_cast<const char*>(src), bytes, chunk, sink);
    return hipGetLastError();
}

hipError_t launch_tile_read(const TileReadArgs& a, hipStream_t stream) {
    if (a.num_items <= 0) return hipSuccess;
    hipLaunchKernelGGL(tile_read_kernel, dim3((unsigned)a.num_items), dim3(kTileWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
