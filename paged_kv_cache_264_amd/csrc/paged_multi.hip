// Causal attention of several query tokens per sequence over the paged KV
// cache, for gfx950 (CDNA4, wave64, MFMA).
//
// What is computed: sequence b holds N_b cached tokens whose last q_len_b are
// its queries (the k draft tokens that the target model checks in one pass
// when decoding speculatively: caojiahao2.github.io section 6; lazyllm lesson
// 4, the speculative-decoding algorithm; or a chunk of a prompt).  Query j sits
// at position p = N_b - q_len_b + j and attends to positions 0..p:
//     out[row][h] = softmax(scale * q[row][h] . K[0..p]^T) V[0..p]
// The cache is read through the block table (docs.lazyllm.ai lesson 4,
// section 4.2) and reduced with an online softmax over 16-token blocks
// (caojiahao2.github.io section 3.2; FlashAttention's tiling and fused
// score / mask / softmax / value steps, lecture 13 notes).
//
// Mapping onto the hardware: with several queries per kv head, q.K^T is a
// dense contraction, so it runs on the matrix cores.
//   * rows: the (query token, q head) pairs that read one kv head, 16 per
//     tile; a work-group is one (sequence, kv head, row tile, partition) with
//     4 waves, each streaming a contiguous run of the partition's blocks.
//   * scores: S^T = K Q^T, one v_mfma_f32_16x16x32 per 32 channels.  The A
//     operand is the K tile itself (lane l: token l%16, 8 channels), loaded
//     straight from the pool with raw buffer loads; the B operand is Q,
//     loaded once.  The C layout puts a query's 16 scores in the 4 lanes
//     l%16 = query, so the online-softmax max / sum need two lane swaps.
//   * the same C layout is the A operand of v_mfma_f32_16x16x16 for P V, so
//     P never leaves registers.  V is staged in a per-wave LDS tile (row
//     stride 2D + 16 bytes: the 4 lane groups of a transposed read fall on
//     different banks) and read back as the B operand.
//   * tokens past a query's position, past the partition or past the context
//     are masked by select; the 4 waves are merged through LDS at the end.
//     Sequences with one partition write the output directly, longer ones
//     write (m, l, o) partials for the merge kernel.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));

constexpr int kRows = 16;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegBig = -3.0e38f;
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer access
constexpr int kNonTemporal = 2;

template <Elem T> struct Mfma;
template <> struct Mfma<Elem::F16> {
    static __device__ __forceinline__ f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                     __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        const _Float16 a = (_Float16)x, b = (_Float16)y;
        return (uint32_t)__builtin_bit_cast(uint16_t, a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
};
template <> struct Mfma<Elem::BF16> {
    static __device__ __forceinline__ f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                       0);
    }
    static __device__ __forceinline__ f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                         __builtin_bit_cast(s16x4_t, b), c, 0, 0,
                                                         0);
    }
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        const __bf16 a = (__bf16)x, b = (__bf16)y;
        return (uint32_t)__builtin_bit_cast(uint16_t, a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                             kBufferWord3);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <Elem T, int D>
__global__ __launch_bounds__(kThreads) void paged_multi_kernel(MultiArgs a) {
    constexpr int KK = D / 32;          // 16x16x32 MFMAs per score tile
    constexpr int NN = D / 16;          // 16x16x16 MFMAs (output column tiles) per block
    constexpr int VL = D / 32;          // 16-byte V loads per lane per block
    constexpr int ROW = D * 2;          // bytes per token row
    constexpr int TILE = kRows * ROW;   // bytes per (block, kv head) tile
    constexpr int VS = ROW + 16;        // LDS row stride of the staged V tile

    // LDS: the per-wave V stage during the loop, then (same bytes) the output
    // tiles of waves 1..3 for the final merge
    constexpr int kStage = kWaves * kRows * VS;
    constexpr int kMerge = (kWaves - 1) * kRows * D * 4;
    __shared__ __attribute__((aligned(16))) char s_buf[kStage > kMerge ? kStage : kMerge];
    __shared__ float s_m[kWaves][kRows];
    __shared__ float s_l[kWaves][kRows];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4;          // lane group 0..3
    const int col = lane & 15;          // query row (B / C column) of this lane

    // (partition fastest, then row tile, then kv head, then sequence)
    const int NP = a.num_partitions;
    int rest = blockIdx.x;
    const int part = rest % NP;
    rest /= NP;
    const int rt = rest % a.row_tiles;
    rest /= a.row_tiles;
    const int kvh = rest % a.num_kv_heads;
    const int b = rest / a.num_kv_heads;

    const int Hq = a.num_q_heads;
    const int g = Hq / a.num_kv_heads;
    const int q0 = a.query_start_loc[b];
    // query rows must lie in [0, T): a malformed query_start_loc skips rows
    const int q1 = min(a.query_start_loc[b + 1], a.num_tokens);
    const int qlen = a.query_start_loc[b + 1] - q0;  // positions follow the given count
    const int rows_total = q0 < 0 ? 0 : max(0, q1 - q0) * g;
    if (rt * kRows >= rows_total) return;
    const int n_cap = a.max_blocks_per_seq * kBlockSize;
    int n = a.context_lens[b];
    n = n < 0 ? 0 : (n > n_cap ? n_cap : n);
    const int n_parts = partition_count(n, a.partition_size);
    const bool direct_out = n_parts <= 1;
    if (part >= (n_parts > 0 ? n_parts : 1)) return;
    const int span = n_parts > 0 ? partition_span(n, n_parts) : 0;
    const int t_begin = part * span;
    const int t_end = min(n, t_begin + span);

    // this lane's query row (B operand and softmax state)
    const int R = rt * kRows + col;
    const bool row_ok = R < rows_total;
    const int jq = row_ok ? R / g : 0;
    const int hq = kvh * g + (row_ok ? R % g : 0);
    const int pos = n - qlen + jq;      // the query attends to positions 0..pos

    uint4 qv[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qv[kk] = make_uint4(0u, 0u, 0u, 0u);
        if (row_ok)
            qv[kk] = *reinterpret_cast<const uint4*>(
                static_cast<const char*>(a.q) +
                (((size_t)(q0 + jq) * Hq + hq) * D + kk * 32 + grp * 8) * 2);
    }

    float m = kNegBig, l = 0.f;
    f32x4_t o[NN];
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // this wave's contiguous run of the partition's blocks
    const int blk_begin = t_begin / kBlockSize;
    const int blk_end = (t_end + kBlockSize - 1) / kBlockSize;
    const int nblk = blk_end - blk_begin;
    const int per_wave = (nblk + kWaves - 1) / kWaves;
    const int my0 = blk_begin + wave * per_wave;
    const int n_my = max(0, min(per_wave, blk_end - my0));
    const int32_t* table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
    const float c = a.scale_log2;
    char* vst = s_buf + wave * kRows * VS;

    struct Regs {
        uint4 k[KK], v[VL];
        int jb;
        bool ok;
    };
    auto load = [&](Regs& r, int i) {
        r.jb = my0 + i;
        const int phys = i < n_my ? table[my0 + i] : -1;
        r.ok = i < n_my && phys >= 0 && (int64_t)phys < a.num_blocks;
        const size_t tile = (size_t)(r.ok ? phys : 0) * a.num_kv_heads + kvh;
        const int bytes = r.ok ? TILE : 0;
        const __amdgpu_buffer_rsrc_t kr = rsrc(static_cast<const char*>(a.k_cache) + tile * TILE, bytes);
        const __amdgpu_buffer_rsrc_t vr = rsrc(static_cast<const char*>(a.v_cache) + tile * TILE, bytes);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) r.k[kk] = ld16(kr, col * ROW + (kk * 32 + grp * 8) * 2);
#pragma unroll
        for (int u = 0; u < VL; ++u) r.v[u] = ld16(vr, (u * 64 + lane) * 16);
    };
    auto compute = [&](const Regs& r) {
        // S^T[token 4*grp + i][query col]
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s = Mfma<T>::qk(r.k[kk], qv[kk], s);
        float sv[4];
        float mx = kNegBig;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = r.jb * kBlockSize + grp * 4 + i;
            const bool valid = r.ok && row_ok && t < t_end && t <= pos;
            sv[i] = valid ? s[i] * c : -INFINITY;
            mx = fmaxf(mx, sv[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mn);
        float p[4], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(sv[i] - mn);
            ps += p[i];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        l = fmaf(l, alpha, ps);
        m = mn;
        // rows of the O tile held by this lane are queries 4*grp + i
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, grp * 4 + i);
        // stage V (natural layout) in this wave's LDS tile; rows past the
        // partition are zeroed (their weight is 0, but 0 * NaN would not be)
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            const int ch = u * 64 + lane;                  // 16-byte chunk of the tile
            const int tok = ch / (D / 8), d0 = (ch % (D / 8)) * 8;
            const bool keep = r.jb * kBlockSize + tok < t_end;
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            const uint4 v = r.v[u];
            *reinterpret_cast<uint4*>(vst + tok * VS + d0 * 2) =
                make_uint4(keep ? v.x : z.x, keep ? v.y : z.y, keep ? v.z : z.z, keep ? v.w : z.w);
        }
        __asm__ volatile("" ::: "memory");
        const uint2 pa = make_uint2(Mfma<T>::pack(p[0], p[1]), Mfma<T>::pack(p[2], p[3]));
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
            const char* base = vst + (grp * 4) * VS + (nn * 16 + col) * 2;
            const uint32_t v0 = *reinterpret_cast<const uint16_t*>(base);
            const uint32_t v1 = *reinterpret_cast<const uint16_t*>(base + VS);
            const uint32_t v2 = *reinterpret_cast<const uint16_t*>(base + 2 * VS);
            const uint32_t v3 = *reinterpret_cast<const uint16_t*>(base + 3 * VS);
            const uint2 vb = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
#pragma unroll
            for (int i = 0; i < 4; ++i) o[nn][i] *= al[i];
            o[nn] = Mfma<T>::pv(pa, vb, o[nn]);
        }
        __asm__ volatile("" ::: "memory");
    };

    if (n_my > 0) {
        Regs ra, rb;
        load(ra, 0);
        for (int i = 0; i < n_my; i += 2) {
            load(rb, i + 1);
            compute(ra);
            load(ra, i + 2);
            if (i + 1 < n_my) compute(rb);
        }
    }

    // ---- merge the 4 waves (wave 0 keeps its tile in registers) ------------
    __syncthreads();  // every wave is done with its V stage
    float* s_o = reinterpret_cast<float*>(s_buf);  // [wave - 1][row][D]
    if (grp == 0) {
        s_m[wave][col] = m;
        s_l[wave][col] = l;
    }
    if (wave > 0) {
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_o[((wave - 1) * kRows + grp * 4 + i) * D + nn * 16 + col] = o[nn][i];
    }
    __syncthreads();
    if (wave != 0) return;

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int qr = grp * 4 + i;                 // query row of o[.][i]
        const int Rr = rt * kRows + qr;
        if (Rr >= rows_total) continue;
        float M = kNegBig;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][qr]);
        float f[kWaves], L = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            f[w] = fast_exp2(s_m[w][qr] - M);
            L = fmaf(s_l[w][qr], f[w], L);
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const size_t orow = (size_t)(q0 + Rr / g) * Hq + kvh * g + Rr % g;
        const size_t pi = orow * NP + part;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
            const int d = nn * 16 + col;
            float O = o[nn][i] * f[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) O = fmaf(s_o[((w - 1) * kRows + qr) * D + d], f[w], O);
            if (direct_out)
                store_elem<T>(a.out, orow * D + d, O * inv);
            else
                a.o_part[pi * D + d] = O * inv;
        }
        if (!direct_out && col == 0) {
            a.m_part[pi] = M * kLn2;
            a.l_part[pi] = L;
        }
    }
}

// Long runs of queries (prefill chunks): a work-group owns 4 waves x RW row
// tiles of 16 rows and walks every block of its partition up to the last
// position any of its rows attends to.  Each 16-token K/V block is fetched
// once per work-group (one 16-byte chunk per thread), staged in
// double-buffered padded LDS tiles, and every wave reads the K operand and the
// V operand once per block and reuses them for its RW row tiles; one barrier
// per block.  Each wave owns its rows for the whole partition, so there is no
// merge between waves.
template <Elem T, int D, int RW>
__global__ __launch_bounds__(kThreads) void paged_multi_tiled_kernel(MultiArgs a) {
    constexpr int KK = D / 32;
    constexpr int NN = D / 16;
    constexpr int ROW = D * 2;
    constexpr int TILE = kRows * ROW;
    constexpr int LS = ROW + 16;                    // padded LDS row stride
    constexpr int CH = TILE / 16;                   // 16-byte chunks per tile
    constexpr int CPT = (CH + kThreads - 1) / kThreads;
    constexpr int WG_ROWS = kWaves * kRows * RW;

    __shared__ __attribute__((aligned(16))) char s_k[2][kRows * LS];
    __shared__ __attribute__((aligned(16))) char s_v[2][kRows * LS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4;
    const int col = lane & 15;

    const int NP = a.num_partitions;
    int rest = blockIdx.x;
    const int part = rest % NP;
    rest /= NP;
    const int rg = rest % a.row_tiles;
    rest /= a.row_tiles;
    const int kvh = rest % a.num_kv_heads;
    const int b = rest / a.num_kv_heads;

    const int Hq = a.num_q_heads;
    const int g = Hq / a.num_kv_heads;
    const int q0 = a.query_start_loc[b];
    const int q1 = min(a.query_start_loc[b + 1], a.num_tokens);
    const int qlen = a.query_start_loc[b + 1] - q0;
    const int rows_total = q0 < 0 ? 0 : max(0, q1 - q0) * g;
    const int wg_r0 = rg * WG_ROWS;
    if (wg_r0 >= rows_total) return;
    const int n_cap = a.max_blocks_per_seq * kBlockSize;
    int n = a.context_lens[b];
    n = n < 0 ? 0 : (n > n_cap ? n_cap : n);
    const int n_parts = partition_count(n, a.partition_size);
    const bool direct_out = n_parts <= 1;
    if (part >= (n_parts > 0 ? n_parts : 1)) return;
    const int span = n_parts > 0 ? partition_span(n, n_parts) : 0;
    const int t_begin = part * span;
    const int t_end = min(n, t_begin + span);
    // the last position any row of this work-group attends to
    const int r_last = min(wg_r0 + WG_ROWS, rows_total) - 1;
    const int t_stop = min(t_end, max(n - qlen + r_last / g + 1, 0));
    const int blk_begin = t_begin / kBlockSize;
    const int blk_stop = t_stop > t_begin ? (t_stop + kBlockSize - 1) / kBlockSize : blk_begin;
    const int32_t* table = a.block_tables + (size_t)b * a.max_blocks_per_seq;
    const float c = a.scale_log2;

    // this wave's row tiles
    const int w_r0 = wg_r0 + wave * kRows * RW;
    bool row_ok[RW];
    int pos[RW];
    uint4 qv[RW][KK];
    float m[RW], l[RW];
    f32x4_t o[RW][NN];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const int R = w_r0 + rr * kRows + col;
        row_ok[rr] = R < rows_total;
        const int jq = row_ok[rr] ? R / g : 0;
        const int hq = kvh * g + (row_ok[rr] ? R % g : 0);
        pos[rr] = n - qlen + jq;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qv[rr][kk] = make_uint4(0u, 0u, 0u, 0u);
            if (row_ok[rr])
                qv[rr][kk] = *reinterpret_cast<const uint4*>(
                    static_cast<const char*>(a.q) +
                    (((size_t)(q0 + jq) * Hq + hq) * D + kk * 32 + grp * 8) * 2);
        }
        m[rr] = kNegBig;
        l[rr] = 0.f;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) o[rr][nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    auto gload = [&](int jb, uint4 (&kc)[CPT], uint4 (&vc)[CPT]) {
        const int phys = table[jb];
        const bool ok = phys >= 0 && (int64_t)phys < a.num_blocks;
        const size_t tile = (size_t)(ok ? phys : 0) * a.num_kv_heads + kvh;
        const int bytes = ok ? TILE : 0;
        const __amdgpu_buffer_rsrc_t kr = rsrc(static_cast<const char*>(a.k_cache) + tile * TILE, bytes);
        const __amdgpu_buffer_rsrc_t vr = rsrc(static_cast<const char*>(a.v_cache) + tile * TILE, bytes);
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
            const int ch = cc * kThreads + tid;
            const int off = ch < CH ? ch * 16 : TILE;     // past the tile: reads zeros
            kc[cc] = ld16(kr, off);
            vc[cc] = ld16(vr, off);
        }
    };
    auto lstore = [&](int buf, int jb, const uint4 (&kc)[CPT], const uint4 (&vc)[CPT]) {
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
            const int ch = cc * kThreads + tid;
            if (ch < CH) {
                const int tok = ch / (ROW / 16), off = (ch % (ROW / 16)) * 16;
                // rows past the partition are zeroed: weight 0 times NaN would not be 0
                const bool keep = jb * kBlockSize + tok < t_end;
                const uint4 kx = kc[cc], vx = vc[cc];
                *reinterpret_cast<uint4*>(s_k[buf] + tok * LS + off) =
                    make_uint4(keep ? kx.x : 0u, keep ? kx.y : 0u, keep ? kx.z : 0u,
                               keep ? kx.w : 0u);
                *reinterpret_cast<uint4*>(s_v[buf] + tok * LS + off) =
                    make_uint4(keep ? vx.x : 0u, keep ? vx.y : 0u, keep ? vx.z : 0u,
                               keep ? vx.w : 0u);
            }
        }
    };
    auto compute = [&](int buf, int jb) {
        uint4 ka[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            ka[kk] = *reinterpret_cast<const uint4*>(s_k[buf] + col * LS + (kk * 32 + grp * 8) * 2);
        uint2 vb[NN];
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
            const char* base = s_v[buf] + (grp * 4) * LS + (nn * 16 + col) * 2;
            const uint32_t v0 = *reinterpret_cast<const uint16_t*>(base);
            const uint32_t v1 = *reinterpret_cast<const uint16_t*>(base + LS);
            const uint32_t v2 = *reinterpret_cast<const uint16_t*>(base + 2 * LS);
            const uint32_t v3 = *reinterpret_cast<const uint16_t*>(base + 3 * LS);
            vb[nn] = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
        }
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s = Mfma<T>::qk(ka[kk], qv[rr][kk], s);
            float sv[4], mx = kNegBig;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = jb * kBlockSize + grp * 4 + i;
                const bool valid = row_ok[rr] && t < t_end && t <= pos[rr];
                sv[i] = valid ? s[i] * c : -INFINITY;
                mx = fmaxf(mx, sv[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = fmaxf(m[rr], mx);
            const float alpha = fast_exp2(m[rr] - mn);
            float p[4], ps = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(sv[i] - mn);
                ps += p[i];
            }
            ps += __shfl_xor(ps, 16);
            ps += __shfl_xor(ps, 32);
            l[rr] = fmaf(l[rr], alpha, ps);
            m[rr] = mn;
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, grp * 4 + i);
            const uint2 pa = make_uint2(Mfma<T>::pack(p[0], p[1]), Mfma<T>::pack(p[2], p[3]));
#pragma unroll
            for (int nn = 0; nn < NN; ++nn) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[rr][nn][i] *= al[i];
                o[rr][nn] = Mfma<T>::pv(pa, vb[nn], o[rr][nn]);
            }
        }
    };

    if (blk_begin < blk_stop) {
        uint4 kc[CPT], vc[CPT];
        gload(blk_begin, kc, vc);
        lstore(0, blk_begin, kc, vc);
        __syncthreads();
        for (int jb = blk_begin; jb < blk_stop; ++jb) {
            const int buf = (jb - blk_begin) & 1;
            const bool more = jb + 1 < blk_stop;
            if (more) gload(jb + 1, kc, vc);
            compute(buf, jb);
            if (more) lstore(buf ^ 1, jb + 1, kc, vc);
            __syncthreads();
        }
    }

    // ---- epilogue: each wave writes its own rows ---------------------------
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qr = grp * 4 + i;
            const float lr = __shfl(l[rr], qr);
            const float mr = __shfl(m[rr], qr);
            const int R = w_r0 + rr * kRows + qr;
            if (R >= rows_total) continue;
            const float inv = lr > 0.f ? 1.f / lr : 0.f;
            const size_t orow = (size_t)(q0 + R / g) * Hq + kvh * g + R % g;
            const size_t pi = orow * NP + part;
#pragma unroll
            for (int nn = 0; nn < NN; ++nn) {
                const int d = nn * 16 + col;
                if (direct_out)
                    store_elem<T>(a.out, orow * D + d, o[rr][nn][i] * inv);
                else
                    a.o_part[pi * D + d] = o[rr][nn][i] * inv;
            }
            if (!direct_out && col == 0) {
                a.m_part[pi] = mr * kLn2;
                a.l_part[pi] = lr;
            }
        }
    }
}

constexpr int kTiledRW = 2;                 // row tiles per wave in the tiled kernel
constexpr int kTiledMinRows = 64;           // rows per (sequence, kv head) that select it

template <Elem T>
hipError_t launch_d(const MultiArgs& a, int d, int64_t grid, hipStream_t s) {
    const dim3 g((unsigned)grid), blk(kThreads);
    switch (d) {
    case 64: hipLaunchKernelGGL((paged_multi_kernel<T, 64>), g, blk, 0, s, a); break;
    case 128: hipLaunchKernelGGL((paged_multi_kernel<T, 128>), g, blk, 0, s, a); break;
    case 256: hipLaunchKernelGGL((paged_multi_kernel<T, 256>), g, blk, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <Elem T>
hipError_t launch_tiled(const MultiArgs& a, int d, int64_t grid, hipStream_t s) {
    const dim3 g((unsigned)grid), blk(kThreads);
    switch (d) {
    case 64: hipLaunchKernelGGL((paged_multi_tiled_kernel<T, 64, kTiledRW>), g, blk, 0, s, a); break;
    case 128: hipLaunchKernelGGL((paged_multi_tiled_kernel<T, 128, kTiledRW>), g, blk, 0, s, a); break;
    case 256: hipLaunchKernelGGL((paged_multi_tiled_kernel<T, 256, 1>), g, blk, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int64_t multi_row_groups(int max_rows, int head_dim) {
    if (max_rows < kTiledMinRows) return (max_rows + kRows - 1) / kRows;
    const int rw = head_dim == 256 ? 1 : kTiledRW;
    const int per = kWaves * kRows * rw;
    return (max_rows + per - 1) / per;
}

hipError_t launch_paged_multi(const MultiArgs& a, int dtype, int head_dim, hipStream_t stream) {
    const int64_t grid =
        (int64_t)a.num_seqs * a.num_kv_heads * a.row_tiles * a.num_partitions;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool tiled = a.max_rows >= kTiledMinRows;
    const Elem e = static_cast<Elem>(dtype);
    if (e == Elem::F16)
        return tiled ? launch_tiled<Elem::F16>(a, head_dim, grid, stream)
                     : launch_d<Elem::F16>(a, head_dim, grid, stream);
    if (e == Elem::BF16)
        return tiled ? launch_tiled<Elem::BF16>(a, head_dim, grid, stream)
                     : launch_d<Elem::BF16>(a, head_dim, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
