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
//     4 waves (6 or 8 for one query per sequence), each streaming a contiguous run of the partition's blocks.
//   * scores: S^T = K Q^T, one v_mfma_f32_16x16x32 per 32 channels.  The A
//     operand is the K tile (lane l: token l%16, 8 channels), fetched from
//     the pool in token order and staged in a per-wave LDS tile; the B
//     operand is Q, loaded once.  The C layout puts a query's 16 scores in
//     the 4 lanes l%16 = query, so the online-softmax max / sum need two
//     lane swaps.
//   * the output is accumulated transposed, O^T = V^T P^T, on
//     v_mfma_f32_16x16x16: the score C layout is then the B operand as it
//     stands (P never leaves registers) and the accumulator column of a lane
//     is its own query, so rescaling needs no lane exchange.  V is staged in
//     a per-wave LDS tile in token order and read back as the V^T operand by
//     the LDS transpose read (see the long-run kernel below).
//   * the running max is shared by the 4 lanes of a query and reduced across
//     them only when a score exceeds it; each lane sums its own tokens and
//     the 4 partial sums are added once at the end.
//   * tokens past a query's position, past the partition or past the context
//     are masked by select; the waves are merged through LDS at the end.
//     Sequences with one partition write the output directly, longer ones
//     write (m, l, o) partials for the merge kernel.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_quant.h"

namespace pkv {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));

constexpr int kRows = 16;
// Waves per work-group of the short-run kernel.  Runs of several queries use
// 4 (8 measured slower on MI355X: verify 381.7 -> 389.2 us per launch,
// shared-prefix sampling decode 97.0 -> 98.8 us).  A single query per
// sequence (decode of 4-63 q heads per kv head) fills at most one 16-row
// tile, so its work-groups are few and short of loads in flight: more waves
// each stream a share of the item's blocks.  Over a 16-bit cache 6 (two
// work-groups of 168 registers fit a CU; against 8, one per CU: 64 q / 8 kv
// heads bf16 x 64 sequences 104.3 -> 103.2 us, 32 q / 4 kv heads 62.5 ->
// 59.9, 32 q / 2 kv heads x 16 19.6 -> 18.5); over a quantized cache 8
// (6 measured 3-17% slower: its per-block widening wants the waves).  Four
// waves measured slower for both (127.1 against 118.0 us at 8, bf16).
constexpr int kWavesRuns = 4;
constexpr int kWavesOneQuery16 = 6;
constexpr int kWavesOneQueryQ = 8;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegBig = -3.0e38f;
// The running max of a row is the reference the weights are taken against,
// exp2(c s - c m): any reference gives the same softmax once the sum and the
// output use the same one.  It is moved (and the sum and output rescaled)
// only when a score exceeds it by more than kSlack in exp2 units, so a weight
// is at most 2^kSlack (exact in fp32 and in the 16-bit P operand's range), and
// the rescale, which touches every output accumulator of the wave, runs about
// once per row after the first blocks instead of whenever a row's max grows.
constexpr float kSlack = 8.0f;
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer access
constexpr int kNonTemporal = 2;
constexpr unsigned kXcds = 8;              // accelerator complex dies of the chip
// s_waitcnt immediate that waits for at most n outstanding vector memory
// operations and for nothing else (gfx9 layout: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

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
    static __device__ __forceinline__ f32x4_t pv32(const uint4& a, const uint4& b, f32x4_t c) {
        return qk(a, b, c);
    }
    // two floats to a pair of fp16, nearest even (one v_cvt_pk_f16_f32)
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, f16x2_t));
    }
    // the pair back to floats (exact)
    static __device__ __forceinline__ void unpack(uint32_t w, float& x, float& y) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, w);
        x = (float)h[0];
        y = (float)h[1];
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
    static __device__ __forceinline__ f32x4_t pv32(const uint4& a, const uint4& b, f32x4_t c) {
        return qk(a, b, c);
    }
    // two floats to a pair of bf16, nearest even (one v_cvt_pk_bf16_f32)
    static __device__ __forceinline__ uint32_t pack(float x, float y) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
    }
    // the pair back to floats (exact: a bf16 is the top half of an fp32)
    static __device__ __forceinline__ void unpack(uint32_t w, float& x, float& y) {
        x = __builtin_bit_cast(float, w << 16);
        y = __builtin_bit_cast(float, w & 0xffff0000u);
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
// two 8-byte loads at off and off + 8 (arrays that are only 8-byte aligned)
// (the builtin returns a generic two-element vector, taken apart by
// subscript: assigned to an ext_vector_type, only its first element survived)
__device__ __forceinline__ float4 ld8x2(__amdgpu_buffer_rsrc_t r, int off) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    const auto b = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8, 0, 0);
    return make_float4(__builtin_bit_cast(float, (unsigned)a[0]), __builtin_bit_cast(float, (unsigned)a[1]),
                       __builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}
// 16 bytes per lane from the buffer straight into LDS: lane l's land at
// lds + 16 l (lds is wave-uniform); bytes outside the buffer window arrive
// as zeros.  Counted by vmcnt, like any vector memory load.
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, char* lds, int voffset) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voffset, 0, 0, 0);
}

// Two e4m3 codes (bytes 0, 1 of w, or 2, 3 with HI) as a pair of T, exactly
// (gfx950's scaled convert with scale 1: every non-NaN code pair, both word
// selects and both output types, matched the fp32 convert and a round-trip
// pack on the GPU)
template <Elem T, bool HI> __device__ __forceinline__ uint32_t fp8x2_to(uint32_t w) {
    if constexpr (T == Elem::F16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// 16 codes of an 8-bit cache (INT8, or e4m3 FP8) as 16 values of the 16-bit
// MFMA type T, in order: both formats' values are exact in fp16 and in bf16
// (integers up to 127; e4m3's 4 significant bits and exponents 2^-9..2^8)
template <Elem T, Elem CE>
__device__ __forceinline__ void widen16(const uint4& w, uint4& lo, uint4& hi) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (CE == Elem::F8) {
            out[2 * i] = fp8x2_to<T, false>(in[i]);
            out[2 * i + 1] = fp8x2_to<T, true>(in[i]);
        } else {  // byte-select converts of the sign-extended codes, then a pack
            out[2 * i] = Mfma<T>::pack((float)(int8_t)(in[i] & 0xffu),
                                       (float)(int8_t)((in[i] >> 8) & 0xffu));
            out[2 * i + 1] = Mfma<T>::pack((float)(int8_t)((in[i] >> 16) & 0xffu),
                                           (float)(int8_t)(in[i] >> 24));
        }
    }
    lo = make_uint4(out[0], out[1], out[2], out[3]);
    hi = make_uint4(out[4], out[5], out[6], out[7]);
}

// 32 codes of a 4-bit cache (two per byte, element 2k in the low nibble of
// byte k) as 32 values code * 2^-9 of the 16-bit type T, in order: a byte c
// <= 15 read as an e4m3 code is exactly c * 2^-9 (1..7 the subnormals, 8..15
// the normals of exponent -6), so one scaled fp8 convert widens two codes
template <Elem T>
__device__ __forceinline__ void widen32_u4(const uint4& w, uint4 out[4]) {
    const uint32_t in[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = in[i] & 0x0F0F0F0Fu;         // elements 8i, 8i+2, 8i+4, 8i+6
        const uint32_t hi = (in[i] >> 4) & 0x0F0F0F0Fu;  // elements 8i+1, 8i+3, ..
        // bytes in element order: (8i, 8i+1, 8i+2, 8i+3) and (8i+4, .., 8i+7)
        const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
        const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        out[i] = make_uint4(fp8x2_to<T, false>(a), fp8x2_to<T, true>(a), fp8x2_to<T, false>(b),
                            fp8x2_to<T, true>(b));
    }
}
constexpr float kU4Unscale = 512.0f;        // undoes widen32_u4's 2^-9
constexpr float kInv15 = 1.0f / 15.0f;      // 4-bit step = range / 15

// T: the q (and MFMA operand) type; CE: the cache's, T itself, an 8-bit
// format with an fp32 scale per (slot, kv head), or 4-bit codes with an
// fp32 (x_min, range) per (slot, kv head), widened to T as the tiles are
// staged.  XP: the weights enter P.V as two 16-bit parts
// (MultiArgs::exact_p)
template <Elem T, Elem CE, int D, bool XP, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void paged_multi_kernel(MultiArgs a) {
    constexpr int kThreads = kWaves * 64;
    constexpr bool kQ8 = CE == Elem::I8 || CE == Elem::F8;
    constexpr bool kU4 = CE == Elem::U4;
    static_assert(CE == T || kQ8 || kU4, "cache of the q type, 8-bit or 4-bit");
    constexpr int KK = D / 32;          // 16x16x32 MFMAs per score tile
    constexpr int NN = D / 16;          // 16x16x16 MFMAs (output column tiles) per block
    constexpr int ROW = D * 2;          // bytes per staged (16-bit) token row
    constexpr int CROW = kU4 ? D / 2 : kQ8 ? D : ROW;  // bytes per token row in the cache
    constexpr int CTILE = kRows * CROW; // cache bytes per (block, kv head) tile
    constexpr int VL = CTILE / 1024;    // 16-byte loads per lane per tile
    static_assert(VL >= 1, "a tile is at least one 1 KiB wave load");
    constexpr int CPR = CROW / 16;      // 16-byte chunks per cache row
    constexpr int WID = kU4 ? 64 : kQ8 ? 32 : 16;  // staged bytes per 16-byte cache chunk
    // LDS row stride of the staged V tile: the 16 lanes of a transpose read
    // address 4 tokens x 4 channel quads; rows 8 words apart (mod 64) put
    // them on distinct banks
    constexpr int VS = ROW + 32;
    // LDS row stride of the staged K tile: 16 lanes reading 16 bytes of 16
    // token rows fall on distinct banks
    constexpr int KS = ROW + 16;

    // LDS: the per-wave K and V stages during the loop, then (same bytes) the
    // output tiles of waves 1.. for the final merge
    constexpr int kStage = kWaves * kRows * (VS + KS);
    constexpr int kMerge = (kWaves - 1) * kRows * D * 4;
    __shared__ __attribute__((aligned(16))) char s_buf[kStage > kMerge ? kStage : kMerge];
    __shared__ float s_m[kWaves][kRows];
    __shared__ float s_l[kWaves][kRows];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4;          // lane group 0..3
    const int col = lane & 15;          // query row (B / C column) of this lane

    // (partition fastest, then row tile, then kv head, then sequence), the
    // sequences in longest-first order (by partition length) so that the
    // work-groups dispatched last are the shortest; every work-group ranks
    // the sequences itself (one per thread, keys read eight per LDS round
    // trip)
    const int NP = a.num_partitions;
    int rest = blockIdx.x;
    const int part = rest % NP;
    rest /= NP;
    const int rt = rest % a.row_tiles;
    rest /= a.row_tiles;
    int kvh = rest % a.num_kv_heads;
    int b = rest / a.num_kv_heads;
    // With one work-group per (sequence, kv head), work-groups go to the 8
    // XCDs round-robin and XCD x would read kv heads x, x + 8, ...; taken
    // through the decode kernel's bijection it reads heads 2 x and 2 x + 1
    // of each 16, whose tiles of a block lie next to each other in the pool
    // (verify workload: 381.7 against 389.5 us per launch, same output).
    if (NP * a.row_tiles == 1 && (a.num_kv_heads & 15) == 0)
        kvh = (kvh & ~15) | ((kvh >> 3) & 1) | ((kvh & 7) << 1);
    static_assert(kThreads >= kScheduleMaxSeqs, "one thread per ranked sequence");
    __shared__ __align__(16) int s_key[kScheduleMaxSeqs];
    __shared__ int s_order[kScheduleMaxSeqs];
    // a key packs the partition span in blocks above 255 - index (longer
    // first, then lower index): distinct keys, and a branch-free rank
    if (a.num_seqs <= kScheduleMaxSeqs && a.max_blocks_per_seq < (1 << 23)) {
        const int n_cap0 = a.max_blocks_per_seq * kBlockSize;
        int key = -1;
        if (threadIdx.x < a.num_seqs) {
            int s0 = threadIdx.x;
            if (a.group_rows) {  // a group's context is its first member's
                s0 = a.query_start_loc[threadIdx.x];
                s0 = s0 >= 0 && s0 < a.num_tokens ? s0 : -1;
            }
            const int nn = s0 < 0 ? 0 : min(max(a.context_lens[s0], 0), n_cap0);
            const int c = partition_count(nn, a.partition_size);
            key = (c > 0 ? partition_span(nn, c) / kBlockSize : 0) << 8 | (255 - threadIdx.x);
        }
        // every entry is written; those past the batch (key -1) rank nothing
        if (threadIdx.x < kScheduleMaxSeqs) s_key[threadIdx.x] = key;
        __syncthreads();
        if (threadIdx.x < a.num_seqs) {
            int r = 0;
            const int nj = (a.num_seqs + 3) & ~3;  // <= kScheduleMaxSeqs
#pragma unroll 2
            for (int j = 0; j < nj; j += 4) {
                const int4 kk = *reinterpret_cast<const int4*>(&s_key[j]);
                r += (kk.x > key) + (kk.y > key) + (kk.z > key) + (kk.w > key);
            }
            s_order[r] = threadIdx.x;
        }
        __syncthreads();
        b = s_order[b];
    }

    const int Hq = a.num_q_heads;
    const int g = Hq / a.num_kv_heads;
    const int q0 = a.one_query ? b : a.query_start_loc[b];
    // query rows must lie in [0, T): a malformed query_start_loc skips rows
    const int q1 = min(a.one_query ? b + 1 : a.query_start_loc[b + 1], a.num_tokens);
    // positions follow the given count
    const int qlen = a.one_query ? 1 : a.query_start_loc[b + 1] - q0;
    const int rows_total = q0 < 0 ? 0 : max(0, q1 - q0) * g;
    if (rt * kRows >= rows_total) return;
    // the sequence whose length and block table the rows read (a group's
    // first member; q0 < num_tokens here, as the tile has rows)
    const int seq0 = a.group_rows ? q0 : b;
    const int n_cap = a.max_blocks_per_seq * kBlockSize;
    int n = a.context_lens[seq0];
    n = n < 0 ? 0 : (n > n_cap ? n_cap : n);
    const int n_parts = partition_count(n, a.partition_size);
    const bool direct_out = n_parts <= 1 && !a.partials_only;
    if (part >= (n_parts > 0 ? n_parts : 1)) return;
    const int span = n_parts > 0 ? partition_span(n, n_parts) : 0;
    const int t_begin = part * span;
    const int t_end = min(n, t_begin + span);
    // The step's new token (one query per sequence, k_new given): position
    // n - 1, row row_new of block jb_new.  If this partition holds it, every
    // lane keeps the 16 cache bytes of that row that it would load (chunk
    // l % CPR): the row itself for a 16-bit cache; for a quantized cache its
    // codes, from the cache write's own quantizer over the row's D / 8 lanes,
    // with the row's scale or (x_min, range).  They replace what the cache
    // holds when the block is computed, so no work-group depends on another's
    // store; row tile 0 makes the store.
    const bool append = a.one_query && !a.group_rows && a.k_new != nullptr && n >= 1 &&
                        t_end == n;  // uniform: the last partition
    const int jb_new = append ? (n - 1) / kBlockSize : -1;
    const int row_new = (n - 1) & (kBlockSize - 1);
    constexpr int kRowsPerLoad = 64 / CPR;          // rows per 1 KiB wave load
    constexpr int LPR = D / 8;                      // the quantizer's lanes per row
    const bool new_lane = lane / CPR == row_new % kRowsPerLoad;
    uint4 k_nw = make_uint4(0u, 0u, 0u, 0u), v_nw = make_uint4(0u, 0u, 0u, 0u);
    uint2 kq_st = make_uint2(0u, 0u), vq_st = make_uint2(0u, 0u);  // lane < LPR: its codes
    float k_s0 = 0.f, k_s1 = 0.f, v_s0 = 0.f, v_s1 = 0.f;  // the scale, or (x_min, range)
    if (append) {
        const size_t row = (size_t)b * a.num_kv_heads + kvh;
        if constexpr (CE == T) {
            const size_t at = (row * D + (lane % CPR) * 8) * 2;
            k_nw = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + at);
            v_nw = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + at);
        } else {
            // lane l quantizes elements 8 (l % LPR) .. + 7, as the cache write does
            const size_t at = (row * D + (lane % LPR) * 8) * 2;
            const uint4 kr = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + at);
            const uint4 vr = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + at);
            const uint32_t kw[4] = {kr.x, kr.y, kr.z, kr.w}, vw[4] = {vr.x, vr.y, vr.z, vr.w};
            float kx[8], vx[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Mfma<T>::unpack(kw[i], kx[2 * i], kx[2 * i + 1]);
                Mfma<T>::unpack(vw[i], vx[2 * i], vx[2 * i + 1]);
            }
            // (the codes are gathered into chunks when the block is computed)
            if constexpr (kU4) {
                kq_st = make_uint2(quantize8_u4<LPR>(kx, k_s0, k_s1), 0u);
                vq_st = make_uint2(quantize8_u4<LPR>(vx, v_s0, v_s1), 0u);
            } else {
                kq_st = quantize8<CE, LPR>(kx, k_s0);
                vq_st = quantize8<CE, LPR>(vx, v_s0);
            }
        }
    }
    // the last query of the sequence sits at position n - 1 (causal), or every
    // query sees the whole context
    const int pos_of_last = a.causal ? n - 1 : 0x3fffffff;

    // this lane's query row (B operand and softmax state)
    const int R = rt * kRows + col;
    const bool row_ok = R < rows_total;
    const int jq = row_ok ? R / g : 0;
    const int hq = kvh * g + (row_ok ? R % g : 0);
    const int pos = pos_of_last - (qlen - 1) + jq;  // the query attends to positions 0..pos

    // Scores stay in raw units (q . k); the softmax works on c * s with
    // c = scale * log2(e), applied inside the exponent by one FMA.  A
    // negative scale is taken as |scale| on negated queries (exact), and c
    // is kept above zero so that a masked score (-inf) still gives weight 0.
    const bool neg_scale = a.scale_log2 < 0.f;
    const float c = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
    uint4 qv[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        qv[kk] = make_uint4(0u, 0u, 0u, 0u);
        if (row_ok)
            qv[kk] = *reinterpret_cast<const uint4*>(
                static_cast<const char*>(a.q) +
                (((size_t)(q0 + jq) * Hq + hq) * D + kk * 32 + grp * 8) * 2);
        if (neg_scale) {
            const uint32_t sg = 0x80008000u;  // sign bits of both 16-bit elements
            qv[kk] = make_uint4(qv[kk].x ^ sg, qv[kk].y ^ sg, qv[kk].z ^ sg, qv[kk].w ^ sg);
        }
    }
    // 4-bit caches: q . (x_min + step c) = step (q . c) + x_min sum(q), and
    // the weights' x_min part, sum over tokens of p x_min, kept per lane
    float qsum = 0.f, pxm = 0.f;
    if constexpr (kU4) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const uint32_t w4[4] = {qv[kk].x, qv[kk].y, qv[kk].z, qv[kk].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x, y;
                Mfma<T>::unpack(w4[j], x, y);
                qsum += x + y;
            }
        }
        qsum += __shfl_xor(qsum, 16);
        qsum += __shfl_xor(qsum, 32);
    }

    float m = kNegBig, cm = c * kNegBig, l = 0.f;  // max of raw scores, c times it, sum
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
    const int32_t* table = a.block_tables + (size_t)seq0 * a.max_blocks_per_seq;
    char* vst = s_buf + wave * kRows * VS;
    char* kst = s_buf + kWaves * kRows * VS + wave * kRows * KS;
    // the last position any row of this tile attends to, and the first
    const int pos_min = pos_of_last - (qlen - 1) + min(rt * kRows, rows_total - 1) / g;
    // the address this lane gives the V^T transpose read: token 4 grp +
    // (lane / 4) % 4, channels 4 (lane % 4) .. + 3 of each 16 (in each
    // 16-lane group, lane 16 G + 4 a + c receives as its element e element c
    // of what lane 16 G + a + 4 e addresses, so lane 16 grp + col receives
    // channel 16 nn + col of tokens 4 grp .. 4 grp + 3)
    const int v_off = (4 * grp + ((lane >> 2) & 3)) * VS + (lane & 3) * 8;

    struct Regs {
        uint4 k[VL], v[VL];
        // 8-bit caches: the scales of tokens 4 grp .. 4 grp + 3; 4-bit: their
        // (x_min, range) pairs, tokens 4 grp, 4 grp + 1 in ks / vs, the
        // other two in ks2 / vs2
        float4 ks, vs, ks2, vs2;
        int jb, phys;
        bool ok;
    };
    // The block ids of this wave's run, 64 at a time in one register (lane j
    // holds id j of the current 64) and taken out with readlane.  A table
    // read per block is a vector load, and waiting for it would also wait
    // for the K/V loads of the blocks in flight.
    int ids = -1;
    auto fetch_ids = [&](int i0) {
        const int j = i0 + lane;
        ids = j < n_my ? table[my0 + j] : -1;
    };
    fetch_ids(0);
    auto load = [&](Regs& r, int i) {
        r.jb = my0 + i;
        if ((i & 63) == 0 && i > 0 && i < n_my) fetch_ids(i);  // uniform
        const int phys = i < n_my ? __builtin_amdgcn_readlane(ids, i & 63) : -1;
        r.ok = i < n_my && phys >= 0 && (int64_t)phys < a.num_blocks;
        r.phys = phys;
        const size_t tile = (size_t)(r.ok ? phys : 0) * a.num_kv_heads + kvh;
        const int bytes = r.ok ? CTILE : 0;
        const __amdgpu_buffer_rsrc_t kr = rsrc(static_cast<const char*>(a.k_cache) + tile * CTILE, bytes);
        const __amdgpu_buffer_rsrc_t vr = rsrc(static_cast<const char*>(a.v_cache) + tile * CTILE, bytes);
        if constexpr (kQ8) {
            const int sb = r.ok ? kRows * 4 : 0;
            const uint4 ks = ld16(rsrc(a.k_scale + tile * kRows, sb), grp * 16);
            const uint4 vs = ld16(rsrc(a.v_scale + tile * kRows, sb), grp * 16);
            r.ks = __builtin_bit_cast(float4, ks);
            r.vs = __builtin_bit_cast(float4, vs);
        }
        if constexpr (kU4) {
            const int sb = r.ok ? kRows * 8 : 0;
            const __amdgpu_buffer_rsrc_t kq = rsrc(a.k_scale + tile * kRows * 2, sb);
            const __amdgpu_buffer_rsrc_t vq = rsrc(a.v_scale + tile * kRows * 2, sb);
            // (the pairs are 8-byte aligned: 8-byte loads)
            r.ks = ld8x2(kq, grp * 32);
            r.ks2 = ld8x2(kq, grp * 32 + 16);
            r.vs = ld8x2(vq, grp * 32);
            r.vs2 = ld8x2(vq, grp * 32 + 16);
        }
        // both tiles in token order, 1 KiB per wave load (the MFMA operand
        // order, 16 rows x 64 bytes per load, streams less well from HBM)
#pragma unroll
        for (int u = 0; u < VL; ++u) r.k[u] = ld16(kr, (u * 64 + lane) * 16);
#pragma unroll
        for (int u = 0; u < VL; ++u) r.v[u] = ld16(vr, (u * 64 + lane) * 16);
    };
    auto compute = [&](Regs& r) {
        if (append && r.ok && r.jb == jb_new) {  // uniform: the new token's block
            if constexpr (kU4) {
                // chunk c of the row (32 codes): quantizer lanes 4 c .. 4 c + 3
                const int c0 = (lane % CPR) * 4;
                k_nw = make_uint4(__shfl(kq_st.x, c0), __shfl(kq_st.x, c0 + 1),
                                  __shfl(kq_st.x, c0 + 2), __shfl(kq_st.x, c0 + 3));
                v_nw = make_uint4(__shfl(vq_st.x, c0), __shfl(vq_st.x, c0 + 1),
                                  __shfl(vq_st.x, c0 + 2), __shfl(vq_st.x, c0 + 3));
            } else if constexpr (kQ8) {
                // chunk c of the row (16 codes): quantizer lanes 2 c and 2 c + 1
                const int c0 = (lane % CPR) * 2;
                k_nw = make_uint4(__shfl(kq_st.x, c0), __shfl(kq_st.y, c0),
                                  __shfl(kq_st.x, c0 + 1), __shfl(kq_st.y, c0 + 1));
                v_nw = make_uint4(__shfl(vq_st.x, c0), __shfl(vq_st.y, c0),
                                  __shfl(vq_st.x, c0 + 1), __shfl(vq_st.y, c0 + 1));
            }
#pragma unroll
            for (int u = 0; u < VL; ++u)
                if (new_lane && u == row_new / kRowsPerLoad) {
                    r.k[u] = k_nw;
                    r.v[u] = v_nw;
                }
            // the row's scale (or pair): token row_new is entry row_new % 4 of
            // lane group row_new / 4
            const int e = row_new & 3;
            if (kQ8 && grp == row_new / 4) {
                r.ks.x = e == 0 ? k_s0 : r.ks.x;
                r.ks.y = e == 1 ? k_s0 : r.ks.y;
                r.ks.z = e == 2 ? k_s0 : r.ks.z;
                r.ks.w = e == 3 ? k_s0 : r.ks.w;
                r.vs.x = e == 0 ? v_s0 : r.vs.x;
                r.vs.y = e == 1 ? v_s0 : r.vs.y;
                r.vs.z = e == 2 ? v_s0 : r.vs.z;
                r.vs.w = e == 3 ? v_s0 : r.vs.w;
            }
            if (kU4 && grp == row_new / 4) {
                // entries 0, 1 in ks / vs, 2, 3 in ks2 / vs2; (x_min, range)
                // of an even entry in x, y, of an odd one in z, w (selects
                // only: a reference into the register set would put it in
                // memory)
                const bool e0 = e == 0, e1 = e == 1, e2 = e == 2, e3 = e == 3;
                r.ks.x = e0 ? k_s0 : r.ks.x;
                r.ks.y = e0 ? k_s1 : r.ks.y;
                r.ks.z = e1 ? k_s0 : r.ks.z;
                r.ks.w = e1 ? k_s1 : r.ks.w;
                r.ks2.x = e2 ? k_s0 : r.ks2.x;
                r.ks2.y = e2 ? k_s1 : r.ks2.y;
                r.ks2.z = e3 ? k_s0 : r.ks2.z;
                r.ks2.w = e3 ? k_s1 : r.ks2.w;
                r.vs.x = e0 ? v_s0 : r.vs.x;
                r.vs.y = e0 ? v_s1 : r.vs.y;
                r.vs.z = e1 ? v_s0 : r.vs.z;
                r.vs.w = e1 ? v_s1 : r.vs.w;
                r.vs2.x = e2 ? v_s0 : r.vs2.x;
                r.vs2.y = e2 ? v_s1 : r.vs2.y;
                r.vs2.z = e3 ? v_s0 : r.vs2.z;
                r.vs2.w = e3 ? v_s1 : r.vs2.w;
            }
            if (rt == 0) {
                const size_t srow = ((size_t)r.phys * a.num_kv_heads + kvh) * kRows + row_new;
                char* kc = static_cast<char*>(a.k_cache_w);
                char* vc = static_cast<char*>(a.v_cache_w);
                if constexpr (CE == T) {
                    if (new_lane) {
                        const size_t at = srow * ROW + (lane % CPR) * 16;
                        *reinterpret_cast<uint4*>(kc + at) = k_nw;
                        *reinterpret_cast<uint4*>(vc + at) = v_nw;
                    }
                } else if (lane < LPR) {
                    if constexpr (kU4) {
                        *reinterpret_cast<uint32_t*>(kc + srow * (D / 2) + lane * 4) = kq_st.x;
                        *reinterpret_cast<uint32_t*>(vc + srow * (D / 2) + lane * 4) = vq_st.x;
                        if (lane == 0) {
                            *reinterpret_cast<float2*>(a.k_scale_w + 2 * srow) = make_float2(k_s0, k_s1);
                            *reinterpret_cast<float2*>(a.v_scale_w + 2 * srow) = make_float2(v_s0, v_s1);
                        }
                    } else {
                        *reinterpret_cast<uint2*>(kc + srow * D + lane * 8) = kq_st;
                        *reinterpret_cast<uint2*>(vc + srow * D + lane * 8) = vq_st;
                        if (lane == 0) {
                            a.k_scale_w[srow] = k_s0;
                            a.v_scale_w[srow] = v_s0;
                        }
                    }
                }
            }
        }
        // K through this wave's LDS tile into the MFMA A operand (lane:
        // token col, channels 32 kk + 8 grp .. + 7)
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            const int ch = u * 64 + lane;  // 16-byte chunk ch % CPR of token ch / CPR
            char* dst = kst + (ch / CPR) * KS + (ch % CPR) * WID;
            if constexpr (kU4) {
                uint4 w4[4];
                widen32_u4<T>(r.k[u], w4);
#pragma unroll
                for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(dst + 16 * j) = w4[j];
            } else if constexpr (kQ8) {
                uint4 lo, hi;
                widen16<T, CE>(r.k[u], lo, hi);
                *reinterpret_cast<uint4*>(dst) = lo;
                *reinterpret_cast<uint4*>(dst + 16) = hi;
            } else {
                *reinterpret_cast<uint4*>(dst) = r.k[u];
            }
        }
        __asm__ volatile("" ::: "memory");
        // S^T[token 4*grp + i][query col]
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            s = Mfma<T>::qk(*reinterpret_cast<const uint4*>(kst + col * KS + (kk * 32 + grp * 8) * 2),
                            qv[kk], s);
        float sv[4] = {s[0], s[1], s[2], s[3]};
        if constexpr (kQ8) {  // q . (code * scale) = scale * (q . code)
            sv[0] *= r.ks.x;
            sv[1] *= r.ks.y;
            sv[2] *= r.ks.z;
            sv[3] *= r.ks.w;
        }
        if constexpr (kU4) {  // step (q . code) + x_min sum(q), step = range / 15
            const float xm[4] = {r.ks.x, r.ks.z, r.ks2.x, r.ks2.z};
            const float rg[4] = {r.ks.y, r.ks.w, r.ks2.y, r.ks2.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sv[i] = fmaf(sv[i], rg[i] * kInv15 * kU4Unscale, xm[i] * qsum);
        }
        // masks only where the block reaches the partition end or the causal
        // diagonal of some row of the tile (uniform test)
        const int t_hi = (r.jb + 1) * kBlockSize;
        const bool full = r.ok && t_hi <= t_end && t_hi <= pos_min + 1;
        if (!full) {
            const int t_lim = (r.ok && row_ok) ? min(t_end, pos + 1) : 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sv[i] = r.jb * kBlockSize + grp * 4 + i < t_lim ? sv[i] : -INFINITY;
        }
        float mx = kNegBig;
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[i]);
        // shared reference max, reduced across the query's 4 lanes only
        // when some score exceeds it by more than kSlack; l is this lane's
        // share of the sum
        const bool grew = __builtin_amdgcn_ballot_w64(fmaf(mx, c, -cm) > kSlack) != 0;
        float alpha = 1.f;
        if (grew) {
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mn = fmaxf(m, mx);
            alpha = fast_exp2((m - mn) * c);
            m = mn;
            cm = c * mn;
        }
        float p[4], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(fmaf(sv[i], c, -cm));
            ps += p[i];
        }
        l = fmaf(l, alpha, ps);
        // stage V (natural layout) in this wave's LDS tile; rows past the
        // partition are zeroed (their weight is 0, but 0 * NaN would not be)
        const bool tail = t_hi > t_end;  // uniform
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            const int ch = u * 64 + lane;                  // 16-byte chunk of the tile
            const int tok = ch / CPR;
            char* dst = vst + tok * VS + (ch % CPR) * WID;
            uint4 v = r.v[u];
            if (tail && r.jb * kBlockSize + tok >= t_end) v = make_uint4(0u, 0u, 0u, 0u);
            if constexpr (kU4) {
                uint4 w4[4];
                widen32_u4<T>(v, w4);
#pragma unroll
                for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(dst + 16 * j) = w4[j];
            } else if constexpr (kQ8) {
                uint4 lo, hi;
                widen16<T, CE>(v, lo, hi);
                *reinterpret_cast<uint4*>(dst) = lo;
                *reinterpret_cast<uint4*>(dst + 16) = hi;
            } else {
                *reinterpret_cast<uint4*>(dst) = v;
            }
        }
        __asm__ volatile("" ::: "memory");
        if constexpr (kQ8) {
            // the weight of a token's codes is p times its V scale; a token
            // past the partition keeps weight 0 whatever its scale slot holds
            const float vs4[4] = {r.vs.x, r.vs.y, r.vs.z, r.vs.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p[i] = r.jb * kBlockSize + grp * 4 + i < t_end ? p[i] * vs4[i] : 0.f;
        }
        if constexpr (kU4) {
            // the codes' weight is p step (times 2^9 for the widening), and
            // p x_min adds to every channel; tokens past the partition add
            // nothing whatever their pair holds
            const float xm[4] = {r.vs.x, r.vs.z, r.vs2.x, r.vs2.z};
            const float rg[4] = {r.vs.y, r.vs.w, r.vs2.y, r.vs2.w};
            float add = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool in = r.jb * kBlockSize + grp * 4 + i < t_end;
                add = in ? fmaf(p[i], xm[i], add) : add;
                p[i] = in ? p[i] * (rg[i] * kInv15 * kU4Unscale) : 0.f;
            }
            pxm = fmaf(pxm, alpha, add);
        }
        const uint2 pa = make_uint2(Mfma<T>::pack(p[0], p[1]), Mfma<T>::pack(p[2], p[3]));
        // with exact_p the rest of each weight, lo = p - hi, as a second
        // 16-bit operand: |lo| <= 2^-8 |p| (bf16) or 2^-11 |p| (fp16), and
        // its own rounding leaves 2^-16 |p| or 2^-22 |p| (2^-25 absolute for
        // an fp16 subnormal lo)
        uint2 pl = make_uint2(0u, 0u);
        if constexpr (XP) {
            float h0, h1, h2, h3;
            Mfma<T>::unpack(pa.x, h0, h1);
            Mfma<T>::unpack(pa.y, h2, h3);
            pl = make_uint2(Mfma<T>::pack(p[0] - h0, p[1] - h1), Mfma<T>::pack(p[2] - h2, p[3] - h3));
        }
        if (grew) {
#pragma unroll
            for (int nn = 0; nn < NN; ++nn) o[nn] *= alpha;
        }
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
            typedef __attribute__((address_space(3))) s16x4_v lds_s16x4;
            const s16x4_v vt =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vst + v_off + nn * 32));
            // O^T = V^T P^T: the accumulator column is the lane's own query
            o[nn] = Mfma<T>::pv(__builtin_bit_cast(uint2, vt), pa, o[nn]);
            if constexpr (XP) o[nn] = Mfma<T>::pv(__builtin_bit_cast(uint2, vt), pl, o[nn]);
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

    // ---- merge the waves (wave 0 keeps its tile in registers) --------------
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if constexpr (kU4) {  // the x_min part of every channel of the lane's query
        pxm += __shfl_xor(pxm, 16);
        pxm += __shfl_xor(pxm, 32);
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) o[nn] += pxm;
    }
    __syncthreads();  // every wave is done with its V stage
    float* s_o = reinterpret_cast<float*>(s_buf);  // [wave - 1][query][D]
    if (grp == 0) {
        s_m[wave][col] = cm;  // in log2 units
        s_l[wave][col] = l;
    }
    if (wave > 0) {
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
            *reinterpret_cast<float4*>(&s_o[((wave - 1) * kRows + col) * D + nn * 16 + grp * 4]) =
                make_float4(o[nn][0], o[nn][1], o[nn][2], o[nn][3]);
    }
    __syncthreads();
    if (wave != 0) return;

    // lane: query col, channels 16 nn + 4 grp + i
    const int Rr = rt * kRows + col;
    if (Rr >= rows_total) return;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][col]);
    float f[kWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        f[w] = fast_exp2(s_m[w][col] - M);
        L = fmaf(s_l[w][col], f[w], L);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const size_t orow = (size_t)(q0 + Rr / g) * Hq + kvh * g + Rr % g;
    const size_t pi = orow * NP + part;
#pragma unroll
    for (int nn = 0; nn < NN; ++nn) {
        const int d0 = nn * 16 + grp * 4;
        float O[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) O[i] = o[nn][i] * f[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            const float4 x = *reinterpret_cast<const float4*>(&s_o[((w - 1) * kRows + col) * D + d0]);
            O[0] = fmaf(x.x, f[w], O[0]);
            O[1] = fmaf(x.y, f[w], O[1]);
            O[2] = fmaf(x.z, f[w], O[2]);
            O[3] = fmaf(x.w, f[w], O[3]);
        }
        if (direct_out) {
            *reinterpret_cast<uint2*>(static_cast<char*>(a.out) + (orow * D + d0) * 2) =
                make_uint2(Mfma<T>::pack(O[0] * inv, O[1] * inv), Mfma<T>::pack(O[2] * inv, O[3] * inv));
        } else {
            *reinterpret_cast<float4*>(a.o_part + pi * D + d0) =
                make_float4(O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv);
        }
    }
    if (!direct_out && grp == 0) {
        a.m_part[pi] = M * kLn2;
        a.l_part[pi] = L;
    }
}

// Long runs of queries (prefill chunks): a work-group owns NW waves x RW
// row tiles of 16 rows and walks every block of its partition up to the last
// position any of its rows attends to.  The K/V blocks are fetched once per
// work-group, four at a time (one load step), straight from the pool into
// one of two LDS stages; the step is computed as two halves of two blocks,
// each one softmax update, and every wave reads the K and V operands once
// and uses them for its RW row tiles.  One barrier per load step.  The
// output is accumulated transposed,
// O^T = V^T P^T: the P operand is then the score tile as it leaves the first
// MFMA and each lane's accumulator column is its own query, so rescaling and
// normalizing need no lane exchange.  The V^T operand comes from the
// token-major V tile through the LDS transpose read (ds_read_b64_tr_b16):
// in each 16-lane group, lane 16 G + 4 a + c receives, as its element e,
// element c of the 8 bytes that lane 16 G + a + 4 e addresses.  So when lane
// 16 G + a + 4 e addresses channels 16 nn + 4 a .. + 3 of token 4 G + e,
// lane 16 G + col receives channel 16 nn + col of tokens 4 G .. 4 G + 3:
// one read per block and 16 channels.  Each wave owns its rows for the whole
// partition, so there is no merge between waves.
template <Elem T, int D, int RW, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RW == 1 && D <= 128 ? 4 : 2)))
void paged_multi_tiled_kernel(MultiArgs a) {
    constexpr int KK = D / 32;
    constexpr int NN = D / 16;
    constexpr int KB = D <= 128 ? 2 : 1;            // 16-token blocks per softmax update
    constexpr int KL = 2 * KB;                      // 16-token blocks per load step
    constexpr int ROW = D * 2;
    constexpr int TILE = kRows * ROW;
    constexpr int SUBS = TILE / 1024;               // 1 KiB wave loads per tile
    constexpr int IPW = 2 * KL * SUBS / NW;         // wave loads per step and wave
    static_assert((2 * KL * SUBS) % NW == 0, "the loads of a step split evenly over the waves");
    constexpr int STAGE = 2 * KL * TILE;            // the K tiles, then the V tiles, of one step
    constexpr int WG_ROWS = NW * kRows * RW;

    // two stages: the step being computed, and the next one (its loads are
    // issued at the top of this step and waited for at the top of the next)
    __shared__ __attribute__((aligned(16))) char s_b0[STAGE];
    __shared__ __attribute__((aligned(16))) char s_b1[STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4;
    const int col = lane & 15;

    // Work-groups go to the XCDs round-robin in launch order.  Renumbered so
    // that the row groups of one (sequence, partition, kv head), which read
    // the same K/V blocks, go to one XCD one after the other and share its
    // L2, while successive (sequence, partition, kv head) groups still go
    // round-robin (the XCDs stay balanced when sequence lengths differ).
    const int NP = a.num_partitions;
    unsigned item = blockIdx.x;
    {
        const unsigned R = (unsigned)a.row_tiles;
        const unsigned whole = gridDim.x / R / kXcds * kXcds;  // groups in whole rounds
        if (item < whole * R) {
            const unsigned x = item % kXcds, y = item / kXcds;
            item = ((y / R) * kXcds + x) * R + y % R;
        }
    }
    int rest = (int)item;
    const int rg = rest % a.row_tiles;
    rest /= a.row_tiles;
    const int part = rest % NP;
    rest /= NP;
    const int kvh = rest % a.num_kv_heads;
    // Sequences in longest-first order (by partition length), so that the
    // work-groups dispatched last are the shortest and the ragged tail of
    // the launch is small.  Every work-group ranks the sequences itself
    // (one per thread, in LDS).
    static_assert(NW * 64 >= kScheduleMaxSeqs, "one thread per ranked sequence");
    __shared__ __align__(16) int s_key[kScheduleMaxSeqs];
    __shared__ int s_order[kScheduleMaxSeqs];
    int b = rest / a.num_kv_heads;
    // (keys as in the short-run kernel: span in blocks above 255 - index)
    if (a.num_seqs <= kScheduleMaxSeqs && a.max_blocks_per_seq < (1 << 23)) {
        const int n_cap0 = a.max_blocks_per_seq * kBlockSize;
        int key = -1;
        if (tid < a.num_seqs) {
            int s0 = tid;
            if (a.group_rows) {  // a group's context is its first member's
                s0 = a.query_start_loc[tid];
                s0 = s0 >= 0 && s0 < a.num_tokens ? s0 : -1;
            }
            const int nn = s0 < 0 ? 0 : min(max(a.context_lens[s0], 0), n_cap0);
            const int c = partition_count(nn, a.partition_size);
            key = (c > 0 ? partition_span(nn, c) / kBlockSize : 0) << 8 | (255 - tid);
        }
        if (tid < kScheduleMaxSeqs) s_key[tid] = key;
        __syncthreads();
        if (tid < a.num_seqs) {
            int r = 0;
            const int nj = (a.num_seqs + 3) & ~3;  // <= kScheduleMaxSeqs
            for (int j = 0; j < nj; j += 4) {
                const int4 kk = *reinterpret_cast<const int4*>(&s_key[j]);
                r += (kk.x > key) + (kk.y > key) + (kk.z > key) + (kk.w > key);
            }
            s_order[r] = tid;
        }
        __syncthreads();
        b = s_order[b];
    }

    const int Hq = a.num_q_heads;
    const int g = Hq / a.num_kv_heads;
    const int q0 = a.one_query ? b : a.query_start_loc[b];
    const int q1 = min(a.one_query ? b + 1 : a.query_start_loc[b + 1], a.num_tokens);
    const int qlen = a.one_query ? 1 : a.query_start_loc[b + 1] - q0;
    const int rows_total = q0 < 0 ? 0 : max(0, q1 - q0) * g;
    const int wg_r0 = rg * WG_ROWS;
    if (wg_r0 >= rows_total) return;
    // the sequence whose length and block table the rows read (a group's
    // first member; q0 < num_tokens here, as the work-group has rows)
    const int seq0 = a.group_rows ? q0 : b;
    const int n_cap = a.max_blocks_per_seq * kBlockSize;
    int n = a.context_lens[seq0];
    n = n < 0 ? 0 : (n > n_cap ? n_cap : n);
    const int n_parts = partition_count(n, a.partition_size);
    const bool direct_out = n_parts <= 1 && !a.partials_only;
    if (part >= (n_parts > 0 ? n_parts : 1)) return;
    const int span = n_parts > 0 ? partition_span(n, n_parts) : 0;
    const int t_begin = part * span;
    const int t_end = min(n, t_begin + span);
    // the last query of the sequence sits at position n - 1 (causal), or every
    // query sees the whole context
    const int pos_of_last = a.causal ? n - 1 : 0x3fffffff;
    // the last position any row of this work-group attends to
    const int r_last = min(wg_r0 + WG_ROWS, rows_total) - 1;
    const int t_stop = min(t_end, max(pos_of_last - (qlen - 1) + r_last / g + 1, 0));
    const int blk_begin = t_begin / kBlockSize;
    const int blk_stop = t_stop > t_begin ? (t_stop + kBlockSize - 1) / kBlockSize : blk_begin;
    const int32_t* table = a.block_tables + (size_t)seq0 * a.max_blocks_per_seq;
    // Scores stay in raw units (q . k); the softmax works on c * s with
    // c = scale * log2(e), applied inside the exponent by one FMA.  A
    // negative scale is taken as |scale| on negated queries (exact), and c
    // is kept above zero so that a masked score (-inf) still gives weight 0.
    const bool neg_scale = a.scale_log2 < 0.f;
    const float c = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);

    // this wave's row tiles; lane column `col` is one query row of each tile
    const int w_r0 = wg_r0 + wave * kRows * RW;
    bool row_ok[RW];
    int pos[RW];
    int tile_pos_min[RW];   // the earliest position of a tile's rows (its first row)
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
        tile_pos_min[rr] = pos_of_last - (qlen - 1) + min(w_r0 + rr * kRows, rows_total - 1) / g;
    uint4 qv[RW][KK];
    float m[RW], cm[RW], l[RW];  // running max of raw scores, c times it, sum
    f32x4_t o[RW][NN];  // O^T: o[rr][nn][i] = O[row col][d = 16 nn + 4 grp + i]
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const int R = w_r0 + rr * kRows + col;
        row_ok[rr] = R < rows_total;
        const int jq = row_ok[rr] ? R / g : 0;
        const int hq = kvh * g + (row_ok[rr] ? R % g : 0);
        pos[rr] = pos_of_last - (qlen - 1) + jq;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            qv[rr][kk] = make_uint4(0u, 0u, 0u, 0u);
            if (row_ok[rr])
                qv[rr][kk] = *reinterpret_cast<const uint4*>(
                    static_cast<const char*>(a.q) +
                    (((size_t)(q0 + jq) * Hq + hq) * D + kk * 32 + grp * 8) * 2);
            if (neg_scale) {
                const uint32_t sg = 0x80008000u;  // sign bits of both 16-bit elements
                qv[rr][kk] = make_uint4(qv[rr][kk].x ^ sg, qv[rr][kk].y ^ sg, qv[rr][kk].z ^ sg,
                                        qv[rr][kk].w ^ sg);
            }
        }
        m[rr] = kNegBig;
        cm[rr] = c * kNegBig;
        l[rr] = 0.f;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) o[rr][nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // LDS tiles are token rows of ROW bytes without padding.  The 16-byte
    // chunk c of token t's row sits in chunk slot c ^ swz(t) of that row
    // (swz_k in K tiles, swz_v in V tiles), chosen so that the lanes the LDS
    // serves in one cycle hit distinct banks (64 banks of 4 bytes).  Measured
    // on gfx950 with read-only kernels: a 16-byte read serves lanes 0-7
    // together with 24-31 (and 8-15 with 16-23, likewise in the upper half),
    // which for the K operand read (lane: token col, chunk 4 kk + grp) asks
    // for distinct swz_k(t) over 16 rows and no collision between swz_k(t)
    // and swz_k(t + 8) ^ 1; the transpose read serves lanes 0-31 together (8
    // tokens x one 32-byte piece each), which asks for distinct swz_v(t) / 2
    // over each 8 tokens.  The two conditions exclude each other, hence two
    // layouts: with one swizzle for both the K reads ran at 0.63 of the
    // conflict-free rate.  (The 128-byte rows of head_dim 64 keep one layout
    // for both tiles.)
    auto swz_v = [](int t) {
        return ROW == 128 ? ((2 * t) ^ (3 * (t >> 2))) & 7
                          : 2 * (t & 7) + (((t & 7) >> 2) ^ (t >> 3));
    };
    auto swz_k = [](int t) { return ROW == 128 ? ((2 * t) ^ (3 * (t >> 2))) & 7 : t & 15; };
    // this lane's LDS offsets inside a tile: the K operand (token col,
    // channels 32 kk + 8 grp .. + 7) and the address it gives the V^T
    // transpose read (token 4 grp + (lane / 4) % 4, channels 16 nn + 4 (lane
    // % 4) .. + 3: in each 16-lane group, lane 16 G + 4 a + c receives as its
    // element e element c of what lane 16 G + a + 4 e addresses)
    int k_off[KK], v_off[NN];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) k_off[kk] = col * ROW + 16 * ((kk * 4 + grp) ^ swz_k(col));
    {
        const int tv = 4 * grp + ((lane >> 2) & 3), qa = lane & 3;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
            v_off[nn] = tv * ROW + 16 * ((2 * nn + (qa >> 1)) ^ swz_v(tv)) + 8 * (qa & 1);
    }

    // Loads of the KL blocks from jb0 on, straight from the pool into the LDS
    // stage dst: 2 KL tiles of 1 KiB wave loads, IPW per wave.  Lane l of a
    // wave load fills bytes 16 l .. 16 l + 15 of its kilobyte, so it fetches
    // the chunk that the swizzle puts there.  The buffer window ends at the
    // partition end: rows past it (and a block past the run, or a bad block
    // id) arrive as zeros, so no score or weight meets a stale or NaN value.
    const __attribute__((address_space(4))) int32_t* table_c =
        (const __attribute__((address_space(4))) int32_t*)table;
    // The IPW loads of a wave fall in one tile, so each wave needs one block
    // id per step; it is a scalar load (constant address space: the table is
    // not written here, and waiting for it never waits for the K/V loads),
    // issued a step before the loads that use it.
    static_assert(SUBS % IPW == 0, "a wave's loads of a step lie in one tile");
    auto load_id = [&](int jb0) {
        return table_c[min(jb0 + (wave * IPW / SUBS) % KL, blk_stop - 1)];
    };
    // Block ids at or past nb_lim are refused (the pool's block count, capped
    // to the int range); the K and V bases of this kv head's tiles and the
    // stride from one block to the next.  The descriptor arithmetic is all
    // scalar and branch-free.
    const unsigned nb_lim = (unsigned)(a.num_blocks < 0x7fffffff ? a.num_blocks : 0x7fffffff);
    const char* const k_base = static_cast<const char*>(a.k_cache) + (size_t)kvh * TILE;
    const char* const v_base = static_cast<const char*>(a.v_cache) + (size_t)kvh * TILE;
    const size_t blk_stride = (size_t)a.num_kv_heads * TILE;
    auto issue = [&](char* dst, int jb0, int id) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int u = wave * IPW + i;            // wave-uniform
            const int tt = u / SUBS, r = u % SUBS;   // tile (K tiles first), kilobyte
            const int jb = jb0 + tt % KL;
            const bool ok = (jb < blk_stop) & ((unsigned)id < nb_lim);
            int rows = t_end - jb * kBlockSize;
            rows = rows < 0 ? 0 : rows;
            rows = rows > kRows ? kRows : rows;
            // wave-uniform by construction; said so, or the descriptor is
            // built in vector registers and the load wrapped in a loop
            rows = __builtin_amdgcn_readfirstlane(ok ? rows : 0);
            const char* base = (tt < KL ? k_base : v_base) + (size_t)(ok ? (unsigned)id : 0u) * blk_stride;
            const __amdgpu_buffer_rsrc_t rs = rsrc(base, rows * ROW);
            const int at = r * 1024 + lane * 16;
            const int t = at / ROW, slot = (at % ROW) / 16;
            load_to_lds16(rs, dst + tt * TILE + r * 1024,
                          t * ROW + 16 * (slot ^ (tt < KL ? swz_k(t) : swz_v(t))));
        }
    };
    // KB blocks from jb0 on: K tiles at kbuf, V tiles at vbuf
    auto compute = [&](const char* kbuf, const char* vbuf, int jb0) {
        // 1. scores of every row tile: S^T[token 4 grp + i][query col]
        f32x4_t s[RW][KB];
        {
            uint4 ka[KB][KK];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[kb][kk] = *reinterpret_cast<const uint4*>(kbuf + kb * TILE + k_off[kk]);
#pragma unroll
            for (int rr = 0; rr < RW; ++rr)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    s[rr][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        s[rr][kb] = Mfma<T>::qk(ka[kb][kk], qv[rr][kk], s[rr][kb]);
                }
        }
        // V^T operands of the step, read once for every row tile (the lane
        // receives channel 16 nn + col of tokens 4 grp .. 4 grp + 3)
        uint2 vw[NN][KB];
#pragma unroll
        for (int nn = 0; nn < NN; ++nn)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                typedef __attribute__((address_space(3))) s16x4_v lds_s16x4;
                const s16x4_v t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vbuf + kb * TILE + v_off[nn]));
                vw[nn][kb] = __builtin_bit_cast(uint2, t);
            }
        // 2. per row tile: online softmax over the step's KB * 16 tokens, then
        //    O^T += V^T P^T.  The P·V products of one tile run on the matrix
        //    cores while the next tile's softmax is computed.
        const int t_hi = (jb0 + KB) * kBlockSize;       // one past the step's last token
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            // Masking only where the step reaches the partition end or the
            // causal diagonal of some row of the tile (uniform test).
            const bool full = t_hi <= t_end && t_hi <= tile_pos_min[rr] + 1;
            float sv[KB][4], mx = kNegBig;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[kb][i] = s[rr][kb][i];
            if (!full) {
                // a lane's tokens lie below t_lim: its row's position + 1 and the partition end
                const int t_lim = row_ok[rr] ? min(t_end, pos[rr] + 1) : 0;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = (jb0 + kb) * kBlockSize + grp * 4 + i;
                        sv[kb][i] = t < t_lim ? sv[kb][i] : -INFINITY;
                    }
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[kb][i]);
            // The reference max m is shared by a query's 4 lanes; the
            // cross-lane max is needed only when some score exceeds it by
            // more than kSlack, and then acc is rescaled (otherwise alpha is 1).
            if (__builtin_amdgcn_ballot_w64(fmaf(mx, c, -cm[rr]) > kSlack) != 0) {
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mn = fmaxf(m[rr], mx);
                const float alpha = fast_exp2((m[rr] - mn) * c);
                m[rr] = mn;
                cm[rr] = c * mn;
                l[rr] *= alpha;
#pragma unroll
                for (int nn = 0; nn < NN; ++nn) o[rr][nn] *= alpha;
            }
            // l is this lane's share of the sum (its own tokens), reduced
            // across the 4 lanes at the end
            uint2 pb[KB];
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = fast_exp2(fmaf(sv[kb][i], c, -cm[rr]));
                    ps += p[i];
                }
                pb[kb] = make_uint2(Mfma<T>::pack(p[0], p[1]), Mfma<T>::pack(p[2], p[3]));
            }
            l[rr] += ps;
#pragma unroll
            for (int nn = 0; nn < NN; ++nn) {
                if constexpr (KB == 2) {
                    // one 16x16x32 MFMA over both blocks: contraction index 8 grp + j
                    // is token 4 grp + j of block 0 (j < 4) or 4 grp + j - 4 of
                    // block 1, in the A (V^T) and the B (P^T) operand alike
                    const uint4 va = make_uint4(vw[nn][0].x, vw[nn][0].y, vw[nn][1].x, vw[nn][1].y);
                    const uint4 pbb = make_uint4(pb[0].x, pb[0].y, pb[1].x, pb[1].y);
                    o[rr][nn] = Mfma<T>::pv32(va, pbb, o[rr][nn]);
                } else {
                    o[rr][nn] = Mfma<T>::pv(vw[nn][0], pb[0], o[rr][nn]);
                }
            }
        }
    };

    // Load steps of KL blocks over two LDS stages.  At the top of a step a
    // wave waits for all its loads (those of this step); after the barrier
    // every wave's have landed and no wave still reads the other stage, which
    // then takes the loads of the next step, issued before this step's
    // compute.  (With deeper prefetch the compiler, which cannot tell the LDS
    // stages apart, waits for every load issued earlier before the first LDS
    // read anyway.)  A plain s_barrier: a fence would also wait for the newer
    // loads.  Past the run the loads fetch zeros.
    const int n_steps = (blk_stop - blk_begin + KL - 1) / KL;
    if (n_steps > 0) {
        issue(s_b0, blk_begin, load_id(blk_begin));
        int id_next = load_id(blk_begin + KL);  // for the loads issued at step 0
        auto step = [&](const char* cur, char* nxt, int st) {
            __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
            __builtin_amdgcn_s_barrier();
            const int id = id_next;
            id_next = load_id(blk_begin + (st + 2) * KL);
            issue(nxt, blk_begin + (st + 1) * KL, id);
#pragma unroll
            for (int h = 0; h < KL / KB; ++h)
                compute(cur + h * KB * TILE, cur + (KL + h * KB) * TILE, blk_begin + st * KL + h * KB);
        };
        for (int st = 0; st < n_steps; st += 2) {
            step(s_b0, s_b1, st);
            if (st + 1 < n_steps) step(s_b1, s_b0, st + 1);
        }
        // no load may still write this work-group's LDS when its waves end
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    }

    // ---- epilogue: each lane writes 4 consecutive channels of its own row --
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        l[rr] += __shfl_xor(l[rr], 16);
        l[rr] += __shfl_xor(l[rr], 32);
    }
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
        const int R = w_r0 + rr * kRows + col;
        if (R >= rows_total) continue;
        const float inv = l[rr] > 0.f ? 1.f / l[rr] : 0.f;
        const size_t orow = (size_t)(q0 + R / g) * Hq + kvh * g + R % g;
        const size_t pi = orow * NP + part;
#pragma unroll
        for (int nn = 0; nn < NN; ++nn) {
            const int d0 = nn * 16 + grp * 4;
            if (direct_out) {
                const uint2 w = make_uint2(Mfma<T>::pack(o[rr][nn][0] * inv, o[rr][nn][1] * inv),
                                           Mfma<T>::pack(o[rr][nn][2] * inv, o[rr][nn][3] * inv));
                *reinterpret_cast<uint2*>(static_cast<char*>(a.out) + (orow * D + d0) * 2) = w;
            } else {
                float4 w = make_float4(o[rr][nn][0] * inv, o[rr][nn][1] * inv,
                                       o[rr][nn][2] * inv, o[rr][nn][3] * inv);
                *reinterpret_cast<float4*>(a.o_part + pi * D + d0) = w;
            }
        }
        if (!direct_out && grp == 0) {
            a.m_part[pi] = cm[rr] * kLn2;
            a.l_part[pi] = l[rr];
        }
    }
}

constexpr int kTiledRW = 1;                 // row tiles per wave in the tiled kernel
constexpr int kTiledWaves = 8;              // waves per work-group of the tiled kernel
constexpr int kTiledMinRows = 64;           // rows per (sequence, kv head) that select it

template <Elem T, Elem CE, int D>
hipError_t launch_dw(const MultiArgs& a, int64_t grid, hipStream_t s) {
    const dim3 g((unsigned)grid);
    if constexpr (CE != T) {
        // 8- and 4-bit caches: the decode route only (one query, two-part
        // weights); a 4-bit tile at head_dim 64 is half a wave load
        if (!a.one_query || !a.exact_p) return hipErrorInvalidValue;
    }
    if constexpr (CE == Elem::U4 && D < 128) {
        return hipErrorInvalidValue;
    } else {
    // (at head_dim 256 more than four waves would spill registers to memory)
    constexpr int WQ = CE == T ? kWavesOneQuery16 : kWavesOneQueryQ;
    if constexpr (D <= 128) {
        if (a.one_query) {
            const dim3 blk(WQ * 64);
            if (a.exact_p) hipLaunchKernelGGL((paged_multi_kernel<T, CE, D, true, WQ>), g, blk, 0, s, a);
            else if constexpr (CE == T)
                hipLaunchKernelGGL((paged_multi_kernel<T, T, D, false, WQ>), g, blk, 0, s, a);
            return hipGetLastError();
        }
    }
    const dim3 blk(kWavesRuns * 64);
    if (a.exact_p) hipLaunchKernelGGL((paged_multi_kernel<T, CE, D, true, kWavesRuns>), g, blk, 0, s, a);
    else if constexpr (CE == T)
        hipLaunchKernelGGL((paged_multi_kernel<T, T, D, false, kWavesRuns>), g, blk, 0, s, a);
    return hipGetLastError();
    }
}

template <Elem T, Elem CE>
hipError_t launch_d(const MultiArgs& a, int d, int64_t grid, hipStream_t s) {
    switch (d) {
    case 64: return launch_dw<T, CE, 64>(a, grid, s);
    case 128: return launch_dw<T, CE, 128>(a, grid, s);
    case 256: return launch_dw<T, CE, 256>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

template <Elem T>
hipError_t launch_tiled(const MultiArgs& a, int d, int64_t grid, hipStream_t s) {
    const dim3 g((unsigned)grid), blk(kTiledWaves * 64);
    switch (d) {
    case 64: hipLaunchKernelGGL((paged_multi_tiled_kernel<T, 64, kTiledRW, kTiledWaves>), g, blk, 0, s, a); break;
    case 128: hipLaunchKernelGGL((paged_multi_tiled_kernel<T, 128, kTiledRW, kTiledWaves>), g, blk, 0, s, a); break;
    case 256: hipLaunchKernelGGL((paged_multi_tiled_kernel<T, 256, 1, kTiledWaves>), g, blk, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int64_t multi_row_groups(int max_rows, int head_dim) {
    if (max_rows < kTiledMinRows) return (max_rows + kRows - 1) / kRows;
    const int rw = head_dim == 256 ? 1 : kTiledRW;
    const int per = kTiledWaves * kRows * rw;
    return (max_rows + per - 1) / per;
}

hipError_t launch_paged_multi(const MultiArgs& a, int dtype, int cache_dtype, int head_dim,
                              hipStream_t stream) {
    const int64_t grid =
        (int64_t)a.num_seqs * a.num_kv_heads * a.row_tiles * a.num_partitions;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool tiled = a.max_rows >= kTiledMinRows;
    const Elem e = static_cast<Elem>(dtype), ce = static_cast<Elem>(cache_dtype);
    if (ce == e) {
        if (e == Elem::F16)
            return tiled ? launch_tiled<Elem::F16>(a, head_dim, grid, stream)
                         : launch_d<Elem::F16, Elem::F16>(a, head_dim, grid, stream);
        if (e == Elem::BF16)
            return tiled ? launch_tiled<Elem::BF16>(a, head_dim, grid, stream)
                         : launch_d<Elem::BF16, Elem::BF16>(a, head_dim, grid, stream);
        return hipErrorInvalidValue;
    }
    if (tiled || !(a.k_scale && a.v_scale)) return hipErrorInvalidValue;
    if (e == Elem::F16 && ce == Elem::I8) return launch_d<Elem::F16, Elem::I8>(a, head_dim, grid, stream);
    if (e == Elem::F16 && ce == Elem::F8) return launch_d<Elem::F16, Elem::F8>(a, head_dim, grid, stream);
    if (e == Elem::BF16 && ce == Elem::I8) return launch_d<Elem::BF16, Elem::I8>(a, head_dim, grid, stream);
    if (e == Elem::BF16 && ce == Elem::F8) return launch_d<Elem::BF16, Elem::F8>(a, head_dim, grid, stream);
    if (e == Elem::F16 && ce == Elem::U4) return launch_d<Elem::F16, Elem::U4>(a, head_dim, grid, stream);
    if (e == Elem::BF16 && ce == Elem::U4) return launch_d<Elem::BF16, Elem::U4>(a, head_dim, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
