// C ABI of libpkv: argument validation, launch configuration and workspace
// layout.  Every entry point checks what the host can see before it enqueues
// anything, never allocates, frees or synchronizes, and reports failures as a
// pkv_status plus a thread-local message.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {
thread_local char g_err[512] = "";
}  // namespace

pkv_status fail(pkv_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

pkv_status ok() {
    g_err[0] = '\0';
    return PKV_OK;
}

const char* last_error() { return g_err; }

}  // namespace pkv

namespace {

using pkv::fail;
using pkv::ok;

pkv_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_float(pkv_dtype d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }

// 1-byte codes with one fp32 scale per (slot, kv head)
bool is_scaled(pkv_dtype d) { return d == PKV_I8 || d == PKV_F8_E4M3; }

// quantized caches: per-row scale arrays required (4-bit: (x_min, range) pairs)
bool is_quantized(pkv_dtype d) { return is_scaled(d) || d == PKV_U4; }

// bytes of one cache row of head_dim elements
int64_t row_bytes(pkv_dtype d, int head_dim) {
    return d == PKV_F32 ? 4LL * head_dim : d == PKV_U4 ? head_dim / 2 : is_scaled(d) ? head_dim : 2LL * head_dim;
}

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int heads_per_tile(int g, pkv_dtype cache) {
    const int cap = cache == PKV_U4 ? 2 : is_scaled(cache) ? 4 : 8;
    for (int t = cap; t > 1; t >>= 1)
        if (g % t == 0) return t;
    return 1;
}

int num_partitions(int mbs, int P) { return (int)(((int64_t)mbs * pkv::kBlockSize + P - 1) / P); }

// Blocks of a sequence a decode can touch: all of them, or with a sliding
// window of W positions at most W / 16 + 2 (the window's first block may start
// mid-block and the partitions split from that block on).
int window_blocks(int mbs, int window) {
    if (window <= 0) return mbs;
    const int64_t wb = (int64_t)window / pkv::kBlockSize + 2;
    return wb < mbs ? (int)wb : mbs;
}

// Workspace layout: the fp32 partials m [B][Hq][NP], l [B][Hq][NP] and
// o [B][Hq][NP][D], each region 256-byte aligned.
struct WorkspaceLayout {
    size_t m_off, l_off, o_off, total;
};

WorkspaceLayout layout(int B, int Hq, int D, int NP) {
    WorkspaceLayout w;
    const size_t pl = (size_t)B * Hq * NP;
    w.m_off = 0;
    w.l_off = align256(w.m_off + pl * sizeof(float));
    w.o_off = align256(w.l_off + pl * sizeof(float));
    w.total = align256(w.o_off + pl * D * sizeof(float));
    return w;
}

// shape checks shared by the decode entry points
pkv_status check_decode(const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* block_tables,
                        int mbs, const int32_t* context_lens, int B, int Hq, int Hkv, int D,
                        int block_size, int64_t num_blocks, pkv_dtype q_dtype,
                        pkv_dtype cache_dtype) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || mbs <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE,
                    "need num_seqs >= 0 and positive num_q_heads, num_kv_heads, "
                    "max_blocks_per_seq, num_blocks (got %d, %d, %d, %d, %lld)",
                    B, Hq, Hkv, mbs, (long long)num_blocks);
    if (Hq % Hkv != 0)
        return fail(PKV_ERR_SHAPE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", Hq,
                    Hkv);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (only 16)", block_size);
    if (!head_dim_ok(D))
        return fail(PKV_ERR_UNSUPPORTED, "head_dim %d unsupported (64, 128, 256)", D);
    const bool pair_ok = (is_float(q_dtype) && cache_dtype == q_dtype) ||
                         ((q_dtype == PKV_F16 || q_dtype == PKV_BF16) && is_quantized(cache_dtype));
    if (cache_dtype == PKV_U4 && D == 64)
        return fail(PKV_ERR_UNSUPPORTED, "4-bit caches need head_dim 128 or 256");
    if (!pair_ok)
        return fail(PKV_ERR_DTYPE, "unsupported (q_dtype, cache_dtype) = (%d, %d)", (int)q_dtype,
                    (int)cache_dtype);
    if (B == 0) return ok();
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens)
        return fail(PKV_ERR_NULL, "q, k_cache, v_cache, block_tables and context_lens are required");
    if (is_quantized(cache_dtype) && (!k_scale || !v_scale))
        return fail(PKV_ERR_NULL, "k_scale and v_scale are required for an INT8 / FP8 / 4-bit cache");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKV_ERR_SHAPE, "q, k_cache and v_cache must be 16-byte aligned");
    // a 4-bit row's (x_min, range) pair is read as one 8-byte word
    if (cache_dtype == PKV_U4 &&
        ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 7u))
        return fail(PKV_ERR_SHAPE, "4-bit k_scale and v_scale must be 8-byte aligned");
    if ((int64_t)Hkv * num_blocks * pkv::kBlockSize * D > (int64_t)1 << 62)
        return fail(PKV_ERR_SHAPE, "pool too large");
    return ok();
}

pkv::DecodeArgs make_args(const void* q, const void* k_cache, const void* v_cache,
                          const float* k_scale, const float* v_scale, const int32_t* block_tables,
                          int mbs, const int32_t* context_lens, int B, int Hq, int Hkv,
                          int64_t num_blocks, float scale, int P, int NP, int n_tiles) {
    pkv::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_blocks = num_blocks;
    a.num_seqs = B;
    a.num_q_heads = Hq;
    a.num_kv_heads = Hkv;
    a.max_blocks_per_seq = mbs;
    a.partition_size = P;
    a.num_partitions = NP;
    a.n_tiles = n_tiles;
    a.longest_first = B <= pkv::kScheduleMaxSeqs && mbs < (1 << 23) ? 1 : 0;
    a.scale_log2 = scale * 1.44269504088896340736f;
    return a;
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status s) {
    switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "invalid or inconsistent sizes";
    case PKV_ERR_DTYPE: return "unsupported dtype or dtype pairing";
    case PKV_ERR_UNSUPPORTED: return "head_dim or block_size outside the supported set";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_CAPACITY: return "too few free blocks in the pool";
    case PKV_ERR_SEQUENCE: return "unknown or already existing sequence id";
    default: return "unknown status";
    }
}

const char* pkv_last_error(void) { return pkv::last_error(); }

}  // extern "C"

namespace {
// The smallest power of two in [256, cap] that cuts the longest context of a
// launch with `count` work-groups per partition into about `wgs` in all.
int pow2_partition(int64_t count, int64_t max_tokens, int64_t wgs, int cap) {
    const int64_t want = (max_tokens * count + wgs - 1) / wgs;  // tokens per work-group
    int P = 256;
    while (P < cap && P < want) P <<= 1;
    return P;
}

// Decodes with 16-bit q of 8 to 63 q heads per kv head over a cache of q's
// dtype, or 4 to 63 over a quantized one (INT8, FP8; 4-bit from head_dim
// 128), run on the matrix cores (the short-run multi-query kernel; see
// decode_mfma).  Measured, fused step of 64 sequences U[512, 4096], decode
// kernel against matrix cores: 4 q heads per kv head, INT8 / bf16 q 86.0 vs
// 66.7 us, FP8 95.1 vs 72.0, 4-bit 81.6 vs 66.0, bf16 cache (128 x
// U[1024, 8192]) 365.4 vs 367.3; 2 per kv head, INT8 125.4 vs 135.1, 4-bit
// 88.9 vs 128.1.
bool decode_on_matrix_cores(int g, int window, pkv_dtype q_dtype, pkv_dtype cache_dtype) {
    const bool quant = cache_dtype == PKV_I8 || cache_dtype == PKV_F8_E4M3 || cache_dtype == PKV_U4;
    return window == 0 && g >= (quant ? 4 : 8) && g < 64 &&
           (q_dtype == PKV_F16 || q_dtype == PKV_BF16) && (cache_dtype == q_dtype || quant);
}

// Measured on MI355X: a work-group pays a chain of dependent memory round
// trips (context length, block ids, first K/V tiles) before it streams, and
// a split adds the merge launch, so long partitions stream best; they are cut
// only as far as needed to give the chip about as many work-groups as it
// holds at once, counted at the maximum context: 1024 for one-head tiles
// (two 8-wave work-groups per CU), 256 for tiles of several q heads (their
// registers leave room for one per CU; work-groups counted as the decode
// launches them, num_seqs x num_q_heads / heads per tile), and for the
// decodes on the matrix cores their own (below).  Partitions of
// at most 4096 tokens, or 8192 once the batch has 1024 (sequence, kv head)
// items.  Sweeps of the fused step over powers of two (same box), µs at the
// size this picks, and in brackets at the size a rule of 2048 work-groups
// per (sequence, kv head) item picked: GQA 32/8 4 x 32k 85.9 (109.1), 8 x
// 32k 169.9 (182.0), 1 x 32k 26.4 (40.3), 16 x U[1024, 8192] 59.9 (68.1),
// 64 x U[512, 4096] 90.0 (119.2); one-head tiles: 64 sequences x 4 heads
// 55.0 (57.0), 16 x U[512, 4096] 89.0 (91.4), 32 x U[1024, 8192] x 8 heads
// 106.0 (106.3), 16 x U[4096, 16384] x 16 heads 203.2 (204.5); 32 q / 4 kv
// heads x 64 sequences, INT8 83.1 (102.5 at half the size), 32 q / 2 kv
// heads x 32 sequences, 4-bit 53.8 (71.1).  Each the best size or within
// 1.2% of it, but for 8 x U[512, 4096]: 61.0 unsplit against 64.9 here.
int decode_default_partition(int num_seqs, int num_q_heads, int num_kv_heads,
                             int max_blocks_per_seq, pkv_dtype cache_dtype) {
    const int g = num_q_heads / num_kv_heads;
    const int64_t items = (int64_t)num_seqs * num_kv_heads;
    const int64_t max_tokens = (int64_t)max_blocks_per_seq * pkv::kBlockSize;
    const int cap = items >= 1024 ? 8192 : 4096;
    // (q's dtype is not an argument: an 8-bit cache is taken with 16-bit q)
    if (decode_on_matrix_cores(g, 0, is_float(cache_dtype) ? cache_dtype : PKV_F16, cache_dtype)) {
        // 8-wave work-groups, one per 16-row tile and partition: about 256
        // of them (512 once there are 1024 tiles) at the longest context.
        // Sweeps of the step over powers of two, µs at the size this picks
        // and in brackets at the size of the 4-wave multi-query rule: 64 q /
        // 8 kv heads bf16, 64 x U[512, 4096] 105.9 (105.9), 8 x U[8k, 16k]
        // 73.5 (81.9), 256 x U[512, 4096] 399.3 (399.3); 32 q / 1 kv head
        // bf16 64 x U[512, 4096] 42.6 (46.0); 32 q / 2 kv heads 16 x U[512,
        // 4096] 21.6; 32 q / 4 kv heads 64 x U[512, 4096] 67.1 (66.5).
        const int64_t rows = items * ((g + 15) / 16);  // 16-row tiles
        return pow2_partition(rows, max_tokens, rows >= 1024 ? 512 : 256,
                              rows >= 1024 ? 8192 : 4096);
    }
    if (g == 1) {
        const int P = pow2_partition(items, max_tokens, 1024, cap);
        // over at most 1024 tokens: no split (the merge launch costs more
        // than it parallelizes: 1 x 1k 16.3 -> 14.2 us, 16 x 1k 44.7 -> 41.3)
        return max_tokens <= 1024 && P < max_tokens ? 1024 : P;
    }
    const int64_t wgs = (int64_t)num_seqs * (num_q_heads / heads_per_tile(g, cache_dtype));
    return pow2_partition(wgs, max_tokens, 256, cap);
}
}  // namespace

extern "C" {

int pkv_default_partition_size(int num_seqs, int num_q_heads, int num_kv_heads,
                               int max_blocks_per_seq, pkv_dtype cache_dtype) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        num_q_heads % num_kv_heads != 0 || !(is_float(cache_dtype) || is_quantized(cache_dtype)))
        return 0;
    return decode_default_partition(num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq,
                                    cache_dtype);
}

size_t pkv_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_blocks_per_seq, int partition_size,
                                 pkv_dtype cache_dtype) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        num_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim) || partition_size < 0 ||
        partition_size % pkv::kBlockSize != 0 ||
        !(is_float(cache_dtype) || is_quantized(cache_dtype)))
        return 0;
    const int P = partition_size ? partition_size
                                 : decode_default_partition(num_seqs, num_q_heads, num_kv_heads,
                                                            max_blocks_per_seq, cache_dtype);
    return layout(num_seqs, num_q_heads, head_dim, num_partitions(max_blocks_per_seq, P)).total;
}

pkv_status pkv_kv_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                              float* k_scale, float* v_scale, const int64_t* slot_mapping,
                              int64_t num_tokens, int num_kv_heads, int head_dim, int block_size,
                              int64_t num_blocks, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                              hipStream_t stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE,
                    "need num_tokens >= 0, num_kv_heads > 0 and num_blocks > 0 (got %lld, %d, %lld)",
                    (long long)num_tokens, num_kv_heads, (long long)num_blocks);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (only 16)", block_size);
    if (!head_dim_ok(head_dim))
        return fail(PKV_ERR_UNSUPPORTED, "head_dim %d unsupported (64, 128, 256)", head_dim);
    if (cache_dtype == PKV_U4 && head_dim == 64)
        return fail(PKV_ERR_UNSUPPORTED, "4-bit caches need head_dim 128 or 256");
    if (!is_float(src_dtype) || !(cache_dtype == src_dtype || is_quantized(cache_dtype)))
        return fail(PKV_ERR_DTYPE, "unsupported (src_dtype, cache_dtype) = (%d, %d)",
                    (int)src_dtype, (int)cache_dtype);
    if (num_tokens == 0) return ok();
    if (!k || !v || !k_cache || !v_cache || !slot_mapping)
        return fail(PKV_ERR_NULL, "k, v, k_cache, v_cache and slot_mapping are required");
    if (is_quantized(cache_dtype) && (!k_scale || !v_scale))
        return fail(PKV_ERR_NULL, "k_scale and v_scale are required for an INT8 / FP8 / 4-bit cache");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKV_ERR_SHAPE, "k, v, k_cache and v_cache must be 16-byte aligned");
    // a 4-bit row's (x_min, range) pair is stored as one 8-byte word
    if (cache_dtype == PKV_U4 &&
        ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 7u))
        return fail(PKV_ERR_SHAPE, "4-bit k_scale and v_scale must be 8-byte aligned");
    pkv::CacheWriteArgs a{k, v, k_cache, v_cache, k_scale, v_scale, slot_mapping, nullptr,
                          nullptr, 0, num_tokens, num_blocks, num_kv_heads};
    return hip_status(
        pkv::launch_kv_cache_write(a, (int)src_dtype, (int)cache_dtype, head_dim, stream),
        "kv_cache_write launch");
}

pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                           const int32_t* copy_pairs, int64_t num_pairs, int num_kv_heads,
                           int head_dim, int block_size, int64_t num_blocks,
                           pkv_dtype cache_dtype, hipStream_t stream) {
    if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE,
                    "need num_pairs >= 0, num_kv_heads > 0 and num_blocks > 0 (got %lld, %d, %lld)",
                    (long long)num_pairs, num_kv_heads, (long long)num_blocks);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (only 16)", block_size);
    if (!head_dim_ok(head_dim))
        return fail(PKV_ERR_UNSUPPORTED, "head_dim %d unsupported (64, 128, 256)", head_dim);
    if (!is_float(cache_dtype) && !is_quantized(cache_dtype))
        return fail(PKV_ERR_DTYPE, "unsupported cache_dtype %d", (int)cache_dtype);
    if (num_pairs == 0) return ok();
    if (!k_cache || !v_cache || !copy_pairs)
        return fail(PKV_ERR_NULL, "k_cache, v_cache and copy_pairs are required");
    if (is_quantized(cache_dtype) && (!k_scale || !v_scale))
        return fail(PKV_ERR_NULL, "k_scale and v_scale are required for an INT8 / FP8 / 4-bit cache");
    if (!aligned16(k_cache) || !aligned16(v_cache) ||
        (is_quantized(cache_dtype) && (!aligned16(k_scale) || !aligned16(v_scale))))
        return fail(PKV_ERR_SHAPE, "caches and scales must be 16-byte aligned");
    pkv::CopyBlocksArgs a{};
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_scale = is_quantized(cache_dtype) ? k_scale : nullptr;
    a.v_scale = is_quantized(cache_dtype) ? v_scale : nullptr;
    a.pairs = copy_pairs;
    a.num_pairs = num_pairs;
    a.num_blocks = num_blocks;
    a.block_bytes = (int64_t)num_kv_heads * pkv::kBlockSize * row_bytes(cache_dtype, head_dim);
    a.scale_bytes = is_quantized(cache_dtype)
                        ? (int64_t)num_kv_heads * pkv::kBlockSize * (cache_dtype == PKV_U4 ? 8 : 4)
                        : 0;
    if (a.block_bytes > ((int64_t)1 << 40) / num_blocks)
        return fail(PKV_ERR_SHAPE, "pool too large");
    const hipError_t e = pkv::launch_copy_blocks(a, stream);
    if (e == hipErrorInvalidValue)
        return fail(PKV_ERR_SHAPE, "too many copy pairs for one launch (%lld)",
                    (long long)num_pairs);
    return hip_status(e, "copy_blocks launch");
}

}  // extern "C"

namespace {

// Phase 2 (merge of partials) for a decode with the given sliding window.
pkv_status reduce_impl(void* out, const float* m_part, const float* l_part, const float* o_part,
                       const int32_t* context_lens, int num_seqs, int num_q_heads, int head_dim,
                       int partition_size, int num_partitions_, int skip_single_partition,
                       pkv_dtype out_dtype, int window, hipStream_t stream) {
    if (num_seqs < 0 || num_q_heads <= 0 || num_partitions_ <= 0)
        return fail(PKV_ERR_SHAPE, "need num_seqs >= 0, positive num_q_heads and num_partitions");
    if (partition_size <= 0 || partition_size % pkv::kBlockSize != 0)
        return fail(PKV_ERR_SHAPE, "partition_size %d is not a positive multiple of 16",
                    partition_size);
    if (!head_dim_ok(head_dim))
        return fail(PKV_ERR_UNSUPPORTED, "head_dim %d unsupported (64, 128, 256)", head_dim);
    if (!is_float(out_dtype)) return fail(PKV_ERR_DTYPE, "out_dtype must be F32, F16 or BF16");
    if (num_seqs == 0) return ok();
    if (!out || !m_part || !l_part || !o_part || !context_lens)
        return fail(PKV_ERR_NULL, "out, m_part, l_part, o_part and context_lens are required");
    if (!aligned16(o_part)) return fail(PKV_ERR_SHAPE, "o_part must be 16-byte aligned");
    pkv::ReduceArgs a{};
    a.out = out;
    a.m_part = m_part;
    a.l_part = l_part;
    a.o_part = o_part;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.partition_size = partition_size;
    a.num_partitions = num_partitions_;
    a.skip_single = skip_single_partition ? 1 : 0;
    a.window = window;
    a.query_start_loc = nullptr;
    a.num_rows = num_seqs;
    return hip_status(pkv::launch_paged_reduce(a, (int)out_dtype, head_dim, stream),
                      "paged_attn_reduce launch");
}

// Phase 1, optionally with the append of each sequence's new token.
pkv_status decode_phase1(void* out, float* m_part, float* l_part, float* o_part, const void* q,
                         const void* k_new, const void* v_new, const void* k_cache,
                         const void* v_cache, const float* k_scale, const float* v_scale,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                         int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                         float scale, int partition_size, int num_partitions_, pkv_dtype q_dtype,
                         pkv_dtype cache_dtype, int window, hipStream_t stream) {
    pkv_status s = check_decode(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, block_size, num_blocks, q_dtype,
                                cache_dtype);
    if (s != PKV_OK) return s;
    if (partition_size <= 0 || partition_size % pkv::kBlockSize != 0)
        return fail(PKV_ERR_SHAPE, "partition_size %d is not a positive multiple of 16",
                    partition_size);
    const int NP = num_partitions(window_blocks(max_blocks_per_seq, window), partition_size);
    if (num_partitions_ < NP)
        return fail(PKV_ERR_SHAPE, "num_partitions %d < ceil(max_blocks_per_seq*16/P) = %d",
                    num_partitions_, NP);
    if (num_seqs == 0) return ok();
    if (!m_part || !l_part || !o_part)
        return fail(PKV_ERR_NULL, "m_part, l_part and o_part are required");
    if (out && !aligned16(out)) return fail(PKV_ERR_SHAPE, "out must be 16-byte aligned");
    const int gt = heads_per_tile(num_q_heads / num_kv_heads, cache_dtype);
    pkv::DecodeArgs a = make_args(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                  max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                  num_kv_heads, num_blocks, scale, partition_size,
                                  num_partitions_, num_q_heads / gt);
    a.out = out;
    a.k_new = k_new;
    a.v_new = v_new;
    a.m_part = m_part;
    a.l_part = l_part;
    a.o_part = o_part;
    a.window = window;
    return hip_status(pkv::launch_paged_decode(a, (int)q_dtype, (int)cache_dtype, head_dim, gt,
                                               stream),
                      "paged decode launch");
}

// The decode of q-head groups of 8 (4 over a quantized cache) to 63 per kv head (16-bit q; a cache of
// q's dtype, INT8 or FP8; no window) on the matrix cores: the decode
// kernel's tiles of 8 heads keep 8 dot products per K row in vector
// registers and run at about half the HBM rate, while the short-run
// multi-query kernel takes a kv head's 8..63 heads as MFMA rows (8-bit codes
// widened to q's dtype as they are staged, exactly; the K scale multiplies
// the score, the V scale the weight).  Its softmax weights enter P.V as two
// 16-bit parts (exact_p), so the result keeps the decode's precision.  With
// new tokens, the launch stores each sequence's row at its context end and
// computes with the given row (one launch, as the decode kernel's append; for
// a quantized cache the row is quantized by the cache write's own
// quantizer, so the stored bytes are the same).  Measured (decode of U[512, 4096]
// contexts, fp16 / bf16): 64 q / 8 kv heads x 64 sequences 145-147 ->
// 103 us, x 256 sequences 585-591 -> 367 us, 32 q / 4 kv heads x 64
// sequences 113-115 -> 63 us (the multi-query kernel with 16-bit weights);
// 4 q heads per kv head stay on the decode kernel (368 us either way).
pkv_status decode_mfma(void* out, float* m, float* l, float* o, const void* q, const void* k_new,
                       const void* v_new, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale,
                       const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* context_lens, int num_seqs, int num_q_heads,
                       int num_kv_heads, int head_dim, int64_t num_blocks, float scale, int P,
                       int NP, pkv_dtype dtype, pkv_dtype cache_dtype, hipStream_t stream) {
    const bool quant = cache_dtype != dtype;  // INT8 / FP8 / 4-bit codes with scales
    const int g = num_q_heads / num_kv_heads;
    pkv::MultiArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start_loc = nullptr;
    a.m_part = m;
    a.l_part = l;
    a.o_part = o;
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.partition_size = P;
    a.num_partitions = NP;
    a.row_tiles = (int)pkv::multi_row_groups(g, head_dim);
    a.max_rows = g;
    a.num_tokens = num_seqs;
    a.causal = 1;
    a.one_query = 1;
    a.exact_p = 1;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_cache_w = k_new ? const_cast<void*>(k_cache) : nullptr;
    a.v_cache_w = k_new ? const_cast<void*>(v_cache) : nullptr;
    a.k_scale = quant ? k_scale : nullptr;
    a.v_scale = quant ? v_scale : nullptr;
    a.k_scale_w = quant && k_new ? const_cast<float*>(k_scale) : nullptr;
    a.v_scale_w = quant && k_new ? const_cast<float*>(v_scale) : nullptr;
    a.scale_log2 = scale * 1.44269504088896340736f;
    if ((int64_t)num_seqs * num_kv_heads * a.row_tiles * NP > 0x7fffffff)
        return fail(PKV_ERR_SHAPE, "too many work items for one launch");
    return hip_status(pkv::launch_paged_multi(a, (int)dtype, (int)cache_dtype, head_dim, stream),
                      "paged decode (matrix cores) launch");
}

// Phase 1 with direct output, then the merge of sequences with > 1 partition.
pkv_status decode_both_phases(void* out, const void* q, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache, const float* k_scale,
                              const float* v_scale, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                              int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                              int64_t num_blocks, float scale, int partition_size,
                              void* workspace, size_t workspace_bytes, pkv_dtype q_dtype,
                              pkv_dtype cache_dtype, int window, hipStream_t stream) {
    pkv_status s = check_decode(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, block_size, num_blocks, q_dtype,
                                cache_dtype);
    if (s != PKV_OK) return s;
    if (partition_size < 0 || partition_size % pkv::kBlockSize != 0)
        return fail(PKV_ERR_SHAPE, "partition_size %d is not 0 or a positive multiple of 16",
                    partition_size);
    if (num_seqs == 0) return ok();
    if (!out) return fail(PKV_ERR_NULL, "out is required");
    if (!aligned16(out)) return fail(PKV_ERR_SHAPE, "out must be 16-byte aligned");
    const int mbs_eff = window_blocks(max_blocks_per_seq, window);
    const int P = partition_size ? partition_size
                                 : decode_default_partition(num_seqs, num_q_heads, num_kv_heads,
                                                            mbs_eff, cache_dtype);
    const int NP = num_partitions(mbs_eff, P);
    const WorkspaceLayout w = layout(num_seqs, num_q_heads, head_dim, NP);
    if (!workspace || workspace_bytes < w.total)
        return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    char* ws = static_cast<char*>(workspace);
    float* m = reinterpret_cast<float*>(ws + w.m_off);
    float* l = reinterpret_cast<float*>(ws + w.l_off);
    float* o = reinterpret_cast<float*>(ws + w.o_off);
    if (decode_on_matrix_cores(num_q_heads / num_kv_heads, window, q_dtype, cache_dtype))
        s = decode_mfma(out, m, l, o, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                        block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, num_blocks, scale, P, NP, q_dtype, cache_dtype,
                        stream);
    else
        s = decode_phase1(out, m, l, o, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                          block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, scale, P, NP, q_dtype,
                          cache_dtype, window, stream);
    if (s != PKV_OK) return s;
    if (NP == 1) return ok();  // every sequence was finished in phase 1
    return reduce_impl(out, m, l, o, context_lens, num_seqs, num_q_heads, head_dim, P, NP, 1,
                       q_dtype, window, stream);
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attn_decode_partials(void* out, float* m_part, float* l_part, float* o_part,
                                          const void* q, const void* k_cache, const void* v_cache,
                                          const float* k_scale, const float* v_scale,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* context_lens, int num_seqs,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int64_t num_blocks, float scale,
                                          int partition_size, int num_partitions_,
                                          pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                          hipStream_t stream) {
    return decode_phase1(out, m_part, l_part, o_part, q, nullptr, nullptr, k_cache, v_cache,
                         k_scale, v_scale, block_tables, max_blocks_per_seq, context_lens,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                         scale, partition_size, num_partitions_, q_dtype, cache_dtype, 0, stream);
}

pkv_status pkv_paged_attn_reduce(void* out, const float* m_part, const float* l_part,
                                 const float* o_part, const int32_t* context_lens, int num_seqs,
                                 int num_q_heads, int head_dim, int partition_size,
                                 int num_partitions_, int skip_single_partition,
                                 pkv_dtype out_dtype, hipStream_t stream) {
    return reduce_impl(out, m_part, l_part, o_part, context_lens, num_seqs, num_q_heads,
                       head_dim, partition_size, num_partitions_, skip_single_partition,
                       out_dtype, 0, stream);
}

pkv_status pkv_paged_attn_decode(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int64_t num_blocks, float scale, int partition_size,
                                 void* workspace, size_t workspace_bytes, pkv_dtype q_dtype,
                                 pkv_dtype cache_dtype, hipStream_t stream) {
    return decode_both_phases(out, q, nullptr, nullptr, k_cache, v_cache, k_scale, v_scale,
                              block_tables, max_blocks_per_seq, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                              partition_size, workspace, workspace_bytes, q_dtype, cache_dtype,
                              0, stream);
}

pkv_status pkv_paged_attn_decode_append(void* out, const void* q, const void* k_new,
                                        const void* v_new, void* k_cache, void* v_cache,
                                        float* k_scale, float* v_scale,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens, int num_seqs,
                                        int num_q_heads, int num_kv_heads, int head_dim,
                                        int block_size, int64_t num_blocks, float scale,
                                        int partition_size, void* workspace,
                                        size_t workspace_bytes, pkv_dtype q_dtype,
                                        pkv_dtype cache_dtype, hipStream_t stream) {
    if (num_seqs > 0 && (!k_new || !v_new))
        return fail(PKV_ERR_NULL, "k_new and v_new are required");
    if (num_seqs > 0 && (!aligned16(k_new) || !aligned16(v_new)))
        return fail(PKV_ERR_SHAPE, "k_new and v_new must be 16-byte aligned");
    return decode_both_phases(out, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                              block_tables, max_blocks_per_seq, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                              partition_size, workspace, workspace_bytes, q_dtype, cache_dtype,
                              0, stream);
}

pkv_status pkv_paged_attn_decode_sliding(void* out, const void* q, const void* k_new,
                                         const void* v_new, void* k_cache, void* v_cache,
                                         float* k_scale, float* v_scale,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* context_lens, int num_seqs,
                                         int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int64_t num_blocks, float scale,
                                         int sliding_window, int partition_size, void* workspace,
                                         size_t workspace_bytes, pkv_dtype q_dtype,
                                         pkv_dtype cache_dtype, hipStream_t stream) {
    if (sliding_window < 0)
        return fail(PKV_ERR_SHAPE, "sliding_window %d < 0", sliding_window);
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(PKV_ERR_NULL, "k_new and v_new must both be given or both be NULL");
    if (num_seqs > 0 && k_new && (!aligned16(k_new) || !aligned16(v_new)))
        return fail(PKV_ERR_SHAPE, "k_new and v_new must be 16-byte aligned");
    return decode_both_phases(out, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                              block_tables, max_blocks_per_seq, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                              partition_size, workspace, workspace_bytes, q_dtype, cache_dtype,
                              sliding_window, stream);
}

size_t pkv_multi_workspace_size(int num_query_tokens, int num_q_heads, int head_dim,
                                int max_blocks_per_seq, int partition_size) {
    if (num_query_tokens < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 ||
        !head_dim_ok(head_dim) || partition_size <= 0 || partition_size % pkv::kBlockSize != 0)
        return 0;
    return layout(num_query_tokens, num_q_heads, head_dim,
                  num_partitions(max_blocks_per_seq, partition_size))
        .total;
}

int pkv_multi_default_partition_size(int num_seqs, int max_query_len, int num_q_heads,
                                     int num_kv_heads, int max_blocks_per_seq) {
    if (num_seqs < 0 || max_query_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        num_q_heads % num_kv_heads != 0)
        return 0;
    const int64_t rows = (int64_t)max_query_len * (num_q_heads / num_kv_heads);
    const int64_t tiles = (rows + 15) / 16;
    const int64_t items = (int64_t)num_seqs * tiles * num_kv_heads;
    // About 512 work-groups of 4 waves at the longest context (1024 once
    // the items fill the chip).  Sweeps over all powers of two (same box),
    // 8 or 4 queries per sequence: the size this picks was the best on all
    // six shapes; µs, and in brackets at the size a 2048-work-group rule
    // picked: 8 x U[512, 4096] 32 heads 63.4 (84.3), 2 x 16k 88.3 (101.8),
    // GQA 32/8 16 x U[1024, 8192] 109.3 (122.5), 4 x 32k 90.0 (110.4);
    // 64 x U[512, 4096] GQA and MHA unchanged (within 0.1% of the best).
    return pow2_partition(items, (int64_t)max_blocks_per_seq * pkv::kBlockSize,
                          items >= 1024 ? 1024 : 512, items >= 1024 ? 8192 : 4096);
}

}  // extern "C"

namespace {

// The prefix piece of a shared-prefix decode: its partition size and count,
// and the workspace: fp32 partials of the prefix (m, l [B][Hq][NP],
// o [B][Hq][NP][D]) and a region for the own positions' partials (m, l
// [B][Hq], o [B][Hq][D]) that the decode launch is given but, with its one
// partition and an output to merge into, never writes; each region 256-byte
// aligned.
struct SharedPrefixLayout {
    int P, NP;
    size_t m0, l0, o0, m1, l1, o1, total;
};

bool shared_prefix_layout(int B, int G, int max_group, int Hq, int Hkv, int D, int mbs,
                          SharedPrefixLayout& w) {
    // a group's rows share one tile, so the prefix has few work items (groups
    // x kv heads); the default rule would cut them into short partitions,
    // yet each split adds partials and a merge.  Counting every group four
    // times gives longer partitions (measured on the 16-prompt x 4-sample
    // workload with 1x / 2x / 4x the groups: 3 / 2 / 1 partitions, 108.6 /
    // 99.9 / 97.5 us)
    w.P = pkv_multi_default_partition_size(G > 0x7fffffff / 4 ? 0x7fffffff : G * 4, max_group,
                                           Hq, Hkv, mbs);
    if (w.P <= 0) return false;
    w.NP = num_partitions(mbs, w.P);
    const size_t pre = (size_t)B * Hq * w.NP, own = (size_t)B * Hq;
    w.m0 = 0;
    w.l0 = align256(w.m0 + pre * sizeof(float));
    w.o0 = align256(w.l0 + pre * sizeof(float));
    w.m1 = align256(w.o0 + pre * D * sizeof(float));
    w.l1 = align256(w.m1 + own * sizeof(float));
    w.o1 = align256(w.l1 + own * sizeof(float));
    w.total = align256(w.o1 + own * D * sizeof(float));
    return true;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attn_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int num_seqs, int num_query_tokens, int max_query_len,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int64_t num_blocks, float scale, int partition_size,
                                void* workspace, size_t workspace_bytes, pkv_dtype q_dtype,
                                pkv_dtype cache_dtype, hipStream_t stream) {
    if (num_seqs < 0 || num_query_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE,
                    "need num_seqs, num_query_tokens >= 0 and positive num_q_heads, num_kv_heads, "
                    "max_blocks_per_seq, num_blocks");
    if (num_q_heads % num_kv_heads != 0)
        return fail(PKV_ERR_SHAPE, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                    num_q_heads, num_kv_heads);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (only 16)", block_size);
    if (!head_dim_ok(head_dim))
        return fail(PKV_ERR_UNSUPPORTED, "head_dim %d unsupported (64, 128, 256)", head_dim);
    if (!((q_dtype == PKV_F16 || q_dtype == PKV_BF16) && cache_dtype == q_dtype))
        return fail(PKV_ERR_DTYPE, "multi-query attention needs (F16,F16) or (BF16,BF16), got "
                                   "(%d, %d)", (int)q_dtype, (int)cache_dtype);
    if (partition_size < 0 || partition_size % pkv::kBlockSize != 0)
        return fail(PKV_ERR_SHAPE, "partition_size %d is not 0 or a positive multiple of 16",
                    partition_size);
    if (num_seqs == 0 || num_query_tokens == 0) return ok();
    if (max_query_len <= 0)
        return fail(PKV_ERR_SHAPE, "max_query_len must be positive");
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
        return fail(PKV_ERR_NULL, "out, q, k_cache, v_cache, block_tables, context_lens and "
                                  "query_start_loc are required");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return fail(PKV_ERR_SHAPE, "q, out, k_cache and v_cache must be 16-byte aligned");
    const int g = num_q_heads / num_kv_heads;
    if ((int64_t)max_query_len * g > 0x7fffffff)
        return fail(PKV_ERR_SHAPE, "max_query_len * num_q_heads / num_kv_heads too large");
    const int max_rows = max_query_len * g;
    const int64_t row_tiles = pkv::multi_row_groups(max_rows, head_dim);
    const int P = partition_size ? partition_size
                                 : pkv_multi_default_partition_size(num_seqs, max_query_len,
                                                                    num_q_heads, num_kv_heads,
                                                                    max_blocks_per_seq);
    const int NP = num_partitions(max_blocks_per_seq, P);
    const WorkspaceLayout w = layout(num_query_tokens, num_q_heads, head_dim, NP);
    if (NP > 1) {
        if (!workspace || workspace_bytes < w.total)
            return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                        workspace ? workspace_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    if ((int64_t)num_seqs * num_kv_heads * row_tiles * NP > 0x7fffffff)
        return fail(PKV_ERR_SHAPE, "too many work items for one launch");
    char* ws = static_cast<char*>(workspace);
    pkv::MultiArgs a{};
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start_loc = query_start_loc;
    a.m_part = NP > 1 ? reinterpret_cast<float*>(ws + w.m_off) : nullptr;
    a.l_part = NP > 1 ? reinterpret_cast<float*>(ws + w.l_off) : nullptr;
    a.o_part = NP > 1 ? reinterpret_cast<float*>(ws + w.o_off) : nullptr;
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.partition_size = P;
    a.num_partitions = NP;
    a.row_tiles = (int)row_tiles;
    a.max_rows = max_rows;
    a.num_tokens = num_query_tokens;
    a.causal = 1;
    a.scale_log2 = scale * 1.44269504088896340736f;
    pkv_status s = hip_status(pkv::launch_paged_multi(a, (int)q_dtype, (int)q_dtype, head_dim, stream),
                              "paged multi-query launch");
    if (s != PKV_OK || NP == 1) return s;
    pkv::ReduceArgs r{};
    r.out = out;
    r.m_part = a.m_part;
    r.l_part = a.l_part;
    r.o_part = a.o_part;
    r.context_lens = context_lens;
    r.num_seqs = num_seqs;
    r.num_q_heads = num_q_heads;
    r.partition_size = P;
    r.num_partitions = NP;
    r.skip_single = 1;
    r.window = 0;
    r.query_start_loc = query_start_loc;
    r.num_rows = num_query_tokens;
    return hip_status(pkv::launch_paged_reduce(r, (int)q_dtype, head_dim, stream),
                      "paged_attn_reduce launch");
}

size_t pkv_shared_prefix_workspace_size(int num_seqs, int num_groups, int max_group_size,
                                        int num_q_heads, int num_kv_heads, int head_dim,
                                        int max_blocks_per_seq) {
    if (num_seqs < 0 || num_groups < 0 || max_group_size <= 0 || num_q_heads <= 0 ||
        num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || !head_dim_ok(head_dim) ||
        max_blocks_per_seq <= 0)
        return 0;
    SharedPrefixLayout w;
    if (!shared_prefix_layout(num_seqs, num_groups, max_group_size, num_q_heads, num_kv_heads,
                              head_dim, max_blocks_per_seq, w))
        return 0;
    return w.total;
}

pkv_status pkv_paged_attn_decode_shared_prefix(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* prefix_lens, const int32_t* group_start, int num_groups, int max_group_size,
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int64_t num_blocks, float scale, void* workspace, size_t workspace_bytes, pkv_dtype q_dtype,
    pkv_dtype cache_dtype, hipStream_t stream) {
    pkv_status s = check_decode(q, k_cache, v_cache, nullptr, nullptr, block_tables,
                                max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, block_size, num_blocks, q_dtype,
                                cache_dtype);
    if (s != PKV_OK) return s;
    if (!((q_dtype == PKV_F16 || q_dtype == PKV_BF16) && cache_dtype == q_dtype))
        return fail(PKV_ERR_DTYPE, "shared-prefix decode needs (F16,F16) or (BF16,BF16), got "
                                   "(%d, %d)", (int)q_dtype, (int)cache_dtype);
    if (num_groups < 0 || max_group_size <= 0)
        return fail(PKV_ERR_SHAPE, "need num_groups >= 0 and max_group_size > 0 (got %d, %d)",
                    num_groups, max_group_size);
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(PKV_ERR_NULL, "k_new and v_new must both be given or both be NULL");
    if (num_seqs == 0) return ok();
    if (num_groups == 0 || num_groups > num_seqs)
        return fail(PKV_ERR_SHAPE, "need 1 <= num_groups <= num_seqs (got %d, %d)", num_groups,
                    num_seqs);
    if (!out || !prefix_lens || !group_start)
        return fail(PKV_ERR_NULL, "out, prefix_lens and group_start are required");
    if (!aligned16(out) || (k_new && (!aligned16(k_new) || !aligned16(v_new))))
        return fail(PKV_ERR_SHAPE, "out, k_new and v_new must be 16-byte aligned");
    const int g = num_q_heads / num_kv_heads;
    if ((int64_t)max_group_size * g > 0x7fffffff)
        return fail(PKV_ERR_SHAPE, "max_group_size * num_q_heads / num_kv_heads too large");
    SharedPrefixLayout w;
    if (!shared_prefix_layout(num_seqs, num_groups, max_group_size, num_q_heads, num_kv_heads,
                              head_dim, max_blocks_per_seq, w))
        return fail(PKV_ERR_SHAPE, "no partition size for these sizes");
    if (!workspace || workspace_bytes < w.total)
        return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                    w.total);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const int max_rows = max_group_size * g;
    const int64_t row_tiles = pkv::multi_row_groups(max_rows, head_dim);
    if ((int64_t)num_groups * num_kv_heads * row_tiles * w.NP > 0x7fffffff)
        return fail(PKV_ERR_SHAPE, "too many work items for one launch");
    char* ws = static_cast<char*>(workspace);
    float* m0 = reinterpret_cast<float*>(ws + w.m0);
    float* l0 = reinterpret_cast<float*>(ws + w.l0);
    float* o0 = reinterpret_cast<float*>(ws + w.o0);
    float* m1 = reinterpret_cast<float*>(ws + w.m1);
    float* l1 = reinterpret_cast<float*>(ws + w.l1);
    float* o1 = reinterpret_cast<float*>(ws + w.o1);
    const float scale_log2 = scale * 1.44269504088896340736f;

    // the shared prefix: a group's queries are the rows of one tile per kv
    // head; no causal mask (every query follows the whole prefix)
    pkv::MultiArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = prefix_lens;
    a.query_start_loc = group_start;
    a.m_part = m0;
    a.l_part = l0;
    a.o_part = o0;
    a.num_blocks = num_blocks;
    a.num_seqs = num_groups;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.partition_size = w.P;
    a.num_partitions = w.NP;
    a.row_tiles = (int)row_tiles;
    a.max_rows = max_rows;
    a.num_tokens = num_seqs;
    a.causal = 0;
    a.partials_only = 1;
    a.group_rows = 1;
    a.scale_log2 = scale_log2;
    s = hip_status(pkv::launch_paged_multi(a, (int)q_dtype, (int)q_dtype, head_dim, stream),
                   "shared-prefix launch");
    if (s != PKV_OK) return s;

    // each sequence's own positions (with the append), one partition
    const int gt = heads_per_tile(g, cache_dtype);
    const int own_p = (max_blocks_per_seq < 0x7fffffff / pkv::kBlockSize ? max_blocks_per_seq
                                                                         : 0x7fffffff /
                                                                               pkv::kBlockSize) *
                      pkv::kBlockSize;
    pkv::DecodeArgs d = make_args(q, k_cache, v_cache, nullptr, nullptr, block_tables,
                                  max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                  num_kv_heads, num_blocks, scale, own_p, 1, num_q_heads / gt);
    // ... which merges its result with the prefix partials into `out` itself
    d.out = out;
    d.k_new = k_new;
    d.v_new = v_new;
    d.m_part = m1;
    d.l_part = l1;
    d.o_part = o1;
    d.seq_start = prefix_lens;
    d.pre_m = m0;
    d.pre_l = l0;
    d.pre_o = o0;
    d.pre_np = w.NP;
    d.pre_partition_size = w.P;
    return hip_status(pkv::launch_paged_decode(d, (int)q_dtype, (int)cache_dtype, head_dim, gt,
                                               stream),
                      "own-positions decode launch");
}

}  // extern "C"

// ---- decode with the fused append into a library-owned scratch array -------
// For callers that cannot allocate device memory.  The partials of a split
// decode live in `scratch`, a static device array of kStaticScratchBytes that
// every GPU the library runs on holds from the load of this code until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address is looked up once per GPU with
// hipGetSymbolAddress (that GPU current) and only that address is handed to
// kernels.  Calls on one GPU share the array (overlapping calls race); the
// decode writes every partial it later reads, so nothing is cleared.

namespace {

constexpr size_t kStaticScratchBytes = PKV_STATIC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the GPU that `stream` runs on.
pkv_status scratch_on(hipStream_t stream, void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (stream != nullptr) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(stream, &sd);
        if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
        dev = sd;
    }
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(PKV_ERR_UNSUPPORTED, "device %d beyond the %d the static scratch serves", dev,
                    kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_status(e, "hipGetDevice");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return hip_status(e, "hipSetDevice");
        void* p = nullptr;
        const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess)
            return hip_status(e, "hipSetDevice");
        if (es != hipSuccess) return hip_status(es, "hipGetSymbolAddress(scratch)");
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u))
            return fail(PKV_ERR_HIP, "static scratch address %p is not 256-byte aligned", p);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ok();
}

}  // namespace

extern "C" {

pkv_status pkv_paged_attn_decode_append_static(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
    void* v_cache, float* k_scale, float* v_scale, const int32_t* block_tables,
    int max_blocks_per_seq, const int32_t* context_lens, int num_seqs, int num_q_heads,
    int num_kv_heads, int head_dim, int block_size, int64_t num_blocks, float scale,
    int partition_size, pkv_dtype q_dtype, pkv_dtype cache_dtype, hipStream_t stream) {
    pkv_status s = check_decode(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                num_kv_heads, head_dim, block_size, num_blocks, q_dtype,
                                cache_dtype);
    if (s != PKV_OK) return s;
    if (partition_size < 0 || partition_size % pkv::kBlockSize != 0)
        return fail(PKV_ERR_SHAPE, "partition_size %d is not 0 or a positive multiple of 16",
                    partition_size);
    if (num_seqs == 0) return ok();
    if (!k_new || !v_new) return fail(PKV_ERR_NULL, "k_new and v_new are required");
    if (!aligned16(k_new) || !aligned16(v_new))
        return fail(PKV_ERR_SHAPE, "k_new and v_new must be 16-byte aligned");
    const size_t need = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  max_blocks_per_seq, partition_size, cache_dtype);
    if (need > kStaticScratchBytes)
        return fail(PKV_ERR_WORKSPACE,
                    "the partials of this call need %zu bytes, more than the %zu-byte static "
                    "scratch (fewer sequences or partitions per call, or the workspace entry "
                    "point)",
                    need, kStaticScratchBytes);
    void* ws = nullptr;
    s = scratch_on(stream, &ws);
    if (s != PKV_OK) return s;
    return decode_both_phases(out, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                              block_tables, max_blocks_per_seq, context_lens, num_seqs,
                              num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                              partition_size, ws, kStaticScratchBytes, q_dtype, cache_dtype, 0,
                              stream);
}

}  // extern "C"

// ---- read-only measurement helpers ------------------------------------------

extern "C" {

pkv_status pkv_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    if (bytes < 0) return fail(PKV_ERR_SHAPE, "bytes %lld < 0", (long long)bytes);
    if (bytes == 0) return ok();
    if (!src || !sink) return fail(PKV_ERR_NULL, "src and sink are required");
    if (!aligned16(src)) return fail(PKV_ERR_SHAPE, "src must be 16-byte aligned");
    return hip_status(pkv::launch_stream_read(src, bytes, sink, stream), "stream_read launch");
}

pkv_status pkv_tile_read(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                         const int32_t* items, int num_items, int num_kv_heads, int head_dim,
                         int64_t num_blocks, pkv_dtype cache_dtype, uint32_t* sink,
                         hipStream_t stream) {
    if (num_items < 0 || num_seqs < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0)
        return fail(PKV_ERR_SHAPE, "need num_items, num_seqs >= 0 and positive num_kv_heads, "
                                   "max_blocks_per_seq, num_blocks");
    if (!is_float(cache_dtype) && !is_quantized(cache_dtype))
        return fail(PKV_ERR_DTYPE, "unsupported cache_dtype %d", (int)cache_dtype);
    if (!head_dim_ok(head_dim) || pkv::kBlockSize * row_bytes(cache_dtype, head_dim) != 4096)
        return fail(PKV_ERR_UNSUPPORTED, "tile_read reads 4 KiB (block, kv head) tiles only");
    if (num_items == 0) return ok();
    if (!k_cache || !v_cache || !block_tables || !context_lens || !items || !sink)
        return fail(PKV_ERR_NULL, "every pointer is required");
    if (!aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(items) & 7u))
        return fail(PKV_ERR_SHAPE, "caches must be 16-byte and items 8-byte aligned");
    pkv::TileReadArgs a{};
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.items = reinterpret_cast<const int2*>(items);
    a.num_items = num_items;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.tile_bytes = 4096;
    a.num_blocks = num_blocks;
    a.sink = sink;
    return hip_status(pkv::launch_tile_read(a, stream), "tile_read launch");
}

pkv_status pkv_mfma_rate(int groups, int rounds, uint32_t* sink, hipStream_t stream) {
    if (groups <= 0 || rounds <= 0 || groups > (1 << 20))
        return fail(PKV_ERR_SHAPE, "need 0 < groups <= 2^20 and rounds > 0");
    if (!sink) return fail(PKV_ERR_NULL, "sink is required");
    return hip_status(pkv::launch_mfma_rate(groups, rounds, sink, stream), "mfma_rate launch");
}

pkv_status pkv_lds_read_rate(int pattern, int groups, int rounds, uint32_t* sink,
                             hipStream_t stream) {
    if (pattern < 0 || pattern > 3) return fail(PKV_ERR_SHAPE, "pattern %d is not 0..3", pattern);
    if (groups <= 0 || rounds <= 0 || groups > (1 << 20))
        return fail(PKV_ERR_SHAPE, "need 0 < groups <= 2^20 and rounds > 0");
    if (!sink) return fail(PKV_ERR_NULL, "sink is required");
    return hip_status(pkv::launch_lds_rate(pattern, groups, rounds, sink, stream), "lds_read_rate launch");
}

}  // extern "C"

