// Host-side interfaces between the C ABI (pkv_api.hip) and the kernel
// translation units.  Internal to libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Thread-local error reporting shared by every entry point: fail() records a
// message and returns s; ok() clears it.
pkv_status fail(pkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pkv_status ok();
const char* last_error();

constexpr int kBlockSize = 16;   // tokens per KV block

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const void* k_new;   // [B][Hkv][D] new token of each sequence (q dtype), or nullptr
    const void* v_new;
    float* m_part;       // [B][Hq][NP]
    float* l_part;       // [B][Hq][NP]
    float* o_part;       // [B][Hq][NP][D]
    int64_t num_blocks;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int max_blocks_per_seq;
    int partition_size;  // tokens, multiple of 16
    int num_partitions;  // NP: partial-array stride
    int n_tiles;         // num_q_heads / heads_per_tile
    int longest_first;   // schedule work longest-first (needs num_seqs <= kScheduleMaxSeqs
                         // and max_blocks_per_seq < 2^23, for the packed rank key)
    int window;          // > 0: attend to the last `window` positions only
    const int32_t* seq_start;  // [B] first position attended, or nullptr (0)
    // With seq_start and an output: the partials of the positions before the
    // start ([B][Hq][pre_np], natural-log m), merged into the output here
    const float* pre_m;
    const float* pre_l;
    const float* pre_o;  // [B][Hq][pre_np][D]
    int pre_np;
    int pre_partition_size;
    float scale_log2;    // softmax scale * log2(e)
};

// Sequences ranked in LDS by the work-group schedulers (one per thread; the
// work-groups that rank have at least this many threads).
constexpr int kScheduleMaxSeqs = 256;

// Balanced split of an n-token context into ceil(n / P) partitions: every
// partition but the last spans `partition_span` tokens, a multiple of the
// block size and at most P, and no partition is empty.
__host__ __device__ inline int partition_count(int n, int P) { return n <= 0 ? 0 : (n + P - 1) / P; }
__host__ __device__ inline int partition_span(int n, int count) {
    const int per = (n + count - 1) / count;
    return (per + kBlockSize - 1) / kBlockSize * kBlockSize;
}

// Sliding window of `window` positions (0: none) over an n-token context: the
// first position attended to, and the block-aligned start of the tokens that
// the partitions split (positions base..n-1; those below the first are
// masked).
__host__ __device__ inline int window_begin(int n, int window) {
    return (window > 0 && n > window) ? n - window : 0;
}
__host__ __device__ inline int window_base(int n, int window) {
    return window_begin(n, window) / kBlockSize * kBlockSize;
}
// The first position sequence b attends to: the window's, or a later start
// given per sequence (the positions before it are attended to elsewhere, as
// a shared prefix is).
__device__ inline int attend_begin(int n, int window, const int32_t* seq_start, int b) {
    int lo = window_begin(n, window);
    if (seq_start != nullptr) {
        const int s = min(max(seq_start[b], 0), n);
        lo = max(lo, s);
    }
    return lo;
}

// Phase 1 of split-context decode.  With a.out set, sequences whose context
// fits in one partition (or is empty) get their final output in a.out and
// write no partial; with a.out == nullptr every non-empty partition writes its
// partial.  Returns hipErrorInvalidValue for a combination with no kernel.
hipError_t launch_paged_decode(const DecodeArgs& a, int q_dtype, int cache_dtype, int head_dim,
                               int heads_per_tile, hipStream_t stream);

struct MultiArgs {
    void* out;                       // [T][Hq][D], written for sequences with one partition
    const void* q;                   // [T][Hq][D]
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* query_start_loc;  // [B + 1]
    float* m_part;                   // [T][Hq][NP]
    float* l_part;
    float* o_part;                   // [T][Hq][NP][D]
    int64_t num_blocks;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int max_blocks_per_seq;
    int partition_size;
    int num_partitions;
    int row_tiles;                   // row groups per (sequence, kv head): multi_row_groups()
    int max_rows;                    // max_query_len * Hq / Hkv (selects the kernel)
    int num_tokens;                  // T: rows of q / out (query rows outside are skipped)
    int causal;                      // 0: every query row attends to the whole context
    int partials_only;               // 1: (m, l, o) partials even for one partition
    // 1: b indexes groups of sequences (rows query_start_loc[b] .. are the
    // group's sequences, one query each); the group's context is the length
    // context_lens[query_start_loc[b]] and the block table of that first
    // sequence, shared by all its members
    int group_rows;
    // 1: sequence b has one query, row b of q (a decode; query_start_loc is
    // not read)
    int one_query;
    // 1: the softmax weights enter the P.V products as two 16-bit parts,
    // p = hi + lo (hi = p rounded, lo = the rest rounded), so the products
    // carry fp32-level weights instead of weights rounded to 16 bits
    int exact_p;
    // With one_query: the step's new K and V rows [B][Hkv][D] (q's 16-bit
    // dtype), or null.  Sequence b's row is position context_lens[b] - 1;
    // the work-groups that read its block take the row (quantized as the
    // cache write does, for a quantized cache) from here instead of the
    // cache, and the one of row tile 0 stores it into k_cache_w / v_cache_w
    // (the pools k_cache / v_cache, writable).
    const void* k_new;
    const void* v_new;
    void* k_cache_w;
    void* v_cache_w;
    // quantized caches (one query per sequence): INT8 / FP8, the fp32 scale
    // of every (slot, kv head), [num_blocks][Hkv][16]; 4-bit, the fp32
    // (x_min, range) pair of every (slot, kv head), [num_blocks][Hkv][16][2];
    // null otherwise
    const float* k_scale;
    const float* v_scale;
    // with k_new over a quantized cache: k_scale / v_scale, writable (the
    // new row's scale or pair is stored there)
    float* k_scale_w;
    float* v_scale_w;
    float scale_log2;
};

// Work-groups along the query rows of one (sequence, kv head): 16-row tiles
// for short query runs, 8 waves x 16 x RW rows for long ones.
int64_t multi_row_groups(int max_rows, int head_dim);

// Multi-query causal attention (fp16 / bf16 caches).  Returns
// hipErrorInvalidValue for a combination with no kernel.
// dtype: q's (the MFMA operand type); cache_dtype: the same, or a quantized
// format with scales (the short-run kernel with one query per sequence only)
hipError_t launch_paged_multi(const MultiArgs& a, int dtype, int cache_dtype, int head_dim,
                              hipStream_t stream);

struct ReduceArgs {
    void* out;
    const float* m_part;
    const float* l_part;
    const float* o_part;
    const int32_t* context_lens;
    int num_seqs;
    int num_q_heads;
    int partition_size;
    int num_partitions;
    int skip_single;     // sequences with <= 1 partition already hold their output
    int window;          // sliding window of the decode that wrote the partials (0: none)
    // multi-query partials: rows are query tokens; the sequence of token r is
    // the b with query_start_loc[b] <= r < query_start_loc[b + 1] (nullptr:
    // row r belongs to sequence r)
    const int32_t* query_start_loc;
    int num_rows;        // output rows: num_seqs, or the number of query tokens
};

hipError_t launch_paged_reduce(const ReduceArgs& a, int out_dtype, int head_dim,
                               hipStream_t stream);

struct CacheWriteArgs {
    const void* k;
    const void* v;
    void* k_cache;
    void* v_cache;
    float* k_scale;
    float* v_scale;
    const int64_t* slot_mapping;
    // used when slot_mapping is null: token b is sequence b's new token, at
    // position context_lens[b] - 1 of its block table (no store when the
    // length is 0 or the block id is out of range)
    const int32_t* block_tables;
    const int32_t* context_lens;
    int max_blocks_per_seq;
    int64_t num_tokens;
    int64_t num_blocks;
    int num_kv_heads;
};

hipError_t launch_kv_cache_write(const CacheWriteArgs& a, int src_dtype, int cache_dtype,
                                 int head_dim, hipStream_t stream);

struct CopyBlocksArgs {
    void* k_cache;
    void* v_cache;
    float* k_scale;      // nullptr unless the cache holds INT8 codes
    float* v_scale;
    const int32_t* pairs;  // [num_pairs][2] (src, dst)
    int64_t num_pairs;
    int64_t num_blocks;
    int64_t block_bytes;   // bytes of one block of one tensor (all kv heads), multiple of 16
    int64_t scale_bytes;   // bytes of one block's scale row (all kv heads), or 0
};

// Returns hipErrorInvalidValue if the grid would not fit.
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

// Read-only measurement kernels (read_ceiling.hip).
struct TileReadArgs {
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int2* items;     // (sequence, kv head) per work-group
    int num_items;
    int num_seqs;
    int num_kv_heads;
    int max_blocks_per_seq;
    int tile_bytes;        // bytes of one (block, kv head) tile: 4096
    int64_t num_blocks;
    unsigned* sink;
};
hipError_t launch_stream_read(const void* src, int64_t bytes, unsigned* sink, hipStream_t stream);
hipError_t launch_tile_read(const TileReadArgs& a, hipStream_t stream);
hipError_t launch_mfma_rate(int groups, int rounds, unsigned* sink, hipStream_t stream);
hipError_t launch_lds_rate(int pattern, int groups, int rounds, unsigned* sink, hipStream_t stream);


}  // namespace pkv
