/*
 * pkv.h -- C ABI of the paged KV-cache decode-attention library (libpkv.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are the four web pages on paged KV
 * caches; each entry point names the passage it implements):
 *
 *  - The KV cache of every sequence is cut into fixed-size blocks of
 *    `block_size` = 16 tokens that live anywhere in a pre-allocated pool; a
 *    per-sequence block table maps logical block j to a physical block id
 *    ("Efficient AI Lecture 13" notes, section "PagedAttention", its four
 *    numbered steps; docs.lazyllm.ai lesson 4, section 4.2).
 *  - Decode attention for one new query token per sequence:
 *        out[b][h] = softmax(scale * q[b][h] . K^T) V
 *    over the context_lens[b] cached tokens of the kv head that q head h
 *    reads; paging leaves the equation unchanged (lazyllm section 4.2, the
 *    "attention invariance" equation with Q of shape 1 x d).
 *  - Long contexts are split into partitions whose partial softmax results
 *    (max score, sum of exponentials, normalized weighted sum) are merged
 *    exactly; this is the running-max / running-sum rearrangement of online
 *    softmax (caojiahao2.github.io, section 3.2; juejin "LLM Engineer's
 *    Handbook", the FlashAttention-2 passage of "optimized attention").
 *  - Optional INT8 KV cache: symmetric quantization with one fp32 scale per
 *    (token slot, kv head), s = max|x| / 127, code = round(x / s)
 *    (lazyllm section 5.3; juejin absmax passage with its worked example).
 *  - Optional FP8 (e4m3) KV cache, the wider-range alternative the same
 *    section names (and the juejin page lists among serving-engine features):
 *    the same per-(slot, kv head) scale with 448, the format's largest value,
 *    in place of 127; code = e4m3 nearest to x / s.
 *  - Optional 4-bit KV cache (INT4 KV quantization, caojiahao2 section 2.3)
 *    by the linear b-bit formula of lazyllm section 3.2 with b = 4 over each
 *    (slot, kv head) row: code = round((x - x_min) / (x_max - x_min) * 15),
 *    value = x_min + code / 15 * (x_max - x_min).
 *
 * Tensor layouts (row-major, all device memory unless stated):
 *    q, out          [num_seqs][num_q_heads][head_dim]             q_dtype
 *    k_cache,v_cache [num_blocks][num_kv_heads][block_size][head_dim] cache_dtype
 *    k_scale,v_scale [num_blocks][num_kv_heads][block_size]        float (INT8 / FP8 only)
 *    block_tables    [num_seqs][max_blocks_per_seq]                int32
 *    context_lens    [num_seqs]                                    int32
 *    slot_mapping    [num_tokens]                                  int64
 *  A slot is physical_block * block_size + offset.  q head h reads kv head
 *  h / (num_q_heads / num_kv_heads).
 *
 * Conventions shared by every entry point:
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *    legacy default stream).  No entry point allocates, frees or
 *    synchronizes.  All pointers are borrowed until the enqueued work
 *    completes; the caller owns every buffer.
 *  - Argument errors that the host can see are reported before anything is
 *    enqueued: the call returns a non-zero pkv_status and pkv_last_error()
 *    describes it.  A failed kernel launch returns PKV_ERR_HIP.
 *  - Device-resident data cannot be checked on the host without a
 *    synchronization, so the kernels defend themselves instead:
 *    context_lens[b] is clamped to [0, max_blocks_per_seq * block_size],
 *    block ids outside [0, num_blocks) contribute nothing, and slots outside
 *    the pool are skipped.  Such inputs are caller errors and their results
 *    are unspecified, but no access leaves the buffers described here.
 *  - Supported: block_size 16; head_dim 64, 128 or 256; (q_dtype,
 *    cache_dtype) in {(F32,F32), (F16,F16), (BF16,BF16), (F16,I8),
 *    (BF16,I8), (F16,F8_E4M3), (BF16,F8_E4M3), (F16,U4), (BF16,U4)} (U4:
 *    head_dim 128 or 256); num_q_heads a multiple of num_kv_heads.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_ERR_NULL = 1,        /* a required pointer is NULL                      */
    PKV_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be,
                                or inconsistent with another                     */
    PKV_ERR_DTYPE = 3,       /* unsupported dtype or dtype pairing               */
    PKV_ERR_UNSUPPORTED = 4, /* head_dim / block_size outside the support set    */
    PKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required       */
    PKV_ERR_HIP = 6,         /* the HIP runtime reported an error                */
    PKV_ERR_CAPACITY = 7,    /* the block pool has too few free blocks           */
    PKV_ERR_SEQUENCE = 8     /* unknown sequence id, or one that already exists  */
} pkv_status;

/* PKV_F8_E4M3: 8-bit floating point e4m3 (OCP "E4M3FN": bias 7, 3 mantissa
 * bits, no infinities, largest finite value 448), one byte per element.
 * PKV_U4: 4-bit codes 0..15, two per byte (element 2i in the low nibble of
 * byte i): a cache row of head_dim elements takes head_dim / 2 bytes, and the
 * scale arrays hold two floats per (slot, kv head), (x_min, x_max - x_min):
 * [num_blocks][num_kv_heads][block_size][2]. */
typedef enum {
    PKV_F32 = 0,
    PKV_F16 = 1,
    PKV_BF16 = 2,
    PKV_I8 = 3,
    PKV_F8_E4M3 = 4,
    PKV_U4 = 5
} pkv_dtype;

/*
 * Slot-mapped cache append ("when a new token is generated only its keys and
 * values are computed and added to the cache": juejin "LLM Engineer's
 * Handbook", section "KV cache"), with optional INT8 quantize-on-write
 * (lazyllm lesson 4, section 5.3; juejin absmax passage).
 *
 *  k, v          [num_tokens][num_kv_heads][head_dim], src_dtype (F32|F16|BF16)
 *  k_cache/v_cache  pool (see layout above), cache_dtype == src_dtype, I8,
 *                F8_E4M3 or U4
 *  k_scale/v_scale  required iff cache_dtype is I8, F8_E4M3 or U4, else
 *                ignored (may be NULL); U4: 8-byte aligned (each row's
 *                (x_min, range) pair is stored as one 8-byte word), else
 *                PKV_ERR_SHAPE
 *  slot_mapping  token i goes to block slot/16, offset slot%16 for every kv
 *                head; slot < 0 skips the token.  Slots must be distinct.
 *
 * INT8 rows: amax = max_d |x_d|; s = amax / 127 (IEEE single division);
 * code_d = clamp(round_half_even(x_d / s), -127, 127); amax == 0 stores s = 0
 * and zero codes.  FP8 rows: s = amax / 448; code_d = the e4m3 value nearest
 * to clamp(x_d / s, -448, 448), ties to even.  U4 rows: range = max - min;
 * code_d = clamp(round_half_even((x_d - min) / range * 15), 0, 15), each
 * operation in IEEE single precision left to right; (min, range) stored;
 * range == 0 stores zero codes.  Bytes of other slots are not touched.
 */
pkv_status pkv_kv_cache_write(const void* k, const void* v, void* k_cache, void* v_cache,
                              float* k_scale, float* v_scale, const int64_t* slot_mapping,
                              int64_t num_tokens, int num_kv_heads, int head_dim, int block_size,
                              int64_t num_blocks, pkv_dtype src_dtype, pkv_dtype cache_dtype,
                              hipStream_t stream);

/*
 * Partition size (tokens, a multiple of 16) that pkv_paged_attn_decode (and
 * the other decode entry points) use when passed partition_size == 0, for a
 * cache of cache_dtype.  A power of two in [256, 8192], chosen from the sizes
 * and the tile the decode takes (one q head, several q heads of a kv head,
 * or the matrix-core path with 16-bit q of 8 to 63 q heads per kv head over
 * a cache of q's dtype, or 4 to 63 over an INT8, FP8 or 4-bit one; for the
 * quantized caches the size assumes 16-bit q).  Returns 0 for invalid arguments.
 */
int pkv_default_partition_size(int num_seqs, int num_q_heads, int num_kv_heads,
                               int max_blocks_per_seq, pkv_dtype cache_dtype);

/*
 * Bytes of workspace pkv_paged_attn_decode needs for these sizes and cache
 * dtype (partition_size 0 means the default above).  Returns 0 for invalid
 * sizes.
 * The workspace holds the fp32 partial results of sequences longer than one
 * partition; it needs no initialization and its contents after a call are
 * unspecified.  Two decode calls that may run at the same time must not share
 * a workspace.
 */
size_t pkv_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_blocks_per_seq, int partition_size,
                                 pkv_dtype cache_dtype);

/*
 * Single-query decode attention over the paged cache (lazyllm lesson 4,
 * section 4.2 equation; "Efficient AI Lecture 13", "PagedAttention" steps),
 * split over context partitions of `partition_size` tokens whose partial
 * softmax results are merged exactly (online softmax: caojiahao2 section 3.2).
 * Enqueues pkv_paged_attn_decode_partials with `out` set (sequences that fit
 * in one partition are finished there) followed by pkv_paged_attn_reduce with
 * skip_single_partition = 1, using the workspace for the partials.  With
 * 16-bit q and 8 to 63 q heads per kv head over a cache of q's dtype, or 4 to
 * 63 over an INT8, FP8 or 4-bit one, the first phase runs on the matrix cores
 * instead (the kv head's q heads as
 * matrix rows, the softmax weights entered as two 16-bit parts), to the same
 * error bound.
 *
 *  out               [num_seqs][num_q_heads][head_dim], q_dtype, written
 *  q                 [num_seqs][num_q_heads][head_dim], q_dtype
 *  k_scale, v_scale  required iff cache_dtype is I8, F8_E4M3 or U4; for U4
 *                    8-byte aligned (PKV_ERR_SHAPE otherwise)
 *  scale             the softmax scale, normally 1/sqrt(head_dim)
 *  partition_size    0 (library choice) or a positive multiple of 16
 *  workspace         >= pkv_decode_workspace_size(...) bytes, 256-byte aligned
 *
 * context_lens[b] == 0 writes zeros for sequence b.  Only block-table entries
 * j < ceil(context_lens[b] / 16) are read, and only slots of those blocks that
 * lie below context_lens[b]; everything else in the pool may hold any bytes,
 * NaN included.  (For a U4 cache the scale pairs of the other slots of those
 * blocks, and of block 0, may be loaded too; they never reach the result.)
 * Outputs are rounded to q_dtype with round-to-nearest-even.
 * The result does not depend on where blocks sit in the pool (bit for bit),
 * and repeated calls give bit-identical results.
 */
pkv_status pkv_paged_attn_decode(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int64_t num_blocks, float scale, int partition_size,
                                 void* workspace, size_t workspace_bytes, pkv_dtype q_dtype,
                                 pkv_dtype cache_dtype, hipStream_t stream);

/*
 * One decode step in one call: append each sequence's new token, then attend
 * (the cache append of juejin "LLM Engineer's Handbook", section "KV cache",
 * fused with the attention above).  For every sequence with N_b =
 * context_lens[b] >= 1, position N_b - 1 is the new token: its rows
 * k_new[b], v_new[b] ([num_seqs][num_kv_heads][head_dim], q_dtype) are
 * written into slot (block_tables[b][(N_b - 1) / 16], (N_b - 1) % 16) —
 * quantized exactly as pkv_kv_cache_write does for an INT8 / FP8 cache — and the
 * attention over positions 0..N_b-1 uses them.  Result and cache contents are
 * those of pkv_kv_cache_write with those slots followed by
 * pkv_paged_attn_decode; the attention does not wait for the stored copy.
 * Other arguments as for pkv_paged_attn_decode.
 */
pkv_status pkv_paged_attn_decode_append(void* out, const void* q, const void* k_new,
                                        const void* v_new, void* k_cache, void* v_cache,
                                        float* k_scale, float* v_scale,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens, int num_seqs,
                                        int num_q_heads, int num_kv_heads, int head_dim,
                                        int block_size, int64_t num_blocks, float scale,
                                        int partition_size, void* workspace,
                                        size_t workspace_bytes, pkv_dtype q_dtype,
                                        pkv_dtype cache_dtype, hipStream_t stream);

/*
 * pkv_paged_attn_decode_append without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * that must not call an allocator, harnesses that forbid it.  The caller
 * passes inputs and outputs only.  The split-context partials go to a static
 * device array of PKV_STATIC_SCRATCH_BYTES (32 MiB) that every GPU the library
 * runs on holds from the first call on that GPU until the process ends; its
 * address is looked up on that first call (the GPU of `stream`).  The entry
 * point calls no allocator.
 *  - A call whose partials need more than PKV_STATIC_SCRATCH_BYTES
 *    (pkv_decode_workspace_size > PKV_STATIC_SCRATCH_BYTES) returns
 *    PKV_ERR_WORKSPACE before enqueueing anything.
 *  - Every call on one GPU uses the same array and it keeps the last call's
 *    contents: calls that overlap in time on one GPU (different streams, or
 *    host threads) race and must be serialized by the caller.  Nothing needs
 *    clearing between calls.
 * Other arguments, results and errors as for pkv_paged_attn_decode_append.
 */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
pkv_status pkv_paged_attn_decode_append_static(void* out, const void* q, const void* k_new,
                                               const void* v_new, void* k_cache, void* v_cache,
                                               float* k_scale, float* v_scale,
                                               const int32_t* block_tables,
                                               int max_blocks_per_seq,
                                               const int32_t* context_lens, int num_seqs,
                                               int num_q_heads, int num_kv_heads, int head_dim,
                                               int block_size, int64_t num_blocks, float scale,
                                               int partition_size, pkv_dtype q_dtype,
                                               pkv_dtype cache_dtype, hipStream_t stream);

/*
 * Sliding-window decode: as pkv_paged_attn_decode (k_new == v_new == NULL) or
 * pkv_paged_attn_decode_append (both given), but each sequence attends only to
 * its last `sliding_window` positions, [max(0, N_b - sliding_window), N_b)
 * (caojiahao2.github.io section 2.3: keep only the most recent window of the
 * KV cache, for a fixed memory footprint).  sliding_window == 0 means no
 * window.  Only block-table entries from (N_b - sliding_window) / 16 on are
 * read, so blocks before the window may already be released (entries -1;
 * pkv_bm_release_before).  The partitions split the positions from the
 * window's first block on.  Partition default and workspace are those of
 * pkv_paged_attn_decode with max_blocks_per_seq replaced by
 * min(max_blocks_per_seq, sliding_window / 16 + 2), the most blocks a window
 * touches: workspace_bytes >= pkv_decode_workspace_size(num_seqs, num_q_heads,
 * num_kv_heads, head_dim, that value, partition_size, cache_dtype).
 */
pkv_status pkv_paged_attn_decode_sliding(void* out, const void* q, const void* k_new,
                                         const void* v_new, void* k_cache, void* v_cache,
                                         float* k_scale, float* v_scale,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* context_lens, int num_seqs,
                                         int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int64_t num_blocks, float scale,
                                         int sliding_window, int partition_size, void* workspace,
                                         size_t workspace_bytes, pkv_dtype q_dtype,
                                         pkv_dtype cache_dtype, hipStream_t stream);

/*
 * Causal attention of several query tokens per sequence: the verification
 * pass of speculative decoding, in which the target model scores k draft
 * tokens in one forward pass (caojiahao2.github.io section 6; lazyllm lesson
 * 4, the speculative-decoding algorithm), or a prefill chunk.  The queries of
 * sequence b are rows query_start_loc[b] .. query_start_loc[b+1]-1 of q
 * ([T][num_q_heads][head_dim], T = num_query_tokens = query_start_loc[B]);
 * they are its last q_len_b positions, already written into the cache, so
 * query j sits at position p = N_b - q_len_b + j (N_b = context_lens[b]) and
 *     out[row][h] = softmax(scale * q[row][h] . K[0..p]^T) V[0..p].
 * A query with p < 0 (q_len_b > N_b, a caller error) gets a zero row.
 *  query_start_loc  int32 [num_seqs + 1], device, non-decreasing
 *  max_query_len    >= every q_len_b (sizes the grid; rows beyond a
 *                   sequence's own count exit at once)
 *  partition_size   0 = pkv_multi_default_partition_size(...)
 *  workspace        >= pkv_multi_workspace_size(T, Hq, D, MBS, P) bytes,
 *                   256-byte aligned, when the context splits into more than
 *                   one partition (ceil(MBS * 16 / P) > 1); may be NULL
 *                   otherwise
 * Supported: (q_dtype, cache_dtype) in {(F16,F16), (BF16,BF16)}; head_dim 64,
 * 128, 256.  Runs on the matrix cores; the softmax weights are rounded to the
 * q dtype before they multiply V (one more rounding than
 * pkv_paged_attn_decode; relative 2^-11 for F16, 2^-8 for BF16).
 */
pkv_status pkv_paged_attn_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int num_seqs, int num_query_tokens, int max_query_len,
                                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                int64_t num_blocks, float scale, int partition_size,
                                void* workspace, size_t workspace_bytes, pkv_dtype q_dtype,
                                pkv_dtype cache_dtype, hipStream_t stream);

/* Workspace bytes for pkv_paged_attn_multi (0 for invalid sizes). */
size_t pkv_multi_workspace_size(int num_query_tokens, int num_q_heads, int head_dim,
                                int max_blocks_per_seq, int partition_size);

/* Partition size pkv_paged_attn_multi uses for partition_size == 0 (0 for
 * invalid sizes). */
int pkv_multi_default_partition_size(int num_seqs, int max_query_len, int num_q_heads,
                                     int num_kv_heads, int max_blocks_per_seq);

/*
 * Single-query decode of groups of sequences that continue one prompt (the
 * samples of parallel sampling or beam search share the prompt's blocks:
 * "Efficient AI Lecture 13" notes, section "PagedAttention", on sharing
 * between sequences of one request; docs.lazyllm.ai lesson 4, section 4.2):
 * each shared prefix block is read once for all the group's queries instead
 * of once per sequence.  The result is the decode of pkv_paged_attn_decode
 * (with the new token appended when k_new / v_new are given, as
 * pkv_paged_attn_decode_append): attention over positions
 * 0 .. context_lens[b] - 1.  It is computed as two exact pieces merged by the
 * online-softmax rule (caojiahao2.github.io section 3.2): the prefix
 * 0 .. prefix_lens[b] - 1 for all queries of a group at once on the matrix
 * cores (the group's rows of one kv head form one operand tile), and each
 * sequence's own positions prefix_lens[b] .. context_lens[b] - 1.
 *  group_start   [num_groups + 1] int32 on the device: the sequences of group
 *                g are group_start[g] .. group_start[g + 1] - 1 (consecutive;
 *                group_start[0] = 0, group_start[num_groups] = num_seqs)
 *  prefix_lens   [num_seqs] int32 on the device: the group's shared prefix
 *                length, equal for all members; the prefix is read through
 *                the block table of the group's first sequence, so the
 *                members' table entries for those positions must be the same
 *                physical blocks (as after pkv_bm_fork), and the prefix must
 *                end before the appended token (prefix_lens[b] <
 *                context_lens[b] with k_new)
 *  max_group_size >= every group's size (sizes the prefix launch)
 *  workspace     >= pkv_shared_prefix_workspace_size(...) bytes, 256-byte
 *                aligned (fp32 partials of both pieces)
 * Other arguments as pkv_paged_attn_decode_append (k_new, v_new may be NULL).
 * Supported: (q_dtype, cache_dtype) in {(F16,F16), (BF16,BF16)}; head_dim 64,
 * 128, 256.  The prefix piece rounds its softmax weights to the q dtype before
 * they multiply V (as pkv_paged_attn_multi).  A group of one sequence, or a
 * prefix of 0, is the plain decode.  Violated contracts (groups that do not
 * share the first member's prefix blocks, prefix_lens beyond the context)
 * give wrong results, not faults: every position read is bounds-checked
 * against the pool.
 */
pkv_status pkv_paged_attn_decode_shared_prefix(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* prefix_lens, const int32_t* group_start, int num_groups, int max_group_size,
    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
    int64_t num_blocks, float scale, void* workspace, size_t workspace_bytes, pkv_dtype q_dtype,
    pkv_dtype cache_dtype, hipStream_t stream);

/* Workspace bytes for pkv_paged_attn_decode_shared_prefix (0 for invalid
 * sizes). */
size_t pkv_shared_prefix_workspace_size(int num_seqs, int num_groups, int max_group_size,
                                        int num_q_heads, int num_kv_heads, int head_dim,
                                        int max_blocks_per_seq);

/*
 * Phase 1 of the split-context decode: per-partition partial results (for a
 * caller that merges them itself, e.g. partitions computed on several
 * devices, or that times the phases apart).  The N_b = context_lens[b] tokens
 * of sequence b are cut into ceil(N_b / P) partitions (P = partition_size) of
 * equal length rounded up to whole blocks, span_b = 16 * ceil(ceil(N_b /
 * count) / 16) <= P, so no partition is a short stub; partition p holds tokens
 * [p * span_b, min((p + 1) * span_b, N_b)).  For partition p and q head h:
 *    m_part[b][h][p]    = max_t s_t,  s_t = scale * (q . k_t)  (natural units)
 *    l_part[b][h][p]    = sum_t exp(s_t - m)
 *    o_part[b][h][p][:] = sum_t exp(s_t - m) v_t / l
 * Arrays are fp32 with num_partitions entries per (b, h); num_partitions must
 * be >= ceil(max_blocks_per_seq * 16 / P).  Entries of partitions
 * p >= ceil(N_b / P) are not written.  partition_size must be given (no
 * default).  Work is dispatched longest partition first when num_seqs <= 256.
 * out == NULL: every non-empty partition writes its partial.  out != NULL
 * ([num_seqs][num_q_heads][head_dim], q_dtype): sequences with
 * N_b <= partition_size get their final attention output in `out` (zeros for
 * N_b == 0) and write no partial.
 */
pkv_status pkv_paged_attn_decode_partials(void* out, float* m_part, float* l_part, float* o_part,
                                          const void* q, const void* k_cache, const void* v_cache,
                                          const float* k_scale, const float* v_scale,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* context_lens, int num_seqs,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int64_t num_blocks, float scale,
                                          int partition_size, int num_partitions,
                                          pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                          hipStream_t stream);

/*
 * Phase 2: exact merge of partials laid out as written by
 * pkv_paged_attn_decode_partials (derived from the running-max / running-sum
 * rule of online softmax, caojiahao2 section 3.2):
 *    M = max_p m_p;  w_p = l_p exp(m_p - M);  out = sum_p w_p o_p / sum_p w_p
 * over the ceil(N_b / partition_size) partitions of sequence b (the merge
 * does not depend on where the partition boundaries lie).  N_b == 0
 * writes zeros.  skip_single_partition != 0 leaves `out` of sequences with at
 * most one partition untouched (phase 1 with an output pointer finished
 * them).  out is [num_seqs][num_q_heads][head_dim] in out_dtype (F32|F16|BF16),
 * rounded to nearest even.  o_part must be 16-byte aligned (PKV_ERR_SHAPE
 * otherwise): its rows are read as 16-byte pieces.
 */
pkv_status pkv_paged_attn_reduce(void* out, const float* m_part, const float* l_part,
                                 const float* o_part, const int32_t* context_lens, int num_seqs,
                                 int num_q_heads, int head_dim, int partition_size,
                                 int num_partitions, int skip_single_partition,
                                 pkv_dtype out_dtype, hipStream_t stream);

/*
 * Host block manager: the pool of physical blocks and the block table of
 * every sequence ("Efficient AI Lecture 13" notes, section "PagedAttention":
 * blocks allocated on demand, stored anywhere, found through a block table;
 * lazyllm lesson 4, section 4.2: a per-request page table over one global
 * pool with dynamic allocation and release), with sharing of a common prefix
 * between sequences that continue one prompt (lecture 13, the advantages of
 * PagedAttention: shared prompt prefixes reuse physical blocks, for parallel
 * sampling and beam search; juejin "LLM Engineer's Handbook", section
 * "optimized attention").
 *
 * Sharing is by reference count.  pkv_bm_fork gives the child the parent's
 * blocks (every count + 1).  A block whose count is above 1 is never written:
 * when a sequence appends into a partly filled last block that it shares, the
 * manager takes a fresh block, asks the caller to copy the shared block into
 * it (a copy pair), and moves the sequence to the copy (copy-on-write).  A
 * block returns to the free list when its count reaches 0.  With this rule the
 * pool holds exactly one physical block per distinct (logical block, contents)
 * pair over the live sequences, the least any manager can use.
 *
 * The manager lives in host memory and calls no HIP function; it is not
 * thread-safe (one caller at a time per manager).  Sequence ids are any
 * int64 the caller chooses.  Every function checks its arguments and leaves
 * the manager unchanged when it returns an error.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks (>= 1) free blocks of block_size (16) tokens.  The
 * caller owns *out and releases it with pkv_bm_destroy. */
pkv_status pkv_bm_create(int64_t num_blocks, int block_size, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/* A new sequence with no tokens.  PKV_ERR_SEQUENCE if seq_id exists. */
pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id);

/* child_id starts as a copy of parent_id's table (shared blocks, no data
 * moved).  PKV_ERR_SEQUENCE if the parent is unknown or the child exists. */
pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Drop a sequence; blocks no other sequence holds become free. */
pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);

/*
 * Reserve room for num_tokens[i] new tokens at the end of sequence
 * seq_ids[i], for i in order (an id may repeat).  Host arrays:
 *  slot_mapping  [sum num_tokens] int64 or NULL: the slot of each new token,
 *                sequence by sequence, in position order (the layout
 *                pkv_kv_cache_write reads)
 *  copy_pairs    [max_copies][2] int32 (source block, destination block):
 *                copies the caller must make, before writing the new tokens,
 *                with pkv_copy_blocks; at most one per entry of seq_ids
 *  num_copies    number of pairs written
 * PKV_ERR_CAPACITY if the free blocks do not suffice, PKV_ERR_SHAPE if
 * max_copies is too small; nothing changes then.
 */
pkv_status pkv_bm_append(pkv_block_manager* bm, const int64_t* seq_ids, const int32_t* num_tokens,
                         int num_seqs, int64_t* slot_mapping, int32_t* copy_pairs,
                         int64_t max_copies, int64_t* num_copies);

/* Block tables and lengths of the listed sequences (host arrays):
 * block_tables [num_seqs][max_blocks_per_seq] int32, entries past a
 * sequence's last block set to -1; context_lens [num_seqs] int32.
 * PKV_ERR_SHAPE if a sequence has more than max_blocks_per_seq blocks or more
 * than INT32_MAX tokens. */
pkv_status pkv_bm_block_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                               int max_blocks_per_seq, int32_t* block_tables,
                               int32_t* context_lens);

/* A sequence decoded through a sliding window no longer needs its positions
 * before `position`: every whole block that ends at or before `position` (and
 * is not the sequence's last block) is released and its table entry becomes
 * -1.  Blocks other sequences still hold stay allocated. */
pkv_status pkv_bm_release_before(pkv_block_manager* bm, int64_t seq_id, int64_t position);

/* Free blocks left; -1 for a NULL manager. */
int64_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);

/* Tokens held by a sequence; -1 if unknown. */
int64_t pkv_bm_sequence_length(const pkv_block_manager* bm, int64_t seq_id);

/*
 * Copy whole blocks inside the pool, for the copy pairs of pkv_bm_append:
 * for every pair (src, dst) of copy_pairs ([num_pairs][2] int32, device
 * memory), the num_kv_heads tiles of block src in k_cache and v_cache (and
 * their scale rows when cache_dtype is I8, F8_E4M3 or U4) are copied to block dst.  Pairs
 * with an id outside [0, num_blocks) or src == dst are skipped.  A block may
 * not be the destination of one pair and the source or destination of
 * another in the same call.  Asynchronous on `stream` like the calls above.
 */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                           const int32_t* copy_pairs, int64_t num_pairs, int num_kv_heads,
                           int head_dim, int block_size, int64_t num_blocks,
                           pkv_dtype cache_dtype, hipStream_t stream);

/* Static description of a status code. */
const char* pkv_status_string(pkv_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the thread's next pkv_* call. */
const char* pkv_last_error(void);

/*
 * Read-only measurement helpers: the HBM read rate the decode's bytes can be
 * fetched at on this GPU, reported beside the decode's own rate as context.
 * Neither computes anything; a word of `sink` (device, 4 bytes) is written
 * only in the practically impossible case that the bytes read fold to a fixed
 * constant, which keeps the loads from being optimized away.
 *
 * pkv_stream_read: a plain streaming read of `bytes` bytes from `src`
 * (device, 16-byte aligned), contiguous chunks per work-group, non-temporal
 * 16-byte loads.
 *
 * pkv_tile_read: the decode's access pattern without its arithmetic: one
 * work-group per entry of `items` (device int32 [num_items][2], (sequence,
 * kv head), 8-byte aligned; entries outside [0, num_seqs) x [0, num_kv_heads)
 * are skipped), which reads the K and V (block, kv head) tiles of that
 * sequence's context_lens[b] tokens through its block table, up to the last
 * token, in the order the items are listed.  4 KiB tiles only (16 tokens x
 * head_dim x element size = 4096 bytes, e.g. fp16 at head_dim 128), else
 * PKV_ERR_UNSUPPORTED.  Other arguments as for pkv_paged_attn_decode.
 */
pkv_status pkv_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
pkv_status pkv_tile_read(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                         const int32_t* items, int num_items, int num_kv_heads, int head_dim,
                         int64_t num_blocks, pkv_dtype cache_dtype, uint32_t* sink,
                         hipStream_t stream);

/*
 * Rate measurement helpers for the matrix-core kernels, reported beside the
 * chunked-prefill kernel's rate as context.  `sink` as above; `groups`
 * work-groups (1 .. 2^20), `rounds` > 0, else PKV_ERR_SHAPE.
 *
 * pkv_mfma_rate: work-groups of 256 threads; every wave issues `rounds`
 * rounds of 8 independent v_mfma_f32_16x16x32_f16 (16,384 flops each) into
 * its own accumulators, with no memory traffic: flops = groups x 4 x rounds
 * x 8 x 16384.  The rate the matrix cores sustain at the clock the chip holds
 * under that load.
 *
 * pkv_lds_read_rate: work-groups of 512 threads over 32 KiB of LDS; every
 * wave reads 8 KiB per round with one of the chunked-prefill kernel's operand
 * reads: pattern 0 the 16-byte K operand read on the K tile layout, 1 the same
 * read on the V tile layout, 2 the V^T transpose read (ds_read_b64_tr_b16) on
 * the V layout, 3 the transpose read on the K layout; bytes = groups x 8 x
 * rounds x 8192.  Other patterns: PKV_ERR_SHAPE.
 */
pkv_status pkv_mfma_rate(int groups, int rounds, uint32_t* sink, hipStream_t stream);
pkv_status pkv_lds_read_rate(int pattern, int groups, int rounds, uint32_t* sink,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
