// Host block manager: free-list pool of physical blocks, per-sequence block
// tables, prefix sharing by reference count with copy-on-write of a shared,
// partly filled last block.  Pure host code (no HIP calls).
//
// Paging as the "Efficient AI Lecture 13" notes describe it (section
// "PagedAttention": blocks allocated on demand, stored anywhere, reached
// through a block table) and the lazyllm lesson 4, section 4.2 (one page
// table per request over a global pool with dynamic allocation and release);
// sharing of the blocks of a common prompt between its continuations
// (lecture 13, the advantages listed for PagedAttention).
//
// Data layout: one flat refcount array and a LIFO free stack over the pool
// (O(1) take and release, no per-block allocation), and per sequence a vector
// of block ids plus its token count.  An append first plans the whole batch
// (blocks and copies it needs, with the reference counts it would leave), so
// a batch that does not fit changes nothing.
#include <limits.h>
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

struct pkv_block_manager {
    struct Seq {
        std::vector<int32_t> blocks;
        int64_t len = 0;
    };
    int64_t num_blocks = 0;
    int block_size = 16;
    std::vector<int32_t> refs;       // reference count per physical block
    std::vector<int32_t> free_ids;   // stack of free blocks; back() is taken next
    std::unordered_map<int64_t, Seq> seqs;

    int32_t take() {
        const int32_t b = free_ids.back();
        free_ids.pop_back();
        refs[b] = 1;
        return b;
    }
    void release(int32_t b) {
        if (--refs[b] == 0) free_ids.push_back(b);
    }
    int64_t blocks_for(int64_t len) const { return (len + block_size - 1) / block_size; }
};

using pkv::fail;
using pkv::ok;

extern "C" {

pkv_status pkv_bm_create(int64_t num_blocks, int block_size, pkv_block_manager** out) {
    if (!out) return fail(PKV_ERR_NULL, "out is NULL");
    *out = nullptr;
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (only 16)", block_size);
    if (num_blocks <= 0 || num_blocks > INT32_MAX)
        return fail(PKV_ERR_SHAPE, "num_blocks must be in [1, 2^31 - 1] (got %lld)",
                    (long long)num_blocks);
    pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
    if (!bm) return fail(PKV_ERR_CAPACITY, "host allocation failed");
    try {
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->refs.assign((size_t)num_blocks, 0);
        bm->free_ids.resize((size_t)num_blocks);
        // lowest ids are taken first
        for (int64_t i = 0; i < num_blocks; ++i)
            bm->free_ids[(size_t)i] = (int32_t)(num_blocks - 1 - i);
    } catch (const std::bad_alloc&) {
        delete bm;
        return fail(PKV_ERR_CAPACITY, "host allocation failed");
    }
    *out = bm;
    return ok();
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return fail(PKV_ERR_NULL, "manager is NULL");
    if (bm->seqs.count(seq_id))
        return fail(PKV_ERR_SEQUENCE, "sequence %lld exists", (long long)seq_id);
    bm->seqs.emplace(seq_id, pkv_block_manager::Seq{});
    return ok();
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id) {
    if (!bm) return fail(PKV_ERR_NULL, "manager is NULL");
    auto p = bm->seqs.find(parent_id);
    if (p == bm->seqs.end())
        return fail(PKV_ERR_SEQUENCE, "parent sequence %lld unknown", (long long)parent_id);
    if (bm->seqs.count(child_id))
        return fail(PKV_ERR_SEQUENCE, "sequence %lld exists", (long long)child_id);
    pkv_block_manager::Seq child = p->second;   // copy before emplace may rehash
    for (int32_t b : child.blocks)
        if (b >= 0) ++bm->refs[b];
    bm->seqs.emplace(child_id, std::move(child));
    return ok();
}

pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return fail(PKV_ERR_NULL, "manager is NULL");
    auto s = bm->seqs.find(seq_id);
    if (s == bm->seqs.end())
        return fail(PKV_ERR_SEQUENCE, "sequence %lld unknown", (long long)seq_id);
    for (int32_t b : s->second.blocks)
        if (b >= 0) bm->release(b);
    bm->seqs.erase(s);
    return ok();
}

pkv_status pkv_bm_append(pkv_block_manager* bm, const int64_t* seq_ids, const int32_t* num_tokens,
                         int num_seqs, int64_t* slot_mapping, int32_t* copy_pairs,
                         int64_t max_copies, int64_t* num_copies) {
    if (!bm || !num_copies) return fail(PKV_ERR_NULL, "manager and num_copies are required");
    if (num_seqs < 0) return fail(PKV_ERR_SHAPE, "num_seqs < 0");
    *num_copies = 0;
    if (num_seqs == 0) return ok();
    if (!seq_ids || !num_tokens) return fail(PKV_ERR_NULL, "seq_ids and num_tokens are required");
    if (max_copies > 0 && !copy_pairs)
        return fail(PKV_ERR_NULL, "copy_pairs is NULL with max_copies > 0");

    // Plan: count the blocks and copies the batch needs, in order, with the
    // reference-count changes earlier entries make.  Once a sequence has
    // received tokens in this batch its last block is its own.
    using Seq = pkv_block_manager::Seq;
    std::unordered_map<int64_t, int64_t> planned_len;   // sequences touched so far
    std::unordered_map<int32_t, int32_t> ref_drop;      // shared blocks left by a copy
    int64_t need_blocks = 0, need_copies = 0;
    for (int i = 0; i < num_seqs; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end())
            return fail(PKV_ERR_SEQUENCE, "sequence %lld unknown", (long long)seq_ids[i]);
        const int32_t n = num_tokens[i];
        if (n < 0) return fail(PKV_ERR_SHAPE, "num_tokens[%d] = %d < 0", i, n);
        if (n == 0) continue;
        const Seq& s = it->second;
        auto pl = planned_len.find(seq_ids[i]);
        const bool touched = pl != planned_len.end();
        const int64_t len = touched ? pl->second : s.len;
        if (!touched && len % bm->block_size != 0) {
            const int32_t last = s.blocks.back();
            auto d = ref_drop.find(last);
            const int32_t refs = bm->refs[last] - (d == ref_drop.end() ? 0 : d->second);
            if (refs > 1) {
                ++need_blocks;
                ++need_copies;
                ++ref_drop[last];
            }
        }
        need_blocks += bm->blocks_for(len + n) - bm->blocks_for(len);
        planned_len[seq_ids[i]] = len + n;
    }
    if (need_blocks > (int64_t)bm->free_ids.size())
        return fail(PKV_ERR_CAPACITY, "batch needs %lld blocks, %lld free", (long long)need_blocks,
                    (long long)bm->free_ids.size());
    if (need_copies > max_copies)
        return fail(PKV_ERR_SHAPE, "batch needs %lld copy pairs, room for %lld",
                    (long long)need_copies, (long long)max_copies);
    for (auto& kv : planned_len)
        if (bm->blocks_for(kv.second) > INT32_MAX)
            return fail(PKV_ERR_SHAPE, "sequence %lld would exceed 2^31 blocks",
                        (long long)kv.first);

    // Apply (cannot fail any more).
    int64_t slot_pos = 0, copies = 0;
    for (int i = 0; i < num_seqs; ++i) {
        const int32_t n = num_tokens[i];
        if (n == 0) continue;
        Seq& s = bm->seqs[seq_ids[i]];
        if (s.len % bm->block_size != 0) {
            int32_t& last = s.blocks.back();
            if (bm->refs[last] > 1) {
                const int32_t dst = bm->take();
                copy_pairs[2 * copies] = last;
                copy_pairs[2 * copies + 1] = dst;
                ++copies;
                --bm->refs[last];
                last = dst;
            }
        }
        const int64_t end = s.len + n;
        while ((int64_t)s.blocks.size() < bm->blocks_for(end)) s.blocks.push_back(bm->take());
        if (slot_mapping)
            for (int64_t t = s.len; t < end; ++t)
                slot_mapping[slot_pos++] =
                    (int64_t)s.blocks[(size_t)(t / bm->block_size)] * bm->block_size +
                    t % bm->block_size;
        s.len = end;
    }
    *num_copies = copies;
    return ok();
}

pkv_status pkv_bm_block_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                               int max_blocks_per_seq, int32_t* block_tables,
                               int32_t* context_lens) {
    if (!bm) return fail(PKV_ERR_NULL, "manager is NULL");
    if (num_seqs < 0 || max_blocks_per_seq <= 0)
        return fail(PKV_ERR_SHAPE, "need num_seqs >= 0 and max_blocks_per_seq > 0");
    if (num_seqs == 0) return ok();
    if (!seq_ids || !block_tables || !context_lens)
        return fail(PKV_ERR_NULL, "seq_ids, block_tables and context_lens are required");
    for (int i = 0; i < num_seqs; ++i) {
        auto it = bm->seqs.find(seq_ids[i]);
        if (it == bm->seqs.end())
            return fail(PKV_ERR_SEQUENCE, "sequence %lld unknown", (long long)seq_ids[i]);
        if ((int64_t)it->second.blocks.size() > max_blocks_per_seq || it->second.len > INT32_MAX)
            return fail(PKV_ERR_SHAPE, "sequence %lld has %zu blocks, table width %d",
                        (long long)seq_ids[i], it->second.blocks.size(), max_blocks_per_seq);
    }
    for (int i = 0; i < num_seqs; ++i) {
        const auto& s = bm->seqs.find(seq_ids[i])->second;
        int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
        const int nb = (int)s.blocks.size();
        for (int j = 0; j < nb; ++j) row[j] = s.blocks[(size_t)j];
        for (int j = nb; j < max_blocks_per_seq; ++j) row[j] = -1;
        context_lens[i] = (int32_t)s.len;
    }
    return ok();
}

pkv_status pkv_bm_release_before(pkv_block_manager* bm, int64_t seq_id, int64_t position) {
    if (!bm) return fail(PKV_ERR_NULL, "manager is NULL");
    auto it = bm->seqs.find(seq_id);
    if (it == bm->seqs.end())
        return fail(PKV_ERR_SEQUENCE, "sequence %lld unknown", (long long)seq_id);
    auto& s = it->second;
    const int64_t full = s.len / bm->block_size;   // whole blocks; the last partial one stays
    int64_t drop = position > 0 ? position / bm->block_size : 0;
    if (drop > full) drop = full;
    for (int64_t j = 0; j < drop; ++j) {
        int32_t& b = s.blocks[(size_t)j];
        if (b >= 0) {
            bm->release(b);
            b = -1;
        }
    }
    return ok();
}

int64_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) {
    return bm ? (int64_t)bm->free_ids.size() : -1;
}

int64_t pkv_bm_sequence_length(const pkv_block_manager* bm, int64_t seq_id) {
    if (!bm) return -1;
    auto it = bm->seqs.find(seq_id);
    return it == bm->seqs.end() ? -1 : it->second.len;
}

}  // extern "C"
