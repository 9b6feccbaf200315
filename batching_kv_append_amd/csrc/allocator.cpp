// Host block allocator: free list + reference counts over the physical
// blocks of one paged KV pool.
//
// The pages describe the cache as fixed-size blocks handed out on demand and
// recorded in per-sequence block tables (clvsit.github.io AWS SageMaker page,
// section "PagedAttention 批处理": a new physical block only when the current
// one is full; klklkl10086.github.io kv_cache post, section "Paged
// Attention": equal-size blocks, block tables, sharing by editing tables).
// Reference counts make sharing safe: a block listed in several tables (a
// common prefix, written once) stays allocated until the last table drops it.
//
// Host-only C++17; no HIP calls.  The free list is a stack, so ids freed last
// are reused first (good for cache locality of recently-touched blocks).
#include <cstdint>
#include <new>
#include <vector>

#include "kvc.h"
#include "kvc_status.h"

struct kvc_allocator {
    int32_t block_size = 0;
    std::vector<int32_t> free_stack;  // ids of free blocks; top = back()
    std::vector<int32_t> refcount;    // per block; 0 = free
};

extern "C" int kvc_allocator_create(int32_t num_blocks, int32_t block_size, kvc_allocator** out) {
    if (!out) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_allocator_create: out is NULL");
    *out = nullptr;
    if (num_blocks < 1 || block_size < 1)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_allocator_create: num_blocks and block_size must be >= 1");
    kvc_allocator* a = new (std::nothrow) kvc_allocator;
    if (!a) return kvc_fail(KVC_ERR_OOM, "kvc_allocator_create: host allocation failed");
    try {
        a->block_size = block_size;
        a->refcount.assign(num_blocks, 0);
        a->free_stack.resize(num_blocks);
        // block 0 on top: a fresh allocator hands out 0, 1, 2, ...
        for (int32_t i = 0; i < num_blocks; ++i) a->free_stack[i] = num_blocks - 1 - i;
    } catch (...) {
        delete a;
        return kvc_fail(KVC_ERR_OOM, "kvc_allocator_create: host allocation failed");
    }
    *out = a;
    return KVC_OK;
}

extern "C" void kvc_allocator_destroy(kvc_allocator* a) { delete a; }

extern "C" int kvc_alloc_blocks(kvc_allocator* a, int32_t n, int32_t* out_ids) {
    if (!a) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_alloc_blocks: allocator is NULL");
    if (n < 0) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_alloc_blocks: n < 0");
    if (n == 0) return KVC_OK;
    if (!out_ids) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_alloc_blocks: out_ids is NULL");
    if ((size_t)n > a->free_stack.size())
        return kvc_fail(KVC_ERR_OOM, "kvc_alloc_blocks: not enough free blocks");
    for (int32_t i = 0; i < n; ++i) {
        int32_t id = a->free_stack.back();
        a->free_stack.pop_back();
        a->refcount[id] = 1;
        out_ids[i] = id;
    }
    return KVC_OK;
}

static bool valid_id(const kvc_allocator* a, int32_t id) {
    return id >= 0 && (size_t)id < a->refcount.size();
}

extern "C" int kvc_share_blocks(kvc_allocator* a, const int32_t* ids, int32_t n) {
    if (!a) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_share_blocks: allocator is NULL");
    if (n < 0 || (n > 0 && !ids)) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_share_blocks: bad id list");
    for (int32_t i = 0; i < n; ++i)
        if (!valid_id(a, ids[i]) || a->refcount[ids[i]] <= 0)
            return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_share_blocks: id out of range or not allocated");
    for (int32_t i = 0; i < n; ++i) {
        if (a->refcount[ids[i]] == INT32_MAX) {
            for (int32_t j = 0; j < i; ++j) --a->refcount[ids[j]];  // undo
            return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_share_blocks: reference count overflow");
        }
        ++a->refcount[ids[i]];
    }
    return KVC_OK;
}

extern "C" int kvc_free_blocks(kvc_allocator* a, const int32_t* ids, int32_t n) {
    if (!a) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_free_blocks: allocator is NULL");
    if (n < 0 || (n > 0 && !ids)) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_free_blocks: bad id list");
    // Validate the whole list first (an id may appear several times).
    for (int32_t i = 0; i < n; ++i) {
        if (!valid_id(a, ids[i]) || a->refcount[ids[i]] <= 0)
            return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_free_blocks: id out of range or already free");
    }
    for (int32_t i = 0; i < n; ++i) --a->refcount[ids[i]];
    bool underflow = false;
    for (int32_t i = 0; i < n; ++i) underflow |= a->refcount[ids[i]] < 0;
    if (underflow) {
        for (int32_t i = 0; i < n; ++i) ++a->refcount[ids[i]];  // undo
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_free_blocks: id listed more often than it is referenced");
    }
    try {
        a->free_stack.reserve(a->refcount.size());
    } catch (...) {
        for (int32_t i = 0; i < n; ++i) ++a->refcount[ids[i]];
        return kvc_fail(KVC_ERR_OOM, "kvc_free_blocks: host allocation failed");
    }
    // Push each block whose count reached 0 exactly once (an id may be listed
    // several times): mark pushed blocks with -1, then restore them to 0.
    for (int32_t i = 0; i < n; ++i) {
        if (a->refcount[ids[i]] == 0) {
            a->free_stack.push_back(ids[i]);
            a->refcount[ids[i]] = -1;
        }
    }
    for (int32_t i = 0; i < n; ++i)
        if (a->refcount[ids[i]] == -1) a->refcount[ids[i]] = 0;
    return KVC_OK;
}

extern "C" int32_t kvc_num_free_blocks(const kvc_allocator* a) {
    return a ? (int32_t)a->free_stack.size() : -1;
}

extern "C" int32_t kvc_num_blocks(const kvc_allocator* a) {
    return a ? (int32_t)a->refcount.size() : -1;
}

extern "C" int32_t kvc_allocator_block_size(const kvc_allocator* a) {
    return a ? a->block_size : -1;
}

extern "C" int32_t kvc_block_refcount(const kvc_allocator* a, int32_t id) {
    if (!a || !valid_id(a, id)) return -1;
    return a->refcount[id];
}

extern "C" int kvc_extend_table(kvc_allocator* a, int32_t* row, int32_t max_blocks,
                                int32_t* held, int64_t new_len) {
    if (!a || !row || !held) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_extend_table: NULL argument");
    if (max_blocks < 0 || *held < 0 || *held > max_blocks || new_len < 0)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_extend_table: bad sizes");
    const int64_t need = (new_len + a->block_size - 1) / a->block_size;
    if (need > max_blocks)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_extend_table: row too short for new_len");
    if (need <= *held) return KVC_OK;
    const int32_t more = (int32_t)(need - *held);
    int rc = kvc_alloc_blocks(a, more, row + *held);
    if (rc != KVC_OK) return rc;
    *held += more;
    return KVC_OK;
}

// Just-in-time growth of a whole step's rows in one call (the same rule per
// row as kvc_extend_table), all or nothing: every row is checked and the
// blocks counted before any is taken.
extern "C" int kvc_extend_tables(kvc_allocator* a, int32_t* table, int32_t max_blocks,
                                 int32_t* held, const int64_t* new_lens, int32_t num_seqs) {
    if (!a) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_extend_tables: allocator is NULL");
    if (num_seqs < 0 || max_blocks < 0)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_extend_tables: bad sizes");
    if (num_seqs > 0 && (!table || !held || !new_lens))
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_extend_tables: NULL argument");
    int64_t total = 0;
    for (int32_t s = 0; s < num_seqs; ++s) {
        if (held[s] < 0 || held[s] > max_blocks || new_lens[s] < 0)
            return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_extend_tables: bad sizes");
        const int64_t need = (new_lens[s] + a->block_size - 1) / a->block_size;
        if (need > max_blocks)
            return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_extend_tables: row too short for new_len");
        if (need > held[s]) total += need - held[s];
    }
    if (total > (int64_t)a->free_stack.size())
        return kvc_fail(KVC_ERR_OOM, "kvc_extend_tables: not enough free blocks");
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t need = (new_lens[s] + a->block_size - 1) / a->block_size;
        int32_t* row = table + (int64_t)s * max_blocks;
        for (int64_t i = held[s]; i < need; ++i) {
            const int32_t id = a->free_stack.back();
            a->free_stack.pop_back();
            a->refcount[id] = 1;
            row[i] = id;
        }
        if (need > held[s]) held[s] = (int32_t)need;
    }
    return KVC_OK;
}

// Copy-on-write.  Sharing is done by editing tables (klklkl10086.github.io
// kv_cache post, section "Paged Attention"), and a contiguous cache cannot
// share at all (same post, section "连续内存分配", beam search).  A shared block
// that one sharer is about to write into is first copied, so the others keep
// their contents: the writer takes a fresh block, drops its reference to the
// shared one, and copies the contents on the device (kvc_copy_blocks).
extern "C" int kvc_cow_block(kvc_allocator* a, int32_t id, int32_t* out_id, int32_t* copied) {
    if (!a || !out_id || !copied) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_cow_block: NULL argument");
    if (!valid_id(a, id) || a->refcount[id] <= 0)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_cow_block: id out of range or free");
    if (a->refcount[id] == 1) {  // sole owner: write in place
        *out_id = id;
        *copied = 0;
        return KVC_OK;
    }
    if (a->free_stack.empty()) return kvc_fail(KVC_ERR_OOM, "kvc_cow_block: no free block");
    const int32_t nid = a->free_stack.back();
    a->free_stack.pop_back();
    a->refcount[nid] = 1;
    --a->refcount[id];  // > 0: other sharers remain
    *out_id = nid;
    *copied = 1;
    return KVC_OK;
}

extern "C" int kvc_fork_table(kvc_allocator* a, const int32_t* parent_row, int64_t len,
                              int32_t* child_row, int32_t max_blocks, int32_t* child_held,
                              int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies) {
    if (!a || !parent_row || !child_row || !child_held || !copy_src || !copy_dst || !n_copies)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_fork_table: NULL argument");
    if (len < 0 || max_blocks < 0) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_fork_table: bad sizes");
    const int64_t nb = (len + a->block_size - 1) / a->block_size;
    if (nb > max_blocks) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_fork_table: row too short for len");
    const bool partial = len % a->block_size != 0;
    const int32_t full = (int32_t)(partial ? nb - 1 : nb);
    for (int32_t i = 0; i < nb; ++i)
        if (!valid_id(a, parent_row[i]) || a->refcount[parent_row[i]] <= 0)
            return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_fork_table: parent id out of range or free");
    if (partial && a->free_stack.empty()) return kvc_fail(KVC_ERR_OOM, "kvc_fork_table: no free block");
    int rc = kvc_share_blocks(a, parent_row, full);  // all or nothing by itself
    if (rc != KVC_OK) return rc;
    for (int32_t i = 0; i < full; ++i) child_row[i] = parent_row[i];
    *n_copies = 0;
    if (partial) {  // the child will write into the last block: its own copy
        int32_t nid = 0;
        rc = kvc_alloc_blocks(a, 1, &nid);  // cannot fail: checked above
        if (rc != KVC_OK) {
            for (int32_t i = 0; i < full; ++i) --a->refcount[parent_row[i]];
            return rc;
        }
        child_row[full] = nid;
        copy_src[0] = parent_row[full];
        copy_dst[0] = nid;
        *n_copies = 1;
    }
    *child_held = (int32_t)nb;
    return KVC_OK;
}

extern "C" int64_t kvc_cache_bytes(int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t elem_bytes) {
    if (num_blocks < 0 || block_size < 0 || num_kv_heads < 0 || head_dim < 0 || elem_bytes < 0)
        return -1;
    return 2 * num_blocks * block_size * (int64_t)num_kv_heads * head_dim * elem_bytes;
}
