// Host continuous-batching scheduler: each step admits, chunks and retires
// requests under a token budget and writes the ragged step's host arrays
// (cu_seqlens_q, context_lens, block_table) for kvc_paged_attention_varlen.
//
// Policy, following the continuous-batching article (news.myit.tw, section
// "Continuous batching": all active rows of a step form one ragged batch, and
// dynamic scheduling replaces a finished sequence at once; section "Chunked
// prefill": a prompt larger than the step's budget is split into chunks) and
// the PagedAttention page (clvsit.github.io, "PagedAttention 批处理": a new
// physical block only when the current one is full):
//   1. every generating sequence gets one decode row, oldest first;
//   2. sequences still inside their prompt get the next chunk of it;
//   3. waiting requests are admitted first come first served while the budget,
//      the sequence slots and the block reservation allow.
// Blocks are taken just in time through the allocator.  On admission a
// request reserves the blocks its whole life can need (prompt + max_new - 1
// cached tokens), so an admitted sequence never runs out of blocks and no
// preemption is needed; the reservation is a count, not physical blocks.
//
// A prompt's last chunk produces the first generated token; each decode row
// feeds the previous token and produces the next.  A sequence finishes when
// it has produced max_new tokens (its last token is never fed back), and its
// blocks return to the allocator in kvc_scheduler_complete.
//
// Host-only C++17; no HIP calls.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <vector>

#include "kvc.h"
#include "kvc_status.h"

namespace {

struct Seq {
    int64_t id = 0;
    int32_t prompt = 0, max_new = 0;
    int32_t cached = 0;     // tokens in the cache
    int32_t generated = 0;  // tokens produced so far
    int32_t reserved = 0;   // blocks reserved and not yet taken
    int32_t rows = 0;       // rows in the planned step
    std::vector<int32_t> row;  // block table row: held ids
};

}  // namespace

struct kvc_scheduler {
    kvc_allocator* alloc = nullptr;
    int32_t budget = 0, max_seqs = 0, max_blocks = 0, block_size = 0;
    std::deque<Seq> waiting;
    std::vector<Seq> running;      // admission order
    int64_t reserved = 0;          // sum of Seq::reserved over running
    bool pending = false;          // a planned step not yet completed
    std::vector<int32_t> planned;  // running indices of the planned rows, in row order
};

static int64_t blocks_for(const kvc_scheduler* s, int64_t tokens) {
    return (tokens + s->block_size - 1) / s->block_size;
}

extern "C" int kvc_scheduler_create(kvc_allocator* a, int32_t token_budget, int32_t max_seqs,
                                    int32_t max_blocks_per_seq, kvc_scheduler** out) {
    if (!out) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_create: out is NULL");
    *out = nullptr;
    if (!a || token_budget < 1 || max_seqs < 1 || max_blocks_per_seq < 1)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_create: bad arguments");
    kvc_scheduler* s = new (std::nothrow) kvc_scheduler;
    if (!s) return kvc_fail(KVC_ERR_OOM, "kvc_scheduler_create: host allocation failed");
    s->alloc = a;
    s->budget = token_budget;
    s->max_seqs = max_seqs;
    s->max_blocks = max_blocks_per_seq;
    s->block_size = kvc_allocator_block_size(a);
    *out = s;
    return KVC_OK;
}

extern "C" void kvc_scheduler_destroy(kvc_scheduler* s) {
    if (!s) return;
    for (Seq& q : s->running)  // blocks still held go back to the allocator
        if (!q.row.empty()) (void)kvc_free_blocks(s->alloc, q.row.data(), (int32_t)q.row.size());
    delete s;
}

extern "C" int kvc_scheduler_add(kvc_scheduler* s, int64_t request_id, int32_t prompt_len,
                                 int32_t max_new_tokens) {
    if (!s) return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_add: scheduler is NULL");
    if (prompt_len < 1 || max_new_tokens < 1)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_add: prompt_len and max_new_tokens must be >= 1");
    const int64_t need = blocks_for(s, (int64_t)prompt_len + max_new_tokens - 1);
    if (need > s->max_blocks)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_add: request longer than a table row");
    if (need > kvc_num_blocks(s->alloc))
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_add: request larger than the pool");
    try {
        Seq q;
        q.id = request_id;
        q.prompt = prompt_len;
        q.max_new = max_new_tokens;
        s->waiting.push_back(std::move(q));
    } catch (...) {
        return kvc_fail(KVC_ERR_OOM, "kvc_scheduler_add: host allocation failed");
    }
    return KVC_OK;
}

// Give sequence q `rows` more rows: grow its table row to cover the cached
// tokens plus the new ones (the reservation guarantees the blocks).
static int grow(kvc_scheduler* s, Seq& q, int32_t rows) {
    const int64_t need = blocks_for(s, (int64_t)q.cached + rows);
    int32_t held = (int32_t)q.row.size();
    if (need <= held) return KVC_OK;
    const int32_t more = (int32_t)(need - held);
    try {
        q.row.resize(need);
    } catch (...) {
        return kvc_fail(KVC_ERR_OOM, "kvc_scheduler_step: host allocation failed");
    }
    int rc = kvc_alloc_blocks(s->alloc, more, q.row.data() + held);
    if (rc != KVC_OK) {
        q.row.resize(held);
        return rc;
    }
    q.reserved -= more;
    s->reserved -= more;
    return KVC_OK;
}

extern "C" int kvc_scheduler_step(kvc_scheduler* s, int32_t* cu_seqlens_q, int32_t* context_lens,
                                  int32_t* block_table, int64_t* request_ids, int32_t* num_seqs,
                                  int32_t* total_q, int32_t* max_q_len, int32_t* max_context_len) {
    if (!s || !cu_seqlens_q || !context_lens || !block_table || !request_ids || !num_seqs ||
        !total_q || !max_q_len || !max_context_len)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_step: NULL argument");
    if (s->pending)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_step: the previous step is not completed");
    s->planned.clear();
    for (Seq& q : s->running) q.rows = 0;
    int32_t left = s->budget;
    auto plan = [&](int32_t i, int32_t rows) -> int {
        if (int rc = grow(s, s->running[i], rows)) return rc;
        s->running[i].rows = rows;
        s->planned.push_back(i);
        left -= rows;
        return KVC_OK;
    };
    const int32_t nrun = (int32_t)s->running.size();
    // 1. decode rows of generating sequences, oldest first
    for (int32_t i = 0; i < nrun && left > 0 && (int32_t)s->planned.size() < s->max_seqs; ++i)
        if (s->running[i].cached >= s->running[i].prompt)
            if (int rc = plan(i, 1)) return rc;
    // 2. next chunks of prompts in progress
    for (int32_t i = 0; i < nrun && left > 0 && (int32_t)s->planned.size() < s->max_seqs; ++i) {
        Seq& q = s->running[i];
        if (q.cached < q.prompt)
            if (int rc = plan(i, std::min(q.prompt - q.cached, left))) return rc;
    }
    // 3. admissions, first come first served (a head that does not fit blocks the queue)
    while (!s->waiting.empty() && left > 0 && (int32_t)s->planned.size() < s->max_seqs) {
        Seq& w = s->waiting.front();
        const int64_t need = blocks_for(s, (int64_t)w.prompt + w.max_new - 1);
        if (kvc_num_free_blocks(s->alloc) - s->reserved < need) break;
        try {
            s->running.push_back(std::move(w));
        } catch (...) {
            return kvc_fail(KVC_ERR_OOM, "kvc_scheduler_step: host allocation failed");
        }
        s->waiting.pop_front();
        Seq& q = s->running.back();
        q.reserved = (int32_t)need;
        s->reserved += need;
        if (int rc = plan((int32_t)s->running.size() - 1, std::min(q.prompt, left))) return rc;
    }
    // the step's arrays, rows in plan order
    const int32_t n = (int32_t)s->planned.size();
    int32_t t = 0, mq = 0, mc = 0;
    cu_seqlens_q[0] = 0;
    for (int32_t k = 0; k < n; ++k) {
        const Seq& q = s->running[s->planned[k]];
        context_lens[k] = q.cached;
        request_ids[k] = q.id;
        t += q.rows;
        cu_seqlens_q[k + 1] = t;
        mq = std::max(mq, q.rows);
        mc = std::max(mc, q.cached);
        int32_t* r = block_table + (int64_t)k * s->max_blocks;
        std::copy(q.row.begin(), q.row.end(), r);
        std::fill(r + q.row.size(), r + s->max_blocks, -1);
    }
    *num_seqs = n;
    *total_q = t;
    *max_q_len = mq;
    *max_context_len = mc;
    s->pending = n > 0;
    return KVC_OK;
}

extern "C" int kvc_scheduler_complete(kvc_scheduler* s, int64_t* finished_ids, int32_t* n_finished) {
    if (!s || !finished_ids || !n_finished)
        return kvc_fail(KVC_ERR_INVALID_ARG, "kvc_scheduler_complete: NULL argument");
    *n_finished = 0;
    if (!s->pending) return KVC_OK;
    for (int32_t i : s->planned) {
        Seq& q = s->running[i];
        const bool was_prefill = q.cached < q.prompt;
        q.cached += q.rows;
        if (!was_prefill || q.cached == q.prompt) ++q.generated;  // last chunk or decode row
        q.rows = 0;
    }
    // retire finished sequences (order of the rest is kept)
    size_t keep = 0;
    for (size_t i = 0; i < s->running.size(); ++i) {
        Seq& q = s->running[i];
        if (q.generated >= q.max_new) {
            finished_ids[(*n_finished)++] = q.id;
            (void)kvc_free_blocks(s->alloc, q.row.data(), (int32_t)q.row.size());
            s->reserved -= q.reserved;
            continue;
        }
        if (keep != i) s->running[keep] = std::move(q);
        ++keep;
    }
    s->running.resize(keep);
    s->planned.clear();
    s->pending = false;
    return KVC_OK;
}

extern "C" int32_t kvc_scheduler_num_waiting(const kvc_scheduler* s) {
    return s ? (int32_t)s->waiting.size() : -1;
}

extern "C" int32_t kvc_scheduler_num_running(const kvc_scheduler* s) {
    return s ? (int32_t)s->running.size() : -1;
}
