// Host-only driver for the block allocator, built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_allocator.py.
// Exercises every allocator entry point, including the failure paths, and
// checks the free-list/refcount invariants after each operation.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "kvc.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "CHECK failed line %d: %s\n", __LINE__, #c); \
            std::exit(1);                                                 \
        }                                                                 \
    } while (0)

static void invariants(const kvc_allocator* a) {
    int32_t nb = kvc_num_blocks(a), used = 0;
    for (int32_t i = 0; i < nb; ++i) {
        int32_t r = kvc_block_refcount(a, i);
        CHECK(r >= 0);
        used += r > 0;
    }
    CHECK(used + kvc_num_free_blocks(a) == nb);
}

int main() {
    kvc_allocator* a = nullptr;
    CHECK(kvc_allocator_create(0, 16, &a) == KVC_ERR_INVALID_ARG && a == nullptr);
    CHECK(kvc_allocator_create(100, 16, &a) == KVC_OK && a);
    invariants(a);
    std::vector<int32_t> ids(100);
    CHECK(kvc_alloc_blocks(a, 101, ids.data()) == KVC_ERR_OOM);
    CHECK(kvc_num_free_blocks(a) == 100);
    CHECK(kvc_alloc_blocks(a, 60, ids.data()) == KVC_OK);
    invariants(a);
    CHECK(kvc_alloc_blocks(a, 41, ids.data() + 60) == KVC_ERR_OOM);
    CHECK(kvc_num_free_blocks(a) == 40);
    CHECK(kvc_share_blocks(a, ids.data(), 10) == KVC_OK);
    CHECK(kvc_block_refcount(a, ids[0]) == 2);
    // double free of a shared block is fine once, not three times
    int32_t trip[3] = {ids[0], ids[0], ids[0]};
    CHECK(kvc_free_blocks(a, trip, 3) == KVC_ERR_INVALID_ARG);
    CHECK(kvc_block_refcount(a, ids[0]) == 2);
    CHECK(kvc_free_blocks(a, trip, 2) == KVC_OK);
    CHECK(kvc_block_refcount(a, ids[0]) == 0);
    invariants(a);
    CHECK(kvc_free_blocks(a, trip, 1) == KVC_ERR_INVALID_ARG);
    int32_t bad = 100;
    CHECK(kvc_free_blocks(a, &bad, 1) == KVC_ERR_INVALID_ARG);
    CHECK(kvc_share_blocks(a, &bad, 1) == KVC_ERR_INVALID_ARG);
    CHECK(kvc_block_refcount(a, -1) == -1);
    // extend a table row just in time
    std::vector<int32_t> row(8, -1);
    int32_t held = 0;
    CHECK(kvc_extend_table(a, row.data(), 8, &held, 1) == KVC_OK && held == 1);
    CHECK(kvc_extend_table(a, row.data(), 8, &held, 16) == KVC_OK && held == 1);
    CHECK(kvc_extend_table(a, row.data(), 8, &held, 17) == KVC_OK && held == 2);
    CHECK(kvc_extend_table(a, row.data(), 8, &held, 129) == KVC_ERR_INVALID_ARG && held == 2);
    {  // the batched form: two rows at once, then all or nothing on a too-short row
        std::vector<int32_t> tab(2 * 8, -1);
        int32_t hs[2] = {0, 0};
        const int64_t lens[2] = {17, 33};
        const int free0 = kvc_num_free_blocks(a);
        CHECK(kvc_extend_tables(a, tab.data(), 8, hs, lens, 2) == KVC_OK && hs[0] == 2 && hs[1] == 3);
        CHECK(kvc_num_free_blocks(a) == free0 - 5);
        const int64_t too_long[2] = {20, 8 * 16 + 1};
        CHECK(kvc_extend_tables(a, tab.data(), 8, hs, too_long, 2) == KVC_ERR_INVALID_ARG);
        CHECK(hs[0] == 2 && hs[1] == 3 && kvc_num_free_blocks(a) == free0 - 5);
        CHECK(kvc_free_blocks(a, tab.data(), 2) == KVC_OK);
        CHECK(kvc_free_blocks(a, tab.data() + 8, 3) == KVC_OK);
        CHECK(kvc_num_free_blocks(a) == free0);
        invariants(a);
    }
    // random churn
    std::mt19937 rng(1);
    std::vector<int32_t> live;
    for (int it = 0; it < 20000; ++it) {
        int op = rng() % 4;
        if (op == 0) {
            int32_t n = rng() % 5;
            std::vector<int32_t> got(n + 1);
            int free0 = kvc_num_free_blocks(a);
            int rc = kvc_alloc_blocks(a, n, got.data());
            if (n > free0) CHECK(rc == KVC_ERR_OOM && kvc_num_free_blocks(a) == free0);
            else {
                CHECK(rc == KVC_OK);
                for (int i = 0; i < n; ++i) live.push_back(got[i]);
            }
        } else if (op == 1 && !live.empty()) {
            int32_t id = live[rng() % live.size()];
            CHECK(kvc_share_blocks(a, &id, 1) == KVC_OK);
            live.push_back(id);
        } else if (op == 2 && !live.empty()) {  // copy-on-write of one held reference
            size_t k = rng() % live.size();
            int32_t nid = -1, copied = -1;
            const int32_t rc0 = kvc_block_refcount(a, live[k]);
            const int free0 = kvc_num_free_blocks(a);
            int rc = kvc_cow_block(a, live[k], &nid, &copied);
            if (rc0 == 1) {
                CHECK(rc == KVC_OK && nid == live[k] && copied == 0);
            } else if (free0 == 0) {
                CHECK(rc == KVC_ERR_OOM && kvc_block_refcount(a, live[k]) == rc0);
            } else {
                CHECK(rc == KVC_OK && copied == 1 && nid != live[k]);
                CHECK(kvc_block_refcount(a, live[k]) == rc0 - 1 && kvc_block_refcount(a, nid) == 1);
                live[k] = nid;  // the reference moved to the copy
            }
        } else if (!live.empty()) {
            size_t k = rng() % live.size();
            int32_t id = live[k];
            live[k] = live.back();
            live.pop_back();
            CHECK(kvc_free_blocks(a, &id, 1) == KVC_OK);
        }
        if (it % 1000 == 0) invariants(a);
    }
    kvc_allocator_destroy(a);
    // fork of a 40-token row (block 16): 2 shared + 1 copied block
    CHECK(kvc_allocator_create(8, 16, &a) == KVC_OK);
    std::vector<int32_t> parent(4, -1), child(4, -1);
    int32_t ph = 0, chh = 0, src = -1, dst = -1, nc = -1;
    CHECK(kvc_extend_table(a, parent.data(), 4, &ph, 40) == KVC_OK && ph == 3);
    CHECK(kvc_fork_table(a, parent.data(), 40, child.data(), 4, &chh, &src, &dst, &nc) == KVC_OK);
    CHECK(chh == 3 && nc == 1 && src == parent[2] && dst == child[2] && child[0] == parent[0]);
    CHECK(kvc_block_refcount(a, parent[0]) == 2 && kvc_block_refcount(a, parent[2]) == 1);
    CHECK(kvc_fork_table(a, parent.data(), 40, child.data(), 2, &chh, &src, &dst, &nc) == KVC_ERR_INVALID_ARG);
    CHECK(kvc_free_blocks(a, parent.data(), 3) == KVC_OK && kvc_free_blocks(a, child.data(), 3) == KVC_OK);
    CHECK(kvc_num_free_blocks(a) == 8);
    invariants(a);
    kvc_allocator_destroy(a);
    kvc_allocator_destroy(nullptr);
    CHECK(kvc_cache_bytes(1, 1, 32, 128, 2) == 16384);
    std::printf("allocator driver ok\n");
    return 0;
}
