// Randomised stress of the host block pool (include/pa_pool.h), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
// After every operation the pool's accounting is checked against the tables
// it exports: free + used blocks = pool size, each block's count = the number
// of live tables holding it, each table ceil(length / B) blocks, and every
// slot a call hands out lies in the sequence's own last block.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pa_pool.h"

static uint64_t state = 88172645463325252ull;
static uint32_t rnd(uint32_t n) {   // xorshift64
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)(state % n);
}

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            std::exit(1);                                               \
        }                                                               \
    } while (0)

int main() {
    const int NB = 257, B = 4, MAXB = 64;
    std::vector<int32_t> order(NB);
    for (int i = 0; i < NB; ++i) order[i] = (i * 37) % NB;   // a permutation (37 coprime to 257)
    pa_pool *pool = nullptr;
    CHECK(pa_pool_create(NB, B, order.data(), &pool) == PA_OK);
    CHECK(pa_pool_create(0, B, nullptr, &pool) != PA_OK);
    std::vector<int> live;
    std::vector<int32_t> slots(64), pairs(2 * 64), tables, lens;
    for (int step = 0; step < 20000; ++step) {
        const uint32_t op = rnd(100);
        if (op < 10 || live.empty()) {
            int s = -1;
            CHECK(pa_seq_create(pool, &s) == PA_OK && s >= 0);
            live.push_back(s);
        } else if (op < 20) {
            int c = -1;
            const int p = live[rnd((uint32_t)live.size())];
            CHECK(pa_seq_fork(pool, p, &c) == PA_OK);
            live.push_back(c);
        } else if (op < 55) {
            const int s = live[rnd((uint32_t)live.size())];
            const int n = (int)rnd(9);
            const int before = pa_seq_length(pool, s);
            int32_t src = 0, dst = 0;
            const pa_status st = pa_seq_append(pool, s, n, slots.data(), &src, &dst);
            if (st == PA_OK) {
                CHECK(pa_seq_length(pool, s) == before + n);
                if (src >= 0) CHECK(dst >= 0 && src != dst && pa_pool_refcount(pool, dst) == 1);
            } else {
                CHECK(st == PA_ERR_NO_BLOCKS && pa_seq_length(pool, s) == before);
            }
        } else if (op < 75) {
            // a batch of distinct live sequences, one token each
            std::vector<int> batch;
            for (int s : live)
                if (rnd(3) == 0 && (int)batch.size() < 64) batch.push_back(s);
            int np = -1;
            const pa_status st = pa_seq_append_batch(pool, batch.data(), (int)batch.size(),
                                                     slots.data(), pairs.data(), &np);
            CHECK(st == PA_OK || st == PA_ERR_NO_BLOCKS);
            if (st == PA_OK) CHECK(np >= 0 && np <= (int)batch.size());
            if (batch.size() >= 2) {   // a repeated id is refused, nothing changes
                std::vector<int> dup = {batch[0], batch[0]};
                const int freeb = pa_pool_num_free(pool);
                CHECK(pa_seq_append_batch(pool, dup.data(), 2, slots.data(), pairs.data(), &np) ==
                      PA_ERR_BAD_ID);
                CHECK(pa_pool_num_free(pool) == freeb);
            }
        } else if (op < 95) {
            const uint32_t k = rnd((uint32_t)live.size());
            CHECK(pa_seq_release(pool, live[k]) == PA_OK);
            CHECK(pa_seq_release(pool, live[k]) == PA_ERR_BAD_ID);
            live.erase(live.begin() + k);
        } else {
            CHECK(pa_seq_append(pool, 1 << 30, 1, slots.data(), nullptr, nullptr) != PA_OK);
            CHECK(pa_pool_refcount(pool, NB) == -1 && pa_pool_refcount(pool, -1) == -1);
        }
        // accounting
        const int n = (int)live.size();
        tables.assign((size_t)n * MAXB + 1, 0);
        lens.assign((size_t)n + 1, 0);
        const pa_status st = pa_pool_export(pool, live.data(), n, MAXB, -7, tables.data(), lens.data());
        if (st == PA_ERR_SHAPE) {   // a table outgrew the export width: drop the longest
            int longest = 0;
            for (int i = 1; i < n; ++i)
                if (pa_seq_length(pool, live[i]) > pa_seq_length(pool, live[longest])) longest = i;
            CHECK(pa_seq_release(pool, live[longest]) == PA_OK);
            live.erase(live.begin() + longest);
            continue;
        }
        CHECK(st == PA_OK);
        std::vector<int> count(NB, 0);
        for (int i = 0; i < n; ++i) {
            const int L = lens[i], nb = (L + B - 1) / B;
            CHECK(pa_seq_num_blocks(pool, live[i]) == nb);
            for (int j = 0; j < MAXB; ++j) {
                const int32_t b = tables[(size_t)i * MAXB + j];
                if (j < nb) {
                    CHECK(b >= 0 && b < NB);
                    ++count[b];
                } else {
                    CHECK(b == -7);
                }
            }
        }
        int used = 0;
        for (int b = 0; b < NB; ++b) {
            CHECK(pa_pool_refcount(pool, b) == count[b]);
            used += count[b] > 0;
        }
        CHECK(used + pa_pool_num_free(pool) == NB);
    }
    for (int s : live) CHECK(pa_seq_release(pool, s) == PA_OK);
    CHECK(pa_pool_num_free(pool) == NB);
    pa_pool_destroy(pool);
    std::printf("pool stress ok\n");
    return 0;
}
