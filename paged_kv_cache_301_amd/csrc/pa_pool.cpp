// pa_pool.cpp -- host block pool: free stack, reference counts, block tables,
// copy-on-write (page "PagedAttention by hand", sections "Why divide memory
// into physical blocks?" and "Memory Sharing (Copy-on-Write)").
//
// Plain host C++.  Every public call validates, then checks that the free
// stack can supply everything the call needs, and only then mutates, so a
// failed call leaves the pool unchanged.
#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_pool.h"

struct pa_pool {
    int NB = 0;
    int B = 0;
    std::vector<int32_t> free_stack;     // back() is handed out next
    std::vector<int32_t> refcount;       // per physical block
    struct Seq {
        bool live = false;
        int64_t len = 0;
        std::vector<int32_t> table;
    };
    std::vector<Seq> seqs;               // index = sequence id
    mutable std::mutex mu;

    bool live(int s) const { return s >= 0 && s < (int)seqs.size() && seqs[s].live; }

    // Fresh blocks taken by appending n tokens to sequence s (copy included).
    int64_t blocks_needed(int s, int64_t n) const {
        if (n == 0) return 0;
        const Seq &q = seqs[s];
        const int64_t room = (int64_t)q.table.size() * B - q.len;   // free slots in the last block
        const int64_t rest = n - room;
        const int64_t fresh = rest > 0 ? (rest + B - 1) / B : 0;
        const bool cow = room > 0 && refcount[q.table.back()] > 1;
        return fresh + (cow ? 1 : 0);
    }

    int32_t take() {
        const int32_t b = free_stack.back();
        free_stack.pop_back();
        refcount[b] = 1;
        return b;
    }

    // Append one token; the caller has checked that blocks are available.
    int32_t append_one(int s, int32_t *cow_src, int32_t *cow_dst) {
        Seq &q = seqs[s];
        const int64_t pos = q.len;
        const int64_t j = pos / B, off = pos % B;
        if (j == (int64_t)q.table.size()) {
            q.table.push_back(take());                 // last block full: on demand
        } else if (refcount[q.table[j]] > 1) {
            const int32_t shared = q.table[j];         // shared: copy on write
            const int32_t fresh = take();
            refcount[shared] -= 1;
            q.table[j] = fresh;
            *cow_src = shared;
            *cow_dst = fresh;
        }
        q.len = pos + 1;
        return (int32_t)((int64_t)q.table[j] * B + off);
    }
};

extern "C" {

pa_status pa_pool_create(int num_blocks, int block_size, const int32_t *free_order,
                         pa_pool **out) {
    if (!out) return PA_ERR_NULL;
    if (num_blocks <= 0 || block_size <= 0) return PA_ERR_SHAPE;
    if ((int64_t)num_blocks * block_size > INT32_MAX) return PA_ERR_SHAPE;   // slots are int32
    std::vector<int32_t> order(num_blocks);
    if (free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int i = 0; i < num_blocks; ++i) {
            const int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) return PA_ERR_SHAPE;
            seen[b] = 1;
            order[i] = b;
        }
    } else {
        for (int i = 0; i < num_blocks; ++i) order[i] = i;
    }
    pa_pool *p = new (std::nothrow) pa_pool;
    if (!p) return PA_ERR_NO_BLOCKS;
    p->NB = num_blocks;
    p->B = block_size;
    p->free_stack.assign(order.rbegin(), order.rend());
    p->refcount.assign(num_blocks, 0);
    *out = p;
    return PA_OK;
}

void pa_pool_destroy(pa_pool *pool) { delete pool; }

int pa_pool_num_free(const pa_pool *pool) {
    if (!pool) return -1;
    std::lock_guard<std::mutex> g(pool->mu);
    return (int)pool->free_stack.size();
}

int pa_pool_refcount(const pa_pool *pool, int block) {
    if (!pool || block < 0 || block >= pool->NB) return -1;
    std::lock_guard<std::mutex> g(pool->mu);
    return pool->refcount[block];
}

pa_status pa_seq_create(pa_pool *pool, int *seq) {
    if (!pool || !seq) return PA_ERR_NULL;
    std::lock_guard<std::mutex> g(pool->mu);
    if (pool->seqs.size() >= (size_t)INT32_MAX) return PA_ERR_SHAPE;
    pool->seqs.emplace_back();
    pool->seqs.back().live = true;
    *seq = (int)pool->seqs.size() - 1;
    return PA_OK;
}

pa_status pa_seq_fork(pa_pool *pool, int parent, int *child) {
    if (!pool || !child) return PA_ERR_NULL;
    std::lock_guard<std::mutex> g(pool->mu);
    if (!pool->live(parent)) return PA_ERR_BAD_ID;
    if (pool->seqs.size() >= (size_t)INT32_MAX) return PA_ERR_SHAPE;
    pa_pool::Seq c;
    c.live = true;
    c.len = pool->seqs[parent].len;
    c.table = pool->seqs[parent].table;
    for (int32_t b : c.table) pool->refcount[b] += 1;
    pool->seqs.push_back(std::move(c));
    *child = (int)pool->seqs.size() - 1;
    return PA_OK;
}

pa_status pa_seq_append(pa_pool *pool, int seq, int n, int32_t *slots, int32_t *copy_src,
                        int32_t *copy_dst) {
    if (!pool || !copy_src || !copy_dst) return PA_ERR_NULL;
    if (n < 0) return PA_ERR_SHAPE;
    if (n > 0 && !slots) return PA_ERR_NULL;
    std::lock_guard<std::mutex> g(pool->mu);
    if (!pool->live(seq)) return PA_ERR_BAD_ID;
    if (pool->seqs[seq].len + n > (int64_t)INT32_MAX) return PA_ERR_SHAPE;
    if (pool->blocks_needed(seq, n) > (int64_t)pool->free_stack.size()) return PA_ERR_NO_BLOCKS;
    *copy_src = *copy_dst = -1;
    for (int i = 0; i < n; ++i) slots[i] = pool->append_one(seq, copy_src, copy_dst);
    return PA_OK;
}

pa_status pa_seq_append_batch(pa_pool *pool, const int *seqs, int n, int32_t *slots,
                              int32_t *pairs, int *n_pairs) {
    if (!pool || !n_pairs) return PA_ERR_NULL;
    if (n < 0) return PA_ERR_SHAPE;
    if (n > 0 && (!seqs || !slots || !pairs)) return PA_ERR_NULL;
    std::lock_guard<std::mutex> g(pool->mu);
    std::vector<int> ids(seqs, seqs + n);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end()) return PA_ERR_BAD_ID;
    // Exact count of fresh blocks: an earlier copy in this batch lowers a
    // shared block's count, so a later sharer may write in place.
    int64_t need = 0;
    std::unordered_map<int32_t, int32_t> dropped;   // block -> copies already taken from it
    for (int i = 0; i < n; ++i) {
        if (!pool->live(seqs[i])) return PA_ERR_BAD_ID;
        const pa_pool::Seq &q = pool->seqs[seqs[i]];
        if (q.len + 1 > (int64_t)INT32_MAX) return PA_ERR_SHAPE;
        if (q.len == (int64_t)q.table.size() * pool->B) {
            ++need;                                      // last block full (or none)
            continue;
        }
        const int32_t last = q.table.back();
        int32_t &taken = dropped[last];
        if (pool->refcount[last] - taken > 1) {
            ++need;
            ++taken;
        }
    }
    if (need > (int64_t)pool->free_stack.size()) return PA_ERR_NO_BLOCKS;
    int np = 0;
    for (int i = 0; i < n; ++i) {
        int32_t src = -1, dst = -1;
        slots[i] = pool->append_one(seqs[i], &src, &dst);
        if (src >= 0) {
            pairs[2 * np] = src;
            pairs[2 * np + 1] = dst;
            ++np;
        }
    }
    *n_pairs = np;
    return PA_OK;
}

pa_status pa_seq_release(pa_pool *pool, int seq) {
    if (!pool) return PA_ERR_NULL;
    std::lock_guard<std::mutex> g(pool->mu);
    if (!pool->live(seq)) return PA_ERR_BAD_ID;
    pa_pool::Seq &q = pool->seqs[seq];
    for (int32_t b : q.table) {
        if (--pool->refcount[b] == 0) pool->free_stack.push_back(b);
    }
    q.live = false;
    q.len = 0;
    std::vector<int32_t>().swap(q.table);
    return PA_OK;
}

int pa_seq_length(const pa_pool *pool, int seq) {
    if (!pool) return -1;
    std::lock_guard<std::mutex> g(pool->mu);
    return pool->live(seq) ? (int)pool->seqs[seq].len : -1;
}

int pa_seq_num_blocks(const pa_pool *pool, int seq) {
    if (!pool) return -1;
    std::lock_guard<std::mutex> g(pool->mu);
    return pool->live(seq) ? (int)pool->seqs[seq].table.size() : -1;
}

pa_status pa_pool_export(const pa_pool *pool, const int *seqs, int n, int max_blocks,
                         int32_t pad, int32_t *tables, int32_t *lens) {
    if (!pool) return PA_ERR_NULL;
    if (n < 0 || max_blocks < 0) return PA_ERR_SHAPE;
    if (n == 0) return PA_OK;
    if (!seqs || !lens || (max_blocks > 0 && !tables)) return PA_ERR_NULL;
    std::lock_guard<std::mutex> g(pool->mu);
    for (int i = 0; i < n; ++i) {
        if (!pool->live(seqs[i])) return PA_ERR_BAD_ID;
        if ((int64_t)pool->seqs[seqs[i]].table.size() > max_blocks) return PA_ERR_SHAPE;
    }
    for (int i = 0; i < n; ++i) {
        const pa_pool::Seq &q = pool->seqs[seqs[i]];
        int32_t *row = tables + (size_t)i * max_blocks;
        std::copy(q.table.begin(), q.table.end(), row);
        std::fill(row + q.table.size(), row + max_blocks, pad);
        lens[i] = (int32_t)q.len;
    }
    return PA_OK;
}

}  // extern "C"
