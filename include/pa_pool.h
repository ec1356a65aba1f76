/*
 * pa_pool.h -- host-side block pool: free list, reference counts, per-sequence
 * block tables and copy-on-write, for the paged KV cache of libpa_decode.so.
 *
 * What it manages (page "PagedAttention by hand", sections "Why divide memory
 * into physical blocks?" and "Memory Sharing (Copy-on-Write)"; page "Paged
 * Attention > The PagedAttention Algorithm", the block-table description):
 *   - NB physical blocks of B token slots each, all interchangeable; the free
 *     blocks sit on a stack (last freed, first reused);
 *   - one block table per sequence, logical block j -> physical block id;
 *     a block is taken from the free stack only when the sequence's last
 *     block is full (on demand);
 *   - a reference count per physical block: the number of sequences whose
 *     table holds it.  Forking a sequence shares all its blocks (every count
 *     +1).  When a sequence is about to write into a block whose count is
 *     above 1, the pool takes a fresh block, reports the pair
 *     {shared block, fresh block} for the caller to copy (pa_copy_blocks),
 *     drops the shared block's count by 1 and puts the fresh block in the
 *     sequence's table; the write then goes to the fresh block.
 *
 * Policy fixed here (the pages leave it open): the initial free stack pops
 * block 0 first, then 1, 2, ... (or a caller-given order); a released sequence returns its blocks whose
 * count reaches 0 to the stack in table order, so its last block is reused
 * first.  Sequence ids are 0, 1, 2, ... in creation order and never reused.
 *
 * Everything here is host memory and host code; nothing touches the GPU.
 * The device side of one decode step is: pa_copy_blocks(copies), then
 * pa_write_kv(slots) for the new tokens, then pa_decode.  Each pool call is
 * atomic: on a non-OK status the pool is unchanged.  Calls on one pool are
 * serialised by an internal mutex.
 */
#ifndef PA_POOL_H
#define PA_POOL_H

#include <stdint.h>

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_pool pa_pool;   /* opaque */

/* A pool of num_blocks blocks of block_size slots, all free.  free_order
 * (host, optional) is a permutation of 0 .. num_blocks-1 giving the order in
 * which the fresh stack hands blocks out; NULL means 0, 1, 2, ...  *out
 * receives the handle (owned by the caller, released with pa_pool_destroy).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (num_blocks <= 0, block_size <= 0,
 * free_order not a permutation). */
pa_status pa_pool_create(int num_blocks, int block_size, const int32_t *free_order,
                         pa_pool **out);
void pa_pool_destroy(pa_pool *pool);

/* Free blocks on the stack; -1 for a NULL pool. */
int pa_pool_num_free(const pa_pool *pool);

/* Reference count of a physical block (0 = free); -1 for a bad id. */
int pa_pool_refcount(const pa_pool *pool, int block);

/* A new, empty sequence (length 0, no blocks); its id goes to *seq. */
pa_status pa_seq_create(pa_pool *pool, int *seq);

/* A new sequence sharing every block of `parent` (same table, same length);
 * each of those blocks' counts goes up by 1.  Errors: PA_ERR_BAD_ID. */
pa_status pa_seq_fork(pa_pool *pool, int parent, int *child);

/*
 * Reserve slots for the next n tokens of sequence `seq` (positions L .. L+n-1,
 * L its current length) and grow its length by n.  slots[i] (host, n entries)
 * receives block * B + offset for position L + i.  If the first new token
 * falls into a partly filled last block whose count is above 1, that block is
 * copied on write: *copy_src / *copy_dst receive {shared block, fresh block}
 * (both -1 when no copy is needed; only the first token can need one).
 * Errors: PA_ERR_BAD_ID, PA_ERR_SHAPE (n < 0), PA_ERR_NULL, PA_ERR_NO_BLOCKS
 * (the free stack cannot supply every block the call needs).
 */
pa_status pa_seq_append(pa_pool *pool, int seq, int n, int32_t *slots,
                        int32_t *copy_src, int32_t *copy_dst);

/*
 * One decode step for a batch: one new token for each of the n sequences in
 * seqs (distinct ids), in order.  slots[i] receives sequence seqs[i]'s slot;
 * copy-on-write pairs are appended to pairs ([n][2] host capacity) and their
 * number stored in *n_pairs.  All or nothing: PA_ERR_NO_BLOCKS leaves the pool
 * unchanged.  Errors as pa_seq_append, PA_ERR_BAD_ID also for repeated ids.
 */
pa_status pa_seq_append_batch(pa_pool *pool, const int *seqs, int n, int32_t *slots,
                              int32_t *pairs, int *n_pairs);

/* Release a sequence: every block in its table loses one reference; blocks
 * reaching 0 go back on the free stack.  Errors: PA_ERR_BAD_ID. */
pa_status pa_seq_release(pa_pool *pool, int seq);

/* Length in tokens and number of blocks of a live sequence; -1 for a bad id. */
int pa_seq_length(const pa_pool *pool, int seq);
int pa_seq_num_blocks(const pa_pool *pool, int seq);

/*
 * Export the block tables and lengths of n sequences in the decode layout:
 * tables [n][max_blocks] int32 (host), entry j of row i = physical block of
 * logical block j of seqs[i], entries past its block count = pad; lens [n].
 * Errors: PA_ERR_BAD_ID, PA_ERR_NULL, PA_ERR_SHAPE (a table longer than
 * max_blocks, n < 0).
 */
pa_status pa_pool_export(const pa_pool *pool, const int *seqs, int n, int max_blocks,
                         int32_t pad, int32_t *tables, int32_t *lens);

#ifdef __cplusplus
}
#endif

#endif /* PA_POOL_H */
