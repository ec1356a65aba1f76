/*
 * pa_decode.h -- paged decode attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpa_decode.so.  Every pointer argument named *_cache, query,
 * block_tables, seq_lens, out or workspace is a DEVICE pointer owned by the
 * caller; the library allocates nothing.  All compute entry points are
 * asynchronous on `stream` (a hipStream_t; NULL is the default stream) and
 * never synchronise it, except in the checked mode described at
 * pa_get_device_error.  The only device state the library keeps is the small
 * per-device word of that checked mode.
 *
 * The operation (pages "Paged Attention > The PagedAttention Algorithm",
 * sections "Standard Attention vs PagedAttention" and "Optimized CUDA
 * Kernels"; "PagedAttention by hand", sections "Setup" and "Forward pass",
 * Steps 2-4; glossary "PagedAttention", section "How It Works"): for every
 * sequence s and query head h, with L = seq_lens[s] and kv head
 * g = h / (Hq / Hkv),
 *
 *     token t (0 <= t < L) lives in physical block block_tables[s][t / B]
 *     at slot t % B;
 *     x_t  = scale * dot(query[s][h], K[t]);
 *     p_t  = exp(x_t - max_u x_u) / sum_u exp(x_u - max_u x_u);
 *     out[s][h] = sum_t p_t * V[t];
 *
 * and out[s][h] = 0 when L = 0.  Slots at or past L in a sequence's last
 * block, and table entries at or past ceil(L / B), are never read: their
 * contents (NaN included) cannot reach the output.
 *
 * Layouts (row-major, densely packed, element type `dtype`):
 *     query        [S][Hq][D]
 *     key_cache    [NB][Hkv][B][D]
 *     value_cache  [NB][Hkv][B][D]
 *     block_tables [S][max_blocks]   int32
 *     seq_lens     [S]               int32
 *     out          [S][Hq][D]        element type `out_dtype`
 *
 * Preconditions on device data (the caller guarantees them; the attention
 * kernels do not check them): 0 <= seq_lens[s] <= max_blocks * B, and
 * 0 <= block_tables[s][j] < NB for every j < ceil(seq_lens[s] / B).  In the
 * checked mode (PA_CHECK=1 in the environment, or pa_config.check = 1) the
 * library verifies them on the device before any attention kernel runs and
 * returns PA_ERR_DEVICE_CHECK instead of launching ("PagedAttention by
 * hand", section "Forward pass", Step 2: slots past a sequence's context may
 * hold whatever an earlier sequence left there, so lengths and table entries
 * decide what may be read).
 *
 * Arithmetic: fp32 accumulation for fp16 / bf16 inputs; the output is rounded
 * to `out_dtype` (round to nearest even) once, at the end.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Status codes.  Every entry point validates its host-side arguments before
 * launching anything: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED and
 * PA_ERR_WORKSPACE mean nothing was launched, and so does
 * PA_ERR_DEVICE_CHECK.  PA_ERR_HIP means a launch failed; a kernel queued
 * earlier in the same call (e.g. the partition pass before a failing
 * combine) may still run. */
typedef enum {
    PA_OK = 0,
    PA_ERR_NULL = 1,        /* a required pointer is NULL                       */
    PA_ERR_SHAPE = 2,       /* negative / zero size, Hq % Hkv != 0, size overflow,
                               or a launch grid beyond the hardware limits       */
    PA_ERR_UNSUPPORTED = 3, /* dtype, head size or kernel choice not supported  */
    PA_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned       */
    PA_ERR_HIP = 5,         /* the HIP runtime reported an error                */
    PA_ERR_NO_BLOCKS = 6,   /* block pool: not enough free blocks (nothing changed) */
    PA_ERR_BAD_ID = 7,      /* block pool: unknown or released sequence / block id */
    PA_ERR_DEVICE_CHECK = 8,/* checked mode: a length or used table entry breaks
                               the preconditions; no attention kernel ran       */
    PA_ERR_SCRATCH = 9      /* pa_decode_noalloc: the plan needs more partial-
                               result space than PA_NOALLOC_SCRATCH_BYTES        */
} pa_status;

/* Kernel families (pa_config.kernel). */
typedef enum {
    PA_KERNEL_AUTO = 0,     /* library chooses                                   */
    PA_KERNEL_GENERIC = 1,  /* plain kernel: any D <= 512, any B >= 1, any group,
                               fp32 / fp16 / bf16; one pass, no workspace        */
    PA_KERNEL_VALU = 2,     /* tiled kernel: D = 128, fp16 / bf16, B a power of
                               two, groups of 1, 2, 4 or 8 query heads; 16-byte
                               loads of whole block rows, VALU dot products     */
    PA_KERNEL_MFMA = 3      /* grouped-query kernel: D = 128, fp16 / bf16, B a
                               power of two, 1, 2, 4, 8, 16, 32 or 64 query
                               heads per kv head (32 and 64: multi-query,
                               several waves share each K / V tile; 1 and 2
                               only when asked for); the group's q.K and p.V
                               contractions on matrix cores                      */
} pa_kernel;

/* Stages of a call (pa_config.stages, a bit mask). */
enum {
    PA_STAGE_PARTITIONS = 1, /* attention over each context partition           */
    PA_STAGE_COMBINE = 2,    /* log-sum-exp merge of partitions (split plans)   */
    PA_STAGE_ALL = 3
};

/* Optional explicit configuration; a zero-initialised struct means "auto". */
typedef struct {
    int kernel;           /* pa_kernel                                           */
    int partition_tokens; /* 0: automatic.  Otherwise tokens per context
                             partition, a positive multiple of 32.  A value at
                             or above max_blocks * B gives a single-pass plan.   */
    int stages;           /* 0 means PA_STAGE_ALL                                */
    int kv_reuse;         /* 0: K / V rows are streamed with the non-temporal
                             load hint (each row is read once per call: best
                             when sequences share few blocks).  1: ordinary
                             cached loads, for pools where many sequences of
                             the batch share blocks (a common prompt prefix),
                             so repeated rows can hit in L2 / Infinity Cache.
                             Results are identical either way.                  */
    int check;            /* checked mode: 0 follows the PA_CHECK environment
                             variable (on when it is "1"), 1 always checks,
                             -1 never checks.  See pa_get_device_error.          */
    int token_waves;      /* 0: automatic.  1, 2 or 4: waves of one work-group
                             that share each (sequence, kv head, partition)
                             item's tokens, every one streaming every
                             token_waves-th 32-token tile, their softmax
                             states merged in LDS.  Above 1 it needs the VALU
                             kernel with a block size that is a multiple of 4,
                             or the matrix-core kernel with at most 16 query
                             heads per kv head (any block size; the automatic
                             plan keeps blocks of 1 or 2 tokens on one wave)
                             (else PA_ERR_UNSUPPORTED); other values are
                             PA_ERR_SHAPE.  Decode only: the
                             multi-token calls accept 0 or 1.                   */
} pa_config;

/* The plan a call will execute (filled by pa_decode_plan). */
typedef struct {
    int kernel;           /* resolved pa_kernel                                  */
    int partition_tokens; /* tokens per partition (>= max_blocks * B if single)  */
    int max_partitions;   /* partitions per (sequence, head) the grid covers     */
    int split;            /* 1: partial results go to the workspace and a
                             combine stage merges them; 0: single pass          */
    size_t workspace_bytes; /* bytes of device workspace the plan needs (0 if
                               single pass)                                     */
    int token_waves;      /* waves per item (1, 2 or 4; see pa_config)          */
} pa_plan;

/*
 * pa_decode_plan -- resolve the kernel, the context partitioning and the
 * waves per item for a shape.  Host-only: touches no device and launches
 * nothing.  `cfg` may be NULL (automatic).  Returns the same validation
 * status pa_decode_ex would for these sizes and types.  The automatic plan
 * sees only the table width (max_blocks * B), not the lengths: it sizes
 * partitions and token-waves so the items of a batch that fills its tables
 * fill the GPU's resident waves.
 */
pa_status pa_decode_plan(int S, int Hq, int Hkv, int D, int B, int NB,
                         int max_blocks, pa_dtype dtype, pa_dtype out_dtype,
                         const pa_config *cfg, pa_plan *plan);

/*
 * pa_decode_workspace_bytes -- device workspace pa_decode needs for this
 * shape (the automatic plan); 0 when that plan is single pass.  Returns 0 for
 * invalid shapes too (pa_decode then reports the error).
 */
size_t pa_decode_workspace_bytes(int S, int Hq, int Hkv, int D, int B, int NB,
                                 int max_blocks, pa_dtype dtype,
                                 pa_dtype out_dtype);

/*
 * pa_decode -- paged decode attention with the automatic plan.
 *
 * scale      multiplies every dot product (usually 1 / sqrt(D)).
 * out_dtype  dtype or PA_F32.
 * workspace  device buffer of at least pa_decode_workspace_bytes(...) bytes,
 *            256-byte aligned; may be NULL when that size is 0.  Its contents
 *            need no initialisation and are scratch after the call.
 * S = 0 is a no-op returning PA_OK.
 *
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (e.g. D > 512,
 * out_dtype not in {dtype, PA_F32}), PA_ERR_WORKSPACE, PA_ERR_HIP, and in the
 * checked mode PA_ERR_DEVICE_CHECK.
 */
pa_status pa_decode(const void *query, const void *key_cache,
                    const void *value_cache, const int32_t *block_tables,
                    const int32_t *seq_lens, float scale, void *out,
                    int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                    pa_dtype dtype, pa_dtype out_dtype,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_decode_ex -- as pa_decode, with an explicit configuration.
 *
 * cfg->kernel forces a kernel family (PA_ERR_UNSUPPORTED if it cannot run this
 * shape or if a pointer is not 16-byte aligned); cfg->partition_tokens forces
 * the context partition; cfg->stages runs only part of a split plan: running
 * PA_STAGE_PARTITIONS and then PA_STAGE_COMBINE on the same stream, with the
 * same arguments and workspace, equals one PA_STAGE_ALL call.  In a single-pass
 * plan PA_STAGE_COMBINE alone is a no-op.
 */
pa_status pa_decode_ex(const void *query, const void *key_cache,
                       const void *value_cache, const int32_t *block_tables,
                       const int32_t *seq_lens, float scale, void *out,
                       int S, int Hq, int Hkv, int D, int B, int NB,
                       int max_blocks, pa_dtype dtype, pa_dtype out_dtype,
                       const pa_config *cfg, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Bytes of the static device scratch of pa_decode_noalloc (per GPU). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * pa_decode_noalloc -- pa_decode_ex for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and errors as pa_decode_ex
 * without the workspace: the split plan's partial results go to a static
 * device array of PA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends.  The call allocates nothing.
 *
 * Limit: a plan whose workspace (pa_decode_plan's workspace_bytes) exceeds
 * PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_SCRATCH before anything runs; a
 * longer cfg->partition_tokens shrinks it (the workspace holds
 * S * Hq * max_partitions * (D + 2) fp32 values, 256-byte aligned parts).
 * The scratch is shared by every call on one GPU and keeps the last call's
 * partial results: calls that overlap on one GPU (several streams or host
 * threads) race and must be serialised by the caller.
 */
pa_status pa_decode_noalloc(const void *query, const void *key_cache,
                            const void *value_cache, const int32_t *block_tables,
                            const int32_t *seq_lens, float scale, void *out,
                            int S, int Hq, int Hkv, int D, int B, int NB,
                            int max_blocks, pa_dtype dtype, pa_dtype out_dtype,
                            const pa_config *cfg, void *stream);

/*
 * pa_write_kv -- store new tokens' keys and values into their cache slots
 * (page "PagedAttention by hand", section "Setup", Step 1, and the end of
 * "Forward pass": a token's key and value are written into its slot of the
 * sequence's physical block before attention runs).
 *
 *   key, value     [T][Hkv][D]      dtype, device
 *   slot_mapping   [T]              int32, device: block * B + offset; a
 *                                   negative value skips the token
 *   key_cache, value_cache [NB][Hkv][B][D], device, updated in place
 *
 * Bits are copied unchanged.  Slots at or past NB * B are skipped.  Two tokens
 * with the same slot race (one of them wins).  Asynchronous on `stream`.
 * Errors: PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (dtype), PA_ERR_NULL, PA_ERR_HIP.
 */
pa_status pa_write_kv(const void *key, const void *value, const int32_t *slot_mapping,
                      void *key_cache, void *value_cache, int T, int Hkv, int D, int B,
                      int NB, pa_dtype dtype, void *stream);

/*
 * pa_append_kv -- the decode-step form of pa_write_kv: sequence s's new token
 * is the last of its seq_lens[s] tokens (the lengths include it), so its rows
 * go to block block_tables[s][(L - 1) / B], offset (L - 1) % B.
 *
 *   key, value     [S][Hkv][D]      dtype, device
 *   block_tables   [S][max_blocks]  int32, device
 *   seq_lens       [S]              int32, device
 *
 * Sequences with L <= 0, a table position past max_blocks, or a table entry
 * outside [0, NB) are skipped.  Asynchronous on `stream`.
 */
pa_status pa_append_kv(const void *key, const void *value, const int32_t *block_tables,
                       const int32_t *seq_lens, void *key_cache, void *value_cache,
                       int S, int Hkv, int D, int B, int NB, int max_blocks,
                       pa_dtype dtype, void *stream);

/*
 * pa_copy_blocks -- batched whole-block copy inside both caches, the copy step
 * of copy-on-write (page "PagedAttention by hand", section "Memory Sharing
 * (Copy-on-Write)": before a sequence writes into a block that other
 * sequences still use, the block's contents are copied to a fresh block and
 * the write goes to the copy).
 *
 *   pairs   [n][2] int32, device: pairs[i] = {src, dst}; block dst of both
 *           caches becomes a copy of block src (all Hkv heads, all B slots)
 *   key_cache, value_cache [NB][Hkv][B][D], device, updated in place
 *
 * Pairs with src or dst outside [0, NB), or src == dst, are skipped.  The dst
 * blocks must be distinct and no dst may be another pair's src (a block pool
 * never produces either); otherwise the result is unspecified.  Bits are
 * copied unchanged.  Asynchronous on `stream`.  n = 0 is a no-op.
 * Errors: PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (dtype), PA_ERR_NULL, PA_ERR_HIP.
 */
pa_status pa_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs, int n,
                         int Hkv, int D, int B, int NB, pa_dtype dtype, void *stream);

/*
 * pa_check_inputs -- debug check of the device-data preconditions above
 * (0 <= seq_lens[s] <= max_blocks * B; 0 <= block_tables[s][j] < NB for every
 * j < ceil(seq_lens[s] / B)), run on the device without reading K or V.
 *
 *   report   int32[2], device, caller-owned: report[0] = number of offending
 *            sequences, report[1] = smallest offending sequence index
 *            (INT32_MAX if none).  Written by the call (no prior zeroing).
 *
 * Only the table entries a valid length would use are read, so any table is
 * safe to check.  Run it before pa_decode / pa_prefill / pa_append_kv on
 * untrusted inputs and skip the call when report[0] != 0.  Asynchronous on
 * `stream`.  Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_HIP.  S = 0 writes a
 * clean report.
 */
pa_status pa_check_inputs(const int32_t *block_tables, const int32_t *seq_lens, int S,
                          int max_blocks, int B, int NB, int32_t *report, void *stream);

/*
 * pa_get_device_error -- the sticky result of the library's device input
 * check on the current device (the device `stream` belongs to).
 *
 * Checked mode.  When PA_CHECK=1 is set in the environment (read at every
 * call) or pa_config.check = 1, pa_decode, pa_decode_ex and pa_prefill first
 * run the device check of pa_check_inputs (lengths within the table, every
 * used table entry within the pool; for pa_prefill also query_start ordered,
 * from 0 to T, with 0 <= n_s <= min(seq_lens[s], max_query_len)) on
 * `stream`, wait for it (the call synchronises `stream`, so the checked mode
 * cannot be captured in a HIP graph) and, if any sequence fails, return
 * PA_ERR_DEVICE_CHECK without launching an attention kernel: `out` and the
 * workspace are left untouched.  A failing check also sets a per-device
 * error word that stays set until read here.
 *
 * This call synchronises `stream`, returns PA_ERR_DEVICE_CHECK if the word
 * is set (and clears it), PA_OK otherwise, PA_ERR_HIP on a runtime error.
 * `first_bad` may be NULL; otherwise it receives the smallest offending
 * sequence index of the device's most recent check if the word is set and
 * that check failed, else -1.  Checks on one device share the word: calls
 * that overlap on several streams of one device race for it.
 */
pa_status pa_get_device_error(void *stream, int32_t *first_bad);

/* Human-readable name of a status code (static storage). */
const char *pa_status_string(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
