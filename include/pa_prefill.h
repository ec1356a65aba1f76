/*
 * pa_prefill.h -- several new tokens per sequence against the paged cache,
 * causal (a chunked prefill, or several tokens appended at once).
 *
 * The operation (glossary "PagedAttention", section "How It Works": query i
 * attends logical blocks 1 .. ceil(i / B) through the block table; page
 * "Paged Attention > The PagedAttention Algorithm", section "Standard
 * Attention vs PagedAttention", for the attention itself): sequence s has
 * n_s = query_start[s+1] - query_start[s] new tokens, the last n_s of its
 * L_s = seq_lens[s] cached tokens (their K / V already written, e.g. with
 * pa_write_kv).  Query row r = query_start[s] + k (0 <= k < n_s) sits at
 * position P = L_s - n_s + k and, for every query head h with kv head
 * g = h / (Hq / Hkv),
 *
 *     x_t  = scale * dot(query[r][h], K[t])           for t = 0 .. P
 *     out[r][h] = sum_t softmax(x)_t * V[t]
 *
 * i.e. token-level causal attention: the row sees its own token and every
 * earlier one, never a later token of the same chunk, even one in the same
 * block.  With n_s = 1 for every s this is pa_decode.
 *
 * Layouts (row-major, element type `dtype`):
 *     query        [T][Hq][D]      rows grouped by sequence, in order
 *     key_cache / value_cache [NB][Hkv][B][D]
 *     block_tables [S][max_blocks] int32
 *     seq_lens     [S]             int32
 *     query_start  [S+1]           int32, device
 *     out          [T][Hq][D]      element type `out_dtype`
 *
 * Device-data preconditions (the kernels do not check them; the checked mode
 * of pa_decode.h does, before launching): query_start[0] = 0, non-decreasing,
 * query_start[S] = T; 0 <= n_s <= max_query_len; n_s <= L_s <= max_blocks * B
 * when n_s > 0; valid block ids for the first ceil(L_s / B) table entries.
 *
 * Kernels: a matrix-core kernel for D = 128, fp16 / bf16, B a power of two
 * and Hq / Hkv in {1, 2, 4, 8, 16, 32, 64}; every other accepted shape runs
 * the plain kernel (D <= 512, any B, fp32 too).  Long contexts are split
 * into partitions merged per query row; the split needs the workspace that
 * pa_prefill_plan reports (256-byte aligned device memory).
 *
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (also T > 65535 or S > 65535),
 * PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, and in the checked mode
 * PA_ERR_DEVICE_CHECK.  T = 0 or S = 0 is a no-op.  Asynchronous on `stream`
 * (the checked mode synchronises it); nothing is allocated.
 */
#ifndef PA_PREFILL_H
#define PA_PREFILL_H

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Host-only: the plan (kernel, partition, workspace) a call would use.
 * cfg may force PA_KERNEL_GENERIC or PA_KERNEL_MFMA and a partition size
 * (a multiple of 32); cfg->stages and cfg->kv_reuse act as in pa_decode_ex. */
pa_status pa_prefill_plan(int S, int T, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                          int max_query_len, pa_dtype dtype, pa_dtype out_dtype,
                          const pa_config *cfg, pa_plan *plan);

pa_status pa_prefill(const void *query, const void *key_cache, const void *value_cache,
                     const int32_t *block_tables, const int32_t *seq_lens,
                     const int32_t *query_start, float scale, void *out,
                     int S, int T, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                     int max_query_len, pa_dtype dtype, pa_dtype out_dtype,
                     const pa_config *cfg, void *workspace, size_t workspace_bytes,
                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PREFILL_H */
