/*
 * pa_oracle.c -- CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, fp64 statement of
 * what a paged decode-attention call computes.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the library
 * under paged_kv_cache_301_amd/ never calls, links or includes it, and it
 * shares no code, header or constant with that library.
 *
 * What it computes (one output row per sequence s and query head h):
 *
 *   1. Gather (page "Paged Attention > The PagedAttention Algorithm", section
 *      "Standard Attention vs PagedAttention", the reference function): walk
 *      the sequence's logical blocks in order, translate each through the
 *      block table to a physical block, and copy only the tokens that the
 *      context length covers (the last block may be partly filled) into a
 *      contiguous K and V matrix.  Logical token t lives in logical block
 *      t div B at slot t mod B (same page, opening paragraphs: block number
 *      and within-block offset).
 *   2. Standard attention on the contiguous matrices (same section, the
 *      softmax(Q K^T / sqrt(d_k)) V equation): scores x_t = scale * (q . K_t),
 *      softmax with the maximum subtracted first (page "PagedAttention by
 *      hand", Step 3), output = sum_t p_t V_t (same page, Step 4).
 *
 * Readings where the pages are silent:
 *   - KV pool layout is [NB][Hkv][B][D] for both caches.
 *   - Grouped-query attention: query head h reads kv head h / (Hq / Hkv).
 *   - A sequence of length 0 produces an all-zero output row (the reference
 *     function starts from a zero-filled output).
 *   - Table entries past ceil(L / B) are never read.
 *
 * All arithmetic is IEEE double: inputs are widened exactly (fp32, IEEE
 * binary16 and bfloat16 are all exactly representable in double), sums run
 * in index order, exp() is libm's.
 *
 * Parity is pinned by the tests under tests/: the pages' worked example,
 * closed forms, invariants, and equality with unpaged attention computed by a
 * library routine.  Nothing here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element types of q / K / V.  Values match the library's public enum only
 * because both follow the same documented numbering; no header is shared. */
enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* Return codes. */
enum { ORACLE_OK = 0, ORACLE_EINVAL = 1, ORACLE_ENOMEM = 2 };

/* IEEE 754 binary16 -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 -> double: a bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

static double load_elem(const void *base, size_t i, int dtype)
{
    switch (dtype) {
    case ORACLE_F32: return (double)((const float *)base)[i];
    case ORACLE_F16: return oracle_half_to_double(((const uint16_t *)base)[i]);
    default:         return oracle_bf16_to_double(((const uint16_t *)base)[i]);
    }
}

/*
 * Step 1 (gather): copy the first n tokens of sequence s, kv head g, from the
 * paged pools into contiguous [n][D] matrices K and V, walking the logical
 * blocks in order and cutting the last, partly filled one at n.
 */
static void gather_kv(const void *key_cache, const void *value_cache,
                      const int32_t *block_tables, int s, int g, int n,
                      double *K, double *V, int Hkv, int D, int B,
                      int max_blocks, int dtype)
{
    int nblocks = (n + B - 1) / B;
    int t = 0;
    for (int j = 0; j < nblocks; ++j) {
        int phys = block_tables[(size_t)s * max_blocks + j];
        int first = j * B;
        int last = first + B < n ? first + B : n;    /* partly filled last block */
        for (int slot = 0; slot < last - first; ++slot, ++t) {
            size_t base = (((size_t)phys * Hkv + g) * B + slot) * (size_t)D;
            for (int d = 0; d < D; ++d) {
                K[(size_t)t * D + d] = load_elem(key_cache, base + d, dtype);
                V[(size_t)t * D + d] = load_elem(value_cache, base + d, dtype);
            }
        }
    }
}

/*
 * Steps 2-4 (standard attention on contiguous K / V): query row qrow, head h
 * against the first n >= 1 rows of K and V.  Writes D doubles to o.  Returns
 * ORACLE_ENOMEM if a scratch buffer cannot be allocated.
 */
static int attend_gathered(const void *query, const double *K, const double *V,
                           int qrow, int n, double scale, double *o,
                           int h, int Hq, int D, int dtype)
{
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    double *x = malloc(sizeof(double) * (size_t)n);
    double *qv = malloc(sizeof(double) * (size_t)D);
    if (!x || !qv) {
        free(x); free(qv);
        return ORACLE_ENOMEM;
    }

    /* Step 2: scores x_t = scale * q . K_t. */
    for (int d = 0; d < D; ++d)
        qv[d] = load_elem(query, ((size_t)qrow * Hq + h) * D + d, dtype);
    for (int tt = 0; tt < n; ++tt) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qv[d] * K[(size_t)tt * D + d];
        x[tt] = scale * acc;
    }

    /* Step 3: softmax with the maximum subtracted. */
    double m = x[0];
    for (int tt = 1; tt < n; ++tt) if (x[tt] > m) m = x[tt];
    double Z = 0.0;
    for (int tt = 0; tt < n; ++tt) { x[tt] = exp(x[tt] - m); Z += x[tt]; }
    for (int tt = 0; tt < n; ++tt) x[tt] /= Z;

    /* Step 4: probability-weighted sum of the value rows. */
    for (int tt = 0; tt < n; ++tt)
        for (int d = 0; d < D; ++d) o[d] += x[tt] * V[(size_t)tt * D + d];

    free(x); free(qv);
    return ORACLE_OK;
}

/*
 * One output row: query row qrow (query[qrow][h]) attending the first n
 * tokens of sequence s, query head h (gather, then standard attention).
 * Writes D doubles to o.  Decode calls it with qrow = s and n = seq_lens[s].
 * Returns ORACLE_ENOMEM if the gather buffers cannot be allocated.
 */
static int attend_row(const void *query, const void *key_cache,
                      const void *value_cache, const int32_t *block_tables,
                      int qrow, int n, double scale, double *o,
                      int s, int h, int Hq, int Hkv, int D, int B,
                      int max_blocks, int dtype)
{
    int G = Hq / Hkv;
    int g = h / G;                   /* kv head shared by this query head */

    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n <= 0) return ORACLE_OK;

    double *K = malloc(sizeof(double) * (size_t)n * D);
    double *V = malloc(sizeof(double) * (size_t)n * D);
    if (!K || !V) {
        free(K); free(V);
        return ORACLE_ENOMEM;
    }
    gather_kv(key_cache, value_cache, block_tables, s, g, n, K, V, Hkv, D, B,
              max_blocks, dtype);
    int rc = attend_gathered(query, K, V, qrow, n, scale, o, h, Hq, D, dtype);
    free(K); free(V);
    return rc;
}

/*
 * oracle_decode -- paged decode attention in fp64.
 *
 *   query        [S][Hq][D]            element type `dtype`
 *   key_cache    [NB][Hkv][B][D]       element type `dtype`
 *   value_cache  [NB][Hkv][B][D]       element type `dtype`
 *   block_tables [S][max_blocks]       int32 physical block ids
 *   seq_lens     [S]                   int32 context lengths
 *   out          [nrows][D]            double; row r is (s, h) = divmod(rows[r], Hq)
 *   rows         which (s * Hq + h) rows to compute; NULL means all S * Hq rows
 *                in order (then nrows must equal S * Hq).
 *
 * All pointers are host memory owned by the caller.  Returns ORACLE_EINVAL for
 * inconsistent sizes or an out-of-range table entry / length (checked before
 * any arithmetic), ORACLE_ENOMEM if a gather buffer cannot be allocated.
 */
int oracle_decode(const void *query, const void *key_cache,
                  const void *value_cache, const int32_t *block_tables,
                  const int32_t *seq_lens, double scale, double *out,
                  int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                  int dtype, const int32_t *rows, int nrows)
{
    if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0 ||
        NB <= 0 || max_blocks < 0 || nrows < 0)
        return ORACLE_EINVAL;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_EINVAL;
    if (!rows && nrows != S * Hq) return ORACLE_EINVAL;
    for (int r = 0; r < nrows; ++r) {
        int row = rows ? rows[r] : r;
        if (row < 0 || row >= S * Hq) return ORACLE_EINVAL;
        int s = row / Hq;
        int n = seq_lens[s];
        if (n < 0 || (long long)n > (long long)max_blocks * B) return ORACLE_EINVAL;
        for (int j = 0; j < (n + B - 1) / B; ++j) {
            int p = block_tables[(size_t)s * max_blocks + j];
            if (p < 0 || p >= NB) return ORACLE_EINVAL;
        }
    }

    int status = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int row = rows ? rows[r] : r;
        int s = row / Hq;
        int rc = attend_row(query, key_cache, value_cache, block_tables,
                            s, seq_lens[s], scale, out + (size_t)r * D,
                            s, row % Hq, Hq, Hkv, D, B, max_blocks, dtype);
        if (rc != ORACLE_OK) {
#pragma omp atomic write
            status = rc;
        }
    }
    return status;
}

/*
 * oracle_prefill -- several new tokens per sequence, causal, in fp64.
 *
 * Glossary "PagedAttention", section "How It Works": query i attends the
 * logical blocks up to ceil(i / B), i.e. (token-level reading) every token up
 * to and including its own position, the last block cut there.  Sequence s
 * owns query rows query_start[s] .. query_start[s+1]-1, the last
 * n_s = query_start[s+1] - query_start[s] of its L_s = seq_lens[s] tokens;
 * row query_start[s] + k sits at position L_s - n_s + k and attends tokens
 * 0 .. L_s - n_s + k.  Each output row is the decode computation (gather,
 * then standard attention) over that many tokens.
 *
 *   query [T][Hq][D], out [nrows][D] doubles; row r of out is query row
 *   rows[r] / Hq, head rows[r] % Hq (rows NULL: all T * Hq rows in order).
 * Returns ORACLE_EINVAL for inconsistent sizes or offsets, ORACLE_ENOMEM.
 */
int oracle_prefill(const void *query, const void *key_cache,
                   const void *value_cache, const int32_t *block_tables,
                   const int32_t *seq_lens, const int32_t *query_start,
                   double scale, double *out, int S, int T, int Hq, int Hkv,
                   int D, int B, int NB, int max_blocks, int dtype,
                   const int32_t *rows, int nrows)
{
    if (S < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 ||
        B <= 0 || NB <= 0 || max_blocks < 0 || nrows < 0)
        return ORACLE_EINVAL;
    if (dtype != ORACLE_F32 && dtype != ORACLE_F16 && dtype != ORACLE_BF16)
        return ORACLE_EINVAL;
    if (!rows && nrows != T * Hq) return ORACLE_EINVAL;
    if (query_start[0] != 0 || query_start[S] != T) return ORACLE_EINVAL;
    for (int s = 0; s < S; ++s) {
        int n = query_start[s + 1] - query_start[s];
        int L = seq_lens[s];
        if (n < 0 || (n > 0 && (L < n || (long long)L > (long long)max_blocks * B)))
            return ORACLE_EINVAL;
        if (n > 0)
            for (int j = 0; j < (L + B - 1) / B; ++j) {
                int p = block_tables[(size_t)s * max_blocks + j];
                if (p < 0 || p >= NB) return ORACLE_EINVAL;
            }
    }
    for (int r = 0; r < nrows; ++r) {
        int row = rows ? rows[r] : r;
        if (row < 0 || row >= T * Hq) return ORACLE_EINVAL;
    }

    /* The requested rows, bucketed by (sequence, kv head): each bucket's
     * sequence is gathered once (all L_s tokens), and every row attends its
     * own prefix of that gather.  Tokens 0 .. pos of a logical-order gather
     * are exactly a gather of pos + 1 tokens, so each row's arithmetic is
     * the same as gathering for that row alone. */
    int G = Hq / Hkv;
    int nb = S * Hkv;
    int *count = calloc((size_t)nb + 1, sizeof(int));
    int *order = malloc(sizeof(int) * (size_t)(nrows > 0 ? nrows : 1));
    int *seq_of = malloc(sizeof(int) * (size_t)(nrows > 0 ? nrows : 1));
    int *pos_of = malloc(sizeof(int) * (size_t)(nrows > 0 ? nrows : 1));
    if (!count || !order || !seq_of || !pos_of) {
        free(count); free(order); free(seq_of); free(pos_of);
        return ORACLE_ENOMEM;
    }
    for (int r = 0; r < nrows; ++r) {
        int row = rows ? rows[r] : r;
        int t = row / Hq, h = row % Hq;
        int s = 0;                        /* the sequence owning query row t */
        while (query_start[s + 1] <= t) ++s;
        int n = query_start[s + 1] - query_start[s];
        int pos = seq_lens[s] - n + (t - query_start[s]);
        seq_of[r] = s;
        pos_of[r] = pos;
        count[s * Hkv + h / G + 1] += 1;
    }
    for (int k = 0; k < nb; ++k) count[k + 1] += count[k];
    {
        int *fill = malloc(sizeof(int) * (size_t)(nb > 0 ? nb : 1));
        if (!fill) {
            free(count); free(order); free(seq_of); free(pos_of);
            return ORACLE_ENOMEM;
        }
        for (int k = 0; k < nb; ++k) fill[k] = count[k];
        for (int r = 0; r < nrows; ++r) {
            int row = rows ? rows[r] : r;
            order[fill[seq_of[r] * Hkv + (row % Hq) / G]++] = r;
        }
        free(fill);
    }

    int status = ORACLE_OK;
    for (int k = 0; k < nb && status == ORACLE_OK; ++k) {
        int lo = count[k], hi = count[k + 1];
        if (lo == hi) continue;
        int s = k / Hkv, g = k % Hkv;
        int L = seq_lens[s];              /* >= 1: the sequence has query rows */
        double *K = malloc(sizeof(double) * (size_t)L * D);
        double *V = malloc(sizeof(double) * (size_t)L * D);
        if (!K || !V) {
            free(K); free(V);
            status = ORACLE_ENOMEM;
            break;
        }
        gather_kv(key_cache, value_cache, block_tables, s, g, L, K, V, Hkv, D, B,
                  max_blocks, dtype);
#pragma omp parallel for schedule(dynamic, 1)
        for (int i = lo; i < hi; ++i) {
            int r = order[i];
            int row = rows ? rows[r] : r;
            int t = row / Hq, h = row % Hq;
            int pos = pos_of[r];
            int rc = attend_gathered(query, K, V, t, pos + 1, scale, out + (size_t)r * D,
                                     h, Hq, D, dtype);
            if (rc != ORACLE_OK) {
#pragma omp atomic write
                status = rc;
            }
        }
        free(K); free(V);
    }
    free(count); free(order); free(seq_of); free(pos_of);
    return status;
}

/*
 * oracle_write_kv -- store new tokens' keys and values into their cache slots.
 *
 * Page "PagedAttention by hand", section "Setup" (Step 1) and the end of
 * "Forward pass" (Step 4): the current token's key and value are written into
 * its slot of the sequence's physical block before attention runs.
 *
 *   key, value    [T][Hkv][D]        element size esz bytes
 *   slot_mapping  [T]                physical slot = block * B + offset, or
 *                                    negative to skip the token
 *   key_cache, value_cache [NB][Hkv][B][D]
 *
 * Pure data movement: element bytes are copied unchanged.  Slots at or past
 * NB * B are skipped (returned count excludes them).  Returns the number of
 * tokens written.
 */
long long oracle_write_kv(const void *key, const void *value, const int32_t *slot_mapping,
                          void *key_cache, void *value_cache, int T, int Hkv, int D, int B,
                          int NB, int esz)
{
    long long written = 0;
    for (int t = 0; t < T; ++t) {
        long long slot = slot_mapping[t];
        if (slot < 0 || slot >= (long long)NB * B) continue;
        long long block = slot / B, offset = slot % B;
        for (int h = 0; h < Hkv; ++h) {
            size_t src = ((size_t)t * Hkv + h) * (size_t)D * esz;
            size_t dst = (((size_t)block * Hkv + h) * B + offset) * (size_t)D * esz;
            memcpy((char *)key_cache + dst, (const char *)key + src, (size_t)D * esz);
            memcpy((char *)value_cache + dst, (const char *)value + src, (size_t)D * esz);
        }
        ++written;
    }
    return written;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
