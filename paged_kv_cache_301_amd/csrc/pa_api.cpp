// pa_api.cpp -- the C ABI of libpa_decode.so: argument validation, planning
// (kernel family, context partitioning, workspace layout) and launches.
//
// Validation and planning are plain host code with no HIP calls, so they run
// (and are tested) on machines without a GPU.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "pa_internal.h"
#include "pa_measure.h"
#include "pa_prefill.h"

namespace {

using pa::Args;

// Automatic partition size: at least kAutoPartitionMin tokens and at most
// kAutoMaxParts partitions per context (long contexts: fewer, longer
// partitions keep the combine pass and the partial results small), then
// halved (down to kAutoPartitionFloor) while the grid would hold fewer than
// kAutoMinItems waves over (sequence, kv head, partition) items, so small batches still
// occupy 256 CUs.  Contexts of at most kAutoSinglePass tokens run in one pass.
constexpr long long kAutoPartitionMin = 1024;
constexpr long long kAutoMaxParts = 32;
constexpr long long kAutoPartitionFloor = 64;
constexpr long long kAutoMinItems = 4096;
constexpr long long kAutoSinglePass = 256;
// (sequence, kv head) pairs from which the automatic plan runs items on
// four token-waves (see make_plan).
constexpr long long kMultiWavePairs = 512;
// Resident waves of the matrix-core kernel on 256 CUs: 2 per SIMD, 3 for
// its four-wave work-groups (at most 158 VGPRs, 32 KB of LDS per
// work-group).
constexpr long long kResidentWaves = 2048;
long long resident_waves(int waves) { return waves == 4 ? 3072 : kResidentWaves; }
// Resident waves of the VALU kernel: 3 per SIMD (161 VGPRs).
constexpr long long kValuResidentWaves = 3072;

// waves: waves per work-group (the matrix-core kernel runs ceil(G / 16)).
// Measured with the longest-first item order: 1024-token partitions beat 512
// by 2 % (mha_7b), 5 % (gqa_70b) and 8 % (multi-query, whose partial results
// are G * D * 4 bytes per partition) and tie on gqa_long.
// Wide groups (several waves per work-group) have few resident work-groups
// and large partial results, so their partition also doubles while the
// items, counted at the full table width, would exceed a round of resident
// waves by more than a third (batches rarely fill their tables).  On the
// 256-sequence multi-query workload this keeps 1024 tokens at 64 heads
// (cold step 83.0 / 84.6 us against 88.3 / 89.4 at 2048; 1280 gave 80.7 /
// 83.2, 768 87.1 / 88.5) and at 32 heads (3993 vs 3643 GB/s at 1536).
// One-wave items in batches below kMultiWavePairs (sequence, kv head)
// pairs, which get no token-waves, double the same way when their contexts
// are long enough to exceed that at the base partition, and the small-batch
// halving then does not apply.  16 contexts of 16k-32k tokens at 4 heads per
// kv head (128 pairs) take 2048-token partitions, about 1500 items in one
// round, instead of about 3000 in 1.47 rounds at 1024: cold step 221.3 /
// 222.1 -> 213.8 / 213.2 us (B = 16), 224.8 / 225.2 -> 217.5 / 219.6
// (B = 8), 219.1 / 219.8 -> 212.7 / 214.8 (B = 32), A/B on one box.
// Batches that fill a round only at the table width keep the halving to
// two rounds: their tables are mostly empty (one round at the table width
// was slower on 8 sequences of up to 2048 or 4096 tokens, 28.2 -> 29.4 and
// 57.9 -> 61.2 us, and on 32 of 128 - 8192, 69.8 -> 71.9).  The VALU
// kernel counts its own 3072 slots: 8 MHA sequences of 16000 tokens keep
// 1024-token partitions, 332.9 / 333.9 us against 341.0 / 342.3 at 2048.
long long auto_partition(int S, int Hkv, long long max_ctx, int waves, bool valu) {
    if (max_ctx <= kAutoSinglePass) return max_ctx;
    long long part = kAutoPartitionMin;
    while (part * kAutoMaxParts < max_ctx) part *= 2;
    const long long pairs = (long long)S * Hkv;
    auto items = [&](long long p) { return pairs * ((max_ctx + p - 1) / p); };
    const long long resident = resident_waves(waves);
    bool grown = false;   // one-wave items of a small batch made longer
    if (waves > 1) {
        while (part < max_ctx && 3 * items(part) * waves > 4 * resident) part *= 2;
    } else if (pairs < kMultiWavePairs) {
        const long long slots = valu ? kValuResidentWaves : resident;
        while (part < max_ctx && 3 * items(part) > 4 * slots) {
            part *= 2;
            grown = true;
        }
    }
    // small batches: cut finer until the items fill the machine (wide groups
    // settle for one round of resident waves)
    const long long min_waves = waves > 1 ? resident : kAutoMinItems;
    while (!grown && part > kAutoPartitionFloor && items(part) * waves < min_waves) part /= 2;
    return part;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool valid_dtype(int d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }

pa_status validate_shape(int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                         pa_dtype dtype, pa_dtype out_dtype) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0 || max_blocks < 0)
        return PA_ERR_SHAPE;
    if (Hq % Hkv != 0) return PA_ERR_SHAPE;
    if (S > 65535 || Hq > 65535) return PA_ERR_SHAPE;              // launch grid limits
    if ((long long)S * Hq > INT_MAX) return PA_ERR_SHAPE;
    if ((long long)max_blocks * B > INT_MAX) return PA_ERR_SHAPE;  // token index is int32
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return PA_ERR_UNSUPPORTED;
    if (out_dtype != dtype && out_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
    if (D > 512) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

bool supports_valu(int Hq, int Hkv, int D, int B, pa_dtype dt) {
    const int G = Hq / Hkv;
    return D == 128 && (dt == PA_F16 || dt == PA_BF16) && is_pow2(B) &&
           (G == 1 || G == 2 || G == 4 || G == 8);
}

bool supports_mfma(int Hq, int Hkv, int D, int B, pa_dtype dt) {
    const int G = Hq / Hkv;
    return D == 128 && (dt == PA_F16 || dt == PA_BF16) && is_pow2(B) &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64);
}

// Largest partition whose block-table slice fits the LDS copy (the tiled
// kernels stage the table when B % 4 != 0).
long long table_cap(int kernel, int B) {
    const bool staged = (kernel == PA_KERNEL_VALU || kernel == PA_KERNEL_MFMA) && B % 4 != 0;
    return staged ? (long long)pa::kTableLds * B : (long long)INT_MAX;
}

// Token-waves per item of the VALU kernel and of the matrix-core kernel's
// one-wave groups (at most 16 heads): each streams every TW-th 32-token tile
// of the partition, and their softmax states meet in LDS.  The VALU kernel's
// waves need blocks of at least 4 tokens; the matrix-core kernel's also run
// on the table slice staged in LDS for smaller blocks, though only when asked
// for (the automatic plan keeps those on one wave: their partitions are
// capped by the slice, and on 32k-token tables at one kv head per 8 query
// heads, one-token blocks took 244.2 / 251.1 / 259.0 us a cold step on 1 / 2
// / 4 waves, two-token blocks 227.8 / 252.8 / 227.3).
bool multi_wave_items(int kernel, int G, int B) {
    return kernel == PA_KERNEL_VALU ? B % 4 == 0 : kernel == PA_KERNEL_MFMA && G <= 16;
}

// Waves for a partition the planner made multi-wave: at most 1024 tokens
// each (a single-pass partition cut to the longest context can be shorter
// than the four-fold one).  Batch-64 MHA with every context 3000 tokens,
// one pass of 3008: cold step 518.9 / 519.1 us on two waves, 483.3 / 486.4
// on four.
int waves_for_length(long long part) { return part > 2048 ? 4 : part > 1024 ? 2 : 1; }

// Threads per work-group of a decode kernel family (the matrix-core kernel
// runs ceil(G / 16) head waves, times its token-waves).
int decode_threads(int kernel, int G, int tw) {
    if (kernel == PA_KERNEL_MFMA) return 64 * ((G + 15) / 16) * tw;
    if (kernel == PA_KERNEL_VALU) return 64 * tw;
    return 64;
}

// Grid of the tiled decode kernels: 1 = the 1-D live-item grid (every
// work-group decodes its item from the lengths one wave holds, pa_sched.h),
// 0 = the rectangular (sequence x kv head, partition) grid, -1 = neither
// fits the launch limits.
int decode_grid_mode(int S, int Hkv, int parts, int threads) {
    const long long pairs = (long long)S * Hkv;
    if (S <= pa::kSchedMaxSeqs && pa::grid_fits(pairs * parts, threads)) return 1;
    if (pa::grid_fits(pairs, threads) && parts <= pa::kMaxPartitions) return 0;
    return -1;
}

pa_status make_plan(int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                    pa_dtype dtype, pa_dtype out_dtype, const pa_config *cfg, pa_plan *plan) {
    pa_status st = validate_shape(S, Hq, Hkv, D, B, NB, max_blocks, dtype, out_dtype);
    if (st != PA_OK) return st;
    int kernel = cfg ? cfg->kernel : PA_KERNEL_AUTO;
    const int req = cfg ? cfg->partition_tokens : 0;
    if (req < 0 || (req > 0 && req % pa::kTileTokens != 0)) return PA_ERR_SHAPE;
    if (cfg && (cfg->stages < 0 || cfg->stages > PA_STAGE_ALL)) return PA_ERR_SHAPE;
    const int req_tw = cfg ? cfg->token_waves : 0;
    if (req_tw != 0 && req_tw != 1 && req_tw != 2 && req_tw != 4) return PA_ERR_SHAPE;

    switch (kernel) {
    case PA_KERNEL_AUTO:
        // Groups of 4+ heads go to the matrix cores.  Groups of 1 or 2 stay on
        // the VALU kernel: padded to 16 columns, the matrix-core kernel reads
        // the same bytes no faster (mha_7b: 359 vs 355 us median).
        kernel = Hq / Hkv >= 4 && supports_mfma(Hq, Hkv, D, B, dtype) ? PA_KERNEL_MFMA
                 : supports_valu(Hq, Hkv, D, B, dtype) ? PA_KERNEL_VALU
                                                       : PA_KERNEL_GENERIC;
        break;
    case PA_KERNEL_GENERIC:
        break;
    case PA_KERNEL_VALU:
        if (!supports_valu(Hq, Hkv, D, B, dtype)) return PA_ERR_UNSUPPORTED;
        break;
    case PA_KERNEL_MFMA:
        if (!supports_mfma(Hq, Hkv, D, B, dtype)) return PA_ERR_UNSUPPORTED;
        break;
    default:
        return PA_ERR_UNSUPPORTED;
    }

    const int G = Hq / Hkv;
    if (req_tw > 1 && !multi_wave_items(kernel, G, B)) return PA_ERR_UNSUPPORTED;
    const long long max_ctx = (long long)max_blocks * B;
    pa_plan p{};
    bool multi = false;   // the planner chose multi-wave items
    if (kernel != PA_KERNEL_GENERIC) {
        const long long cap = table_cap(kernel, B);
        const int waves = kernel == PA_KERNEL_MFMA ? (Hq / Hkv + 15) / 16 : 1;
        long long part = req > 0 ? req : auto_partition(S, Hkv, max_ctx, waves, kernel == PA_KERNEL_VALU);
        // Token-waves: with at least kMultiWavePairs (sequence, kv head)
        // pairs, a full one-wave partition (not one halved for a small
        // batch) becomes four waves on a partition four times as long, each
        // wave streaming as many tokens as before, with a quarter of the
        // partial results (none when that covers the context).  Cold step
        // µs, one wave -> four, VALU kernel: batch-64 MHA (2048 pairs) 358.7
        // -> 347.0, at two heads per kv head 373.4 -> 352.4, 256 sequences
        // 1519 -> 1450, 32 sequences 192.2 -> 186.7; matrix-core kernel: 64
        // sequences of 16k-32k tokens at 4 heads per kv head (512 pairs) 984
        // -> 892, 64 sequences at 8 heads per kv head (2048 pairs) 406 -> 366,
        // gqa_70b (1024 pairs) 188.1 -> 189.2.  Fewer pairs make too few,
        // too long items to balance: 32 gqa_70b sequences (256 pairs) 68.7
        // -> 78.7, and 16 long contexts sharing a 4096-token prefix (128
        // pairs) 226.3 -> 232.8.  A partition halved for a small batch stays
        // on one wave (8 sequences of up to 2048 tokens: 27.3 against
        // 29.4-31.8 on four).
        if (req == 0 && multi_wave_items(kernel, G, B) && B % 4 == 0 && (long long)S * Hkv >= kMultiWavePairs) {
            if (part >= kAutoPartitionMin && part < max_ctx) {
                part *= 4;
                multi = true;
            } else if (part < kAutoPartitionMin && max_ctx > kAutoSinglePass) {
                // halved for a short-context batch: rather one pass (or 4096-token
                // partitions) on up to four waves, when those still fill a
                // round of resident waves.  128 sequences at 8 heads per kv
                // head, every context 1500 tokens: cold step 163.7 / 164.1 us on
                // 256-token one-wave items, 133.3 / 131.8 in one pass on two
                // waves; every context 3000: 300.1 / 300.5 on 512-token items,
                // 256.2 / 255.9 in one pass on four.
                const long long tw_part = std::min(4 * kAutoPartitionMin, max_ctx);
                const long long tw_waves = (long long)S * Hkv * ((max_ctx + tw_part - 1) / tw_part) *
                                           waves_for_length(tw_part);
                const long long slots =
                    kernel == PA_KERNEL_VALU ? kValuResidentWaves : resident_waves(1);
                if (tw_waves >= slots) {
                    part = tw_part;
                    multi = true;
                }
            }
        }
        if (part >= max_ctx) {   // single pass: one partition covers any context
            part = ((max_ctx > 0 ? max_ctx : 1) + pa::kTileTokens - 1) / pa::kTileTokens * pa::kTileTokens;
        }
        // the partition index is a grid dimension (at most kMaxPartitions)
        const long long min_part = (max_ctx + pa::kMaxPartitions - 1) / pa::kMaxPartitions;
        if (part < min_part) part = (min_part + pa::kTileTokens - 1) / pa::kTileTokens * pa::kTileTokens;
        if (part > cap) part = cap / pa::kTileTokens * pa::kTileTokens;
        if (part > INT_MAX) part = INT_MAX / pa::kTileTokens * pa::kTileTokens;
        const long long parts = max_ctx > 0 ? (max_ctx + part - 1) / part : 1;
        if (parts <= pa::kMaxPartitions) {
            p.kernel = kernel;
            p.partition_tokens = (int)part;
            p.max_partitions = (int)parts;
            p.split = parts > 1 ? 1 : 0;
        } else if (cfg && cfg->kernel != PA_KERNEL_AUTO) {
            return PA_ERR_UNSUPPORTED;   // context too long for this kernel's table staging
        } else {
            kernel = PA_KERNEL_GENERIC;
        }
    }
    if (kernel == PA_KERNEL_GENERIC) {
        // one pass over the whole context; no workspace.  Grid (Hq, S) of
        // 64-thread work-groups: within the limits for every valid shape.
        if (req_tw > 1) return PA_ERR_UNSUPPORTED;   // an automatic kernel fell back
        p.kernel = kernel;
        p.partition_tokens = (int)(max_ctx > 0 ? max_ctx : 1);
        p.max_partitions = 1;
        p.split = 0;
        p.token_waves = 1;
    } else {
        p.token_waves = req_tw > 0 ? req_tw : multi ? waves_for_length(p.partition_tokens) : 1;
        if (decode_grid_mode(S, Hkv, p.max_partitions, decode_threads(kernel, G, p.token_waves)) < 0)
            return PA_ERR_SHAPE;
    }
    if (p.split) {
        const size_t rows = (size_t)S * Hq * p.max_partitions;
        p.workspace_bytes = align256(rows * D * sizeof(float)) + 2 * align256(rows * sizeof(float));
    }
    *plan = p;
    return PA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Checked mode: the config's explicit choice, else PA_CHECK=1 in the
// environment (read at every call, so a process can switch it at run time).
bool check_enabled(const pa_config *cfg) {
    if (cfg && cfg->check > 0) return true;
    if (cfg && cfg->check < 0) return false;
    const char *env = std::getenv("PA_CHECK");
    return env && std::strcmp(env, "1") == 0;
}

// ---------------------------------------------------------------- multi-token

bool supports_prefill_mfma(int Hq, int Hkv, int D, int B, pa_dtype dt) {
    const int G = Hq / Hkv;
    return D == 128 && (dt == PA_F16 || dt == PA_BF16) && is_pow2(B) &&
           (G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64);
}

// Work-groups below which the automatic plan splits contexts: the grid then
// holds fewer than one round of four-wave groups (two per CU).
constexpr long long kPrefillMinGroups = 512;

// Columns per work-group of the multi-token kernel (32 per wave): 64 when
// every sequence's rows fit them, so a 128-column block would be at least
// half empty for every sequence; 256 when the longest chunk fills a
// 256-column block, so each staged sub-tile serves twice the columns (half
// the K / V re-reads of a sequence's query blocks); else 128.  Measured,
// cold µs at 128 / 256 columns: 512 new tokens on the 16-sequence batch at 4
// heads per kv head 1227 / 1169, at 8 heads 2157 / 1970, at 1 head 334 /
// 330; 256 new tokens at 1 head (mha_7b batch) 995 / 919; at G x chunk =
// 256 a tie (192 / 193).
int prefill_columns(int G, int max_query_len) {
    const long long rows = (long long)G * max_query_len;
    if (rows <= pa::kPrefillColumnsNarrow) return pa::kPrefillColumnsNarrow;
    if (rows >= pa::kPrefillColumnsWide) return pa::kPrefillColumnsWide;
    return pa::kPrefillColumns;
}

pa_status make_prefill_plan(int S, int T, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                            int max_query_len, pa_dtype dtype, pa_dtype out_dtype,
                            const pa_config *cfg, pa_plan *plan, int *q_blocks) {
    pa_status st = validate_shape(S, Hq, Hkv, D, B, NB, max_blocks, dtype, out_dtype);
    if (st != PA_OK) return st;
    if (T < 0 || max_query_len < 0 || T > 65535) return PA_ERR_SHAPE;   // rows are grid y
    if (T > 0 && S > 0 && max_query_len == 0) return PA_ERR_SHAPE;
    if ((long long)T * Hq > INT_MAX) return PA_ERR_SHAPE;
    int kernel = cfg ? cfg->kernel : PA_KERNEL_AUTO;
    const int req = cfg ? cfg->partition_tokens : 0;
    if (req < 0 || (req > 0 && req % pa::kTileTokens != 0)) return PA_ERR_SHAPE;
    if (cfg && (cfg->stages < 0 || cfg->stages > PA_STAGE_ALL)) return PA_ERR_SHAPE;
    if (cfg && cfg->token_waves != 0 && cfg->token_waves != 1) return PA_ERR_UNSUPPORTED;
    switch (kernel) {
    case PA_KERNEL_AUTO:
        kernel = supports_prefill_mfma(Hq, Hkv, D, B, dtype) ? PA_KERNEL_MFMA : PA_KERNEL_GENERIC;
        break;
    case PA_KERNEL_GENERIC:
        break;
    case PA_KERNEL_MFMA:
        if (!supports_prefill_mfma(Hq, Hkv, D, B, dtype)) return PA_ERR_UNSUPPORTED;
        break;
    default:
        return PA_ERR_UNSUPPORTED;
    }
    const long long max_ctx = (long long)max_blocks * B;
    pa_plan p{};
    p.token_waves = 1;
    *q_blocks = 0;
    if (kernel == PA_KERNEL_MFMA) {
        const int cols = prefill_columns(Hq / Hkv, max_query_len);
        const int qpb = cols / (Hq / Hkv);
        const long long qb = (max_query_len + qpb - 1) / qpb;
        const long long groups = qb * S * Hkv;
        // grid x: the (sequence, kv head) pairs padded to whole XCD rounds,
        // times the query blocks, of 64 threads per 32 columns
        const long long grid_x = ((long long)S * Hkv + 7) / 8 * 8 * qb;
        if (!pa::grid_fits(grid_x, 2 * cols)) return PA_ERR_SHAPE;
        // one round of resident work-groups: kPrefillMinGroups four-wave ones
        const long long min_groups = kPrefillMinGroups * pa::kPrefillColumns / cols;
        long long part;
        if (req > 0) {
            part = req;
        } else if (groups >= min_groups || max_ctx <= 256) {
            part = max_ctx;                                        // one pass
        } else {
            const long long want = (min_groups + groups - 1) / (groups > 0 ? groups : 1);
            part = (max_ctx + want - 1) / want;
            part = (part + 127) / 128 * 128;
            if (part < 256) part = 256;
        }
        if (part >= max_ctx) part = ((max_ctx > 0 ? max_ctx : 1) + 31) / 32 * 32;
        const long long min_part = (max_ctx + pa::kMaxPartitions - 1) / pa::kMaxPartitions;
        if (part < min_part) part = (min_part + 31) / 32 * 32;
        const long long cap = B % 4 != 0 ? (long long)pa::kTableLds * B : (long long)INT_MAX;
        if (part > cap) part = cap / 32 * 32;
        if (part > INT_MAX) part = INT_MAX / 32 * 32;
        const long long parts = max_ctx > 0 ? (max_ctx + part - 1) / part : 1;
        if (parts > pa::kMaxPartitions) return PA_ERR_UNSUPPORTED;
        p.kernel = kernel;
        p.partition_tokens = (int)part;
        p.max_partitions = (int)parts;
        p.split = parts > 1 ? 1 : 0;
        *q_blocks = (int)qb;
    } else {
        p.kernel = PA_KERNEL_GENERIC;
        p.partition_tokens = (int)(max_ctx > 0 ? max_ctx : 1);
        p.max_partitions = 1;
        p.split = 0;
    }
    if (p.split) {
        const size_t rows = (size_t)T * Hq * p.max_partitions;
        p.workspace_bytes = align256(rows * D * sizeof(float)) + 2 * align256(rows * sizeof(float));
    }
    *plan = p;
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_plan(int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                         pa_dtype dtype, pa_dtype out_dtype, const pa_config *cfg,
                         pa_plan *plan) {
    if (!plan) return PA_ERR_NULL;
    return make_plan(S, Hq, Hkv, D, B, NB, max_blocks, dtype, out_dtype, cfg, plan);
}

size_t pa_decode_workspace_bytes(int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                                 pa_dtype dtype, pa_dtype out_dtype) {
    pa_plan p;
    if (make_plan(S, Hq, Hkv, D, B, NB, max_blocks, dtype, out_dtype, nullptr, &p) != PA_OK)
        return 0;
    return p.workspace_bytes;
}

pa_status pa_decode_ex(const void *query, const void *key_cache, const void *value_cache,
                       const int32_t *block_tables, const int32_t *seq_lens, float scale,
                       void *out, int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                       pa_dtype dtype, pa_dtype out_dtype, const pa_config *cfg,
                       void *workspace, size_t workspace_bytes, void *stream) {
    pa_plan plan;
    pa_status st = make_plan(S, Hq, Hkv, D, B, NB, max_blocks, dtype, out_dtype, cfg, &plan);
    if (st != PA_OK) return st;
    if (S == 0) return PA_OK;
    if (!query || !key_cache || !value_cache || !block_tables || !seq_lens || !out)
        return PA_ERR_NULL;

    if (plan.kernel != PA_KERNEL_GENERIC &&
        !(aligned16(query) && aligned16(key_cache) && aligned16(value_cache) && aligned16(out))) {
        if (cfg && cfg->kernel != PA_KERNEL_AUTO) return PA_ERR_UNSUPPORTED;
        pa_config gen{PA_KERNEL_GENERIC, 0, cfg ? cfg->stages : 0, 0, cfg ? cfg->check : 0};
        st = make_plan(S, Hq, Hkv, D, B, NB, max_blocks, dtype, out_dtype, &gen, &plan);
        if (st != PA_OK) return st;
    }
    const int stages = (cfg && cfg->stages) ? cfg->stages : PA_STAGE_ALL;
    if (plan.split && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
                       workspace_bytes < plan.workspace_bytes))
        return PA_ERR_WORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (check_enabled(cfg)) {
        int bad = 0;
        if (pa::library_check(block_tables, seq_lens, nullptr, S, 0, 0, max_blocks, B, NB, hs,
                              &bad) != hipSuccess)
            return PA_ERR_HIP;
        if (bad) return PA_ERR_DEVICE_CHECK;
    }

    Args a;
    std::memset(&a, 0, sizeof a);
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.out = out;
    a.scale_log2 = scale * 1.4426950408889634f;   // log2(e): exp(x) = 2^(x log2 e)
    a.S = S;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.B = B;
    a.NB = NB;
    a.max_blocks = max_blocks;
    a.log2B = is_pow2(B) ? ilog2(B) : -1;
    a.part_tokens = plan.partition_tokens;
    a.max_parts = plan.max_partitions;
    a.split = plan.split;
    a.stream_kv = (cfg && cfg->kv_reuse) ? 0 : 1;
    // live-item grid when every work-group can decode its item from the
    // lengths held in one wave's registers and the 1-D grid fits (the plan
    // has checked that one of the two grids fits)
    a.token_waves = plan.token_waves;
    a.compact = plan.kernel != PA_KERNEL_GENERIC &&
                decode_grid_mode(S, Hkv, plan.max_partitions,
                                 decode_threads(plan.kernel, Hq / Hkv, plan.token_waves)) == 1;
    if (plan.split) {
        const size_t rows = (size_t)S * Hq * plan.max_partitions;
        char *ws = static_cast<char *>(workspace);
        a.part_o = reinterpret_cast<float *>(ws);
        a.part_m = reinterpret_cast<float *>(ws + align256(rows * D * sizeof(float)));
        a.part_l = reinterpret_cast<float *>(ws + align256(rows * D * sizeof(float)) +
                                             align256(rows * sizeof(float)));
    }

    hipError_t err = hipSuccess;
    if (stages & PA_STAGE_PARTITIONS) {
        switch (plan.kernel) {
        case PA_KERNEL_GENERIC: err = pa::launch_generic(a, dtype, out_dtype, hs); break;
        case PA_KERNEL_VALU: err = pa::launch_valu(a, dtype, out_dtype, hs); break;
        case PA_KERNEL_MFMA: err = pa::launch_mfma(a, dtype, out_dtype, hs); break;
        default: return PA_ERR_UNSUPPORTED;
        }
        if (err != hipSuccess) return PA_ERR_HIP;
    }
    if (plan.split && (stages & PA_STAGE_COMBINE)) {
        err = pa::launch_combine(a, out_dtype, hs);
        if (err != hipSuccess) return PA_ERR_HIP;
    }
    return PA_OK;
}

pa_status pa_prefill_plan(int S, int T, int Hq, int Hkv, int D, int B, int NB, int max_blocks,
                          int max_query_len, pa_dtype dtype, pa_dtype out_dtype,
                          const pa_config *cfg, pa_plan *plan) {
    if (!plan) return PA_ERR_NULL;
    int qb;
    return make_prefill_plan(S, T, Hq, Hkv, D, B, NB, max_blocks, max_query_len, dtype, out_dtype,
                             cfg, plan, &qb);
}

pa_status pa_prefill(const void *query, const void *key_cache, const void *value_cache,
                     const int32_t *block_tables, const int32_t *seq_lens,
                     const int32_t *query_start, float scale, void *out, int S, int T, int Hq,
                     int Hkv, int D, int B, int NB, int max_blocks, int max_query_len,
                     pa_dtype dtype, pa_dtype out_dtype, const pa_config *cfg, void *workspace,
                     size_t workspace_bytes, void *stream) {
    pa_plan plan;
    int qb = 0;
    pa_status st = make_prefill_plan(S, T, Hq, Hkv, D, B, NB, max_blocks, max_query_len, dtype,
                                     out_dtype, cfg, &plan, &qb);
    if (st != PA_OK) return st;
    if (S == 0 || T == 0) return PA_OK;
    if (!query || !key_cache || !value_cache || !block_tables || !seq_lens || !query_start || !out)
        return PA_ERR_NULL;
    if (plan.kernel != PA_KERNEL_GENERIC &&
        !(aligned16(query) && aligned16(key_cache) && aligned16(value_cache) && aligned16(out))) {
        if (cfg && cfg->kernel != PA_KERNEL_AUTO) return PA_ERR_UNSUPPORTED;
        pa_config gen{PA_KERNEL_GENERIC, 0, cfg ? cfg->stages : 0, 0, cfg ? cfg->check : 0};
        st = make_prefill_plan(S, T, Hq, Hkv, D, B, NB, max_blocks, max_query_len, dtype, out_dtype,
                               &gen, &plan, &qb);
        if (st != PA_OK) return st;
    }
    const int stages = (cfg && cfg->stages) ? cfg->stages : PA_STAGE_ALL;
    if (plan.split && (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
                       workspace_bytes < plan.workspace_bytes))
        return PA_ERR_WORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (check_enabled(cfg)) {
        int bad = 0;
        if (pa::library_check(block_tables, seq_lens, query_start, S, T, max_query_len, max_blocks,
                              B, NB, hs, &bad) != hipSuccess)
            return PA_ERR_HIP;
        if (bad) return PA_ERR_DEVICE_CHECK;
    }

    Args a;
    std::memset(&a, 0, sizeof a);
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.out = out;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.S = S;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.B = B;
    a.NB = NB;
    a.max_blocks = max_blocks;
    a.log2B = is_pow2(B) ? ilog2(B) : -1;
    a.part_tokens = plan.partition_tokens;
    a.max_parts = plan.max_partitions;
    a.split = plan.split;
    a.stream_kv = (cfg && cfg->kv_reuse) ? 0 : 1;
    a.query_start = query_start;
    a.T = T;
    a.q_blocks = qb;
    a.prefill_columns = prefill_columns(Hq / Hkv, max_query_len);
    // Longest contexts first when the work-groups take more than one round
    // of the resident ones (two waves per SIMD: 8 / waves per work-group on
    // each of 256 CUs); in one round every work-group starts at once and the
    // order only delays each start by the length lookup.  Chunked-prefill
    // batch (16 sequences of 1024-8192 tokens, the last 512 new, four rounds):
    // 611 -> 628-636 TFLOP/s per step, 650-654 -> 686-694 at 8 heads per kv
    // head; 4 new tokens per sequence (one round): 71 -> 78 us if ordered.
    {
        const long long wgs = ((long long)S * Hkv + 7) / 8 * 8 * qb * plan.max_partitions;
        const long long resident = 256LL * (8 / (2 * a.prefill_columns / 64));
        a.by_length = plan.kernel == PA_KERNEL_MFMA && S <= pa::kSchedMaxSeqs && wgs > resident;
    }
    if (plan.split) {
        const size_t rows = (size_t)T * Hq * plan.max_partitions;
        char *ws = static_cast<char *>(workspace);
        a.part_o = reinterpret_cast<float *>(ws);
        a.part_m = reinterpret_cast<float *>(ws + align256(rows * D * sizeof(float)));
        a.part_l = reinterpret_cast<float *>(ws + align256(rows * D * sizeof(float)) +
                                             align256(rows * sizeof(float)));
    }
    hipError_t err = hipSuccess;
    if (stages & PA_STAGE_PARTITIONS) {
        err = plan.kernel == PA_KERNEL_MFMA ? pa::launch_prefill(a, dtype, out_dtype, hs)
                                            : pa::launch_generic(a, dtype, out_dtype, hs);
        if (err != hipSuccess) return PA_ERR_HIP;
    }
    if (plan.split && (stages & PA_STAGE_COMBINE)) {
        err = pa::launch_combine(a, out_dtype, hs);
        if (err != hipSuccess) return PA_ERR_HIP;
    }
    return PA_OK;
}

pa_status pa_decode(const void *query, const void *key_cache, const void *value_cache,
                    const int32_t *block_tables, const int32_t *seq_lens, float scale, void *out,
                    int S, int Hq, int Hkv, int D, int B, int NB, int max_blocks, pa_dtype dtype,
                    pa_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return pa_decode_ex(query, key_cache, value_cache, block_tables, seq_lens, scale, out, S, Hq,
                        Hkv, D, B, NB, max_blocks, dtype, out_dtype, nullptr, workspace,
                        workspace_bytes, stream);
}

pa_status pa_decode_noalloc(const void *query, const void *key_cache, const void *value_cache,
                            const int32_t *block_tables, const int32_t *seq_lens, float scale,
                            void *out, int S, int Hq, int Hkv, int D, int B, int NB,
                            int max_blocks, pa_dtype dtype, pa_dtype out_dtype,
                            const pa_config *cfg, void *stream) {
    pa_plan plan;
    pa_status st = make_plan(S, Hq, Hkv, D, B, NB, max_blocks, dtype, out_dtype, cfg, &plan);
    if (st != PA_OK) return st;
    if (plan.workspace_bytes > pa::kNoAllocScratchBytes) return PA_ERR_SCRATCH;
    if (S == 0) return PA_OK;
    if (!query || !key_cache || !value_cache || !block_tables || !seq_lens || !out)
        return PA_ERR_NULL;
    void *ws = nullptr;
    if (plan.workspace_bytes &&
        pa::noalloc_scratch(static_cast<hipStream_t>(stream), &ws) != hipSuccess)
        return PA_ERR_HIP;
    return pa_decode_ex(query, key_cache, value_cache, block_tables, seq_lens, scale, out, S, Hq,
                        Hkv, D, B, NB, max_blocks, dtype, out_dtype, cfg, ws,
                        ws ? pa::kNoAllocScratchBytes : 0, stream);
}

static int dtype_size(pa_dtype d) { return d == PA_F32 ? 4 : 2; }

pa_status pa_write_kv(const void *key, const void *value, const int32_t *slot_mapping,
                      void *key_cache, void *value_cache, int T, int Hkv, int D, int B, int NB,
                      pa_dtype dtype, void *stream) {
    if (T < 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0) return PA_ERR_SHAPE;
    if (!pa::grid_fits(T, pa::kKvThreads)) return PA_ERR_SHAPE;            // grid x = token
    if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
    if (T == 0) return PA_OK;
    if (!key || !value || !slot_mapping || !key_cache || !value_cache) return PA_ERR_NULL;
    const hipError_t err = pa::launch_kv_write(key, value, slot_mapping, nullptr, nullptr,
                                               key_cache, value_cache, T, Hkv, D, B, NB, 0,
                                               dtype_size(dtype), static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_append_kv(const void *key, const void *value, const int32_t *block_tables,
                       const int32_t *seq_lens, void *key_cache, void *value_cache, int S,
                       int Hkv, int D, int B, int NB, int max_blocks, pa_dtype dtype,
                       void *stream) {
    if (S < 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0 || max_blocks < 0) return PA_ERR_SHAPE;
    if (!pa::grid_fits(S, pa::kKvThreads)) return PA_ERR_SHAPE;            // grid x = sequence
    if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
    if (S == 0) return PA_OK;
    if (!key || !value || !block_tables || !seq_lens || !key_cache || !value_cache)
        return PA_ERR_NULL;
    const hipError_t err = pa::launch_kv_write(key, value, nullptr, block_tables, seq_lens,
                                               key_cache, value_cache, S, Hkv, D, B, NB,
                                               max_blocks, dtype_size(dtype),
                                               static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs, int n,
                         int Hkv, int D, int B, int NB, pa_dtype dtype, void *stream) {
    if (n < 0 || Hkv <= 0 || D <= 0 || B <= 0 || NB <= 0) return PA_ERR_SHAPE;
    if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
    if (n == 0) return PA_OK;
    if (!key_cache || !value_cache || !pairs) return PA_ERR_NULL;
    const long long block_bytes = (long long)Hkv * B * D * dtype_size(dtype);
    // grid x = pieces of one block
    if (block_bytes > (1LL << 40) ||
        !pa::grid_fits((block_bytes + pa::kCopyPieceBytes - 1) / pa::kCopyPieceBytes, pa::kKvThreads))
        return PA_ERR_SHAPE;
    const hipError_t err = pa::launch_copy_blocks(key_cache, value_cache, pairs, n, block_bytes,
                                                  NB, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_check_inputs(const int32_t *block_tables, const int32_t *seq_lens, int S,
                          int max_blocks, int B, int NB, int32_t *report, void *stream) {
    if (S < 0 || max_blocks < 0 || B <= 0 || NB <= 0) return PA_ERR_SHAPE;
    if (!report) return PA_ERR_NULL;
    if (S > 0 && (!seq_lens || (max_blocks > 0 && !block_tables))) return PA_ERR_NULL;
    const hipError_t err = pa::launch_check(block_tables, seq_lens, S, max_blocks, B, NB, report,
                                            static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_get_device_error(void *stream, int32_t *first_bad) {
    int set = 0, first = -1;
    if (pa::read_device_error(static_cast<hipStream_t>(stream), &set, &first) != hipSuccess) {
        if (first_bad) *first_bad = -1;
        return PA_ERR_HIP;
    }
    if (first_bad) *first_bad = first;
    return set ? PA_ERR_DEVICE_CHECK : PA_OK;
}

pa_status pa_read_bytes(const void *buf, size_t bytes, uint32_t *sink, void *stream) {
    if (bytes == 0) return PA_OK;
    if (!buf || !sink) return PA_ERR_NULL;
    if (bytes % 16 != 0 || !aligned16(buf)) return PA_ERR_SHAPE;
    const hipError_t err = pa::launch_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

const char *pa_status_string(pa_status status) {
    switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid sizes";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape, type or kernel not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime reported an error";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: the block pool has too few free blocks";
    case PA_ERR_BAD_ID: return "PA_ERR_BAD_ID: unknown or released sequence or block id";
    case PA_ERR_SCRATCH:
        return "PA_ERR_SCRATCH: the plan's partial results exceed the static scratch of "
               "pa_decode_noalloc (PA_NOALLOC_SCRATCH_BYTES); use longer partitions";
    case PA_ERR_DEVICE_CHECK:
        return "PA_ERR_DEVICE_CHECK: a sequence length or used block-table entry breaks the "
               "preconditions (checked mode); nothing was launched";
    }
    return "unknown pa_status";
}

}  // extern "C"
