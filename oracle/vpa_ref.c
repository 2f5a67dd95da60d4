/*
 * vpa_ref.c -- CPU oracle for the vocab-parallel greedy argmax and greedy
 * verification.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load this library; the
 * product path never does.  It shares no source with the HIP library.
 *
 * Everything here is the plain definition, written for a reader to check by
 * eye: one thread, scalar loops, values compared as C doubles (every fp32 and
 * bf16 value converts to double exactly, so the order is the exact IEEE order
 * with no flush of subnormals).
 *
 * Sources (pages of the vLLM project, cited by title and section):
 *  [P1] PR #34049 "[Spec Decode] Reduce TP communication for speculative
 *       decoding draft token generation", section "Solution": every TP rank
 *       takes the argmax of its own vocabulary shard, only (max value, global
 *       index) pairs travel, and a final reduction over ranks gives the
 *       global argmax.
 *  [P4] PR #62604 (sharded greedy verification), section "Purpose":
 *       item 1 -- each rank reduces its shard to per-block (max, token id)
 *       statistics whose block boundaries are the global ones of the full
 *       vocabulary (8192 columns for draft positions, 1024 for the bonus
 *       position) even where a block crosses a shard edge, so ties come out
 *       as on the full logits; the gathered statistics give the global
 *       argmax, the accepted tokens, the bonus token and the sampled and
 *       rejected counts; vocabulary below 2^24.
 *       item 2 -- the fused get_top_tokens masks the vocabulary padding and
 *       returns the same token as torch.argmax: on ties the lowest id, and a
 *       NaN beats every number.
 *       section "Test Plan" -- shard statistics are concatenated in rank
 *       order, as a dim-0 all-gather lays them out; placeholder drafts;
 *       unaligned padding; NaN rows stay inside the vocabulary.
 *
 * Readings where the pages leave a step open:
 *  - among several NaNs the lowest id wins (first occurrence, as
 *    torch.argmax);
 *  - -0 and +0 compare equal, so the lower id wins;
 *  - the reported value is the raw fp32 bit pattern of the winning element
 *    (bf16 is widened by appending 16 zero bits), NaN payload and zero sign
 *    kept;
 *  - shards are contiguous, equal-width slices of the padded vocabulary in
 *    rank order; block b covers global columns [b*B, (b+1)*B);
 *  - each shard owns M slots, M being the largest number of blocks any shard
 *    touches; slot j of shard s is block floor(s*W/B)+j cut to the shard and
 *    to the valid vocabulary; an empty slot holds the sentinel
 *    (-inf bits, id INT32_MAX);
 *  - greedy verification accepts the longest prefix of drafts equal to the
 *    target argmax; the next position emits the target argmax (correction or
 *    bonus token); later positions hold -1; sampled = accepted + 1 and
 *    rejected = K - accepted.
 *  - ragged verification: request r carries K_r >= 0 drafts given by
 *    cumulative offsets cu[0..R] (cu[0] = 0, K_r = cu[r+1] - cu[r]); its
 *    logits rows are cu[r]+r .. cu[r]+r+K_r (drafts, then the bonus
 *    position) and its K_r+1 outputs sit at the same offsets; the greedy
 *    rule is the uniform one with K = K_r (K_r = 0 emits the bonus token).
 *  - prefilling requests ([P4] "Test Plan" lists them among the verified
 *    cases but states no rule; the reading taken here): a request flagged as
 *    still prefilling samples nothing, so all K_r+1 of its output slots
 *    hold -1 and sampled = rejected = 0; its target tokens are still
 *    reported.
 *  - synthetic acceptance ([P4] "Purpose" item 1 names it beside the real
 *    acceptance, and "Test Plan" lists it among the verified cases, with no
 *    rule; the reading taken here): the caller may give each request an
 *    accept count a_r.  With a_r >= 0 the first min(a_r, K_r) drafts are
 *    accepted whatever their values (random draws behind a_r are the
 *    caller's); the next position emits its target token as usual; a_r < 0,
 *    or no counts at all, means the real greedy rule.  A prefilling request
 *    still samples nothing.
 *  - optional epilogue of the combined argmax k:
 *    [P2] PR #39419 "[SpecDecode] Reduce TP communication for large-vocab
 *    draft models speculative decoding", note "Refactor local argmax code":
 *    the local argmax is taken first and the draft id then maps to a target
 *    id as k + d2t[k];
 *    [P1] review: a negative logit scale would turn the argmax into an
 *    argmin, so only a positive scale is accepted; it leaves the argmax
 *    unchanged and the reported maximum becomes fp32(value) * scale rounded
 *    to nearest (a NaN is reported unchanged).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define REF_F32 0
#define REF_BF16 1

typedef struct {
    uint32_t val_bits;
    int32_t id;
} ref_stat;

/* fp32 bit pattern of logits element (row, col) of a row-major matrix with
 * row stride ld elements.  bf16 widens to fp32 by appending 16 zero bits. */
static uint32_t ref_bits(const void *x, int dtype, int64_t ld, int64_t row, int64_t col)
{
    int64_t off = row * ld + col;
    if (dtype == REF_BF16) {
        uint16_t h;
        memcpy(&h, (const char *)x + 2 * off, 2);
        return (uint32_t)h << 16;
    }
    uint32_t w;
    memcpy(&w, (const char *)x + 4 * off, 4);
    return w;
}

static double ref_value(uint32_t bits)
{
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* The ordering of [P4] item 2: a NaN beats every number; between two
 * numbers the larger wins; equal numbers (including -0 == +0) and two NaNs
 * are decided by the lower id. */
static int ref_better(double a, int64_t ia, double b, int64_t ib)
{
    int a_nan = isnan(a), b_nan = isnan(b);
    if (a_nan && b_nan)
        return ia < ib;
    if (a_nan)
        return 1;
    if (b_nan)
        return 0;
    if (a > b)
        return 1;
    if (a == b)
        return ia < ib;
    return 0;
}

/* Number of statistic slots per shard: the most blocks that any of the S
 * shards [s*W, (s+1)*W) touches. */
int32_t vpa_ref_stats_slots(int64_t shard_width, int32_t n_shards, int32_t block)
{
    int64_t m = 0;
    for (int32_t s = 0; s < n_shards; ++s) {
        int64_t first = (s * shard_width) / block;
        int64_t last = (s * shard_width + shard_width - 1) / block;
        if (last - first + 1 > m)
            m = last - first + 1;
    }
    return (int32_t)m;
}

/* Full-row argmax over the valid columns [0, vocab) of each row ([P4] item 2;
 * the baseline of [P1] "Problem" that gathers the whole row first). */
void vpa_ref_argmax(const void *x, int dtype, int64_t ld, int64_t n_rows, int64_t vocab,
                    int32_t *ids, uint32_t *val_bits)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t best = 0;
        double best_v = ref_value(ref_bits(x, dtype, ld, r, 0));
        for (int64_t c = 1; c < vocab; ++c) {
            double v = ref_value(ref_bits(x, dtype, ld, r, c));
            if (ref_better(v, c, best_v, best)) {
                best = c;
                best_v = v;
            }
        }
        ids[r] = (int32_t)best;
        val_bits[r] = ref_bits(x, dtype, ld, r, best);
    }
}

/* Per-block statistics of the local shards [P4] item 1.  `x` holds the
 * columns of shards first_shard .. first_shard+n_local-1 side by side, so its
 * column 0 is global column first_shard*W.  `rows` (may be NULL for
 * 0..n_rows-1) selects which rows of x are reduced.  Output layout is
 * rank-major, [n_local][n_rows][M], as a dim-0 all-gather would produce
 * ([P4] "Test Plan"). */
void vpa_ref_block_stats(const void *x, int dtype, int64_t ld, int64_t vocab, int64_t shard_width,
                         int32_t n_shards, int32_t first_shard, int32_t n_local,
                         const int32_t *rows, int64_t n_rows, int32_t block, int32_t m,
                         ref_stat *stats)
{
    (void)n_shards;
    int64_t col0 = (int64_t)first_shard * shard_width;
    for (int32_t sl = 0; sl < n_local; ++sl) {
        int64_t s = first_shard + sl;
        int64_t shard_lo = s * shard_width, shard_hi = shard_lo + shard_width;
        for (int64_t i = 0; i < n_rows; ++i) {
            int64_t row = rows ? rows[i] : i;
            for (int32_t j = 0; j < m; ++j) {
                int64_t b = shard_lo / block + j;
                int64_t lo = b * block, hi = lo + block;
                if (lo < shard_lo)
                    lo = shard_lo;
                if (hi > shard_hi)
                    hi = shard_hi;
                if (hi > vocab)
                    hi = vocab;
                ref_stat st = {0xFF800000u, INT32_MAX};
                if (lo < hi) {
                    int64_t best = lo;
                    double best_v = ref_value(ref_bits(x, dtype, ld, row, lo - col0));
                    for (int64_t c = lo + 1; c < hi; ++c) {
                        double v = ref_value(ref_bits(x, dtype, ld, row, c - col0));
                        if (ref_better(v, c, best_v, best)) {
                            best = c;
                            best_v = v;
                        }
                    }
                    st.val_bits = ref_bits(x, dtype, ld, row, best - col0);
                    st.id = (int32_t)best;
                }
                stats[(sl * n_rows + i) * m + j] = st;
            }
        }
    }
}

/* Rank-order reduction of one row's gathered statistics ([P1] "Solution",
 * step 3): `stats` is [S][rows_total][M]; scan shard by shard, slot by slot,
 * keeping a statistic only when it is strictly better than the one held. */
static ref_stat ref_combine_row(const ref_stat *stats, int32_t n_shards, int64_t rows_total,
                                int64_t row, int32_t m)
{
    ref_stat best = stats[row * m];
    for (int32_t s = 0; s < n_shards; ++s)
        for (int32_t j = 0; j < m; ++j) {
            ref_stat st = stats[((int64_t)s * rows_total + row) * m + j];
            if (ref_better(ref_value(st.val_bits), st.id, ref_value(best.val_bits), best.id))
                best = st;
        }
    return best;
}

void vpa_ref_combine(const ref_stat *stats, int32_t n_shards, int64_t n_rows, int32_t m,
                     int32_t *ids, uint32_t *val_bits)
{
    for (int64_t i = 0; i < n_rows; ++i) {
        ref_stat best = ref_combine_row(stats, n_shards, n_rows, i, m);
        ids[i] = best.id;
        val_bits[i] = best.val_bits;
    }
}

/* Acceptance for one request ([P4] item 1) given the K+1 target tokens.
 * Real acceptance (synth < 0): the drafts are accepted while they equal the
 * target token.  Synthetic acceptance (synth >= 0): the first min(synth, K)
 * drafts are accepted whatever their values.  The position after the
 * accepted ones (the bonus position when all K are accepted) emits its
 * target token. */
static void ref_accept(const int32_t *draft, const int32_t *target, int32_t k, int32_t synth,
                       int32_t *out, int32_t *n_sampled, int32_t *n_rejected)
{
    int32_t n = 0;
    if (synth >= 0)
        n = synth < k ? synth : k;
    else
        while (n < k && draft[n] == target[n])
            ++n;
    for (int32_t j = 0; j <= k; ++j)
        out[j] = j < n ? draft[j] : (j == n ? target[j] : -1);
    *n_sampled = n + 1;
    *n_rejected = k - n;
}

/* A request still prefilling samples nothing: K+1 slots of -1, no sampled
 * and no rejected token. */
static void ref_prefilling(int32_t k, int32_t *out, int32_t *n_sampled, int32_t *n_rejected)
{
    for (int32_t j = 0; j <= k; ++j)
        out[j] = -1;
    *n_sampled = 0;
    *n_rejected = 0;
}

/* Synthetic accept count of request r: accept[r], or -1 (real acceptance)
 * when no counts are given. */
static int32_t ref_synth(const int32_t *accept, int64_t r)
{
    return accept ? accept[r] : -1;
}

/* Greedy verification from gathered statistics: draft stats
 * [S][R*K][m_draft] (row i = request i/K, position i%K) and bonus stats
 * [S][R][m_bonus].  accept (synthetic accept counts, [R]) and target_ids may
 * be NULL. */
void vpa_ref_greedy_verify(const ref_stat *draft_stats, int32_t m_draft, const ref_stat *bonus_stats,
                           int32_t m_bonus, int32_t n_shards, int64_t n_req, int32_t k,
                           const int32_t *draft_ids, const int32_t *accept, int32_t *out_tokens,
                           int32_t *num_sampled, int32_t *num_rejected, int32_t *target_ids)
{
    int32_t tgt[k + 1];
    for (int64_t r = 0; r < n_req; ++r) {
        for (int32_t j = 0; j < k; ++j)
            tgt[j] = ref_combine_row(draft_stats, n_shards, n_req * k, r * k + j, m_draft).id;
        tgt[k] = ref_combine_row(bonus_stats, n_shards, n_req, r, m_bonus).id;
        ref_accept(draft_ids + r * k, tgt, k, ref_synth(accept, r), out_tokens + r * (k + 1),
                   num_sampled + r, num_rejected + r);
        if (target_ids)
            for (int32_t j = 0; j <= k; ++j)
                target_ids[r * (k + 1) + j] = tgt[j];
    }
}

/* Greedy verification straight from the full logits: request r owns rows
 * r*(K+1) .. r*(K+1)+K (K draft positions, then the bonus position), and the
 * target token of each row is its full-row argmax. */
void vpa_ref_greedy_verify_logits(const void *x, int dtype, int64_t ld, int64_t vocab, int64_t n_req,
                                  int32_t k, const int32_t *draft_ids, const int32_t *accept,
                                  int32_t *out_tokens, int32_t *num_sampled, int32_t *num_rejected,
                                  int32_t *target_ids)
{
    int32_t tgt[k + 1];
    uint32_t vb;
    for (int64_t r = 0; r < n_req; ++r) {
        for (int32_t j = 0; j <= k; ++j) {
            const char *row = (const char *)x + (dtype == REF_BF16 ? 2 : 4) * (r * (k + 1) + j) * ld;
            vpa_ref_argmax(row, dtype, ld, 1, vocab, &tgt[j], &vb);
        }
        ref_accept(draft_ids + r * k, tgt, k, ref_synth(accept, r), out_tokens + r * (k + 1),
                   num_sampled + r, num_rejected + r);
        if (target_ids)
            for (int32_t j = 0; j <= k; ++j)
                target_ids[r * (k + 1) + j] = tgt[j];
    }
}

/* Draft-to-target id map ([P2] "Refactor local argmax code"): out[i] =
 * ids[i] + d2t[ids[i]]; an id outside [0, d2t_len) maps to -1. */
void vpa_ref_map_ids(const int32_t *ids, int64_t n, const int64_t *d2t, int64_t d2t_len,
                     int64_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (ids[i] >= 0 && ids[i] < d2t_len) ? (int64_t)ids[i] + d2t[ids[i]] : -1;
}

/* Reported maximum under a positive logit scale: the fp32 product of the
 * value and the scale, rounded to nearest even (the double product is exact,
 * its conversion to float is the one rounding); a NaN is reported as is. */
uint32_t vpa_ref_scale_bits(uint32_t bits, float scale)
{
    double v = ref_value(bits);
    if (isnan(v))
        return bits;
    float prod = (float)(v * (double)scale);
    uint32_t out;
    memcpy(&out, &prod, 4);
    return out;
}

/* Ragged greedy verification from full logits: request r owns rows
 * cu[r]+r .. cu[r]+r+K_r (K_r = cu[r+1]-cu[r] drafts, then the bonus row);
 * draft_ids holds the cu[R] drafts back to back; out_tokens and target_ids
 * hold K_r+1 entries per request at offset cu[r]+r.  prefilling (NULL = none)
 * flags the requests that are still prefilling; accept (NULL = none) holds
 * synthetic accept counts. */
void vpa_ref_greedy_verify_ragged(const void *x, int dtype, int64_t ld, int64_t vocab, int64_t n_req,
                                  const int32_t *cu, const int32_t *draft_ids,
                                  const uint8_t *prefilling, const int32_t *accept,
                                  int32_t *out_tokens, int32_t *num_sampled,
                                  int32_t *num_rejected, int32_t *target_ids)
{
    for (int64_t r = 0; r < n_req; ++r) {
        int32_t k = cu[r + 1] - cu[r];
        int64_t base = (int64_t)cu[r] + r;
        int32_t tgt[k + 1];
        uint32_t vb;
        for (int32_t j = 0; j <= k; ++j) {
            const char *row = (const char *)x + (dtype == REF_BF16 ? 2 : 4) * (base + j) * ld;
            vpa_ref_argmax(row, dtype, ld, 1, vocab, &tgt[j], &vb);
        }
        if (prefilling && prefilling[r])
            ref_prefilling(k, out_tokens + base, num_sampled + r, num_rejected + r);
        else
            ref_accept(draft_ids + cu[r], tgt, k, ref_synth(accept, r), out_tokens + base,
                       num_sampled + r, num_rejected + r);
        if (target_ids)
            for (int32_t j = 0; j <= k; ++j)
                target_ids[base + j] = tgt[j];
    }
}

/* Ragged greedy verification from gathered statistics: draft_stats
 * [S][cu[R]][m_draft] (row cu[r]+j is draft position j of request r),
 * bonus_stats [S][R][m_bonus]; outputs as vpa_ref_greedy_verify_ragged. */
void vpa_ref_greedy_verify_ragged_stats(const ref_stat *draft_stats, int32_t m_draft,
                                        const ref_stat *bonus_stats, int32_t m_bonus,
                                        int32_t n_shards, int64_t n_req, const int32_t *cu,
                                        const int32_t *draft_ids, const uint8_t *prefilling,
                                        const int32_t *accept, int32_t *out_tokens,
                                        int32_t *num_sampled, int32_t *num_rejected,
                                        int32_t *target_ids)
{
    int64_t total = cu[n_req];
    for (int64_t r = 0; r < n_req; ++r) {
        int32_t k = cu[r + 1] - cu[r];
        int64_t base = (int64_t)cu[r] + r;
        int32_t tgt[k + 1];
        for (int32_t j = 0; j < k; ++j)
            tgt[j] = ref_combine_row(draft_stats, n_shards, total, (int64_t)cu[r] + j, m_draft).id;
        tgt[k] = ref_combine_row(bonus_stats, n_shards, n_req, r, m_bonus).id;
        if (prefilling && prefilling[r])
            ref_prefilling(k, out_tokens + base, num_sampled + r, num_rejected + r);
        else
            ref_accept(draft_ids + cu[r], tgt, k, ref_synth(accept, r), out_tokens + base,
                       num_sampled + r, num_rejected + r);
        if (target_ids)
            for (int32_t j = 0; j <= k; ++j)
                target_ids[base + j] = tgt[j];
    }
}
