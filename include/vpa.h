/*
 * vpa.h -- C ABI of the vocab-parallel greedy argmax library for MI355X
 * (gfx950).
 *
 * The library computes, on one GPU, the hot path of greedy speculative
 * decoding with a vocabulary-sharded LM head, as the vLLM pages describe it:
 *
 *  - vLLM PR #34049 "[Spec Decode] Reduce TP communication for speculative
 *    decoding draft token generation", section "Solution": each tensor-
 *    parallel rank takes the argmax of its own vocabulary shard, the ranks
 *    exchange only (max value, global index) pairs, and a final reduction
 *    over the ranks yields the global argmax.
 *  - vLLM PR #62604 (sharded greedy verification and fused get_top_tokens),
 *    section "Purpose": item 1 -- every rank reduces its shard to per-block
 *    (max, token id) statistics with the global block boundaries of the full
 *    vocabulary (8192 columns for draft positions, 1024 for the bonus
 *    position), kept across shard edges; after the statistics are gathered,
 *    one step finishes the global argmax, the acceptance, the bonus token and
 *    the sampled/rejected counts; vocabularies below 2^24.  Item 2 -- the
 *    fused get_top_tokens masks the vocabulary padding and picks the same
 *    token as torch.argmax: the lowest id on ties, and NaN above every
 *    number.  Section "Test Plan" -- shard statistics are laid out in rank
 *    order, as a dim-0 all-gather produces them.
 *
 * Vocabulary shards here are logical: shard s of S holds global columns
 * [s*W, (s+1)*W) of the padded vocabulary (S*W >= V); columns [V, S*W) are
 * padding and are never read.  Statistics of all local shards are written in
 * rank order into one device buffer, the layout a dim-0 all-gather of the
 * per-rank statistics would produce, so a multi-GPU caller can gather them
 * with one collective and run the combining calls unchanged.
 *
 * Conventions shared by every call:
 *  - Pointers named logits, stats, ids, val_bits, mapped, d2t, draft_ids,
 *    accept, out_tokens, num_sampled, num_rejected, target_ids, rows,
 *    draft_rows, bonus_rows, cu, prefilling and workspace are DEVICE memory
 *    owned by the caller.  The library never allocates or frees.
 *  - Every call only enqueues work on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream) and returns without synchronising;
 *    outputs are defined once the stream reaches that point.
 *  - Arguments are validated on the host before any HIP call.  On
 *    VPA_ERR_INVALID or VPA_ERR_UNSUPPORTED nothing has been enqueued and
 *    vpa_last_error() describes the problem.  VPA_ERR_HIP reports a failed
 *    launch; launches of the same call that precede it may have been
 *    enqueued.
 *  - A call with zero rows (or zero requests) returns VPA_OK and enqueues
 *    nothing.
 *  - Logits are row-major: element (row, c) of the local columns sits at
 *    logits[row*ld + c], c counted from the first local shard.  The pointer
 *    must be aligned to the element size; rows may start at any such address.
 *  - Value bits are the fp32 bit pattern of the chosen element (a bf16
 *    pattern h widens to h<<16), NaN payload and the sign of zero kept.
 *  - Results are deterministic: the same inputs give bitwise identical
 *    outputs on every run, whatever the launch shape.
 *  - The library is greedy-only: the argmax is taken over the logits as
 *    given (a logit scale, which must be positive to keep the argmax, is
 *    the caller's; the optional epilogue scale below only rescales the
 *    reported maxima), and sampled requests are routed elsewhere.
 */
#ifndef VPA_H
#define VPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VPA_OK = 0,
    VPA_ERR_INVALID = 1,     /* bad size, geometry, alignment or null pointer */
    VPA_ERR_UNSUPPORTED = 2, /* a dtype the library does not handle */
    VPA_ERR_HIP = 3          /* the HIP runtime refused a launch */
} vpa_status;

typedef enum { VPA_F32 = 0, VPA_BF16 = 1 } vpa_dtype;

/* One (max, token id) statistic, 8 bytes.  An empty slot holds
 * {VPA_EMPTY_BITS, VPA_EMPTY_ID}: -inf with an id above every token, so it
 * loses to every real statistic, -inf included. */
typedef struct {
    uint32_t val_bits; /* fp32 bit pattern of the block's winning value */
    int32_t id;        /* global token id of the winner */
} vpa_stat;

#define VPA_EMPTY_BITS 0xFF800000u
#define VPA_EMPTY_ID 0x7FFFFFFF
#define VPA_MAX_VOCAB (1 << 24) /* the vocabulary must stay below this */
#define VPA_MAX_DRAFTS 4096     /* most draft tokens per request (K) */
#define VPA_MAX_SHARDS (1 << 24) /* most vocabulary shards (S) */

/* Vocabulary geometry: V valid columns, S shards of W columns each. */
typedef struct {
    int64_t vocab;       /* V, 1 <= V < 2^24 */
    int64_t shard_width; /* 1 <= W < 2^31 */
    int32_t n_shards;    /* 1 <= S <= VPA_MAX_SHARDS, S*W >= V (a shard may hold only padding) */
} vpa_vocab;

/* Optional epilogue of the combined argmax k of a row.
 *  d2t    draft-to-target offsets, device int64 [d2t_len], or NULL: the
 *         mapped id is k + d2t[k] (vLLM PR #39419, note "Refactor local argmax
 *         code": the local argmax comes first, the D2T map after it); an id
 *         outside [0, d2t_len) maps to -1.
 *  scale  logit scale, finite and > 0 (1.0 for none).  A positive scale
 *         keeps the argmax (vLLM PR #34049 review: a negative one would turn
 *         it into an argmin), so it only changes the reported maximum, which
 *         becomes the fp32 product value*scale, rounded to nearest even with
 *         subnormals kept; a NaN maximum is reported unchanged. */
typedef struct {
    const int64_t* d2t;
    int64_t d2t_len;
    float scale;
} vpa_epilogue;

/* Statistic slots per shard, M: the largest number of global blocks
 * [b*block, (b+1)*block) that any shard [s*W, (s+1)*W), s < S, touches
 * (PR #62604, "Purpose" item 1: global block boundaries across shard edges).
 * Slot j of shard s is block floor(s*W/block)+j cut to the shard and to
 * [0, V).  Returns -1 on invalid arguments (W < 1, S < 1, S > VPA_MAX_SHARDS,
 * block < 1) or when M would not fit an int32. */
int32_t vpa_stats_slots(int64_t shard_width, int32_t n_shards, int32_t block);

/* Per-block statistics of the local shards (PR #62604, "Purpose" item 1;
 * the per-rank step of PR #34049, "Solution").
 *  logits   [*, ld] of dtype `dtype`; column 0 is global column first_shard*W.
 *           Row stride ld must cover the valid local columns:
 *           ld >= min(n_local_shards*W, V - first_shard*W).
 *  first_shard, n_local_shards  the shard range this call reduces
 *           (0 <= first_shard, first_shard + n_local_shards <= S).  A rank of
 *           a multi-GPU job passes its own rank and 1; one GPU holding every
 *           shard passes 0 and S.
 *  rows     n_rows int32 row indices into logits, or NULL for 0..n_rows-1.
 *           An index outside [0, logits_rows) yields empty statistics for
 *           that row and reads nothing.
 *  logits_rows  number of rows the logits buffer holds: it bounds rows[],
 *           and with rows NULL it must be at least n_rows.
 *  block    global block size (>= 1).
 *  stats    out, [n_local_shards][n_rows][M] with M = vpa_stats_slots(W,S,block),
 *           8-byte aligned.  Slot i of shard s describes row rows[i]. */
vpa_status vpa_block_stats(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                           int32_t first_shard, int32_t n_local_shards, const int32_t* rows,
                           int64_t n_rows, int64_t logits_rows, int32_t block, vpa_stat* stats,
                           void* stream);

/* Both statistics of a greedy verification batch in one launch (PR #62604,
 * "Purpose" item 1: draft positions use 8192-column blocks, the bonus
 * position 1024-column blocks).  Request r owns logits rows
 * r*(K+1) .. r*(K+1)+K: K draft positions, then the bonus position; the
 * logits buffer must hold at least n_req*(K+1) rows.
 *  draft_stats  out, [n_local_shards][n_req*K][M_draft], row r*K+j is draft
 *               position j of request r; M_draft = vpa_stats_slots(W,S,block_draft).
 *  bonus_stats  out, [n_local_shards][n_req][M_bonus]; M_bonus likewise.
 * Other arguments as vpa_block_stats; 1 <= k <= VPA_MAX_DRAFTS. */
vpa_status vpa_verify_stats(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                            int32_t first_shard, int32_t n_local_shards, int64_t n_req, int32_t k,
                            int32_t block_draft, int32_t block_bonus, vpa_stat* draft_stats,
                            vpa_stat* bonus_stats, void* stream);

/* Statistics of a verification batch given by two row lists, in one launch:
 * draft rows with block_draft, bonus rows with block_bonus (PR #62604,
 * "Purpose" item 1).  Other arguments as vpa_block_stats; rows outside
 * [0, logits_rows) give empty statistics.
 *  draft_stats  out, [n_local_shards][n_draft_rows][M_draft]
 *  bonus_stats  out, [n_local_shards][n_bonus_rows][M_bonus] */
vpa_status vpa_verify_stats_rows(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                                 int32_t first_shard, int32_t n_local_shards,
                                 const int32_t* draft_rows, int64_t n_draft_rows,
                                 const int32_t* bonus_rows, int64_t n_bonus_rows,
                                 int64_t logits_rows, int32_t block_draft, int32_t block_bonus,
                                 vpa_stat* draft_stats, vpa_stat* bonus_stats, void* stream);

/* Row lists of a ragged verification batch (per-request draft counts).
 *  cu           device int32 [n_req+1], cumulative draft counts: cu[0] = 0,
 *               request r carries K_r = cu[r+1] - cu[r] drafts, cu[n_req] =
 *               total_drafts.  Request r owns logits rows cu[r]+r ..
 *               cu[r]+r+K_r: its K_r draft positions, then its bonus position.
 *  draft_rows   out, int32 [total_drafts]: draft position j of request r at
 *               index cu[r]+j holds row cu[r]+r+j.
 *  bonus_rows   out, int32 [n_req]: row cu[r+1]+r.
 * Offsets that break the rules above give unspecified rows (any row outside
 * the logits then yields empty statistics) but no access out of bounds. */
vpa_status vpa_ragged_rows(const int32_t* cu, int64_t n_req, int64_t total_drafts,
                           int32_t* draft_rows, int32_t* bonus_rows, void* stream);

/* Rank-order combination of gathered statistics into the global argmax
 * (PR #34049, "Solution", step 3).
 *  stats    [n_shards][n_rows][m], e.g. the concatenation of every rank's
 *           vpa_block_stats output (n_shards = S, all shards present).
 *  epi      host pointer to an epilogue, or NULL for none.
 *  ids      out, int32 [n_rows]: the global argmax of each row.
 *  val_bits out, uint32 [n_rows], or NULL: the fp32 bits of the maximum
 *           (scaled by epi->scale).
 *  mapped   out, int64 [n_rows]: k + d2t[k]; required iff epi->d2t is set. */
vpa_status vpa_combine_stats(const vpa_stat* stats, int32_t n_shards, int64_t n_rows, int32_t m,
                             const vpa_epilogue* epi, int32_t* ids, uint32_t* val_bits,
                             int64_t* mapped, void* stream);

/* Workspace bytes vpa_top_tokens needs for n_rows rows (0 if the arguments
 * are invalid or n_rows is 0): enough for either cut of its statistics (see
 * vpa_top_tokens), whatever the dtype and row stride of the call. */
size_t vpa_top_tokens_workspace(vpa_vocab v, int64_t n_rows, int32_t block);

/* Fused draft-side get_top_tokens over every shard of a row (PR #62604,
 * "Purpose" item 2): padding mask, statistics of every row kept in
 * `workspace`, and their combination into the global argmax.  The ids and
 * maxima do not depend on how a row is cut into statistics, so the library
 * picks the cut:
 *  - bf16 batches of at most 409,731,072 bytes of valid columns (1024 rows
 *    of a 200064-entry vocabulary), with V and ld multiples of 8 and a
 *    16-byte aligned logits pointer: one statistic per 4096-column chunk of
 *    a row, from a persistent launch that sweeps the batch;
 *  - otherwise the per-block statistics of all S shards in rank order,
 *    [S][n_rows][M] with the given block size, as vpa_block_stats cuts them.
 *  The workspace's layout is therefore internal.
 *  logits     [n_rows, ld] holding all S shards side by side (global column
 *             c at logits[row*ld + c]); ld >= V.
 *  workspace  device memory of at least vpa_top_tokens_workspace() bytes,
 *             8-byte aligned; its contents on entry do not matter.
 *  epi, ids, val_bits, mapped  as vpa_combine_stats; with epi->d2t set,
 *             d2t_len must be at least V. */
vpa_status vpa_top_tokens(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                          int64_t n_rows, int32_t block, void* workspace, size_t workspace_bytes,
                          const vpa_epilogue* epi, int32_t* ids, uint32_t* val_bits,
                          int64_t* mapped, void* stream);

/* vpa_top_tokens for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as vpa_top_tokens without the workspace: the
 * statistics go to a device array the library holds, one copy of
 * VPA_NOALLOC_WORKSPACE_BYTES per GPU it runs on, kept until the process
 * ends.  The call makes no allocation and no memset; the first call on a
 * device looks the array's address up once (hipGetSymbolAddress).
 *  - A call needing more statistics bytes than VPA_NOALLOC_WORKSPACE_BYTES
 *    (vpa_top_tokens_workspace) returns VPA_ERR_INVALID and enqueues
 *    nothing; at 8192-column blocks that allows 16384 rows of a
 *    200064-entry vocabulary over 8 shards.
 *  - Every call on one GPU shares that GPU's array, and the array keeps the
 *    last call's contents (nothing in it needs to start at zero): calls that
 *    overlap on one GPU (on different streams) race on it and must be
 *    serialised by the caller. */
#define VPA_NOALLOC_WORKSPACE_BYTES ((size_t)4 << 20)
vpa_status vpa_top_tokens_noalloc(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                                  int64_t n_rows, int32_t block, const vpa_epilogue* epi,
                                  int32_t* ids, uint32_t* val_bits, int64_t* mapped,
                                  void* stream);

/* Greedy verification from gathered statistics (PR #62604, "Purpose" item 1
 * and "Test Plan"): the target token of each position is the combined
 * argmax of its row; drafts are accepted while they equal their target;
 * the first differing position -- or position K when all K match -- emits
 * its target token (correction or bonus token); later positions hold -1.
 *  draft_stats  [n_shards][n_req*K][m_draft], bonus_stats [n_shards][n_req][m_bonus]
 *               (the layout vpa_verify_stats writes).
 *  draft_ids    int32 [n_req][K]; any value is legal, -1 marks a placeholder,
 *               and only a value equal to the target token is accepted.
 *  accept       device int32 [n_req], or NULL: synthetic accept counts.  The
 *               same "Purpose" item names synthetic acceptance beside the
 *               real one, and "Test Plan" lists it among the verified cases,
 *               without a rule; the reading here: with accept[r] >= 0 the
 *               first min(accept[r], K) drafts of request r are accepted
 *               whatever their values, and the next position emits its
 *               target token as above; accept[r] < 0 (or NULL) is the real
 *               rule.  Random draws behind the counts are the caller's.
 *  out_tokens   out, int32 [n_req][K+1].
 *  num_sampled  out, int32 [n_req]: accepted + 1.
 *  num_rejected out, int32 [n_req]: K - accepted.
 *  target_ids   out, int32 [n_req][K+1], or NULL: the target token of every
 *               position.
 *  1 <= k <= VPA_MAX_DRAFTS. */
vpa_status vpa_greedy_verify(const vpa_stat* draft_stats, int32_t m_draft,
                             const vpa_stat* bonus_stats, int32_t m_bonus, int32_t n_shards,
                             int64_t n_req, int32_t k, const int32_t* draft_ids,
                             const int32_t* accept, int32_t* out_tokens, int32_t* num_sampled,
                             int32_t* num_rejected, int32_t* target_ids, void* stream);

/* Ragged greedy verification from gathered statistics: as
 * vpa_greedy_verify with a draft count per request.
 *  cu           device int32 [n_req+1] as for vpa_ragged_rows.
 *  draft_stats  [n_shards][total_drafts][m_draft] (row cu[r]+j = draft j of r),
 *  bonus_stats  [n_shards][n_req][m_bonus].
 *  draft_ids    int32 [total_drafts], request r's drafts at cu[r]...
 *  prefilling   device uint8 [n_req], or NULL for none: a nonzero entry marks
 *               a request that is still prefilling.  The PR's "Test Plan"
 *               lists such requests without a rule; the reading here is that
 *               one samples nothing: all K_r+1 of its out_tokens hold -1 and
 *               num_sampled = num_rejected = 0, whatever its accept count.
 *               Its target_ids are written as for any request.
 *  accept       device int32 [n_req], or NULL: synthetic accept counts as for
 *               vpa_greedy_verify, with K_r in place of K.
 *  out_tokens   out, int32 [total_drafts + n_req]: request r's K_r+1 entries
 *               at cu[r]+r (accepted drafts, then the correction or bonus
 *               token, then -1); a request with K_r = 0 emits its bonus token.
 *  num_sampled, num_rejected  out, int32 [n_req]: accepted+1 and K_r-accepted;
 *               both -1 for a request whose offsets are malformed (K_r < 0,
 *               K_r > VPA_MAX_DRAFTS, or outside [0, total_drafts]), which then
 *               writes no tokens, prefilling or not.  Offsets that pass these
 *               checks one by one but decrease across requests make requests
 *               overlap: their outputs are then unspecified, though every
 *               access stays inside the arrays above.
 *  target_ids   out, int32 [total_drafts + n_req] or NULL. */
vpa_status vpa_greedy_verify_ragged(const vpa_stat* draft_stats, int32_t m_draft,
                                    const vpa_stat* bonus_stats, int32_t m_bonus,
                                    int32_t n_shards, int64_t n_req, const int32_t* cu,
                                    int64_t total_drafts, const int32_t* draft_ids,
                                    const uint8_t* prefilling, const int32_t* accept,
                                    int32_t* out_tokens, int32_t* num_sampled,
                                    int32_t* num_rejected, int32_t* target_ids, void* stream);

/* Message describing the last non-OK status returned on the calling thread
 * ("" if none).  The pointer stays valid until the next call on that thread. */
const char* vpa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VPA_H */
