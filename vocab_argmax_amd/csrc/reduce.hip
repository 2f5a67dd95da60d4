// reduce.hip -- the steps after the statistics exchange: rank-order
// combination into the global argmax, and greedy verification.
//
// vLLM PR #34049, "Solution", step 3: a reduction over the gathered
// (max, global index) pairs gives the global argmax.  vLLM PR #62604,
// "Purpose" item 1: one kernel finishes the global argmax, the acceptance,
// the bonus token and the sampled/rejected counts from the gathered per-block
// statistics.
//
// Statistics arrive in rank order, [S][rows][M].  One wavefront reduces one
// row (a combine row, or one position of a verified request): lanes stride
// over the row's S*M statistics, keep the best under the argmax order (key of
// the value bits, then the lower id), and a DPP cross-lane reduction finishes.  The lexicographic
// (key, -id) maximum is order independent, so the result equals a scan in
// rank order that keeps only strictly better statistics; an empty slot
// (-inf, id INT32_MAX) loses to every real statistic.
#include "vpa_device.h"
#include "vpa_internal.h"

namespace vpa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kVerifyMaxThreads = 1024;

// Best statistic of row `row` of a [S][rows_total][m] array; every lane
// returns the same (id, bits).  A lane's statistics are loaded kRowBatch at a
// time before any is compared, so a row of up to 64*kRowBatch statistics
// (the bonus rows' 1024-column blocks: 200-208 of them) costs one memory
// round trip, not one per 64.
constexpr int kRowBatch = 4;

__device__ __forceinline__ void row_best(const vpa_stat* __restrict__ stats, int32_t n_shards,
                                         int64_t rows_total, int64_t row, int32_t m, int lane,
                                         int32_t& id, uint32_t& bits) {
    uint32_t bk = 0, bn = 0, bb = 0;
    const int32_t total = n_shards * m;
    for (int32_t i0 = lane; i0 < total; i0 += 64 * kRowBatch) {
        vpa_stat st[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
            const int32_t idx = i0 + 64 * u;
            if (idx < total) {
                const int32_t s = idx / m;
                const int32_t j = idx - s * m;
                st[u] = stats[((int64_t)s * rows_total + row) * m + j];
            }
        }
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
            if (i0 + 64 * u >= total)
                break;
            const uint32_t k = key_f32(st[u].val_bits);
            const uint32_t n = ~(uint32_t)st[u].id;
            if (k > bk || (k == bk && n > bn)) {
                bk = k;
                bn = n;
                bb = st[u].val_bits;
            }
        }
    }
    wave_best_stat(bk, bn, bb);
    id = (int32_t)~bn;
    bits = bb;
}

// Reported maximum under a positive logit scale: the IEEE fp32 product,
// rounded to nearest even (the kernel runs with fp32 denormals preserved);
// a NaN is passed through untouched.
__device__ __forceinline__ uint32_t scaled_bits(uint32_t bits, float scale) {
    if ((bits & 0x7FFFFFFFu) > 0x7F800000u)
        return bits;
    return __float_as_uint(__fmul_rn(__uint_as_float(bits), scale));
}

// Draft ids of a request, loaded into registers at the start of a
// verification workgroup so that their latency overlaps the reduction of the
// statistics: thread t holds positions t + i*blockDim.x, i < kDraftRegs.
constexpr int kDraftRegs = 4;

__device__ __forceinline__ void load_drafts(const int32_t* __restrict__ drafts, int32_t k,
                                            int32_t (&reg)[kDraftRegs]) {
#pragma unroll
    for (int i = 0; i < kDraftRegs; ++i) {
        const int32_t j = (int32_t)(threadIdx.x + i * blockDim.x);
        reg[i] = j < k ? drafts[j] : 0;
    }
}

// The drafts into LDS: the registers, then any position beyond them
// (requests with more than kDraftRegs * blockDim.x drafts) straight from
// memory.
__device__ __forceinline__ void store_drafts(const int32_t* __restrict__ drafts, int32_t k,
                                             const int32_t (&reg)[kDraftRegs], int32_t* lds) {
#pragma unroll
    for (int i = 0; i < kDraftRegs; ++i) {
        const int32_t j = (int32_t)(threadIdx.x + i * blockDim.x);
        if (j < k)
            lds[j] = reg[i];
    }
    for (int32_t j = (int32_t)(threadIdx.x + kDraftRegs * blockDim.x); j < k;
         j += (int32_t)blockDim.x)
        lds[j] = drafts[j];
}

// Finish one request with the whole workgroup, once its K drafts and K+1
// targets are in LDS (after a barrier) and *first was set to k before that
// barrier.  Accepted drafts: with a synthetic count c >= 0 the first
// min(c, k) whatever their values (vLLM PR #62604, "Purpose" item 1, names
// synthetic acceptance beside the real one, with no rule; this is the
// reading taken), else every position before the first draft that differs
// from its target, found by an LDS minimum over the threads.  The K+1
// outputs are then written in parallel: accepted drafts, the next target,
// -1.  A request that samples nothing (`skip`, a request still prefilling)
// writes -1 everywhere and zero counts.  c and skip are uniform over the
// workgroup, so every thread reaches the same barriers.
__device__ __forceinline__ void finish_request(const int32_t* drafts, const int32_t* targets,
                                               int32_t k, int32_t c, bool skip, int32_t* first,
                                               int32_t* __restrict__ out, int32_t* num_sampled,
                                               int32_t* num_rejected) {
    if (skip) {
        for (int32_t j = threadIdx.x; j <= k; j += (int32_t)blockDim.x)
            out[j] = -1;
        if (threadIdx.x == 0) {
            *num_sampled = 0;
            *num_rejected = 0;
        }
        return;
    }
    int32_t n;
    if (c >= 0) {
        n = c < k ? c : k;
    } else {
        for (int32_t j = threadIdx.x; j < k; j += (int32_t)blockDim.x) {
            if (drafts[j] != targets[j]) {
                atomicMin(first, j);
                break;
            }
        }
        __syncthreads();
        n = *first;
    }
    for (int32_t j = threadIdx.x; j <= k; j += (int32_t)blockDim.x)
        out[j] = j < n ? drafts[j] : (j == n ? targets[j] : -1);
    if (threadIdx.x == 0) {
        *num_sampled = n + 1;
        *num_rejected = k - n;
    }
}

// One wavefront per row; the epilogue (vLLM PR #39419, "Refactor local
// argmax code": map the argmax k to k + d2t[k]; a positive scale changes only
// the reported maximum) runs on lane 0 after the reduction.  (Groups of 8 or
// 32 lanes per row, several rows per wavefront, measured no faster at
// 1024-4096 rows and slower at 32 rows.)
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const vpa_stat* __restrict__ stats, int32_t n_shards, int32_t n_rows, int32_t m,
    const int64_t* __restrict__ d2t, int64_t d2t_len, float scale, int32_t* __restrict__ ids,
    uint32_t* __restrict__ val_bits, int64_t* __restrict__ mapped) {
    const int lane = threadIdx.x & 63;
    const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
    const int32_t row = (int32_t)blockIdx.x * kWaves + wave;
    if (row >= n_rows)
        return;
    int32_t id;
    uint32_t bits;
    row_best(stats, n_shards, n_rows, row, m, lane, id, bits);
    if (lane == 0) {
        ids[row] = id;
        if (val_bits)
            val_bits[row] = scale == 1.0f ? bits : scaled_bits(bits, scale);
        if (mapped)
            mapped[row] = (id >= 0 && id < d2t_len) ? (int64_t)id + d2t[id] : -1;
    }
}

// One workgroup per request r.  Its wavefronts share out the K+1 positions
// (wave w takes positions w, w + nw, ...): the target token of draft position
// j is the best statistic of row r*K+j of draft_stats, that of the bonus
// position the best of row r of bonus_stats.  The targets and the drafts
// meet in LDS; after the barrier the workgroup applies the greedy acceptance
// (finish_request): drafts are accepted while they equal their target (or,
// with a synthetic count, the first accept[r] of them), the next position (or
// position K) emits its target, later positions hold -1.
__global__ __launch_bounds__(kVerifyMaxThreads) void greedy_verify_kernel(
    const vpa_stat* __restrict__ draft_stats, int32_t m_draft,
    const vpa_stat* __restrict__ bonus_stats, int32_t m_bonus, int32_t n_shards, int32_t n_req,
    int32_t k, const int32_t* __restrict__ draft_ids, const int32_t* __restrict__ accept,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ num_sampled,
    int32_t* __restrict__ num_rejected, int32_t* __restrict__ target_ids) {
    extern __shared__ int32_t lds[];   // targets [k+1], drafts [k], first mismatch [1]
    int32_t* targets = lds;
    int32_t* drafts = lds + k + 1;
    int32_t* first = drafts + k;
    const int lane = threadIdx.x & 63;
    const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
    const int32_t n_waves = (int32_t)(blockDim.x >> 6);
    const int32_t r = (int32_t)blockIdx.x;
    const int64_t base = (int64_t)r * (k + 1);
    const int32_t* my_drafts = draft_ids + (int64_t)r * k;
    int32_t reg[kDraftRegs];
    load_drafts(my_drafts, k, reg);
    const int32_t c = accept ? accept[r] : -1;
    for (int32_t j = wave; j <= k; j += n_waves) {
        int32_t tgt;
        uint32_t bits;
        if (j < k)
            row_best(draft_stats, n_shards, (int64_t)n_req * k, (int64_t)r * k + j, m_draft, lane,
                     tgt, bits);
        else
            row_best(bonus_stats, n_shards, n_req, r, m_bonus, lane, tgt, bits);
        if (lane == 0) {
            targets[j] = tgt;
            if (target_ids)
                target_ids[base + j] = tgt;
        }
    }
    store_drafts(my_drafts, k, reg, drafts);
    if (threadIdx.x == 0)
        *first = k;
    __syncthreads();
    finish_request(drafts, targets, k, c, false, first, out_tokens + base, num_sampled + r,
                   num_rejected + r);
}

// Ragged batch: one thread per request writes its row indices.  Every
// index is checked against the buffers, so malformed offsets cannot write
// out of bounds.
__global__ __launch_bounds__(kThreads) void ragged_rows_kernel(const int32_t* __restrict__ cu,
                                                               int32_t n_req, int32_t total,
                                                               int32_t* __restrict__ draft_rows,
                                                               int32_t* __restrict__ bonus_rows) {
    const int32_t r = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    if (r >= n_req)
        return;
    const int32_t lo = cu[r], hi = cu[r + 1];
    const bool ok = 0 <= lo && lo <= hi && hi <= total;
    bonus_rows[r] = ok ? hi + r : -1;
    if (!ok)
        return;
    for (int32_t i = lo; i < hi; ++i)
        draft_rows[i] = i + r;
}

// Ragged verification: one workgroup per request r with K_r = cu[r+1]-cu[r]
// drafts; the wavefronts share out the K_r+1 positions as in the uniform
// kernel, then the workgroup applies the acceptance and writes K_r+1 outputs
// at offset cu[r]+r.  A request flagged in `prefilling` (vLLM PR #62604,
// "Test Plan", lists such requests; read here as sampling nothing) writes -1
// in all its slots and 0 sampled / 0 rejected, whatever its synthetic count;
// its targets are still written.
__global__ __launch_bounds__(kThreads) void greedy_verify_ragged_kernel(
    const vpa_stat* __restrict__ draft_stats, int32_t m_draft,
    const vpa_stat* __restrict__ bonus_stats, int32_t m_bonus, int32_t n_shards, int32_t n_req,
    const int32_t* __restrict__ cu, int32_t total, const int32_t* __restrict__ draft_ids,
    const uint8_t* __restrict__ prefilling, const int32_t* __restrict__ accept,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ num_sampled,
    int32_t* __restrict__ num_rejected, int32_t* __restrict__ target_ids) {
    __shared__ int32_t targets[VPA_MAX_DRAFTS + 1];
    __shared__ int32_t drafts[VPA_MAX_DRAFTS];
    __shared__ int32_t first;
    const int lane = threadIdx.x & 63;
    const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
    const int32_t r = (int32_t)blockIdx.x;
    const int32_t lo = cu[r], hi = cu[r + 1];
    const int32_t k = hi - lo;
    if (!(0 <= lo && lo <= hi && hi <= total && k <= VPA_MAX_DRAFTS)) {
        if (threadIdx.x == 0) {
            num_sampled[r] = -1;
            num_rejected[r] = -1;
        }
        return;   // uniform for the workgroup: no barrier is skipped by part of it
    }
    const int64_t base = (int64_t)lo + r;
    const int32_t* my_drafts = draft_ids + lo;
    int32_t reg[kDraftRegs];
    load_drafts(my_drafts, k, reg);
    const int32_t c = accept ? accept[r] : -1;
    const bool skip = prefilling && prefilling[r];
    for (int32_t j = wave; j <= k; j += kWaves) {
        int32_t tgt;
        uint32_t bits;
        if (j < k)
            row_best(draft_stats, n_shards, total, (int64_t)lo + j, m_draft, lane, tgt, bits);
        else
            row_best(bonus_stats, n_shards, n_req, r, m_bonus, lane, tgt, bits);
        if (lane == 0) {
            targets[j] = tgt;
            if (target_ids)
                target_ids[base + j] = tgt;
        }
    }
    store_drafts(my_drafts, k, reg, drafts);
    if (threadIdx.x == 0)
        first = k;
    __syncthreads();
    finish_request(drafts, targets, k, c, skip, &first, out_tokens + base, num_sampled + r,
                   num_rejected + r);
}

}  // namespace

int64_t combine_threads(int32_t n_rows) {
    return ((int64_t)n_rows + kWaves - 1) / kWaves * kThreads;
}

int64_t greedy_verify_threads(int32_t n_req, int32_t k) {
    const int64_t waves = k + 1 < kVerifyMaxThreads / 64 ? k + 1 : kVerifyMaxThreads / 64;
    return (int64_t)n_req * 64 * waves;
}

int64_t greedy_verify_ragged_threads(int32_t n_req) {
    return (int64_t)n_req * kThreads;
}

hipError_t launch_ragged_rows(const int32_t* cu, int32_t n_req, int32_t total_drafts,
                              int32_t* draft_rows, int32_t* bonus_rows, hipStream_t stream) {
    const dim3 grid((unsigned)((n_req + kThreads - 1) / kThreads));
    return launch(ragged_rows_kernel, grid, dim3(kThreads), 0, stream, cu, n_req, total_drafts,
                  draft_rows, bonus_rows);
}

hipError_t launch_greedy_verify_ragged(const vpa_stat* draft_stats, int32_t m_draft,
                                       const vpa_stat* bonus_stats, int32_t m_bonus,
                                       int32_t n_shards, int32_t n_req, const int32_t* cu,
                                       int32_t total_drafts, const int32_t* draft_ids,
                                       const uint8_t* prefilling, const int32_t* accept,
                                       int32_t* out_tokens, int32_t* num_sampled,
                                       int32_t* num_rejected, int32_t* target_ids,
                                       hipStream_t stream) {
    return launch(greedy_verify_ragged_kernel, dim3((unsigned)n_req), dim3(kThreads), 0, stream,
                  draft_stats, m_draft, bonus_stats, m_bonus, n_shards, n_req, cu, total_drafts,
                  draft_ids, prefilling, accept, out_tokens, num_sampled, num_rejected,
                  target_ids);
}

hipError_t launch_combine(const vpa_stat* stats, int32_t n_shards, int32_t n_rows, int32_t m,
                          const int64_t* d2t, int64_t d2t_len, float scale, int32_t* ids,
                          uint32_t* val_bits, int64_t* mapped, hipStream_t stream) {
    const dim3 grid((unsigned)((n_rows + kWaves - 1) / kWaves));
    return launch(combine_kernel, grid, dim3(kThreads), 0, stream, stats, n_shards, n_rows, m, d2t,
                  d2t_len, scale, ids, val_bits, mapped);
}

hipError_t launch_greedy_verify(const vpa_stat* draft_stats, int32_t m_draft,
                                const vpa_stat* bonus_stats, int32_t m_bonus, int32_t n_shards,
                                int32_t n_req, int32_t k, const int32_t* draft_ids,
                                const int32_t* accept, int32_t* out_tokens, int32_t* num_sampled,
                                int32_t* num_rejected, int32_t* target_ids, hipStream_t stream) {
    const int32_t waves = k + 1 < kVerifyMaxThreads / 64 ? k + 1 : kVerifyMaxThreads / 64;
    return launch(greedy_verify_kernel, dim3((unsigned)n_req), dim3(64 * waves),
                  (size_t)(2 * k + 2) * sizeof(int32_t), stream, draft_stats, m_draft, bonus_stats,
                  m_bonus, n_shards, n_req, k, draft_ids, accept, out_tokens, num_sampled,
                  num_rejected, target_ids);
}

}  // namespace vpa
