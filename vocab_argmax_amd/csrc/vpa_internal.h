// vpa_internal.h -- declarations shared by the HIP sources of libvpa (not
// part of the public C ABI, which is include/vpa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vpa.h"

namespace vpa {

template <typename T>
struct same_type {
    using type = T;
};

// Launch `kernel` and return the status of this launch alone: not an error
// left behind by an earlier, unrelated HIP call, which stays where the
// caller can see it.  Arguments convert to the kernel's parameter types.
template <typename... Params>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds_bytes,
                  hipStream_t stream, typename same_type<Params>::type... args) {
    void* ptrs[] = {(void*)&args..., nullptr};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds_bytes,
                           stream);
}

// One launch's worth of (row, shard, slot) work items for the block-statistics
// kernel.  Item t decodes as row i = t / (n_local*m), local shard
// sl = (t / m) % n_local, slot j = t % m; consecutive items therefore walk a
// row's columns in ascending order.  Each item is scanned by a group of
// 2^lanes_log2 lanes of one wavefront (64 / group size items per wavefront);
// launch_block_stats picks the group size and fills lanes_log2 and n_waves.
struct SegTask {
    const unsigned char* base;  // logits, column 0 = global column col0
    int64_t ld;                 // row stride, elements
    int64_t vocab;              // V
    int64_t shard_width;        // W
    int64_t col0;               // first_shard * W
    int64_t logits_rows;        // rows[] entries must lie in [0, logits_rows)
    const int32_t* rows;        // row list or nullptr
    vpa_stat* stats;            // [n_local][n_rows][m]
    int32_t n_rows;
    int32_t n_items;            // n_rows * n_local * m (< 2^31, checked by the host)
    int32_t first_shard;
    int32_t n_local;
    int32_t block;
    int32_t m;
    int32_t row_k;              // > 0: verification rows with K = row_k (rows ignored)
    int32_t row_bonus;          // with row_k > 0: 1 = bonus rows, 0 = draft rows
    int32_t lanes_log2;         // lanes per item: 3..6 (set by launch_block_stats)
    int32_t n_waves;            // wavefronts this task occupies (set by launch_block_stats)
};

// Statistics of vpa_top_tokens for small bf16 batches (chunk_stats.hip): one
// statistic per chunk of chunk_stats_per_row(V) columns of a row, laid out
// [rows][chunk_stats_per_row(V)].  The logits must be bf16 with V and ld
// multiples of 8 and a 16-byte aligned base.
int32_t chunk_stats_per_row(int64_t vocab);
hipError_t launch_chunk_stats(const void* logits, int64_t ld, int32_t vocab, int32_t n_rows,
                              vpa_stat* stats, hipStream_t stream);

// Launch the block-statistics kernel over the items of t0 followed by those
// of t1 (t1.n_items may be 0).  Both tasks share dtype `esize` (2 or 4).
hipError_t launch_block_stats(int esize, const SegTask& t0, const SegTask& t1, hipStream_t stream);

// Work-items that launch would use (a dispatch holds fewer than 2^32).
int64_t block_stats_threads(int esize, const SegTask& t0, const SegTask& t1);

// Work-items of the other launches, for the same check.
int64_t combine_threads(int32_t n_rows);
int64_t greedy_verify_threads(int32_t n_req, int32_t k);
int64_t greedy_verify_ragged_threads(int32_t n_req);

// Most work-items one dispatch may hold.
constexpr int64_t kMaxDispatchThreads = ((int64_t)1 << 32) - 1;

// Combine with the epilogue already validated: d2t may be null (then mapped
// is null too); scale is finite and positive.
hipError_t launch_combine(const vpa_stat* stats, int32_t n_shards, int32_t n_rows, int32_t m,
                          const int64_t* d2t, int64_t d2t_len, float scale, int32_t* ids,
                          uint32_t* val_bits, int64_t* mapped, hipStream_t stream);

hipError_t launch_greedy_verify(const vpa_stat* draft_stats, int32_t m_draft,
                                const vpa_stat* bonus_stats, int32_t m_bonus, int32_t n_shards,
                                int32_t n_req, int32_t k, const int32_t* draft_ids,
                                const int32_t* accept, int32_t* out_tokens, int32_t* num_sampled,
                                int32_t* num_rejected, int32_t* target_ids, hipStream_t stream);

hipError_t launch_ragged_rows(const int32_t* cu, int32_t n_req, int32_t total_drafts,
                              int32_t* draft_rows, int32_t* bonus_rows, hipStream_t stream);

hipError_t launch_greedy_verify_ragged(const vpa_stat* draft_stats, int32_t m_draft,
                                       const vpa_stat* bonus_stats, int32_t m_bonus,
                                       int32_t n_shards, int32_t n_req, const int32_t* cu,
                                       int32_t total_drafts, const int32_t* draft_ids,
                                       const uint8_t* prefilling, const int32_t* accept,
                                       int32_t* out_tokens, int32_t* num_sampled,
                                       int32_t* num_rejected, int32_t* target_ids,
                                       hipStream_t stream);

}  // namespace vpa
