// block_stats.hip -- per-block (max, token id) statistics of vocabulary
// shards, the HBM-streaming step of the path.
//
// vLLM PR #62604, "Purpose" item 1: each rank reduces its vocabulary shard to
// per-block (max, token id) statistics whose block boundaries are the global
// ones of the full vocabulary, even where a block straddles a shard edge;
// item 2: padding columns are masked.  Here a "segment" is one statistic's
// column range: block b = floor(s*W/B) + j cut to shard s and to [0, V).
//
// Work decomposition (CDNA4, wave64): a segment is scanned by a group of L
// lanes of one wavefront (L = 64 for 8192-column bf16 blocks, down to 8 for
// 1024-column ones), so a lane makes about 16 iterations of 16-byte
// non-temporal loads whatever the block size; four wavefronts per
// workgroup, no LDS accesses and no barriers.  The loads come in chunks of
// U group iterations, software-pipelined: chunk c+1 is issued before chunk
// c is folded, so a wavefront keeps U to 2U loads in flight.  U = 8 for bf16
// (91 VGPRs) and 16 for fp32 (150 VGPRs) measured fastest on MI355X, with
// the launch's LDS reservation holding a CU to 4 wavefronts per SIMD for
// bf16 and 2 for fp32.  Each lane keeps a running best, and a shuffle
// reduction inside the group finishes the segment.  Consecutive groups and
// wavefronts take consecutive segments of a row, so a wavefront reads
// contiguous memory.
// Padding columns [V, S*W) are never read.
//
// Per-lane scan.  Every element becomes an order-preserving unsigned key
// (vpa_device.h); bf16 keys are 16 bits wide and computed two at a time with
// packed 16-bit integer ops.  A bf16 lane folds (key << 16 | 0xFFFF -
// position) with one unsigned max: the largest key wins and, among equal
// keys, the earliest position.  For fp32 a strict greater-than keeps the
// first of equal keys.  The winning position decodes back to a global
// column; the group then takes the lexicographic maximum of (key, -column),
// which is associative and commutative, so any lane layout or chunking gives
// the same statistic.
//
// Alignment.  Rows may start at any element-aligned address (an unaligned
// vocabulary padding makes odd row strides).  The segment's full 16-byte
// vectors are streamed; the at most 2*(16/esize - 1) elements before the
// first and after the last full vector are read one by one.
#include "vpa_device.h"
#include "vpa_internal.h"
#include "vpa_scan.h"

namespace vpa {
namespace {

#ifndef VPA_WAVES_PER_WG
#define VPA_WAVES_PER_WG 4
#endif
#ifndef VPA_PIPE_BF16
#define VPA_PIPE_BF16 8
#endif
#ifndef VPA_PIPE_F32
#define VPA_PIPE_F32 16
#endif
#ifndef VPA_LANE_ITERS
#define VPA_LANE_ITERS 16
#endif
constexpr int kWaves = VPA_WAVES_PER_WG;
constexpr int kThreads = 64 * kWaves;
constexpr int kLaneIters = VPA_LANE_ITERS;   // target iterations per lane of a segment

// LDS reserved per workgroup at launch and never touched by the kernel, by
// element size; it sets how many workgroups share a CU.  bf16: with
// 32 KiB, at most 4 workgroups (16 wavefronts) run per CU on MI355X, where
// the registers would allow 5; per-wavefront timestamps show no more than
// 16 resident wavefronts per CU.  That residency measured 2-3 % faster than
// 5 per CU (no or smaller reservations) and faster than 3 or 2.  fp32
// (150 VGPRs, 3 workgroups per CU by registers): 64 KiB, 2 workgroups per
// CU, measured 2-3 % faster than 32 or 48 KiB.
#ifndef VPA_LDS_RESERVE_KB
#define VPA_LDS_RESERVE_KB 32
#endif
#ifndef VPA_LDS_RESERVE_F32_KB
#define VPA_LDS_RESERVE_F32_KB 64
#endif
template <int ESIZE>
constexpr unsigned kLdsReserve =
    (ESIZE == 2 ? VPA_LDS_RESERVE_KB : VPA_LDS_RESERVE_F32_KB) * 1024u;

// Group iterations per pipelined chunk, by element size.
template <int ESIZE>
constexpr int kPipe = ESIZE == 2 ? VPA_PIPE_BF16 : VPA_PIPE_F32;

// Chunk c+1's loads are issued before chunk c is folded.
template <int ESIZE, int L, int U>
__device__ __forceinline__ void scan_pipelined(gvec_ptr seg, uint32_t n, uint32_t gl, int32_t c0,
                                               uint32_t& bk, int32_t& bc) {
    const uint32_t nit = (n + L - 1) / L;
    const uint32_t chunks = (nit + U - 1) / U;
    u32x4 a[U], b[U];
    load_clamped<ESIZE, L, U>(seg, gl, n - 1, a);
    for (uint32_t c = 0; c + 1 < chunks; ++c) {
        const uint32_t i0 = gl + L * U * c;
        load_clamped<ESIZE, L, U>(seg, i0 + L * U, n - 1, b);
        fold_loaded<ESIZE, L, U>(a, i0, n - 1, c0, bk, bc);
#pragma unroll
        for (int u = 0; u < U; ++u)
            a[u] = b[u];
    }
    fold_loaded<ESIZE, L, U>(a, gl + L * U * (chunks - 1), n - 1, c0, bk, bc);
}

// The statistic of item `item` of task t, computed by the L lanes of the
// group (this lane is lane `gl` of it; with L = 64 the item is uniform).
// Every lane of the wavefront reaches the reduction (no early return), so the
// shuffles read live lanes only.
template <int ESIZE, int L>
__device__ __forceinline__ void segment_stat(const SegTask& t, int32_t item, uint32_t gl) {
    constexpr int VEC = 16 / ESIZE;
    const bool live = item < t.n_items;
    const int32_t it = live ? item : 0;
    const int32_t m = t.m;
    const int32_t j = it % m;
    const int32_t rest = it / m;
    const int32_t sl = rest % t.n_local;
    const int32_t i = rest / t.n_local;

    int64_t row;
    if (t.row_k > 0) {
        const int32_t k = t.row_k;
        row = t.row_bonus ? (int64_t)i * (k + 1) + k : (int64_t)(i / k) * (k + 1) + (i % k);
    } else {
        row = t.rows ? (int64_t)t.rows[i] : (int64_t)i;
    }
    const int64_t shard_lo = ((int64_t)t.first_shard + sl) * t.shard_width;
    const int64_t blo = (shard_lo / t.block + j) * (int64_t)t.block;
    const int64_t lo = blo > shard_lo ? blo : shard_lo;
    int64_t hi = blo + t.block;
    hi = hi < shard_lo + t.shard_width ? hi : shard_lo + t.shard_width;
    hi = hi < t.vocab ? hi : t.vocab;
    const bool work = live && lo < hi && row >= 0 && row < t.logits_rows;

    uint32_t bk = 0;
    int32_t bc = INT32_MAX;
    if (work) {
        // Aligned element index a = buffer element index + mis, so that
        // vector q holds aligned indices [q*VEC, (q+1)*VEC); column = a + D.
        const uintptr_t base = (uintptr_t)t.base;
        const int64_t mis = (int64_t)(base & 15) / ESIZE;
        const int64_t a_lo = row * t.ld + (lo - t.col0) + mis;
        const int64_t D = lo - a_lo;
        const int64_t qa = (a_lo + VEC - 1) / VEC;
        int64_t qb = (a_lo + (hi - lo)) / VEC;
        int64_t head_end, tail_lo;
        if (qa < qb) {
            head_end = qa * VEC + D;
            tail_lo = qb * VEC + D;
        } else {
            head_end = hi;
            tail_lo = hi;
            qb = qa;
        }
        // Edge elements, one by one (at most 2*(VEC-1) of them).
        for (int64_t c = lo + gl; c < head_end; c += L) {
            const uint32_t f = load_bits(t.base, ESIZE, row * t.ld + (c - t.col0));
            take_better(bk, bc, ESIZE == 2 ? key_bf16(f >> 16) : key_f32(f), (int32_t)c);
        }
        for (int64_t c = tail_lo + gl; c < hi; c += L) {
            const uint32_t f = load_bits(t.base, ESIZE, row * t.ld + (c - t.col0));
            take_better(bk, bc, ESIZE == 2 ? key_bf16(f >> 16) : key_f32(f), (int32_t)c);
        }
        // The segment's full vectors, seg[0, n); a segment is at most 2^24
        // elements, so 32-bit offsets suffice.
        const gvec_ptr seg = (gvec_ptr)(base - (uintptr_t)(mis * ESIZE)) + qa;
        const uint32_t n = (uint32_t)(qb - qa);
        const int32_t c0 = (int32_t)(qa * VEC + D);
        if (n > 0)
            scan_pipelined<ESIZE, L, kPipe<ESIZE>>(seg, n, gl, c0, bk, bc);
    }

    group_best_key_col<L>(bk, bc);

    if (gl == 0 && live) {
        vpa_stat st;
        if (!work) {
            st.val_bits = VPA_EMPTY_BITS;
            st.id = VPA_EMPTY_ID;
        } else {
            const bool reread = ESIZE == 2 ? (bk == kKeyNanBf16 || bk == kKeyZeroBf16)
                                           : (bk == kKeyNanF32 || bk == kKeyZeroF32);
            st.val_bits = reread ? load_bits(t.base, ESIZE, row * t.ld + ((int64_t)bc - t.col0))
                                 : (ESIZE == 2 ? bits_of_key_bf16(bk) : bits_of_key_f32(bk));
            st.id = bc;
        }
        t.stats[((int64_t)sl * t.n_rows + i) * m + j] = st;
    }
}

// Task t's items for this wavefront, with groups of 2^LG lanes.
template <int ESIZE, int LG>
__device__ __forceinline__ void wave_items(const SegTask& t, int32_t wave, uint32_t lane) {
    const int32_t item = (wave << (6 - LG)) + (int32_t)(lane >> LG);
    segment_stat<ESIZE, 1 << LG>(t, item, lane & ((1u << LG) - 1));
}

template <int ESIZE>
__device__ __forceinline__ void task_wave(const SegTask& t, int32_t wave, uint32_t lane) {
    switch (t.lanes_log2) {   // uniform: a kernel argument
    case 6:
        wave_items<ESIZE, 6>(t, wave, lane);
        break;
    case 5:
        wave_items<ESIZE, 5>(t, wave, lane);
        break;
    case 4:
        wave_items<ESIZE, 4>(t, wave, lane);
        break;
    default:
        wave_items<ESIZE, 3>(t, wave, lane);
        break;
    }
}

template <int ESIZE>
__global__ __launch_bounds__(kThreads)
#ifdef VPA_WAVES_PER_EU
__attribute__((amdgpu_waves_per_eu(VPA_WAVES_PER_EU)))
#endif
void block_stats_kernel(SegTask t0, SegTask t1) {
    const uint32_t lane = threadIdx.x & 63;
    int32_t wave = (int32_t)blockIdx.x * kWaves +
                   __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
    if (wave < t0.n_waves) {
        task_wave<ESIZE>(t0, wave, lane);
        return;
    }
    wave -= t0.n_waves;
    if (wave < t1.n_waves)
        task_wave<ESIZE>(t1, wave, lane);
}

// Lanes per segment: about kLaneIters 16-byte vectors per lane for the
// longest segment, between 8 lanes (128 contiguous bytes per group load) and
// the full wavefront.
int lanes_log2_for(const SegTask& t, int esize) {
    const int64_t span = t.block < t.shard_width ? t.block : t.shard_width;
    const int64_t vectors = (span * esize + 15) / 16 + 1;
    int lg = 3;
    while (lg < 6 && ((int64_t)1 << (lg + 1)) * kLaneIters <= vectors)
        ++lg;
    return lg;
}

}  // namespace

// Group sizes and wavefront counts of a launch over t0 then t1.
void plan_block_stats(int esize, SegTask& t0, SegTask& t1) {
    for (SegTask* t : {&t0, &t1}) {
        t->lanes_log2 = lanes_log2_for(*t, esize);
        const int32_t per_wave = 1 << (6 - t->lanes_log2);
        t->n_waves = t->n_items > 0 ? (t->n_items + per_wave - 1) / per_wave : 0;
    }
}

int64_t block_stats_threads(int esize, const SegTask& t0_in, const SegTask& t1_in) {
    SegTask t0 = t0_in, t1 = t1_in;
    plan_block_stats(esize, t0, t1);
    const int64_t waves = (int64_t)t0.n_waves + t1.n_waves;
    return (waves + kWaves - 1) / kWaves * kThreads;
}

hipError_t launch_block_stats(int esize, const SegTask& t0_in, const SegTask& t1_in,
                              hipStream_t stream) {
    SegTask t0 = t0_in, t1 = t1_in;
    plan_block_stats(esize, t0, t1);
    const int64_t waves = (int64_t)t0.n_waves + t1.n_waves;
    if (waves <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
    const dim3 block(kThreads);
    return esize == 2 ? launch(block_stats_kernel<2>, grid, block, kLdsReserve<2>, stream, t0, t1)
                      : launch(block_stats_kernel<4>, grid, block, kLdsReserve<4>, stream, t0, t1);
}

}  // namespace vpa
