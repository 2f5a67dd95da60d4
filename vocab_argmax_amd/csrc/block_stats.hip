// block_stats.hip -- per-block (max, token id) statistics of vocabulary
// shards, the HBM-streaming step of the path.
//
// vLLM PR #62604, "Purpose" item 1: each rank reduces its vocabulary shard to
// per-block (max, token id) statistics whose block boundaries are the global
// ones of the full vocabulary, even where a block straddles a shard edge;
// item 2: padding columns are masked.  Here a "segment" is one statistic's
// column range: block b = floor(s*W/B) + j cut to shard s and to [0, V).
//
// Work decomposition (CDNA4, wave64): one wavefront per segment, four
// wavefronts per workgroup, no LDS and no barriers.  A wave streams its
// segment with 16-byte non-temporal loads (one 1 KiB wave-wide load per
// iteration, up to 16 iterations -- 16 KiB -- in flight per wave), keeps a
// running best per lane, and finishes with a shuffle reduction.  Segments of
// a row are consecutive work items, so consecutive waves read consecutive
// memory.  Padding columns [V, S*W) are never read.
//
// Per-lane scan.  Every element becomes an order-preserving unsigned key
// (vpa_device.h); bf16 keys are 16 bits wide and computed two at a time with
// packed 16-bit integer ops.  A bf16 lane folds (key << 16 | 0xFFFF -
// position) with one unsigned max: the largest key wins and, among equal
// keys, the earliest position.  For fp32 a strict greater-than keeps the
// first of equal keys.  The winning position decodes back to a global
// column; the wave then takes the lexicographic maximum of (key, -column),
// which is associative and commutative, so any lane layout or chunking gives
// the same statistic.
//
// Alignment.  Rows may start at any element-aligned address (an unaligned
// vocabulary padding makes odd row strides).  The segment's full 16-byte
// vectors are streamed; the at most 2*(16/esize - 1) elements before the
// first and after the last full vector are read one by one by lanes 0..31.
#include "vpa_device.h"
#include "vpa_internal.h"

namespace vpa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* gvec_ptr;
typedef const uint16_t __attribute__((address_space(1)))* gu16_ptr;
typedef const uint32_t __attribute__((address_space(1)))* gu32_ptr;

__device__ __forceinline__ void take_better(uint32_t& bk, int32_t& bc, uint32_t k, int32_t c) {
    if (k > bk || (k == bk && c < bc)) {
        bk = k;
        bc = c;
    }
}

// One chunk of U wave iterations over the segment's full vectors seg[0, n):
// lane reads seg[i0 + 64*u] for u < U, with i0 = lane + 64*t0.  FULL: every
// such index is below n; otherwise indices are clamped to n-1, which only
// re-reads that vector (a duplicate decodes to the same column, so it cannot
// change the result).  Column of element e of seg[i] = c0 + i*VEC + e.
template <int ESIZE, int U, bool FULL>
__device__ __forceinline__ void scan_chunk(gvec_ptr seg, uint32_t i0, uint32_t ilast, int32_t c0,
                                           uint32_t& bk, int32_t& bc) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t i = i0 + 64 * u;
        if (!FULL)
            i = i < ilast ? i : ilast;
        v[u] = __builtin_nontemporal_load(seg + i);
    }
    if constexpr (ESIZE == 2) {
        // key16 << 16 | (0xFFFF - position): one unsigned max keeps the largest
        // key and, among equal keys, the earliest position of this lane.
        uint32_t best = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t k = keys_bf16x2(v[u][d]);
                const uint32_t pos = u * 8 + d * 2;
                // v_perm_b32 picks bytes of {k, c}: selector 0x05040100 gives
                // (k << 16) | c.lo16, 0x07060100 gives (k & 0xFFFF0000) | c.lo16.
                const uint32_t lo = __builtin_amdgcn_perm(k, 0xFFFFu - pos, 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(k, 0xFFFFu - (pos + 1), 0x07060100u);
                best = max(best, max(lo, hi));
            }
        }
        const uint32_t pos = 0xFFFFu - (best & 0xFFFFu);
        uint32_t i = i0 + 64 * (pos >> 3);
        if (!FULL)
            i = i < ilast ? i : ilast;
        take_better(bk, bc, best >> 16, c0 + (int32_t)(i * 8 + (pos & 7)));
    } else {
        uint32_t ck = 0, cpos = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t k = key_f32(v[u][d]);
                if (k > ck || (u == 0 && d == 0)) {
                    ck = k;
                    cpos = u * 4 + d;
                }
            }
        }
        uint32_t i = i0 + 64 * (cpos >> 2);
        if (!FULL)
            i = i < ilast ? i : ilast;
        take_better(bk, bc, ck, c0 + (int32_t)(i * 4 + (cpos & 3)));
    }
}

template <int ESIZE, int U>
__device__ __forceinline__ void scan_iters(gvec_ptr seg, uint32_t n, uint32_t t0, int lane,
                                           int32_t c0, uint32_t& bk, int32_t& bc) {
    const uint32_t i0 = (uint32_t)lane + 64 * t0;
    if (64 * (t0 + U) <= n)
        scan_chunk<ESIZE, U, true>(seg, i0, n - 1, c0, bk, bc);
    else
        scan_chunk<ESIZE, U, false>(seg, i0, n - 1, c0, bk, bc);
}

__device__ __forceinline__ uint32_t load_bits(const unsigned char* base, int esize, int64_t e) {
    return esize == 2 ? (uint32_t)((gu16_ptr)base)[e] << 16 : ((gu32_ptr)base)[e];
}

template <int ESIZE>
__device__ void segment_stat(const SegTask& t, int32_t item, int lane) {
    constexpr int VEC = 16 / ESIZE;
    const int32_t m = t.m;
    const int32_t j = item % m;
    const int32_t rest = item / m;
    const int32_t sl = rest % t.n_local;
    const int32_t i = rest / t.n_local;
    vpa_stat* out = t.stats + ((int64_t)sl * t.n_rows + i) * m + j;

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
    if (lo >= hi || row < 0 || row >= t.logits_rows) {
        if (lane == 0) {
            vpa_stat e;
            e.val_bits = VPA_EMPTY_BITS;
            e.id = VPA_EMPTY_ID;
            *out = e;
        }
        return;
    }

    // Aligned element index a = buffer element index + mis, so that vector q
    // holds aligned indices [q*VEC, (q+1)*VEC); column = a + D.
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
    // The segment's full vectors, seg[0, n); a segment is at most 2^24
    // elements, so 32-bit offsets suffice.
    const gvec_ptr seg = (gvec_ptr)(base - (uintptr_t)(mis * ESIZE)) + qa;
    const uint32_t n = (uint32_t)(qb - qa);
    const int32_t c0 = (int32_t)(qa * VEC + D);

    uint32_t bk = 0;
    int32_t bc = INT32_MAX;
    {
        const int64_t c = lane < 16 ? lo + lane : tail_lo + (lane - 16);
        const bool has = lane < 16 ? c < head_end : (lane < 32 && c < hi);
        if (has) {
            const uint32_t f = load_bits(t.base, ESIZE, row * t.ld + (c - t.col0));
            bk = ESIZE == 2 ? key_bf16(f >> 16) : key_f32(f);
            bc = (int32_t)c;
        }
    }

    const uint32_t nit = (n + 63) >> 6;   // wave iterations over full vectors
    uint32_t t0 = 0;
    for (; t0 + 16 <= nit; t0 += 16)
        scan_iters<ESIZE, 16>(seg, n, t0, lane, c0, bk, bc);
    if (t0 + 8 <= nit) {
        scan_iters<ESIZE, 8>(seg, n, t0, lane, c0, bk, bc);
        t0 += 8;
    }
    if (t0 + 4 <= nit) {
        scan_iters<ESIZE, 4>(seg, n, t0, lane, c0, bk, bc);
        t0 += 4;
    }
    if (t0 + 2 <= nit) {
        scan_iters<ESIZE, 2>(seg, n, t0, lane, c0, bk, bc);
        t0 += 2;
    }
    if (t0 < nit)
        scan_iters<ESIZE, 1>(seg, n, t0, lane, c0, bk, bc);

    wave_best_key_col(bk, bc);

    uint32_t bits;
    if (ESIZE == 2 ? (bk == kKeyNanBf16 || bk == kKeyZeroBf16)
                   : (bk == kKeyNanF32 || bk == kKeyZeroF32))
        bits = load_bits(t.base, ESIZE, row * t.ld + ((int64_t)bc - t.col0));
    else
        bits = ESIZE == 2 ? bits_of_key_bf16(bk) : bits_of_key_f32(bk);
    if (lane == 0) {
        vpa_stat st;
        st.val_bits = bits;
        st.id = bc;
        *out = st;
    }
}

template <int ESIZE>
__global__ __launch_bounds__(kThreads) void block_stats_kernel(SegTask t0, SegTask t1) {
    const int lane = threadIdx.x & 63;
    const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
    int32_t item = (int32_t)blockIdx.x * kWaves + wave;
    if (item < t0.n_items) {
        segment_stat<ESIZE>(t0, item, lane);
        return;
    }
    item -= t0.n_items;
    if (item < t1.n_items)
        segment_stat<ESIZE>(t1, item, lane);
}

}  // namespace

hipError_t launch_block_stats(int esize, const SegTask& t0, const SegTask& t1, hipStream_t stream) {
    const int64_t items = (int64_t)t0.n_items + t1.n_items;
    if (items <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((items + kWaves - 1) / kWaves));
    const dim3 block(kThreads);
    if (esize == 2)
        hipLaunchKernelGGL(block_stats_kernel<2>, grid, block, 0, stream, t0, t1);
    else
        hipLaunchKernelGGL(block_stats_kernel<4>, grid, block, 0, stream, t0, t1);
    return hipGetLastError();
}

}  // namespace vpa
