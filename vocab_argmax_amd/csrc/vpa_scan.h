// vpa_scan.h -- device helpers shared by the statistics kernels
// (block_stats.hip, chunk_stats.hip): 16-byte vector loads of a span of
// logits, the per-lane fold of loaded values into a running best under the
// argmax order (the larger key, then the smaller column), and the
// cross-lane reduction of that best.
#pragma once

#include "vpa_device.h"

namespace vpa {

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

// The segment's full vectors seg[0, n), n >= 1, in chunks of U group
// iterations: in chunk c the lane reads seg[i0 + L*u] for u < U, with
// i0 = (lane in group) + L*U*c.  Indices past the end are clamped to n-1,
// which only re-reads that vector (a duplicate decodes to the same column,
// so it cannot change the result).  Column of element e of seg[i] =
// c0 + i*VEC + e.
template <int ESIZE, int L, int U>
__device__ __forceinline__ void load_clamped(gvec_ptr seg, uint32_t i0, uint32_t ilast,
                                             u32x4 (&v)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        uint32_t i = i0 + L * u;
        i = i < ilast ? i : ilast;
        v[u] = __builtin_nontemporal_load(seg + i);
    }
}

// Called before vector u of a chunk is folded; the default does nothing.
struct NoPace {
    __device__ __forceinline__ void operator()(int) const {}
};

// Fold one loaded chunk (chunk origin i0) into the lane's running best.
// pace(u) runs before vector u is folded.
template <int ESIZE, int L, int U, typename Pace = NoPace>
__device__ __forceinline__ void fold_loaded(const u32x4 (&v)[U], uint32_t i0, uint32_t ilast,
                                            int32_t c0, uint32_t& bk, int32_t& bc,
                                            Pace pace = Pace()) {
    if constexpr (ESIZE == 2) {
        // key16 << 16 | (0xFFFF - position): one unsigned max keeps the
        // largest key and, among equal keys, the earliest position of this
        // lane.  v_perm_b32 picks bytes of {k, c}: selector 0x05040100 gives
        // (k << 16) | c.lo16, 0x07060100 gives (k & 0xFFFF0000) | c.lo16.
        uint32_t best = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            pace(u);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t k = keys_bf16x2(v[u][d]);
                const uint32_t pos = u * 8 + d * 2;
                const uint32_t lo = __builtin_amdgcn_perm(k, 0xFFFFu - pos, 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(k, 0xFFFFu - (pos + 1), 0x07060100u);
                best = max(best, max(lo, hi));
            }
        }
        const uint32_t pos = 0xFFFFu - (best & 0xFFFFu);
        uint32_t i = i0 + L * (pos >> 3);
        i = i < ilast ? i : ilast;
        take_better(bk, bc, best >> 16, c0 + (int32_t)(i * 8 + (pos & 7)));
    } else {
        uint32_t ck = 0, cpos = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            pace(u);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t k = key_f32(v[u][d]);
                if (k > ck || (u == 0 && d == 0)) {
                    ck = k;
                    cpos = u * 4 + d;
                }
            }
        }
        uint32_t i = i0 + L * (cpos >> 2);
        i = i < ilast ? i : ilast;
        take_better(bk, bc, ck, c0 + (int32_t)(i * 4 + (cpos & 3)));
    }
}

__device__ __forceinline__ uint32_t load_bits(const unsigned char* base, int esize, int64_t e) {
    return esize == 2 ? (uint32_t)((gu16_ptr)base)[e] << 16 : ((gu32_ptr)base)[e];
}

// Group-wide lexicographic maximum of (key, -column) over aligned groups of
// L lanes (L a power of two <= 64), by butterfly shuffles: afterwards every
// lane of a group holds the group's result.  (DPP lane moves were measured
// too: lower latency per wavefront, but 0.5-1 % slower statistics
// launches.)
template <int L>
__device__ __forceinline__ void group_best_key_col(uint32_t& key, int32_t& col) {
#pragma unroll
    for (int off = L >> 1; off >= 1; off >>= 1) {
        const uint32_t ok = __shfl_xor(key, (int)off, 64);
        const int32_t oc = __shfl_xor(col, (int)off, 64);
        take_better(key, col, ok, oc);
    }
}

}  // namespace vpa
