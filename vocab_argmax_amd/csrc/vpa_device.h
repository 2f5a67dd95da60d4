// vpa_device.h -- device helpers shared by the libvpa kernels: the ordering of
// logits values as unsigned integer keys, and wave-level reductions.
//
// The ordering is the one vLLM PR #62604 ("Purpose", item 2) gives for the
// fused get_top_tokens: torch.argmax's, i.e. a larger value wins, every NaN
// beats every number, equal values (-0 and +0 included) and NaNs among
// themselves go to the lowest token id.  Mapping each fp32 bit pattern to a
// key that preserves this order lets every comparison be one unsigned compare
// and keeps values untouched (no canonicalised NaN, no flushed subnormal, no
// zero sign chosen by a float max instruction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vpa {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// Key of an fp32 bit pattern f.  With neg = all ones for a set sign bit:
//   x = f ^ (neg | 0x80000000)       (~f for negatives, f + 2^31 otherwise)
//   y = x + 0xFF800000 + (neg & 1)   (mod 2^32)
// gives -inf -> 0, -0 and +0 -> 0x7F800000, +inf -> 0xFF000000 in value order;
// every NaN lands in (0xFF000000, 2^32) and min(y, 0xFF000001) collapses them
// to one key above +inf.  Real keys are >= 0; an empty candidate is key 0
// with an id above every real one.
constexpr uint32_t kKeyZeroF32 = 0x7F800000u;
constexpr uint32_t kKeyNanF32 = 0xFF000001u;

__device__ __forceinline__ uint32_t key_f32(uint32_t f) {
    const uint32_t neg = (uint32_t)((int32_t)f >> 31);
    const uint32_t x = f ^ (neg | 0x80000000u);
    const uint32_t y = x + ((neg & 1u) | 0xFF800000u);
    return y < kKeyNanF32 ? y : kKeyNanF32;
}

// fp32 bits of a key other than kKeyZeroF32 / kKeyNanF32 (those collapse
// several patterns; the element is re-read instead).
__device__ __forceinline__ uint32_t bits_of_key_f32(uint32_t k) {
    return k > kKeyZeroF32 ? k - kKeyZeroF32 : 0x80000000u | (kKeyZeroF32 - k);
}

// The same map on 16-bit bf16 patterns, for both halves of a 32-bit word at
// once (packed 16-bit ops): -inf -> 0, +-0 -> 0x7F80, +inf -> 0xFF00,
// NaN -> 0xFF01.
constexpr uint32_t kKeyZeroBf16 = 0x7F80u;
constexpr uint32_t kKeyNanBf16 = 0xFF01u;

// v_bitop3_b32 truth tables, operands (a, b, c) weighted 0xF0, 0xCC, 0xAA.
constexpr unsigned kB3XorOr = 0x36;   // b ^ (a | c)
constexpr unsigned kB3AndOr = 0xEA;   // (a & b) | c

__device__ __forceinline__ uint32_t keys_bf16x2(uint32_t w) {
    const uint32_t neg =
        __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> (i16x2){15, 15});
    const uint32_t x = __builtin_amdgcn_bitop3_b32(neg, w, 0x80008000u, kB3XorOr);
    const uint32_t c = __builtin_amdgcn_bitop3_b32(neg, 0x00010001u, 0xFF80FF80u, kB3AndOr);
    const u16x2 y = __builtin_bit_cast(u16x2, x) + __builtin_bit_cast(u16x2, c);
    const u16x2 k = __builtin_elementwise_min(y, (u16x2){(unsigned short)kKeyNanBf16,
                                                         (unsigned short)kKeyNanBf16});
    return __builtin_bit_cast(uint32_t, k);
}

// Scalar form for one bf16 pattern h (16 bits).
__device__ __forceinline__ uint32_t key_bf16(uint32_t h) {
    const uint32_t neg = (h & 0x8000u) ? 0xFFFFu : 0u;
    const uint32_t y = ((h ^ (neg | 0x8000u)) + ((neg & 1u) | 0xFF80u)) & 0xFFFFu;
    return y < kKeyNanBf16 ? y : kKeyNanBf16;
}

// fp32 bits (bf16 widened) of a bf16 key other than kKeyZeroBf16 / kKeyNanBf16.
__device__ __forceinline__ uint32_t bits_of_key_bf16(uint32_t k) {
    const uint32_t h = k > kKeyZeroBf16 ? k - kKeyZeroBf16 : 0x8000u | (kKeyZeroBf16 - k);
    return h << 16;
}

// Cross-lane reductions with DPP lane moves (no LDS round trips).  A step
// moves a value from a partner lane within the same row of 16 lanes
// (quad_perm, row_half_mirror, row_mirror) or broadcasts the last lane of
// a row into the next rows (row_bcast:15, row_bcast:31).  Rows left out by
// row_mask keep their own value, so combining it with itself is a no-op.
// After all six steps, lane 63 holds the wavefront's result.
namespace dpp {
constexpr int kSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kBcast15 = 0x142;    // lane 15 of a row -> the next row
constexpr int kBcast31 = 0x143;    // lane 31 -> rows 2 and 3
}  // namespace dpp

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// One step of the maximum of (key, nid) carrying the winner's value bits;
// `nid` is the bitwise NOT of the token id, so a larger nid is a lower id.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void stat_step(uint32_t& key, uint32_t& nid, uint32_t& bits) {
    const uint32_t ok = dpp_move<CTRL, ROW_MASK>(key);
    const uint32_t on = dpp_move<CTRL, ROW_MASK>(nid);
    const uint32_t ob = dpp_move<CTRL, ROW_MASK>(bits);
    const bool take = ok > key || (ok == key && on > nid);
    key = take ? ok : key;
    nid = take ? on : nid;
    bits = take ? ob : bits;
}

// Wave-wide maximum of (key, nid) with the winner's bits; afterwards every
// lane holds the result.  Start a lane with nothing as (0, 0, any bits).
// Every lane of the wavefront must be active.
__device__ __forceinline__ void wave_best_stat(uint32_t& key, uint32_t& nid, uint32_t& bits) {
    stat_step<dpp::kSwap1, 0xF>(key, nid, bits);
    stat_step<dpp::kSwap2, 0xF>(key, nid, bits);
    stat_step<dpp::kHalfMirror, 0xF>(key, nid, bits);
    stat_step<dpp::kMirror, 0xF>(key, nid, bits);
    stat_step<dpp::kBcast15, 0xA>(key, nid, bits);
    stat_step<dpp::kBcast31, 0xC>(key, nid, bits);
    key = __builtin_amdgcn_readlane(key, 63);
    nid = __builtin_amdgcn_readlane(nid, 63);
    bits = __builtin_amdgcn_readlane(bits, 63);
}

}  // namespace vpa
