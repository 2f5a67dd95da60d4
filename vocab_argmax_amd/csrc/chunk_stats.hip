// chunk_stats.hip -- the statistics launch of vpa_top_tokens for small
// bf16 batches: a persistent grid that strides over fixed chunks of the
// rows.
//
// vpa_top_tokens only needs each row's argmax (vLLM PR #62604, "Purpose"
// item 2, fused get_top_tokens), and the argmax does not depend on how a
// row's columns are cut into statistics: every statistic keeps its largest
// key and, among equal keys, its smallest column, and the combine takes the
// same order over the statistics.  So this launch cuts each row into chunks
// of kChunkCols columns, the last one shorter, and writes one statistic per
// chunk: (value bits, global column) of the chunk's best element, laid out
// [rows][chunks per row], which the combine kernel reduces as one shard of
// chunks-per-row slots.
//
// Work decomposition (CDNA4, wave64).  Chunk c of the flattened (row, chunk)
// space is read by wavefront c mod W, W = the grid's wavefronts, so at any
// time the grid reads consecutive chunks: a window of about W * 8 KiB of
// contiguous logits that sweeps through the batch.  Two workgroups of four
// wavefronts per CU, 8 KiB chunks (eight 1 KiB wavefront loads).
//
// Schedule of a wavefront.  It issues the next chunk's loads, then folds the
// current chunk, vector u of it only once vector u of the next chunk has
// arrived (explicit waits on the vector-memory counter, which counts loads
// in issue order), waits for the rest of the next chunk and writes the
// current chunk's statistic.  So each wavefront has about one chunk in
// flight, the grid about 16 MiB, and its fold overlaps the next chunk's
// arrival.  Among the schedules measured on MI355X (two chunks in flight;
// one chunk folded as soon as it arrives, with statistics kept in
// registers) this one streamed fastest, and it has little to drain at the
// end of the launch: every wavefront finishes within about one chunk of the
// others.  Above about 410 MB per batch the one-shot per-block launch
// (block_stats.hip) streams faster and is used instead.
//
// Requirements (checked by the host): bf16 logits, V and the row stride
// multiples of 8 elements and a 16-byte aligned base, so every chunk is a
// whole number of aligned 16-byte vectors.  Padding columns [V, ld) are
// never read.
#include "vpa_device.h"
#include "vpa_internal.h"
#include "vpa_scan.h"

#include <atomic>

namespace vpa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupsPerCU = 2;
constexpr int kChunkLoads = 8;                    // 1 KiB wavefront loads per chunk
constexpr int kChunkCols = 64 * 8 * kChunkLoads;  // bf16 columns per chunk: 4096
constexpr int kMaxDevices = 64;

// s_waitcnt vmcnt(n) for n in [0, 7], with expcnt and lgkmcnt at their
// maxima (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8).  n is a constant once the caller's loop is unrolled.
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    }
}

// Fold vector u of the current chunk once vector u of the next chunk (the
// kChunkLoads most recent loads) has arrived.  The scheduling barriers keep
// the compiler from moving the fold's instructions across the wait.
struct PaceByNextChunk {
    __device__ __forceinline__ void operator()(int u) const {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt(kChunkLoads - 1 - u);
        __builtin_amdgcn_sched_barrier(0);
    }
};

struct Chunk {
    int32_t row;   // logits row
    int32_t col0;  // first column
    int32_t nv;    // 16-byte vectors, >= 1
};

__device__ __forceinline__ Chunk chunk_at(int32_t c, int32_t per_row, int32_t vocab) {
    Chunk k;
    k.row = c / per_row;
    k.col0 = (c - k.row * per_row) * kChunkCols;
    const int32_t cols = vocab - k.col0 < kChunkCols ? vocab - k.col0 : kChunkCols;
    k.nv = cols / 8;
    return k;
}

__device__ __forceinline__ void load_chunk(const unsigned char* base, int64_t ld, const Chunk& k,
                                           uint32_t lane, u32x4 (&v)[kChunkLoads]) {
    const gvec_ptr p = (gvec_ptr)(base + ((int64_t)k.row * ld + k.col0) * 2);
    load_clamped<2, 64, kChunkLoads>(p, lane, (uint32_t)(k.nv - 1), v);
}

__global__ __launch_bounds__(kThreads) void chunk_stats_kernel(const unsigned char* base,
                                                                int64_t ld, int32_t vocab,
                                                                int32_t per_row, int32_t n_chunks,
                                                                vpa_stat* __restrict__ stats) {
    const int32_t n_waves = (int32_t)gridDim.x * kWaves;
    int32_t c = (int32_t)blockIdx.x * kWaves +
                __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
    const uint32_t lane = threadIdx.x & 63;
    if (c >= n_chunks)
        return;   // uniform for the wavefront
    u32x4 a[kChunkLoads], b[kChunkLoads];
    Chunk ka = chunk_at(c, per_row, vocab);
    load_chunk(base, ld, ka, lane, a);
    for (;;) {
        const int32_t next = c + n_waves;
        const bool more = next < n_chunks;   // uniform
        Chunk kb = ka;
        if (more) {
            kb = chunk_at(next, per_row, vocab);
            load_chunk(base, ld, kb, lane, b);
        }
        uint32_t bk = 0;
        int32_t bc = INT32_MAX;
        fold_loaded<2, 64, kChunkLoads>(a, lane, (uint32_t)(ka.nv - 1), ka.col0, bk, bc,
                                        PaceByNextChunk());
        group_best_key_col<64>(bk, bc);
        const uint32_t key = __builtin_amdgcn_readfirstlane(bk);
        const int32_t col = __builtin_amdgcn_readfirstlane(bc);
        uint32_t bits;
        if (key == kKeyNanBf16 || key == kKeyZeroBf16)   // uniform: NaN payload or zero sign
            bits = __builtin_amdgcn_readfirstlane(load_bits(base, 2, (int64_t)ka.row * ld + col));
        else
            bits = bits_of_key_bf16(key);
        wait_vmcnt(0);   // the rest of the next chunk
        if (lane == 0) {
            vpa_stat st;
            st.val_bits = bits;
            st.id = col;
            stats[c] = st;
        }
        if (!more)
            break;
        for (int u = 0; u < kChunkLoads; ++u)   // a register copy: the next chunk has arrived
            a[u] = b[u];
        ka = kb;
        c = next;
    }
}

std::atomic<int32_t> g_cus[kMaxDevices];

// Compute units of the current device, looked up once per device.
hipError_t cus_of_current_device(int32_t* out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    int32_t n = g_cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        int v = 0;
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        n = v > 0 ? v : 1;
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return hipSuccess;
}

}  // namespace

int32_t chunk_stats_per_row(int64_t vocab) {
    return (int32_t)((vocab + kChunkCols - 1) / kChunkCols);
}

hipError_t launch_chunk_stats(const void* logits, int64_t ld, int32_t vocab, int32_t n_rows,
                              vpa_stat* stats, hipStream_t stream) {
    const int32_t per_row = chunk_stats_per_row(vocab);
    const int64_t n_chunks = (int64_t)n_rows * per_row;
    if (n_chunks <= 0)
        return hipSuccess;
    if (n_chunks > INT32_MAX)
        return hipErrorInvalidValue;   // the host sends only batches far below this
    int32_t cus = 0;
    hipError_t e = cus_of_current_device(&cus);
    if (e != hipSuccess)
        return e;
    int64_t groups = (int64_t)kGroupsPerCU * cus;
    const int64_t needed = (n_chunks + kWaves - 1) / kWaves;
    groups = groups < needed ? groups : needed;
    return launch(chunk_stats_kernel, dim3((unsigned)groups), dim3(kThreads), 0, stream,
                  (const unsigned char*)logits, ld, vocab, per_row, (int32_t)n_chunks, stats);
}

}  // namespace vpa
