// api.hip -- the C ABI of include/vpa.h: host-side validation, sizing and
// launches.  No HIP call happens before every argument has been checked, so
// invalid calls enqueue nothing and can be exercised without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "vpa_internal.h"

// The statistics of vpa_top_tokens_noalloc: a file-scope device array.
// Every GPU the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): it passes the address
// hipGetSymbolAddress returns for the current device, kept per device
// (scratch_of_current_device below).
static __device__ __align__(256) vpa_stat scratch[VPA_NOALLOC_WORKSPACE_BYTES / sizeof(vpa_stat)];

namespace {

thread_local std::string g_last_error;

vpa_status fail(vpa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

vpa_status hip_fail(hipError_t e, const char* what) {
    return fail(VPA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

vpa_status ok() {
    return VPA_OK;
}

// The dtype argument's integer value.  A C caller may pass any int as a
// vpa_dtype, but in C++ loading an enum outside the range of its
// enumerators is undefined (even to pass it on), so every entry point reads
// its dtype argument's bytes as an int first and works with that int.
int dtype_value(const vpa_dtype* dt) {
    static_assert(sizeof(vpa_dtype) == sizeof(int), "vpa_dtype is int-sized");
    int raw;
    memcpy(&raw, dt, sizeof raw);
    return raw;
}

int esize_of(int dt) {
    return dt == VPA_BF16 ? 2 : (dt == VPA_F32 ? 4 : 0);
}

bool aligned(const void* p, size_t a) {
    return ((uintptr_t)p % a) == 0;
}

// Slots per shard M (the most global blocks any shard touches), -1 if invalid.
// At most VPA_MAX_SHARDS shards, so the scan below stays short.
int64_t slots(int64_t w, int64_t s, int64_t b) {
    if (w < 1 || s < 1 || s > VPA_MAX_SHARDS || b < 1)
        return -1;
    int64_t m = 0;
    for (int64_t i = 0; i < s; ++i) {
        const int64_t lo = i * w;
        const int64_t n = (lo + w - 1) / b - lo / b + 1;
        if (n > m)
            m = n;
    }
    return m;
}

vpa_status check_vocab(const vpa_vocab& v) {
    if (v.vocab < 1 || v.vocab >= VPA_MAX_VOCAB)
        return fail(VPA_ERR_INVALID, "vocab %lld outside [1, 2^24)", (long long)v.vocab);
    if (v.shard_width < 1 || v.shard_width > INT32_MAX)
        return fail(VPA_ERR_INVALID, "shard_width %lld outside [1, 2^31)", (long long)v.shard_width);
    if (v.n_shards < 1 || v.n_shards > VPA_MAX_SHARDS)
        return fail(VPA_ERR_INVALID, "n_shards %d outside [1, %d]", (int)v.n_shards,
                    (int)VPA_MAX_SHARDS);
    if ((int64_t)v.n_shards * v.shard_width < v.vocab)
        return fail(VPA_ERR_INVALID, "n_shards*shard_width = %lld does not cover vocab %lld",
                    (long long)((int64_t)v.n_shards * v.shard_width), (long long)v.vocab);
    return ok();
}

vpa_status check_dtype(int dt) {
    if (esize_of(dt) == 0)
        return fail(VPA_ERR_UNSUPPORTED, "dtype %d is not VPA_F32 or VPA_BF16", dt);
    return ok();
}

// Shared checks of the logits-reading calls; fills `t` with the geometry.
vpa_status check_logits_task(int dt, int64_t ld, const vpa_vocab& v, int32_t first_shard,
                             int32_t n_local, int32_t block, vpa::SegTask& t) {
    vpa_status st;
    if ((st = check_dtype(dt)) != VPA_OK)
        return st;
    if ((st = check_vocab(v)) != VPA_OK)
        return st;
    if (first_shard < 0 || n_local < 1 || (int64_t)first_shard + n_local > v.n_shards)
        return fail(VPA_ERR_INVALID, "shard range [%d, %d+%d) outside [0, %d)", (int)first_shard,
                    (int)first_shard, (int)n_local, (int)v.n_shards);
    if (block < 1)
        return fail(VPA_ERR_INVALID, "block %d < 1", (int)block);
    const int64_t col0 = (int64_t)first_shard * v.shard_width;
    int64_t need = (int64_t)n_local * v.shard_width;
    if (v.vocab - col0 < need)
        need = v.vocab - col0;
    if (need < 1)
        need = 1;
    if (ld < need)
        return fail(VPA_ERR_INVALID, "ld %lld < %lld valid local columns", (long long)ld,
                    (long long)need);
    t = vpa::SegTask{};
    t.ld = ld;
    t.vocab = v.vocab;
    t.shard_width = v.shard_width;
    t.col0 = col0;
    t.first_shard = first_shard;
    t.n_local = n_local;
    t.block = block;
    t.m = (int32_t)slots(v.shard_width, v.n_shards, block);
    return ok();
}

// Pointer checks of the logits, made only when there is work (an empty batch
// may pass the NULL data pointer of an empty tensor).
vpa_status check_logits_ptr(const void* logits, int dt) {
    if (!logits)
        return fail(VPA_ERR_INVALID, "logits is NULL");
    if (!aligned(logits, (size_t)esize_of(dt)))
        return fail(VPA_ERR_INVALID, "logits not aligned to its element size");
    return ok();
}

// The epilogue, resolved: no map and scale 1 when epi is NULL.
struct Epi {
    const int64_t* d2t = nullptr;
    int64_t d2t_len = 0;
    float scale = 1.0f;
};

vpa_status check_epilogue(const vpa_epilogue* epi, int64_t min_len, int64_t* mapped, Epi& e) {
    e = Epi{};
    if (epi) {
        if (!(epi->scale > 0.0f) || !isfinite(epi->scale))
            return fail(VPA_ERR_INVALID, "epilogue scale %g is not finite and positive",
                        (double)epi->scale);
        e.scale = epi->scale;
        if (epi->d2t) {
            if (epi->d2t_len < min_len || epi->d2t_len < 1)
                return fail(VPA_ERR_INVALID, "d2t_len %lld < %lld", (long long)epi->d2t_len,
                            (long long)(min_len > 1 ? min_len : 1));
            if (!aligned(epi->d2t, 8))
                return fail(VPA_ERR_INVALID, "d2t not 8-byte aligned");
            e.d2t = epi->d2t;
            e.d2t_len = epi->d2t_len;
        }
    }
    if ((e.d2t != nullptr) != (mapped != nullptr))
        return fail(VPA_ERR_INVALID, "mapped ids are required exactly when a d2t table is given");
    if (mapped && !aligned(mapped, 8))
        return fail(VPA_ERR_INVALID, "mapped not 8-byte aligned");
    return ok();
}

vpa_status check_dispatch(int64_t threads, const char* what) {
    if (threads > vpa::kMaxDispatchThreads)
        return fail(VPA_ERR_INVALID, "%s: %lld work-items exceed one dispatch (2^32 - 1)", what,
                    (long long)threads);
    return ok();
}

vpa_status set_items(vpa::SegTask& t, int64_t n_rows, const char* what) {
    if (n_rows > INT32_MAX)
        return fail(VPA_ERR_INVALID, "%s: %lld rows exceed 2^31-1 per call", what,
                    (long long)n_rows);
    const int64_t per_row = (int64_t)t.n_local * t.m;   // < 2^24 * 2^31
    if (per_row > INT32_MAX || n_rows > INT32_MAX / per_row)
        return fail(VPA_ERR_INVALID, "%s: %lld rows x %lld statistics exceed 2^31-1 per call",
                    what, (long long)n_rows, (long long)per_row);
    const int64_t items = n_rows * per_row;
    t.n_rows = (int32_t)n_rows;
    t.n_items = (int32_t)items;
    return ok();
}

// Batches of bf16 logits up to this size (1024 rows of a 200064-entry
// vocabulary) take their vpa_top_tokens statistics from the chunked launch
// (chunk_stats.hip); larger ones from the per-block launch, which streams
// faster once the batch is large enough to amortise its longer drain.  On
// MI355X the chunked launch measured 0.5-4.7 % faster from 96 to 1024 rows
// of 200064 and slower from 1152.
constexpr int64_t kChunkMaxBytes = (int64_t)1024 * 200064 * 2;

// Whether vpa_top_tokens' statistics of these logits may come from the
// chunked launch, as far as the sizes tell (dtype and alignment aside).
bool chunk_sizes(const vpa_vocab& v, int64_t ld, int64_t n_rows) {
    return v.vocab % 8 == 0 && ld % 8 == 0 && n_rows > 0 &&
           n_rows <= kChunkMaxBytes / (2 * v.vocab);
}

// A validated vpa_top_tokens call: the statistics task over all S shards of
// every row ([S][n_rows][M], as vpa_block_stats cuts them), or, for small
// bf16 batches, the chunked statistics ([n_rows][chunk_m]); the workspace
// bytes it needs, and the resolved epilogue.  (Cutting each row at global
// block edges only, ignoring shard edges, cutting the launch's last rows
// into smaller blocks and cutting each shard into equal parts were
// measured for the per-block launch; none was faster.)
struct TopCall {
    vpa::SegTask task;
    size_t ws_bytes;
    Epi epi;
    int esize;
    bool chunks;
    int32_t chunk_m;
};

vpa_status check_top_tokens(const void* logits, int dtype, int64_t ld, const vpa_vocab& v,
                            int64_t n_rows, int32_t block, const vpa_epilogue* epi,
                            const int32_t* ids, const uint32_t* val_bits, int64_t* mapped,
                            TopCall& c) {
    vpa_status st = check_logits_task(dtype, ld, v, 0, v.n_shards, block, c.task);
    if (st != VPA_OK)
        return st;
    if ((st = check_epilogue(epi, v.vocab, mapped, c.epi)) != VPA_OK)
        return st;
    if (n_rows < 0)
        return fail(VPA_ERR_INVALID, "n_rows %lld < 0", (long long)n_rows);
    if ((st = set_items(c.task, n_rows, "vpa_top_tokens")) != VPA_OK)
        return st;
    c.ws_bytes = (size_t)c.task.n_items * sizeof(vpa_stat);
    if (n_rows == 0)
        return ok();
    if ((st = check_logits_ptr(logits, dtype)) != VPA_OK)
        return st;
    if (!ids || !aligned(ids, 4) || (val_bits && !aligned(val_bits, 4)))
        return fail(VPA_ERR_INVALID, "ids is NULL, or ids/val_bits not 4-byte aligned");
    c.esize = esize_of(dtype);
    c.task.base = (const unsigned char*)logits;
    c.task.logits_rows = n_rows;
    c.chunks = dtype == VPA_BF16 && aligned(logits, 16) && chunk_sizes(v, ld, n_rows);
    c.chunk_m = c.chunks ? vpa::chunk_stats_per_row(v.vocab) : 0;
    if (c.chunks)
        c.ws_bytes = (size_t)n_rows * (size_t)c.chunk_m * sizeof(vpa_stat);
    vpa::SegTask none{};
    if ((st = check_dispatch(vpa::block_stats_threads(c.esize, c.task, none),
                             "vpa_top_tokens (statistics)")) != VPA_OK ||
        (st = check_dispatch(vpa::combine_threads((int32_t)n_rows), "vpa_top_tokens (combine)")) !=
            VPA_OK)
        return st;
    return ok();
}

// The two launches of a checked call, with its statistics in `ws`.
vpa_status launch_top_tokens(TopCall& c, vpa_stat* ws, int32_t* ids, uint32_t* val_bits,
                             int64_t* mapped, hipStream_t stream) {
    c.task.stats = ws;
    vpa::SegTask none{};
    hipError_t e = c.chunks ? vpa::launch_chunk_stats(c.task.base, c.task.ld,
                                                      (int32_t)c.task.vocab, c.task.n_rows, ws,
                                                      stream)
                            : vpa::launch_block_stats(c.esize, c.task, none, stream);
    if (e != hipSuccess)
        return hip_fail(e, "vpa_top_tokens statistics launch");
    if (c.chunks)
        e = vpa::launch_combine(ws, 1, c.task.n_rows, c.chunk_m, c.epi.d2t, c.epi.d2t_len,
                                c.epi.scale, ids, val_bits, mapped, stream);
    else
        e = vpa::launch_combine(ws, c.task.n_local, c.task.n_rows, c.task.m, c.epi.d2t,
                                c.epi.d2t_len, c.epi.scale, ids, val_bits, mapped, stream);
    return e == hipSuccess ? ok() : hip_fail(e, "vpa_top_tokens combine launch");
}

constexpr int kMaxDevices = 64;
std::atomic<vpa_stat*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up once per device.
vpa_status scratch_of_current_device(vpa_stat** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "vpa_top_tokens_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(VPA_ERR_UNSUPPORTED, "vpa_top_tokens_noalloc: device %d beyond the %d supported",
                    dev, kMaxDevices);
    vpa_stat* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return hip_fail(e, "vpa_top_tokens_noalloc: hipGetSymbolAddress(scratch)");
            p = (vpa_stat*)addr;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return ok();
}

}  // namespace

extern "C" {

int32_t vpa_stats_slots(int64_t shard_width, int32_t n_shards, int32_t block) {
    const int64_t m = slots(shard_width, n_shards, block);
    return m > INT32_MAX ? -1 : (int32_t)m;
}

vpa_status vpa_block_stats(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                           int32_t first_shard, int32_t n_local_shards, const int32_t* rows,
                           int64_t n_rows, int64_t logits_rows, int32_t block, vpa_stat* stats,
                           void* stream) {
    const int dt = dtype_value(&dtype);
    vpa::SegTask t;
    vpa_status st = check_logits_task(dt, ld, v, first_shard, n_local_shards, block, t);
    if (st != VPA_OK)
        return st;
    if (n_rows < 0)
        return fail(VPA_ERR_INVALID, "n_rows %lld < 0", (long long)n_rows);
    if (rows ? logits_rows < 0 : logits_rows < n_rows)
        return fail(VPA_ERR_INVALID, "logits_rows %lld too small", (long long)logits_rows);
    if ((st = set_items(t, n_rows, "vpa_block_stats")) != VPA_OK)
        return st;
    if (n_rows == 0)
        return ok();
    if ((st = check_logits_ptr(logits, dt)) != VPA_OK)
        return st;
    if (!stats || !aligned(stats, 8))
        return fail(VPA_ERR_INVALID, "stats is NULL or not 8-byte aligned");
    if (rows && !aligned(rows, 4))
        return fail(VPA_ERR_INVALID, "rows not 4-byte aligned");
    t.base = (const unsigned char*)logits;
    t.rows = rows;
    t.logits_rows = logits_rows;
    t.stats = stats;
    vpa::SegTask none{};
    if ((st = check_dispatch(vpa::block_stats_threads(esize_of(dt), t, none),
                             "vpa_block_stats")) != VPA_OK)
        return st;
    hipError_t e = vpa::launch_block_stats(esize_of(dt), t, none, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "vpa_block_stats launch");
}

vpa_status vpa_verify_stats(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                            int32_t first_shard, int32_t n_local_shards, int64_t n_req, int32_t k,
                            int32_t block_draft, int32_t block_bonus, vpa_stat* draft_stats,
                            vpa_stat* bonus_stats, void* stream) {
    const int dt = dtype_value(&dtype);
    vpa::SegTask td, tb;
    vpa_status st;
    if ((st = check_logits_task(dt, ld, v, first_shard, n_local_shards, block_draft, td)) != VPA_OK)
        return st;
    if ((st = check_logits_task(dt, ld, v, first_shard, n_local_shards, block_bonus, tb)) != VPA_OK)
        return st;
    if (k < 1 || k > VPA_MAX_DRAFTS)
        return fail(VPA_ERR_INVALID, "k %d outside [1, %d]", (int)k, VPA_MAX_DRAFTS);
    if (n_req < 0 || n_req > INT32_MAX / (k + 1))   // n_req * (k+1) <= 2^31-1, no overflow
        return fail(VPA_ERR_INVALID, "n_req %lld out of range", (long long)n_req);
    if ((st = set_items(td, n_req * k, "vpa_verify_stats (draft rows)")) != VPA_OK)
        return st;
    if ((st = set_items(tb, n_req, "vpa_verify_stats (bonus rows)")) != VPA_OK)
        return st;
    if ((int64_t)td.n_items + tb.n_items > INT32_MAX)
        return fail(VPA_ERR_INVALID, "vpa_verify_stats: too many statistics per call");
    if (n_req == 0)
        return ok();
    if ((st = check_logits_ptr(logits, dt)) != VPA_OK)
        return st;
    if (!draft_stats || !bonus_stats || !aligned(draft_stats, 8) || !aligned(bonus_stats, 8))
        return fail(VPA_ERR_INVALID, "draft_stats/bonus_stats NULL or not 8-byte aligned");
    const int64_t logits_rows = n_req * (int64_t)(k + 1);
    td.base = tb.base = (const unsigned char*)logits;
    td.row_k = k;
    td.row_bonus = 0;
    td.logits_rows = logits_rows;
    td.stats = draft_stats;
    tb.row_k = k;
    tb.row_bonus = 1;
    tb.logits_rows = logits_rows;
    tb.stats = bonus_stats;
    if ((st = check_dispatch(vpa::block_stats_threads(esize_of(dt), td, tb),
                             "vpa_verify_stats")) != VPA_OK)
        return st;
    hipError_t e = vpa::launch_block_stats(esize_of(dt), td, tb, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "vpa_verify_stats launch");
}

vpa_status vpa_verify_stats_rows(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                                 int32_t first_shard, int32_t n_local_shards,
                                 const int32_t* draft_rows, int64_t n_draft_rows,
                                 const int32_t* bonus_rows, int64_t n_bonus_rows,
                                 int64_t logits_rows, int32_t block_draft, int32_t block_bonus,
                                 vpa_stat* draft_stats, vpa_stat* bonus_stats, void* stream) {
    const int dt = dtype_value(&dtype);
    vpa::SegTask td, tb;
    vpa_status st;
    if ((st = check_logits_task(dt, ld, v, first_shard, n_local_shards, block_draft, td)) != VPA_OK)
        return st;
    if ((st = check_logits_task(dt, ld, v, first_shard, n_local_shards, block_bonus, tb)) != VPA_OK)
        return st;
    if (n_draft_rows < 0 || n_bonus_rows < 0 || logits_rows < 0)
        return fail(VPA_ERR_INVALID, "negative row count");
    if ((st = set_items(td, n_draft_rows, "vpa_verify_stats_rows (draft rows)")) != VPA_OK)
        return st;
    if ((st = set_items(tb, n_bonus_rows, "vpa_verify_stats_rows (bonus rows)")) != VPA_OK)
        return st;
    if ((int64_t)td.n_items + tb.n_items > INT32_MAX)
        return fail(VPA_ERR_INVALID, "vpa_verify_stats_rows: too many statistics per call");
    if (n_draft_rows == 0 && n_bonus_rows == 0)
        return ok();
    if ((st = check_logits_ptr(logits, dt)) != VPA_OK)
        return st;
    if ((n_draft_rows && (!draft_rows || !aligned(draft_rows, 4) || !draft_stats ||
                          !aligned(draft_stats, 8))) ||
        (n_bonus_rows && (!bonus_rows || !aligned(bonus_rows, 4) || !bonus_stats ||
                          !aligned(bonus_stats, 8))))
        return fail(VPA_ERR_INVALID, "row list or statistics NULL or misaligned");
    td.base = tb.base = (const unsigned char*)logits;
    td.rows = draft_rows;
    td.logits_rows = logits_rows;
    td.stats = draft_stats;
    tb.rows = bonus_rows;
    tb.logits_rows = logits_rows;
    tb.stats = bonus_stats;
    if ((st = check_dispatch(vpa::block_stats_threads(esize_of(dt), td, tb),
                             "vpa_verify_stats_rows")) != VPA_OK)
        return st;
    hipError_t e = vpa::launch_block_stats(esize_of(dt), td, tb, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "vpa_verify_stats_rows launch");
}

vpa_status vpa_ragged_rows(const int32_t* cu, int64_t n_req, int64_t total_drafts,
                           int32_t* draft_rows, int32_t* bonus_rows, void* stream) {
    if (n_req < 0 || total_drafts < 0 || n_req > INT32_MAX || total_drafts > INT32_MAX - n_req)
        return fail(VPA_ERR_INVALID, "n_req %lld / total_drafts %lld out of range",
                    (long long)n_req, (long long)total_drafts);
    if (n_req == 0)
        return ok();
    if (!cu || !bonus_rows || (total_drafts && !draft_rows) || !aligned(cu, 4) ||
        !aligned(bonus_rows, 4) || (draft_rows && !aligned(draft_rows, 4)))
        return fail(VPA_ERR_INVALID, "cu/draft_rows/bonus_rows NULL or not 4-byte aligned");
    hipError_t e = vpa::launch_ragged_rows(cu, (int32_t)n_req, (int32_t)total_drafts, draft_rows,
                                           bonus_rows, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "vpa_ragged_rows launch");
}

vpa_status vpa_combine_stats(const vpa_stat* stats, int32_t n_shards, int64_t n_rows, int32_t m,
                             const vpa_epilogue* epi, int32_t* ids, uint32_t* val_bits,
                             int64_t* mapped, void* stream) {
    if (n_shards < 1 || m < 1 || (int64_t)n_shards * m > INT32_MAX)
        return fail(VPA_ERR_INVALID, "n_shards %d / m %d invalid", (int)n_shards, (int)m);
    if (n_rows < 0 || n_rows > INT32_MAX)
        return fail(VPA_ERR_INVALID, "n_rows %lld out of range", (long long)n_rows);
    Epi e;
    vpa_status st = check_epilogue(epi, 1, mapped, e);
    if (st != VPA_OK)
        return st;
    if (n_rows == 0)
        return ok();
    if (!stats || !aligned(stats, 8))
        return fail(VPA_ERR_INVALID, "stats is NULL or not 8-byte aligned");
    if (!ids || !aligned(ids, 4) || (val_bits && !aligned(val_bits, 4)))
        return fail(VPA_ERR_INVALID, "ids is NULL, or ids/val_bits not 4-byte aligned");
    if ((st = check_dispatch(vpa::combine_threads((int32_t)n_rows), "vpa_combine_stats")) != VPA_OK)
        return st;
    hipError_t he = vpa::launch_combine(stats, n_shards, (int32_t)n_rows, m, e.d2t, e.d2t_len,
                                        e.scale, ids, val_bits, mapped, (hipStream_t)stream);
    return he == hipSuccess ? ok() : hip_fail(he, "vpa_combine_stats launch");
}

size_t vpa_top_tokens_workspace(vpa_vocab v, int64_t n_rows, int32_t block) {
    if (n_rows <= 0 || n_rows > INT32_MAX || v.vocab < 1 || v.vocab >= VPA_MAX_VOCAB ||
        v.n_shards < 1 || v.n_shards > VPA_MAX_SHARDS || v.shard_width < 1 ||
        v.shard_width > INT32_MAX || (int64_t)v.n_shards * v.shard_width < v.vocab)
        return 0;
    const int64_t m = slots(v.shard_width, v.n_shards, block);
    if (m < 1)
        return 0;
    // A call is limited to 2^31-1 statistics; larger sizes get 0 (and the
    // products below cannot overflow: S < 2^25 and M < 2^32).
    const int64_t per_row = (int64_t)v.n_shards * m;
    if (per_row > INT32_MAX || n_rows > INT32_MAX / per_row)
        return 0;
    size_t need = (size_t)(per_row * n_rows) * sizeof(vpa_stat);
    // The row stride and the dtype are not known here: whenever the sizes
    // allow the chunked statistics, the workspace covers them too.
    if (chunk_sizes(v, v.vocab, n_rows)) {
        const size_t chunks = (size_t)n_rows * (size_t)vpa::chunk_stats_per_row(v.vocab) *
                              sizeof(vpa_stat);
        need = chunks > need ? chunks : need;
    }
    return need;
}

vpa_status vpa_top_tokens(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                          int64_t n_rows, int32_t block, void* workspace, size_t workspace_bytes,
                          const vpa_epilogue* epi, int32_t* ids, uint32_t* val_bits,
                          int64_t* mapped, void* stream) {
    const int dt = dtype_value(&dtype);
    TopCall c;
    vpa_status st = check_top_tokens(logits, dt, ld, v, n_rows, block, epi, ids, val_bits,
                                     mapped, c);
    if (st != VPA_OK || n_rows == 0)
        return st;
    if (!workspace || !aligned(workspace, 8) || workspace_bytes < c.ws_bytes)
        return fail(VPA_ERR_INVALID, "workspace NULL, unaligned or smaller than %zu bytes",
                    c.ws_bytes);
    return launch_top_tokens(c, (vpa_stat*)workspace, ids, val_bits, mapped, (hipStream_t)stream);
}

vpa_status vpa_top_tokens_noalloc(const void* logits, vpa_dtype dtype, int64_t ld, vpa_vocab v,
                                  int64_t n_rows, int32_t block, const vpa_epilogue* epi,
                                  int32_t* ids, uint32_t* val_bits, int64_t* mapped,
                                  void* stream) {
    const int dt = dtype_value(&dtype);
    TopCall c;
    vpa_status st = check_top_tokens(logits, dt, ld, v, n_rows, block, epi, ids, val_bits,
                                     mapped, c);
    if (st != VPA_OK || n_rows == 0)
        return st;
    if (c.ws_bytes > (size_t)VPA_NOALLOC_WORKSPACE_BYTES)
        return fail(VPA_ERR_INVALID,
                    "vpa_top_tokens_noalloc: %lld rows need %zu bytes of statistics, more than the "
                    "%zu the library holds (VPA_NOALLOC_WORKSPACE_BYTES); use vpa_top_tokens",
                    (long long)n_rows, c.ws_bytes, (size_t)VPA_NOALLOC_WORKSPACE_BYTES);
    vpa_stat* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != VPA_OK)
        return st;
    return launch_top_tokens(c, ws, ids, val_bits, mapped, (hipStream_t)stream);
}

vpa_status vpa_greedy_verify(const vpa_stat* draft_stats, int32_t m_draft,
                             const vpa_stat* bonus_stats, int32_t m_bonus, int32_t n_shards,
                             int64_t n_req, int32_t k, const int32_t* draft_ids,
                             const int32_t* accept, int32_t* out_tokens, int32_t* num_sampled,
                             int32_t* num_rejected, int32_t* target_ids, void* stream) {
    if (n_shards < 1 || m_draft < 1 || m_bonus < 1 || (int64_t)n_shards * m_draft > INT32_MAX ||
        (int64_t)n_shards * m_bonus > INT32_MAX)
        return fail(VPA_ERR_INVALID, "n_shards %d / m_draft %d / m_bonus %d invalid",
                    (int)n_shards, (int)m_draft, (int)m_bonus);
    if (k < 1 || k > VPA_MAX_DRAFTS)
        return fail(VPA_ERR_INVALID, "k %d outside [1, %d]", (int)k, VPA_MAX_DRAFTS);
    if (n_req < 0 || n_req > INT32_MAX / (k + 1))   // n_req * (k+1) <= 2^31-1, no overflow
        return fail(VPA_ERR_INVALID, "n_req %lld out of range", (long long)n_req);
    if (n_req == 0)
        return ok();
    if (!draft_stats || !bonus_stats || !aligned(draft_stats, 8) || !aligned(bonus_stats, 8))
        return fail(VPA_ERR_INVALID, "draft_stats/bonus_stats NULL or not 8-byte aligned");
    if (!draft_ids || !out_tokens || !num_sampled || !num_rejected)
        return fail(VPA_ERR_INVALID, "draft_ids/out_tokens/num_sampled/num_rejected is NULL");
    if (!aligned(draft_ids, 4) || !aligned(out_tokens, 4) || !aligned(num_sampled, 4) ||
        !aligned(num_rejected, 4) || (target_ids && !aligned(target_ids, 4)) ||
        (accept && !aligned(accept, 4)))
        return fail(VPA_ERR_INVALID, "an int32 array is not 4-byte aligned");
    vpa_status st = check_dispatch(vpa::greedy_verify_threads((int32_t)n_req, k), "vpa_greedy_verify");
    if (st != VPA_OK)
        return st;
    hipError_t e = vpa::launch_greedy_verify(draft_stats, m_draft, bonus_stats, m_bonus, n_shards,
                                             (int32_t)n_req, k, draft_ids, accept, out_tokens,
                                             num_sampled, num_rejected, target_ids,
                                             (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "vpa_greedy_verify launch");
}

vpa_status vpa_greedy_verify_ragged(const vpa_stat* draft_stats, int32_t m_draft,
                                    const vpa_stat* bonus_stats, int32_t m_bonus,
                                    int32_t n_shards, int64_t n_req, const int32_t* cu,
                                    int64_t total_drafts, const int32_t* draft_ids,
                                    const uint8_t* prefilling, const int32_t* accept,
                                    int32_t* out_tokens, int32_t* num_sampled,
                                    int32_t* num_rejected, int32_t* target_ids, void* stream) {
    if (n_shards < 1 || m_draft < 1 || m_bonus < 1 || (int64_t)n_shards * m_draft > INT32_MAX ||
        (int64_t)n_shards * m_bonus > INT32_MAX)
        return fail(VPA_ERR_INVALID, "n_shards %d / m_draft %d / m_bonus %d invalid",
                    (int)n_shards, (int)m_draft, (int)m_bonus);
    if (n_req < 0 || total_drafts < 0 || n_req > INT32_MAX || total_drafts > INT32_MAX - n_req)
        return fail(VPA_ERR_INVALID, "n_req %lld / total_drafts %lld out of range",
                    (long long)n_req, (long long)total_drafts);
    if (n_req == 0)
        return ok();
    if (!cu || !bonus_stats || !out_tokens || !num_sampled || !num_rejected ||
        (total_drafts && (!draft_stats || !draft_ids)))
        return fail(VPA_ERR_INVALID, "a required pointer is NULL");
    if (!aligned(cu, 4) || !aligned(bonus_stats, 8) || (draft_stats && !aligned(draft_stats, 8)) ||
        (draft_ids && !aligned(draft_ids, 4)) || !aligned(out_tokens, 4) ||
        !aligned(num_sampled, 4) || !aligned(num_rejected, 4) ||
        (target_ids && !aligned(target_ids, 4)) || (accept && !aligned(accept, 4)))
        return fail(VPA_ERR_INVALID, "a pointer is misaligned");
    vpa_status st =
        check_dispatch(vpa::greedy_verify_ragged_threads((int32_t)n_req), "vpa_greedy_verify_ragged");
    if (st != VPA_OK)
        return st;
    hipError_t e = vpa::launch_greedy_verify_ragged(
        draft_stats, m_draft, bonus_stats, m_bonus, n_shards, (int32_t)n_req, cu,
        (int32_t)total_drafts, draft_ids, prefilling, accept, out_tokens, num_sampled,
        num_rejected, target_ids, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "vpa_greedy_verify_ragged launch");
}

const char* vpa_last_error(void) {
    return g_last_error.c_str();
}

}  // extern "C"
