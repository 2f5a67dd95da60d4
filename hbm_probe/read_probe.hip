// read_probe.hip -- the practical HBM read ceiling, for reporting beside the
// statistics kernel's roofline.  Not part of the argmax path: libvpa_probe.so
// is built from this file alone (hbm_probe/build.py) and only the benchmark
// and its test load it.
//
// A persistent grid of 256-thread workgroups walks the buffer in 4 KiB chunks
// (one chunk = four 1 KiB wavefront-wide loads, 16-byte non-temporal loads
// as in the statistics kernel), grid-stride, loading chunk c + (grid waves)
// before folding chunk c.  Each thread XORs what it loaded; the XOR of all
// sink words is the XOR of every 32-bit word read, which lets a test check
// that every byte of the read range was read exactly once.  On MI355X two
// workgroups per CU measured fastest among 1-14.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vpa_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* gvec_ptr;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoads = 4;                                  // 1 KiB wavefront loads per chunk
constexpr int64_t kChunkBytes = 64 * 16 * kLoads;          // 4 KiB

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* p, int64_t n_chunks,
                                                              uint32_t* sink) {
    const int64_t n_waves = (int64_t)gridDim.x * kWaves;
    const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    const gvec_ptr g = (gvec_ptr)p;
    u32x4 acc = {0, 0, 0, 0};
    u32x4 a[kLoads], b[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        a[u] = acc;
        b[u] = acc;
    }
    int64_t c = wave;
    if (c < n_chunks) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            a[u] = __builtin_nontemporal_load(g + c * (64 * kLoads) + lane + 64 * u);
    }
    for (; c < n_chunks; c += n_waves) {
        const int64_t nc = c + n_waves;
        if (nc < n_chunks) {
#pragma unroll
            for (int u = 0; u < kLoads; ++u)
                b[u] = __builtin_nontemporal_load(g + nc * (64 * kLoads) + lane + 64 * u);
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            acc ^= a[u];
            a[u] = b[u];
        }
    }
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

int64_t vpa_probe_read_bytes(int64_t bytes) {
    return bytes > 0 ? bytes / kChunkBytes * kChunkBytes : 0;
}

int64_t vpa_probe_sink_words(int32_t n_workgroups) {
    return n_workgroups > 0 ? (int64_t)n_workgroups * kThreads : 0;
}

int vpa_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t n_workgroups,
                   void* stream) {
    const int64_t n_chunks = vpa_probe_read_bytes(bytes) / kChunkBytes;
    if (n_chunks < 1 || !buf || ((uintptr_t)buf & 15) || !sink || ((uintptr_t)sink & 3) ||
        n_workgroups < 1 || n_workgroups > (1 << 20))
        return -1;
    void* args[] = {(void*)&buf, (void*)&n_chunks, (void*)&sink};
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(read_probe_kernel),
                                dim3((unsigned)n_workgroups), dim3(kThreads), args, 0,
                                (hipStream_t)stream);
}

}  // extern "C"
