// Device ceilings for the measurement: how fast a plain kernel streams a large
// buffer out of HBM, reading only.  The decode step's scoring and attention
// kernels are read streams; their bandwidth is reported against the vendor
// peak and against this measured ceiling.
#include <hip/hip_runtime.h>

#include <dlfcn.h>

#include <algorithm>
#include <vector>

#include "shadowkv.h"
#include "skv_device.h"

namespace skv {

// Each thread keeps U independent 16-byte loads in flight per iteration
// (grid-stride, consecutive lanes on consecutive vectors: every wave reads
// whole 1 KiB runs) and folds them into an xor the compiler cannot drop; the
// xor is stored only if it equals `magic`, which the host picks so that no
// store happens in practice, so the kernel moves no bytes but its reads.
template <int U>
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *__restrict__ p, size_t n_vec, uint32_t magic,
                                                         uint32_t *__restrict__ sink) {
    const size_t stride = static_cast<size_t>(gridDim.x) * 256;
    size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (U - 1) * stride < n_vec; i += U * stride) {
        u32x4 t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) t[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= t[u];
    }
    for (; i < n_vec; i += stride) acc ^= p[i];
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (x == magic) sink[0] = x;
}

}  // namespace skv

extern "C" int shadowkv_probe_hbm_read(const void *buf, size_t bytes, int reps, void *stream, double *gbps_out) {
    if (!buf || !gbps_out || reps < 1 || bytes < (1u << 20)) return SKV_E_INVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t n_vec = bytes / 16;
    uint32_t *sink = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = SKV_OK;
    double best = 0.0;
    if (hipMalloc(&sink, 256) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
        hipEventCreate(&e1) != hipSuccess) {
        rc = SKV_E_HIP;
    } else {
        // a few grid sizes and load depths; the best is the ceiling
        const int grids[] = {1024, 2048, 4096, 8192};
        for (int g : grids) {
            for (int u = 0; u < 2 && rc == SKV_OK; ++u) {
                auto launch = [&]() {
                    if (u == 0)
                        hipLaunchKernelGGL(skv::read_probe_kernel<4>, dim3(g), dim3(256), 0, st,
                                           static_cast<const skv::u32x4 *>(buf), n_vec, 0x9e3779b9u, sink);
                    else
                        hipLaunchKernelGGL(skv::read_probe_kernel<8>, dim3(g), dim3(256), 0, st,
                                           static_cast<const skv::u32x4 *>(buf), n_vec, 0x9e3779b9u, sink);
                };
                launch();  // warm
                if (hipEventRecord(e0, st) != hipSuccess) { rc = SKV_E_HIP; break; }
                for (int r = 0; r < reps; ++r) launch();
                float ms = 0.f;
                if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                    hipEventElapsedTime(&ms, e0, e1) != hipSuccess || hipGetLastError() != hipSuccess) {
                    rc = SKV_E_HIP;
                    break;
                }
                best = std::max(best, static_cast<double>(n_vec) * 16.0 * reps / (ms * 1e-3) / 1e9);
            }
        }
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (sink) (void)hipFree(sink);
    *gbps_out = best;
    return rc;
}

extern "C" int shadowkv_probe_host_copies(const void *host, size_t host_bytes, void *dev, size_t chunk_bytes,
                                          int n_chunks, const int64_t *host_chunk, int reps, void *stream,
                                          double *gbps_each, double *gbps_batch) {
    if (!host || !dev || !host_chunk || !gbps_each || !gbps_batch || reps < 1 || n_chunks < 1 || chunk_bytes == 0)
        return SKV_E_INVAL;
    for (int i = 0; i < n_chunks; ++i)
        if (host_chunk[i] < 0 || static_cast<size_t>(host_chunk[i] + 1) * chunk_bytes > host_bytes) return SKV_E_INVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    std::vector<void *> dsts(n_chunks), srcs(n_chunks);
    std::vector<size_t> sizes(n_chunks, chunk_bytes);
    for (int i = 0; i < n_chunks; ++i) {
        srcs[i] = const_cast<char *>(static_cast<const char *>(host)) + static_cast<size_t>(host_chunk[i]) * chunk_bytes;
        dsts[i] = static_cast<char *>(dev) + static_cast<size_t>(i) * chunk_bytes;
    }
    typedef hipError_t (*BatchFn)(void **, void **, size_t *, size_t, hipMemcpyAttributes *, size_t *, size_t,
                                  size_t *, hipStream_t);
    const BatchFn batch_fn = reinterpret_cast<BatchFn>(dlsym(RTLD_DEFAULT, "hipMemcpyBatchAsync"));
    hipEvent_t e0 = nullptr, e1 = nullptr;
    int rc = SKV_OK;
    double best_each = 0.0, best_batch = 0.0;
    const double bytes = static_cast<double>(n_chunks) * chunk_bytes;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        rc = SKV_E_HIP;
    } else {
        for (int r = 0; r < reps && rc == SKV_OK; ++r) {
            float ms = 0.f;
            // one hipMemcpyAsync per chunk
            if (hipEventRecord(e0, st) != hipSuccess) { rc = SKV_E_HIP; break; }
            for (int i = 0; i < n_chunks && rc == SKV_OK; ++i)
                if (hipMemcpyAsync(dsts[i], srcs[i], chunk_bytes, hipMemcpyHostToDevice, st) != hipSuccess) rc = SKV_E_HIP;
            if (rc || hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(&ms, e0, e1) != hipSuccess) { rc = SKV_E_HIP; break; }
            best_each = std::max(best_each, bytes / (ms * 1e-3) / 1e9);
            // one batch of all of them, where the HIP runtime the process
            // loaded has the call (looked up at run time: older runtimes
            // lack it, and a link-time reference would keep the library from
            // loading there)
            if (!batch_fn) continue;
            size_t fail = 0;
            if (hipEventRecord(e0, st) != hipSuccess ||
                batch_fn(dsts.data(), srcs.data(), sizes.data(), n_chunks, nullptr, nullptr, 0, &fail, st) !=
                    hipSuccess ||
                hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(&ms, e0, e1) != hipSuccess) { rc = SKV_E_HIP; break; }
            best_batch = std::max(best_batch, bytes / (ms * 1e-3) / 1e9);
        }
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    *gbps_each = best_each;
    *gbps_batch = best_batch;
    return rc;
}
