// Dispatch-exact kernel timing for benchmarks: when switched on, every walk kernel is launched
// with hipExtLaunchKernel and a pair of HIP events that the dispatch itself records at the
// kernel's start and end, so the measured time excludes the queueing in front of the kernel.
// Host code only; not meant for graph capture.
#include <hip/hip_ext.h>

#include <vector>

#include "internal.hpp"

namespace dspark {

namespace {
struct TimingRing {
    int device = -1;
    std::vector<hipEvent_t> start, stop;
    int64_t launched = 0;  // launches recorded since the last read
};
TimingRing g_ring;

void destroy_ring() {
    for (hipEvent_t e : g_ring.start) (void)hipEventDestroy(e);
    for (hipEvent_t e : g_ring.stop) (void)hipEventDestroy(e);
    g_ring.start.clear();
    g_ring.stop.clear();
    g_ring.launched = 0;
    g_ring.device = -1;
}
}  // namespace

int set_kernel_timing(int64_t n) {
    if (n > 4096) return DSPARK_ERR_INVALID_ARG;
    destroy_ring();
    if (n == 0) return DSPARK_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return DSPARK_ERR_NO_DEVICE;
    }
    for (int64_t i = 0; i < n; ++i) {
        hipEvent_t a = nullptr, b = nullptr;
        if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
            (void)hipGetLastError();
            if (a) (void)hipEventDestroy(a);
            destroy_ring();
            return DSPARK_ERR_LAUNCH;
        }
        g_ring.start.push_back(a);
        g_ring.stop.push_back(b);
    }
    g_ring.device = dev;
    return DSPARK_OK;
}

hipError_t launch_walk_kernel(const void* fn, dim3 grid, dim3 block, void** args, size_t lds,
                              hipStream_t stream) {
    int dev = -1;
    if (!g_ring.start.empty() && hipGetDevice(&dev) == hipSuccess && dev == g_ring.device) {
        const size_t i = (size_t)(g_ring.launched % (int64_t)g_ring.start.size());
        const hipError_t e = hipExtLaunchKernel(fn, grid, block, args, lds, stream,
                                                g_ring.start[i], g_ring.stop[i], 0);
        if (e == hipSuccess) ++g_ring.launched;
        return e;
    }
    return hipLaunchKernel(fn, grid, block, args, lds, stream);
}

int read_kernel_times(float* us, int max, int* count) {
    *count = 0;
    const int64_t ring = (int64_t)g_ring.start.size();
    if (ring == 0) return DSPARK_OK;
    const int64_t n = g_ring.launched < ring ? g_ring.launched : ring;
    const int64_t first = g_ring.launched - n;
    int out = 0;
    for (int64_t j = first; j < g_ring.launched && out < max; ++j) {
        const size_t i = (size_t)(j % ring);
        float ms = 0.0f;
        if (hipEventSynchronize(g_ring.stop[i]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_ring.start[i], g_ring.stop[i]) != hipSuccess) {
            (void)hipGetLastError();
            return DSPARK_ERR_LAUNCH;
        }
        us[out++] = ms * 1000.0f;
    }
    g_ring.launched = 0;
    *count = out;
    return DSPARK_OK;
}

}  // namespace dspark
