// common.hip -- status strings, error plumbing, device attribute cache and the
// small state-copy kernel used for zero-length sequences.
#include <mutex>

#include "mb_internal.h"

namespace mb {

static thread_local int g_last_hip_error = 0;

void set_last_hip_error(int code) { g_last_hip_error = code; }

int device_cu_count() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

__global__ void k_copy_state(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) dst[i] = src ? src[i] : 0.0f;
}

mb_status copy_state(const float* h0, float* h_out, int64_t n, hipStream_t stream) {
    if (!h_out || n <= 0 || h0 == h_out) return MB_OK;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_copy_state, dim3((unsigned)blocks), dim3(256), 0, stream, h0, h_out, n);
    return check_launch();
}

}  // namespace mb

extern "C" const char* mb_status_str(mb_status s) {
    switch (s) {
        case MB_OK: return "ok";
        case MB_ERR_NULL: return "a required pointer is NULL";
        case MB_ERR_SHAPE: return "invalid or unsupported sizes";
        case MB_ERR_DTYPE: return "unsupported dtype";
        case MB_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case MB_ERR_HIP: return "HIP launch failed (see mb_last_hip_error)";
        case MB_ERR_ALIAS: return "an output overlaps an input";
        case MB_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    }
    return "unknown status";
}

extern "C" int mb_last_hip_error(void) { return mb::g_last_hip_error; }

extern "C" int mb_version(void) { return 100; }
