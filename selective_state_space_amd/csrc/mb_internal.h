// mb_internal.h -- helpers shared by the libmb translation units (host
// validation, error plumbing, bf16 conversion).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "mb.h"

namespace mb {

// ---------------------------------------------------------------- errors ----
// Last HIP error seen by a launch in this thread (mb_last_hip_error()).
void set_last_hip_error(int code);

// Check the launch that was just enqueued.
inline mb_status check_launch() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_last_hip_error((int)e);
        return MB_ERR_HIP;
    }
    return MB_OK;
}

// ------------------------------------------------------------ validation ----
struct Span {
    const void* p;
    size_t bytes;
};

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// True when the output span overlaps any of the given input spans.
inline bool overlaps_any(const void* out, size_t nout, const Span* ins, int n_in) {
    for (int i = 0; i < n_in; ++i)
        if (overlaps(out, nout, ins[i].p, ins[i].bytes)) return true;
    return false;
}

inline size_t dtype_size(mb_dtype d) { return d == MB_BF16 ? 2 : 4; }
inline bool dtype_ok(mb_dtype d) { return d == MB_F32 || d == MB_BF16; }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Workspace bytes of the Mamba-1 scan's sequence blocks (0: one block).
size_t m1_scan_workspace(int64_t batch, int64_t L, int64_t D, int64_t N);

// Workspace bytes of the Mamba-1 scan backward (0 for unsupported sizes).
size_t m1_bwd_workspace(int64_t batch, int64_t L, int64_t D, int64_t N);

// Workspace bytes of the Mamba-3 MIMO backward (0 for unsupported sizes).
size_t mimo_bwd_workspace(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R);

// Workspace bytes of the Mamba-3 SISO backward (0 for unsupported sizes).
size_t trap_bwd_workspace(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N);

// Workspace bytes of the Mamba-2 SSD backward (0 for unsupported sizes).
size_t ssd_bwd_workspace(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N);

// Copy h0 (or zeros) into h_out; used for zero-length sequences.
mb_status copy_state(const float* h0, float* h_out, int64_t n, hipStream_t stream);

// ------------------------------------------------------------------ bf16 ----
typedef uint16_t bf16;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float(((uint32_t)v) << 16); }

__device__ __forceinline__ bf16 f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                         // nearest-even
    return (bf16)(u >> 16);
}

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16* p, float v) { *p = f32_to_bf16(v); }

// exp(v) through the hardware base-2 exponential; callers pass v * log2(e).
__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace mb
