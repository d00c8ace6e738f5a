// ssd_prologue.hip -- the Mamba-2 block prologue for gfx950 in one pass over
// HBM: causal depthwise conv1d over the concatenated (x, B, C) channels, SiLU,
// softplus of dt plus its bias, and the split into the SSD's inputs
// (TorchMamba README, API reference: Mamba2Block with d_conv and psi = SiLU;
// Math notes M1 for the exp-Euler discretisation that scales the input by dt
// and gives the log-decay dt A):
//     v_t[c]   = SiLU(conv_b[c] + sum_{k<K} conv_w[c][k] xBC_{t-K+1+k}[c])
//     dt'_t[h] = softplus(dt_t[h] + dt_bias[h])
//     X_t[h][p] = v_t[h P + p] dt'_t[h],  B_t = v_t[H P ..],  C_t = v_t[H P + G N ..]
//     logdecay_t[h] = dt'_t[h] A[h]
// Steps before the call read x_hist (zeros without it), so split sequences
// chain exactly.
//
// Layout and mapping: xBC is channel-last, so a thread owns four adjacent
// channels (one 16-byte load per step, 8 bytes in bf16; the arithmetic is fp32) and a run of kSteps steps, keeping the
// K - 1 previous inputs in registers: every input is read from HBM once, every
// output written once, all accesses coalesced along the channels.  The work is
// HBM-bound; the only arithmetic of note is one exp and one log per output.
// Workgroups are one wave, so the channel blocks tile H P + 2 G N with little
// idle tail (1792 channels: seven full waves of 64 float4 lanes).
#include <hip/hip_runtime.h>

#include "mb.h"
#include "mb_internal.h"

namespace mb {
namespace {

constexpr int kThreads = 64;
constexpr int kSteps = 16;
constexpr int kKMax = 4;

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }
__device__ __forceinline__ float softplus(float v) { return v > 20.0f ? v : log1pf(__expf(v)); }

struct ProArgs {
    const void* xbc;     // activations (xBC, x_hist, X, B, C): fp32 or bf16
    const float* w;
    const float* cb;
    const void* hist;
    const float* dt;
    const float* dtb;
    const float* A;
    void* X;
    void* B;
    void* C;
    float* ld;
    float* dto;
    int L, H, P, G, N, K, cin;
};

// four adjacent activations as fp32, and back
template <typename IO>
__device__ __forceinline__ float4 ld4(const void* p, size_t e) {
    if constexpr (sizeof(IO) == 4) {
        return *(const float4*)((const float*)p + e);
    } else {
        const uint2 u = *(const uint2*)((const bf16*)p + e);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    }
}
template <typename IO>
__device__ __forceinline__ void st4(void* p, size_t e, float v0, float v1, float v2, float v3) {
    if constexpr (sizeof(IO) == 4) {
        *(float4*)((float*)p + e) = make_float4(v0, v1, v2, v3);
    } else {
        const uint32_t u0 = f32_to_bf16(v0) | ((uint32_t)f32_to_bf16(v1) << 16);
        const uint32_t u1 = f32_to_bf16(v2) | ((uint32_t)f32_to_bf16(v3) << 16);
        *(uint2*)((bf16*)p + e) = make_uint2(u0, u1);
    }
}

template <int K, typename IO>
__global__ __launch_bounds__(kThreads) void k_ssd_prologue(ProArgs a) {
    const int c = 4 * (blockIdx.x * kThreads + threadIdx.x);
    if (c >= a.cin) return;
    const int b = blockIdx.z;
    const int t0 = blockIdx.y * kSteps;
    const int t1 = min(a.L, t0 + kSteps);
    const int HP = a.H * a.P, GN = a.G * a.N;
    float w[4][K], bias[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int k = 0; k < K; ++k) w[j][k] = a.w[(size_t)(c + j) * K + k];
        bias[j] = a.cb ? a.cb[c + j] : 0.0f;
    }
    // window: win[k] holds the input of step t - K + 1 + k
    float4 win[K];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
        const int t = t0 - K + 1 + k;
        if (t >= 0)
            win[k] = ld4<IO>(a.xbc, ((size_t)b * a.L + t) * a.cin + c);
        else if (a.hist)
            win[k] = ld4<IO>(a.hist, ((size_t)b * (K - 1) + (K - 1 + t)) * a.cin + c);
        else
            win[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    const int h = c < HP ? c / a.P : 0;
    const float Ah = c < HP ? a.A[h] : 0.0f;
    const float dtbh = (c < HP && a.dtb) ? a.dtb[h] : 0.0f;
    for (int t = t0; t < t1; ++t) {
        const size_t row = (size_t)b * a.L + t;
        win[K - 1] = ld4<IO>(a.xbc, row * a.cin + c);
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float s = bias[j];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float4 q = win[k];
                const float x = j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
                s = fmaf(w[j][k], x, s);
            }
            v[j] = silu(s);
        }
#pragma unroll
        for (int k = 0; k < K - 1; ++k) win[k] = win[k + 1];
        if (c < HP) {
            const float d = softplus(a.dt[row * a.H + h] + dtbh);
            st4<IO>(a.X, row * HP + c, v[0] * d, v[1] * d, v[2] * d, v[3] * d);
            if (c % a.P == 0) {
                a.ld[row * a.H + h] = d * Ah;
                if (a.dto) a.dto[row * a.H + h] = d;
            }
        } else if (c < HP + GN) {
            st4<IO>(a.B, row * GN + (c - HP), v[0], v[1], v[2], v[3]);
        } else {
            st4<IO>(a.C, row * GN + (c - HP - GN), v[0], v[1], v[2], v[3]);
        }
    }
}

}  // namespace
}  // namespace mb

using namespace mb;

extern "C" mb_status mb_ssd_prologue(const void* xBC, const float* conv_w, const float* conv_b,
                                     const void* x_hist, const float* dt, const float* dt_bias,
                                     const float* A, void* X, void* B, void* C, float* logdecay,
                                     float* dt_out, int64_t batch, int64_t L, int64_t H, int64_t P,
                                     int64_t G, int64_t N, int64_t K, mb_dtype dtype, hipStream_t stream) {
    if (!xBC || !conv_w || !dt || !A || !X || !B || !C || !logdecay) return MB_ERR_NULL;
    if (batch < 0 || L < 0 || H < 1 || P < 1 || G < 1 || N < 1 || H % G || P % 4 || N % 4) return MB_ERR_SHAPE;
    if (K < 1 || K > kKMax || batch > 65535) return MB_ERR_SHAPE;
    if (!dtype_ok(dtype)) return MB_ERR_DTYPE;
    const size_t es = dtype_size(dtype);
    const int64_t cin = H * P + 2 * G * N;
    // grid: channel blocks x step runs (at most 65535) x batch
    if (cin > ((int64_t)1 << 28) || (L + kSteps - 1) / kSteps > 65535) return MB_ERR_SHAPE;
    for (const void* p : {(const void*)xBC, (const void*)x_hist, (const void*)X, (const void*)B, (const void*)C})
        if ((uintptr_t)p & 15) return MB_ERR_ALIGN;
    const size_t nx = (size_t)(batch * L * cin) * es, nh = (size_t)(batch * L * H) * 4;
    const Span ins[7] = {{xBC, nx}, {conv_w, (size_t)(cin * K) * 4}, {conv_b, conv_b ? (size_t)cin * 4 : 0},
                         {x_hist, x_hist ? (size_t)(batch * (K - 1) * cin) * es : 0}, {dt, nh},
                         {dt_bias, dt_bias ? (size_t)H * 4 : 0}, {A, (size_t)H * 4}};
    const Span outs[5] = {{X, (size_t)(batch * L * H * P) * es}, {B, (size_t)(batch * L * G * N) * es},
                          {C, (size_t)(batch * L * G * N) * es}, {logdecay, nh}, {dt_out, dt_out ? nh : 0}};
    for (int i = 0; i < 5; ++i) {
        if (overlaps_any(outs[i].p, outs[i].bytes, ins, 7)) return MB_ERR_ALIAS;
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes)) return MB_ERR_ALIAS;
    }
    if (batch == 0 || L == 0) return MB_OK;
    ProArgs a{xBC, conv_w, conv_b, x_hist, dt, dt_bias, A, X, B, C, logdecay, dt_out,
              (int)L, (int)H, (int)P, (int)G, (int)N, (int)K, (int)cin};
    const dim3 grid((unsigned)((cin / 4 + kThreads - 1) / kThreads), (unsigned)((L + kSteps - 1) / kSteps),
                    (unsigned)batch);
    const bool f32 = dtype == MB_F32;
#define MB_PRO(KK)                                                                              \
    if (f32)                                                                                    \
        hipLaunchKernelGGL((k_ssd_prologue<KK, float>), grid, dim3(kThreads), 0, stream, a);   \
    else                                                                                        \
        hipLaunchKernelGGL((k_ssd_prologue<KK, bf16>), grid, dim3(kThreads), 0, stream, a);
    switch (K) {
        case 1: MB_PRO(1) break;
        case 2: MB_PRO(2) break;
        case 3: MB_PRO(3) break;
        default: MB_PRO(4) break;
    }
#undef MB_PRO
    return check_launch();
}
