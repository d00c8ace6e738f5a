// ssd_step.hip -- decode step of the SSD family (Mamba-2, Mamba-3 SISO and
// MIMO) for gfx950: one token per sequence on a state kept in the physical
// (unrotated) frame.
//
// Since plane rotations compose additively, the rotated-frame recurrence of the
// chunked kernels becomes, one token at a time, a recurrence in the unrotated
// B, C that needs only the token's own angle increment (TorchMamba README,
// Math notes M3 SISO and MIMO; Mamba-2 is beta = 0, gamma = 1, no rotation,
// Math notes M2):
//     S' = R(-theta) (alpha S + beta sum_r Bp_r (outer) Xp_r) + gamma sum_r B_r (outer) X_r
//     Y_r = S'^T C_r
// with Bp, Xp the previous token's B and X.  A sequence prefilled by the chunked
// entry points continues exactly: their final state is in the same frame.
//
// Kernel k_ssd_step: one workgroup of 256 threads per (batch, head).  Thread
// (q, g) owns state columns 4q .. 4q + 3 and the row pairs g, g + RG, ...: every
// state access is one 16-byte load and one 16-byte store, a row of the state
// being read by consecutive lanes.  The state is read and written once, so the
// step is bound by HBM.  The sum over state rows of the output goes through LDS.
#include "mb_internal.h"

namespace mb {
namespace {

constexpr int kStepThreads = 256;

// The R ranks of one row, elements e .. e + R - 1 (e a multiple of R, the base
// 16-byte aligned), widened to fp32, with the widest loads the alignment allows.
template <int R, typename IO>
__device__ __forceinline__ void ld_ranks(const IO* p, size_t e, float* o) {
    if constexpr (sizeof(IO) == 4) {
        if constexpr (R >= 4) {
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const float4 v = *(const float4*)((const float*)p + e + i);
                o[i] = v.x; o[i + 1] = v.y; o[i + 2] = v.z; o[i + 3] = v.w;
            }
        } else if constexpr (R == 2) {
            const float2 v = *(const float2*)((const float*)p + e);
            o[0] = v.x; o[1] = v.y;
        } else {
            o[0] = ((const float*)p)[e];
        }
    } else {
        const bf16* q = (const bf16*)p + e;
        if constexpr (R >= 8) {
#pragma unroll
            for (int i = 0; i < R; i += 8) {
                const uint4 v = *(const uint4*)(q + i);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    o[i + 2 * k] = __uint_as_float(w[k] << 16);
                    o[i + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
                }
            }
        } else if constexpr (R == 4) {
            const uint2 v = *(const uint2*)q;
            o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
            o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
        } else if constexpr (R == 2) {
            const uint32_t v = *(const uint32_t*)q;
            o[0] = __uint_as_float(v << 16); o[1] = __uint_as_float(v & 0xffff0000u);
        } else {
            o[0] = to_f32(q[0]);
        }
    }
}

// sin / cos of an angle in radians through the hardware units, which take the
// argument in revolutions; the whole turns are removed first
__device__ __forceinline__ void sincos_turns(float phi, float* s, float* c) {
    float r = phi * 0.15915494309189535f;
    r = r - rintf(r);
    *s = __builtin_amdgcn_sinf(r);
    *c = __builtin_amdgcn_cosf(r);
}

template <int R, bool ROT, typename IO>
__global__ __launch_bounds__(kStepThreads) void k_ssd_step(
    const IO* __restrict__ X, const float* __restrict__ logdecay, const IO* __restrict__ B,
    const IO* __restrict__ C, const float* __restrict__ beta, const float* __restrict__ gamma,
    const float* __restrict__ theta, const IO* __restrict__ X_prev, const IO* __restrict__ B_prev,
    const float* h_in, float* h_out, IO* __restrict__ Y, int H, int P, int G, int N)
{
    extern __shared__ float sY[];   // [RG][P * R] partial outputs
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int NQ = P / 4;                  // column quads
    const int RG = kStepThreads / NQ;      // row-pair groups
    const int tid = threadIdx.x;
    const int q = tid % NQ, rg = tid / NQ;
    const bool on = rg < RG;
    const float a = exp2_fast(logdecay[bh] * kLog2e);
    const float be = beta ? beta[bh] : 0.0f;
    const float ga = gamma ? gamma[bh] : 1.0f;
    const bool prev = be != 0.0f && X_prev != nullptr;

    const size_t xo = (size_t)bh * P * R;
    const size_t bo = ((size_t)b * G + g) * (size_t)N * R;
    float xv[4][R], xp[4][R], y[4][R];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const size_t e = xo + (size_t)(4 * q + j) * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            xv[j][r] = 0.0f;
            xp[j][r] = 0.0f;
            y[j][r] = 0.0f;
        }
        if (on) ld_ranks<R>(X, e, xv[j]);
        if (on && prev) ld_ranks<R>(X_prev, e, xp[j]);
    }

    const size_t so = (size_t)bh * N * P;
    if (on) {
        // row pairs k0, k0 + RG, ... in batches of KU: the batch's state loads are
        // all issued before its first store (in place, a later load may not pass
        // an earlier store, so without batching one pair would be in flight)
        constexpr int KU = 4;
        for (int k0 = rg; 2 * k0 < N; k0 += KU * RG) {
            float4 s0[KU], s1[KU];
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int k = k0 + u * RG;
                s0[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                s1[u] = s0[u];
                if (h_in && 2 * k < N) {
                    s0[u] = *(const float4*)(h_in + so + (size_t)(2 * k) * P + 4 * q);
                    s1[u] = *(const float4*)(h_in + so + (size_t)(2 * k + 1) * P + 4 * q);
                }
            }
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int k = k0 + u * RG;
                if (2 * k >= N) break;
                const int n0 = 2 * k, n1 = 2 * k + 1;
                float t0[4] = {a * s0[u].x, a * s0[u].y, a * s0[u].z, a * s0[u].w};
                float t1[4] = {a * s1[u].x, a * s1[u].y, a * s1[u].z, a * s1[u].w};
                if (prev) {
                    float bp0[R], bp1[R];
                    ld_ranks<R>(B_prev, bo + (size_t)n0 * R, bp0);
                    ld_ranks<R>(B_prev, bo + (size_t)n1 * R, bp1);
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            t0[j] = fmaf(be * bp0[r], xp[j][r], t0[j]);
                            t1[j] = fmaf(be * bp1[r], xp[j][r], t1[j]);
                        }
                }
                if constexpr (ROT) {
                    // R(-theta) on the pair (n0, n1): (c v0 + s v1, -s v0 + c v1)
                    float sn, cs;
                    sincos_turns(theta[(size_t)bh * (N / 2) + k], &sn, &cs);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float v0 = t0[j], v1 = t1[j];
                        t0[j] = fmaf(cs, v0, sn * v1);
                        t1[j] = fmaf(cs, v1, -sn * v0);
                    }
                }
                float b0[R], b1[R], c0[R], c1[R];
                ld_ranks<R>(B, bo + (size_t)n0 * R, b0);
                ld_ranks<R>(B, bo + (size_t)n1 * R, b1);
                ld_ranks<R>(C, bo + (size_t)n0 * R, c0);
                ld_ranks<R>(C, bo + (size_t)n1 * R, c1);
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        t0[j] = fmaf(ga * b0[r], xv[j][r], t0[j]);
                        t1[j] = fmaf(ga * b1[r], xv[j][r], t1[j]);
                    }
                *(float4*)(h_out + so + (size_t)n0 * P + 4 * q) = make_float4(t0[0], t0[1], t0[2], t0[3]);
                *(float4*)(h_out + so + (size_t)n1 * P + 4 * q) = make_float4(t1[0], t1[1], t1[2], t1[3]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < R; ++r) y[j][r] = fmaf(t0[j], c0[r], fmaf(t1[j], c1[r], y[j][r]));
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < R; ++r) sY[(size_t)rg * P * R + (4 * q + j) * R + r] = y[j][r];
    }
    __syncthreads();
    for (int o = tid; o < P * R; o += kStepThreads) {
        float acc = 0.0f;
        for (int g2 = 0; g2 < RG; ++g2) acc += sY[(size_t)g2 * P * R + o];
        store_out(Y + xo + o, acc);
    }
}

template <int R, typename IO>
mb_status launch_step(const void* X, const float* ld, const void* B, const void* C, const float* beta,
                      const float* gamma, const float* theta, const void* Xp, const void* Bp,
                      const float* h_in, float* h_out, void* Y, int64_t batch, int64_t H, int64_t P,
                      int64_t G, int64_t N, hipStream_t stream) {
    const int RG = kStepThreads / (int)(P / 4);
    const size_t lds = (size_t)RG * P * R * sizeof(float);
    const dim3 grid((unsigned)(batch * H)), block(kStepThreads);
    if (theta)
        hipLaunchKernelGGL((k_ssd_step<R, true, IO>), grid, block, lds, stream, (const IO*)X, ld,
                           (const IO*)B, (const IO*)C, beta, gamma, theta, (const IO*)Xp, (const IO*)Bp,
                           h_in, h_out, (IO*)Y, (int)H, (int)P, (int)G, (int)N);
    else
        hipLaunchKernelGGL((k_ssd_step<R, false, IO>), grid, block, lds, stream, (const IO*)X, ld,
                           (const IO*)B, (const IO*)C, beta, gamma, theta, (const IO*)Xp, (const IO*)Bp,
                           h_in, h_out, (IO*)Y, (int)H, (int)P, (int)G, (int)N);
    return check_launch();
}

template <typename IO>
mb_status dispatch_step(int64_t R, const void* X, const float* ld, const void* B, const void* C,
                        const float* beta, const float* gamma, const float* theta, const void* Xp,
                        const void* Bp, const float* h_in, float* h_out, void* Y, int64_t batch,
                        int64_t H, int64_t P, int64_t G, int64_t N, hipStream_t s) {
    switch (R) {
        case 1: return launch_step<1, IO>(X, ld, B, C, beta, gamma, theta, Xp, Bp, h_in, h_out, Y, batch, H, P, G, N, s);
        case 2: return launch_step<2, IO>(X, ld, B, C, beta, gamma, theta, Xp, Bp, h_in, h_out, Y, batch, H, P, G, N, s);
        case 4: return launch_step<4, IO>(X, ld, B, C, beta, gamma, theta, Xp, Bp, h_in, h_out, Y, batch, H, P, G, N, s);
        case 8: return launch_step<8, IO>(X, ld, B, C, beta, gamma, theta, Xp, Bp, h_in, h_out, Y, batch, H, P, G, N, s);
        default: return launch_step<16, IO>(X, ld, B, C, beta, gamma, theta, Xp, Bp, h_in, h_out, Y, batch, H, P, G, N, s);
    }
}

}  // namespace
}  // namespace mb

using namespace mb;

extern "C" mb_status mb_ssd_step(const void* X, const float* logdecay, const void* B, const void* C,
                                 const float* beta, const float* gamma, const float* theta,
                                 const void* X_prev, const void* B_prev, const float* h_in,
                                 float* h_out, void* Y, int64_t batch, int64_t H, int64_t P,
                                 int64_t G, int64_t N, int64_t R, mb_dtype dtype, hipStream_t stream) {
    if (!dtype_ok(dtype)) return MB_ERR_DTYPE;
    if (batch < 0 || H < 1 || G < 1 || H % G || P < 4 || P % 4 || P > 1024 || N < 2 || N % 2 ||
        (R != 1 && R != 2 && R != 4 && R != 8 && R != 16))
        return MB_ERR_SHAPE;
    if (batch > INT32_MAX / H) return MB_ERR_SHAPE;
    if (batch == 0) return MB_OK;
    if (!X || !logdecay || !B || !C || !h_out || !Y) return MB_ERR_NULL;
    if ((X_prev == nullptr) != (B_prev == nullptr)) return MB_ERR_NULL;
    if (((uintptr_t)h_in | (uintptr_t)h_out | (uintptr_t)X | (uintptr_t)X_prev | (uintptr_t)B |
         (uintptr_t)B_prev | (uintptr_t)C | (uintptr_t)Y) & 15)
        return MB_ERR_ALIGN;
    const size_t es = dtype_size(dtype);
    const size_t n_x = (size_t)(batch * H * P * R), n_bc = (size_t)(batch * G * N * R);
    const size_t n_s = (size_t)(batch * H), n_h = (size_t)(batch * H * N * P);
    const Span ins[] = {{X, n_x * es}, {B, n_bc * es}, {C, n_bc * es}, {logdecay, n_s * 4},
                        {beta, beta ? n_s * 4 : 0}, {gamma, gamma ? n_s * 4 : 0},
                        {theta, theta ? n_s * (size_t)(N / 2) * 4 : 0},
                        {X_prev, X_prev ? n_x * es : 0}, {B_prev, B_prev ? n_bc * es : 0},
                        {h_in, h_in ? n_h * 4 : 0}};
    // h_out may be h_in exactly (in place); no other overlap
    if (overlaps_any(h_out, n_h * 4, ins, 9)) return MB_ERR_ALIAS;
    if (h_in && h_in != h_out && overlaps(h_out, n_h * 4, h_in, n_h * 4)) return MB_ERR_ALIAS;
    if (overlaps_any(Y, n_x * es, ins, 10) || overlaps(Y, n_x * es, h_out, n_h * 4)) return MB_ERR_ALIAS;
    return dtype == MB_F32
        ? dispatch_step<float>(R, X, logdecay, B, C, beta, gamma, theta, X_prev, B_prev, h_in, h_out, Y,
                               batch, H, P, G, N, stream)
        : dispatch_step<bf16>(R, X, logdecay, B, C, beta, gamma, theta, X_prev, B_prev, h_in, h_out, Y,
                              batch, H, P, G, N, stream);
}
