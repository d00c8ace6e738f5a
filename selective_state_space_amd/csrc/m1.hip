// m1.hip -- Mamba-1 selective scan and single-token decode step for gfx950.
//
// Recurrence (TorchMamba README, Math notes M1; burn_mamba Mamba1 docs,
// selective_scan / selective_scan_step), exponential-Euler discretisation:
//     h_t[c,n] = exp(dt_t[c] A[c,n]) h_{t-1}[c,n] + dt_t[c] B_t[n] x_t[c]
//     y_t[c]   = sum_n C_t[n] h_t[c,n] + Dskip[c] x_t[c]
//
// Scan layout.  One workgroup owns 16 channels of one batch row and walks the
// whole sequence; each of its 16*NPAD lanes owns one (channel, state) chain, so
// the recurrence needs no cross-lane traffic and 8 batches x 1536 channels fill
// 768 workgroups (three per compute unit).  Per time tile the workgroup stages
// dt, dt*x, x (16 channels) and B, C (shared by all channels) in LDS, prefetching
// the next tile into registers while the current one is computed; each lane
// writes C_t[n] h_t[c,n] into LDS and the sum over n is done by one thread per
// (t, c) output.  One hardware exp2 per (t, c, n) element.
#include "mb_internal.h"

namespace mb {
namespace {

constexpr int kCW = 16;  // channels per workgroup

template <int NPAD, typename IO>
__global__ __launch_bounds__(kCW * NPAD) void k_m1_scan(
    const IO* __restrict__ x, const IO* __restrict__ dt, const float* __restrict__ A,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dskip,
    const float* h0, IO* __restrict__ y, float* h_out, int L, int D, int N, int n_cblk,
    int n_wg)
{
    constexpr int NT = kCW * NPAD;      // threads
    constexpr int T = 256 / NPAD;       // time steps per tile
    constexpr int XE = T * kCW;         // x / dt elements per tile
    constexpr int BE = T * NPAD;        // B / C elements per tile
    constexpr int RX = (XE + NT - 1) / NT;
    constexpr int RB = (BE + NT - 1) / NT;
    constexpr int PSTR = NPAD * kCW + kCW;   // s_p stride per time step (bank skew)

    __shared__ float s_dt[2][T][kCW];
    __shared__ float s_dtx[2][T][kCW];
    __shared__ float s_x[2][T][kCW];
    __shared__ float s_B[2][T][NPAD];
    __shared__ float s_C[2][T][NPAD];
    __shared__ float s_p[T * PSTR];

    // Workgroup -> (batch, channel block).  Workgroups i and i+8 land on the same
    // XCD, so they take adjacent 16-channel blocks and share 128-byte lines in L2.
    int wg = blockIdx.x;
    int full = n_wg / 16 * 16;
    int logical = wg;
    if (wg < full) {
        int g = wg / 16, r = wg % 16;
        logical = g * 16 + (r % 8) * 2 + r / 8;
    }
    const int b = logical / n_cblk;
    const int c0 = (logical % n_cblk) * kCW;

    const int tid = threadIdx.x;
    const int cl = tid % kCW, n = tid / kCW;
    const int c = c0 + cl;
    const bool lane_ok = (c < D) && (n < N);

    const float A2 = lane_ok ? A[(size_t)c * N + n] * kLog2e : 0.0f;
    float h = (lane_ok && h0) ? h0[((size_t)b * D + c) * N + n] : 0.0f;
    const float Dv = (c < D && Dskip) ? Dskip[c] : 0.0f;

    float px[RX], pdt[RX], pB[RB], pC[RB];

    auto load = [&](int k) {
        const int t0 = k * T;
#pragma unroll
        for (int r = 0; r < RX; ++r) {
            int e = tid + r * NT;
            px[r] = 0.0f;
            pdt[r] = 0.0f;
            if (e < XE) {
                int tt = t0 + e / kCW, cc = c0 + e % kCW;
                if (tt < L && cc < D) {
                    size_t off = ((size_t)b * L + tt) * D + cc;
                    px[r] = to_f32(x[off]);
                    pdt[r] = to_f32(dt[off]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            int e = tid + r * NT;
            pB[r] = 0.0f;
            pC[r] = 0.0f;
            if (e < BE) {
                int tt = t0 + e / NPAD, nn = e % NPAD;
                if (tt < L && nn < N) {
                    size_t off = ((size_t)b * L + tt) * N + nn;
                    pB[r] = to_f32(Bm[off]);
                    pC[r] = to_f32(Cm[off]);
                }
            }
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int r = 0; r < RX; ++r) {
            int e = tid + r * NT;
            if (e < XE) {
                int t = e / kCW, cc = e % kCW;
                s_dt[buf][t][cc] = pdt[r];
                s_dtx[buf][t][cc] = pdt[r] * px[r];
                s_x[buf][t][cc] = px[r];
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            int e = tid + r * NT;
            if (e < BE) {
                int t = e / NPAD, nn = e % NPAD;
                s_B[buf][t][nn] = pB[r];
                s_C[buf][t][nn] = pC[r];
            }
        }
    };

    const int ntiles = (L + T - 1) / T;
    if (ntiles > 0) {
        load(0);
        stash(0);
    }
    __syncthreads();
    for (int k = 0; k < ntiles; ++k) {
        const int buf = k & 1;
        if (k + 1 < ntiles) load(k + 1);
        // recurrence: one (channel, state) chain per lane
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float a = exp2_fast(s_dt[buf][t][cl] * A2);
            h = fmaf(a, h, s_dtx[buf][t][cl] * s_B[buf][t][n]);
            s_p[t * PSTR + n * kCW + cl] = s_C[buf][t][n] * h;
        }
        __syncthreads();
        // y_t[c] = sum_n C h + D x, one output per thread per pass
        const int t0 = k * T;
#pragma unroll
        for (int r = 0; r < (T * kCW + NT - 1) / NT; ++r) {
            int o = tid + r * NT;
            if (o < T * kCW) {
                int t = o / kCW;   // o % kCW == cl because NT is a multiple of kCW
                int tt = t0 + t;
                if (tt < L && c < D) {
                    const float* pp = s_p + t * PSTR + cl;
                    float acc = 0.0f;
#pragma unroll
                    for (int nn = 0; nn < NPAD; ++nn) acc += pp[nn * kCW];
                    acc = fmaf(Dv, s_x[buf][t][cl], acc);
                    store_out(&y[((size_t)b * L + tt) * D + c], acc);
                }
            }
        }
        if (k + 1 < ntiles) stash(buf ^ 1);
        __syncthreads();
    }
    if (h_out && lane_ok) h_out[((size_t)b * D + c) * N + n] = h;
}

// Decode step, N a multiple of 4 with N/4 dividing 64: one lane per
// (batch, channel, group of 4 states); 16-byte state loads, so consecutive lanes
// read consecutive 16-byte pieces of the state.  The sum over n is a butterfly
// over the N/4 lanes of a channel.
template <int NQ, typename IO>
__global__ __launch_bounds__(256) void k_m1_step_q(
    const IO* __restrict__ x, const IO* __restrict__ dt, const float* __restrict__ A,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dskip,
    const float* h_in, float* h_out, IO* __restrict__ y, int64_t total, int D)
{
    constexpr int N = NQ * 4;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= total) return;
    const int q = (int)(gid % NQ);
    const int64_t bc = gid / NQ;
    const int64_t b = bc / D;
    const int c = (int)(bc % D);
    const float xv = to_f32(x[bc]);
    const float dtv = to_f32(dt[bc]);
    const float4 hv = *reinterpret_cast<const float4*>(h_in + bc * N + 4 * q);
    const float4 av = *reinterpret_cast<const float4*>(A + (size_t)c * N + 4 * q);
    float bv[4], cv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bv[i] = to_f32(Bm[b * N + 4 * q + i]);
        cv[i] = to_f32(Cm[b * N + 4 * q + i]);
    }
    const float dtx = dtv * xv;
    float4 hn;
    hn.x = fmaf(exp2_fast(dtv * av.x * kLog2e), hv.x, dtx * bv[0]);
    hn.y = fmaf(exp2_fast(dtv * av.y * kLog2e), hv.y, dtx * bv[1]);
    hn.z = fmaf(exp2_fast(dtv * av.z * kLog2e), hv.z, dtx * bv[2]);
    hn.w = fmaf(exp2_fast(dtv * av.w * kLog2e), hv.w, dtx * bv[3]);
    float p = cv[0] * hn.x + cv[1] * hn.y + cv[2] * hn.z + cv[3] * hn.w;
#pragma unroll
    for (int m = 1; m < NQ; m <<= 1) p += __shfl_xor(p, m, 64);
    *reinterpret_cast<float4*>(h_out + bc * N + 4 * q) = hn;
    if (q == 0) {
        float dv = Dskip ? Dskip[c] : 0.0f;
        store_out(&y[bc], fmaf(dv, xv, p));
    }
}

// Decode step for any N: one lane per (batch, channel).
template <typename IO>
__global__ __launch_bounds__(256) void k_m1_step_any(
    const IO* __restrict__ x, const IO* __restrict__ dt, const float* __restrict__ A,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dskip,
    const float* h_in, float* h_out, IO* __restrict__ y, int64_t total, int D, int N)
{
    int64_t bc = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (bc >= total) return;
    const int64_t b = bc / D;
    const int c = (int)(bc % D);
    const float xv = to_f32(x[bc]);
    const float dtv = to_f32(dt[bc]);
    const float dtx = dtv * xv;
    float p = 0.0f;
    for (int n = 0; n < N; ++n) {
        float a = exp2_fast(dtv * A[(size_t)c * N + n] * kLog2e);
        float hn = fmaf(a, h_in[bc * N + n], dtx * to_f32(Bm[b * N + n]));
        h_out[bc * N + n] = hn;
        p = fmaf(to_f32(Cm[b * N + n]), hn, p);
    }
    float dv = Dskip ? Dskip[c] : 0.0f;
    store_out(&y[bc], fmaf(dv, xv, p));
}

template <typename IO>
mb_status launch_scan(const void* x, const void* dt, const float* A, const void* B,
                      const void* C, const float* Dskip, const float* h0, void* y,
                      float* h_out, int64_t batch, int64_t L, int64_t D, int64_t N,
                      hipStream_t stream)
{
    const int n_cblk = (int)((D + kCW - 1) / kCW);
    const int n_wg = (int)(batch * n_cblk);
#define MB_SCAN_LAUNCH(NP)                                                                    \
    hipLaunchKernelGGL((k_m1_scan<NP, IO>), dim3(n_wg), dim3(kCW * NP), 0, stream,            \
                       (const IO*)x, (const IO*)dt, A, (const IO*)B, (const IO*)C, Dskip, h0, \
                       (IO*)y, h_out, (int)L, (int)D, (int)N, n_cblk, n_wg)
    if (N <= 16)
        MB_SCAN_LAUNCH(16);
    else if (N <= 32)
        MB_SCAN_LAUNCH(32);
    else
        MB_SCAN_LAUNCH(64);
#undef MB_SCAN_LAUNCH
    return check_launch();
}

template <typename IO>
mb_status launch_step(const void* x, const void* dt, const float* A, const void* B,
                      const void* C, const float* Dskip, const float* h_in, float* h_out,
                      void* y, int64_t batch, int64_t D, int64_t N, hipStream_t stream)
{
    const int64_t bcs = batch * D;
    const bool aligned = (((uintptr_t)h_in | (uintptr_t)h_out | (uintptr_t)A) & 15) == 0;
#define MB_STEP_Q(NQ)                                                                         \
    do {                                                                                     \
        int64_t total = bcs * NQ;                                                            \
        hipLaunchKernelGGL((k_m1_step_q<NQ, IO>), dim3((unsigned)((total + 255) / 256)),      \
                           dim3(256), 0, stream, (const IO*)x, (const IO*)dt, A,             \
                           (const IO*)B, (const IO*)C, Dskip, h_in, h_out, (IO*)y, total,    \
                           (int)D);                                                          \
    } while (0)
    if (aligned && N == 16)
        MB_STEP_Q(4);
    else if (aligned && N == 8)
        MB_STEP_Q(2);
    else if (aligned && N == 4)
        MB_STEP_Q(1);
    else if (aligned && N == 32)
        MB_STEP_Q(8);
    else if (aligned && N == 64)
        MB_STEP_Q(16);
    else
        hipLaunchKernelGGL((k_m1_step_any<IO>), dim3((unsigned)((bcs + 255) / 256)), dim3(256),
                           0, stream, (const IO*)x, (const IO*)dt, A, (const IO*)B,
                           (const IO*)C, Dskip, h_in, h_out, (IO*)y, bcs, (int)D, (int)N);
#undef MB_STEP_Q
    return check_launch();
}

}  // namespace
}  // namespace mb

using namespace mb;

extern "C" mb_status mb_selective_scan(const void* x, const void* dt, const float* A,
                                       const void* B, const void* C, const float* Dskip,
                                       const float* h0, void* y, float* h_out,
                                       int64_t batch, int64_t L, int64_t D, int64_t N,
                                       mb_dtype dtype, hipStream_t stream)
{
    if (!dtype_ok(dtype)) return MB_ERR_DTYPE;
    if (batch < 0 || L < 0 || D < 0 || N < 1 || N > 64) return MB_ERR_SHAPE;
    if (batch > INT32_MAX || L > INT32_MAX || D > INT32_MAX) return MB_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const size_t n_x = (size_t)(batch * L * D), n_b = (size_t)(batch * L * N);
    const size_t n_h = (size_t)(batch * D * N);
    if (batch * ((D + kCW - 1) / kCW) > INT32_MAX) return MB_ERR_SHAPE;
    if (n_x && (!x || !dt || !y)) return MB_ERR_NULL;
    if (n_b && (!B || !C)) return MB_ERR_NULL;
    if (D > 0 && !A) return MB_ERR_NULL;
    const Span ins[] = {{x, n_x * es}, {dt, n_x * es}, {B, n_b * es}, {C, n_b * es},
                        {A, (size_t)(D * N) * 4}, {Dskip, Dskip ? (size_t)D * 4 : 0},
                        {h0, h0 ? n_h * 4 : 0}};
    if (overlaps_any(y, n_x * es, ins, 7)) return MB_ERR_ALIAS;
    if (h_out) {
        if (overlaps_any(h_out, n_h * 4, ins, 6)) return MB_ERR_ALIAS;
        if (h0 && h0 != h_out && overlaps(h_out, n_h * 4, h0, n_h * 4)) return MB_ERR_ALIAS;
        if (overlaps(h_out, n_h * 4, y, n_x * es)) return MB_ERR_ALIAS;
    }
    if (batch == 0 || D == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, (int64_t)n_h, stream);
    if (dtype == MB_F32)
        return launch_scan<float>(x, dt, A, B, C, Dskip, h0, y, h_out, batch, L, D, N, stream);
    return launch_scan<bf16>(x, dt, A, B, C, Dskip, h0, y, h_out, batch, L, D, N, stream);
}

extern "C" mb_status mb_ssm_step(const void* x, const void* dt, const float* A, const void* B,
                                 const void* C, const float* Dskip, const float* h_in,
                                 float* h_out, void* y, int64_t batch, int64_t D, int64_t N,
                                 mb_dtype dtype, hipStream_t stream)
{
    if (!dtype_ok(dtype)) return MB_ERR_DTYPE;
    if (batch < 0 || D < 0 || N < 1) return MB_ERR_SHAPE;
    if (batch > INT32_MAX || D > INT32_MAX || N > INT32_MAX) return MB_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const size_t n_x = (size_t)(batch * D), n_b = (size_t)(batch * N);
    const size_t n_h = (size_t)(batch * D * N);
    if (n_x && (!x || !dt || !y || !h_in || !h_out || !A)) return MB_ERR_NULL;
    if (n_b && (!B || !C)) return MB_ERR_NULL;
    const Span ins[] = {{x, n_x * es}, {dt, n_x * es}, {B, n_b * es}, {C, n_b * es},
                        {A, (size_t)(D * N) * 4}, {Dskip, Dskip ? (size_t)D * 4 : 0},
                        {h_in, n_h * 4}};
    if (overlaps_any(y, n_x * es, ins, 7)) return MB_ERR_ALIAS;
    if (overlaps_any(h_out, n_h * 4, ins, 6)) return MB_ERR_ALIAS;
    if (h_out != h_in && overlaps(h_out, n_h * 4, h_in, n_h * 4)) return MB_ERR_ALIAS;
    if (overlaps(h_out, n_h * 4, y, n_x * es)) return MB_ERR_ALIAS;
    if (n_x == 0) return MB_OK;
    if (dtype == MB_F32)
        return launch_step<float>(x, dt, A, B, C, Dskip, h_in, h_out, y, batch, D, N, stream);
    return launch_step<bf16>(x, dt, A, B, C, Dskip, h_in, h_out, y, batch, D, N, stream);
}
