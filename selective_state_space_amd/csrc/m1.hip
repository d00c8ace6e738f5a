// m1.hip -- Mamba-1 selective scan and single-token decode step for gfx950.
//
// Recurrence (TorchMamba README, Math notes M1; burn_mamba Mamba1 docs,
// selective_scan / selective_scan_step), exponential-Euler discretisation:
//     h_t[c,n] = exp(dt_t[c] A[c,n]) h_{t-1}[c,n] + dt_t[c] B_t[n] x_t[c]
//     y_t[c]   = sum_n C_t[n] h_t[c,n] + Dskip[c] x_t[c]
//
// Scan layout (detailed at k_m1_scan): a workgroup of 64 x ceil(N/4) lanes owns
// 64 channels of one batch row and walks the whole sequence; each lane keeps
// four (channel, state) chains in registers.  One hardware exp2 per (t, c, n)
// element.
#include "mb_internal.h"

namespace mb {
namespace {

// Buffer resources over one batch row of a tensor: reads at or past the end
// (including the steps past L of the last tile) return zero.
struct Buf {
    __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ Buf make_buf(const void* base, size_t bytes) {
    Buf b;
    b.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
    return b;
}
__device__ __forceinline__ float bload(const Buf& b, int e, float) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(b.r, e * 4, 0, 0));
}
__device__ __forceinline__ float bload(const Buf& b, int e, bf16) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(b.r, e * 2, 0, 0) << 16);
}

// Scan layout.  A workgroup owns 64 channels of one batch row and walks the
// whole sequence; lane l of wave w holds channel c0 + l and the four states
// n = 4w .. 4w + 3, so the step's dt and dt*x serve four states and B_t, C_t
// of the wave's states are the same for all its lanes (one broadcast LDS read
// each).  Per tile of T steps the waves write their partial sums over their
// four states to LDS and, after one barrier, sum them per (t, c).
template <int NW, typename IO>
__global__ __launch_bounds__(64 * NW) void k_m1_scan(
    const IO* __restrict__ x, const IO* __restrict__ dt, const float* __restrict__ A,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dskip,
    const float* h0, IO* __restrict__ y, float* h_out, int L, int D, int N, int n_cg)
{
    constexpr int T = 16;           // steps per tile
    constexpr int NS = 4 * NW;      // states, padded to the waves
    // B / C tiles [B, C][t][n], one array per buffer parity: separate objects,
    // so a copy into one never orders the reads of the other
    __shared__ __attribute__((aligned(16))) float sBC0[2][T][NS];
    __shared__ __attribute__((aligned(16))) float sBC1[2][T][NS];
    __shared__ float sY[2][NW][T][64];                                // partial sums over states

    const int b = blockIdx.x / n_cg, c0 = (blockIdx.x % n_cg) * 64;
    const int tid = threadIdx.x, lane = tid % 64;
    const int w = __builtin_amdgcn_readfirstlane(tid / 64);
    const int c = c0 + lane;
    const bool cok = c < D;
    const size_t row = (size_t)L * D;
    const Buf bx = make_buf(x + (size_t)b * row, row * sizeof(IO));
    const Buf bdt = make_buf(dt + (size_t)b * row, row * sizeof(IO));
    const Buf bB = make_buf(Bm + (size_t)b * L * N, (size_t)L * N * sizeof(IO));
    const Buf bC = make_buf(Cm + (size_t)b * L * N, (size_t)L * N * sizeof(IO));

    float A2[4], h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = 4 * w + q;
        const bool ok = cok && n < N;
        A2[q] = ok ? A[(size_t)c * N + n] * kLog2e : 0.0f;   // states past N: a = 1, no input
        h[q] = (ok && h0) ? h0[((size_t)b * D + c) * N + n] : 0.0f;
    }
    const float Dv = (cok && Dskip) ? Dskip[c] : 0.0f;   // added by wave 0

    // B / C tile staging: thread tid holds element (t, n) = (tid / NS, tid % NS)
    const int bt = tid / NS, bn = tid % NS;
    const bool bok = bn < N;

    float dt_a[T], x_a[T], dt_b[T], x_b[T];
    float nB = 0.0f, nC = 0.0f;
    // fp32: the next tile's B / C go straight into LDS (LDS DMA, one dword per
    // lane into the wave's 64 consecutive slots); bf16 goes through registers
    constexpr bool DMA = sizeof(IO) == 4;
    auto load_bc = [&](int k, float (*dst)[T][NS]) {
        const int t0 = k * T;
        if constexpr (DMA) {
            if (bok && t0 + bt < L) {
                const size_t e = ((size_t)b * L + t0 + bt) * N + bn;
                __builtin_amdgcn_global_load_lds((const void*)(Bm + e),
                    (__attribute__((address_space(3))) void*)(&dst[0][0][0] + 64 * w), 4, 0, 0);
                __builtin_amdgcn_global_load_lds((const void*)(Cm + e),
                    (__attribute__((address_space(3))) void*)(&dst[1][0][0] + 64 * w), 4, 0, 0);
            }
        } else {
            const float lb = bload(bB, (t0 + bt) * N + bn, IO{});
            const float lc = bload(bC, (t0 + bt) * N + bn, IO{});
            nB = bok ? lb : 0.0f;
            nC = bok ? lc : 0.0f;
        }
    };
    auto load = [&](int k, float* pd, float* px, float (*dst)[T][NS]) {
        const int t0 = k * T;
        load_bc(k, dst);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            pd[t] = bload(bdt, (t0 + t) * D + c, IO{});
            px[t] = bload(bx, (t0 + t) * D + c, IO{});
        }
    };
    auto stash_bc = [&](float (*dst)[T][NS]) {
        if constexpr (!DMA) {
            dst[0][bt][bn] = nB;
            dst[1][bt][bn] = nC;
        }
    };
    // states at or past N are never copied: their slots stay zero
    if constexpr (DMA) {
        for (int e = tid; e < 2 * T * NS; e += 64 * NW) {
            (&sBC0[0][0][0])[e] = 0.0f;
            (&sBC1[0][0][0])[e] = 0.0f;
        }
        __syncthreads();
    }
    const int ntiles = (L + T - 1) / T;

    // one tile: T recurrence steps on this lane's four states, partial sums to
    // LDS, the next tile's B / C staged, one barrier, then the sums per (t, c)
    auto tile = [&](int k, const float* pd, const float* px, float* nd, float* nx,
                    float (*cur)[T][NS], float (*nxt)[T][NS]) {
        const int buf = k & 1;
        // unconditional (tiles past the end read zeros) and pinned here, so the
        // next tile's loads stay a full tile ahead of their use
        load(k + 1, nd, nx, nxt);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        // all of the tile's B / C for this wave's states first (broadcast reads),
        // so the LDS latency is paid once per tile rather than once per step
        float4 bqs[T], cqs[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            bqs[t] = *(const float4*)&cur[0][t][4 * w];
            cqs[t] = *(const float4*)&cur[1][t][4 * w];
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float4 bq = bqs[t];
            const float4 cq = cqs[t];
            const float dtv = pd[t];
            const float dtx = dtv * px[t];
            h[0] = fmaf(exp2_fast(dtv * A2[0]), h[0], dtx * bq.x);
            h[1] = fmaf(exp2_fast(dtv * A2[1]), h[1], dtx * bq.y);
            h[2] = fmaf(exp2_fast(dtv * A2[2]), h[2], dtx * bq.z);
            h[3] = fmaf(exp2_fast(dtv * A2[3]), h[3], dtx * bq.w);
            float p = fmaf(cq.x, h[0], fmaf(cq.y, h[1], fmaf(cq.z, h[2], cq.w * h[3])));
            if (w == 0) p = fmaf(Dv, px[t], p);
            sY[buf][w][t][lane] = p;
        }
        if (k + 1 < ntiles) stash_bc(nxt);
        if constexpr (DMA) {
            // the next tile's B / C copies were issued before its 2T dt / x loads
            __builtin_amdgcn_s_waitcnt(((2 * T) & 15) | (((2 * T) >> 4) << 14) | (7 << 4) | (15 << 8));
        }
        __syncthreads();
        const int t0 = k * T;
#pragma unroll
        for (int t = w; t < T; t += NW) {
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < NW; ++v) s += sY[buf][v][t][lane];
            if (cok && t0 + t < L) store_out(&y[((size_t)b * L + t0 + t) * D + c], s);
        }
    };

    if (ntiles > 0) {
        load(0, dt_a, x_a, sBC0);
        stash_bc(sBC0);
    }
    // everything loaded so far (initial state, first tile) has arrived: the
    // waits inside the loop then only cover the tile loads in flight
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    __syncthreads();
    for (int k = 0; k < ntiles; k += 2) {
        tile(k, dt_a, x_a, dt_b, x_b, sBC0, sBC1);
        if (k + 1 < ntiles) tile(k + 1, dt_b, x_b, dt_a, x_a, sBC1, sBC0);
    }
    if (h_out && cok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = 4 * w + q;
            if (n < N) h_out[((size_t)b * D + c) * N + n] = h[q];
        }
    }
}

// Decode step, N a multiple of 4 with N/4 dividing 64: one lane per
// (channel, group of 4 states) of one batch row (grid y = batch, so no
// division by D); 16-byte state loads and stores, streamed past the caches,
// so consecutive lanes move consecutive 16-byte pieces of the state.  The sum
// over n is a butterfly over the N/4 lanes of a channel (DPP within quads).
typedef float f4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float xor_lanes(float v, int m) {
    if (m == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
    if (m == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
    return __shfl_xor(v, m, 64);
}

// Each thread handles K (channel, state-quad) items 256 apart, all loads first,
// so a wave keeps K 16-byte state loads in flight (h_out may alias h_in).
template <int NQ, typename IO, bool VEC_BC, int K>
__global__ __launch_bounds__(256) void k_m1_step_q(
    const IO* __restrict__ x, const IO* __restrict__ dt, const float* __restrict__ A,
    const IO* __restrict__ Bm, const IO* __restrict__ Cm, const float* __restrict__ Dskip,
    const float* h_in, float* h_out, IO* __restrict__ y, int D)
{
    constexpr int N = NQ * 4;
    const int b = blockIdx.y;
    int c[K], q[K];
    bool ok[K];
    size_t bc[K];
    float xv[K], dtv[K];
    f4v hv[K];
    float4 av[K];
    float bv[4], cv[4];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int idx = (blockIdx.x * K + k) * 256 + threadIdx.x;
        c[k] = idx / NQ;
        q[k] = idx % NQ;
        ok[k] = c[k] < D;                 // lanes past D compute on channel 0, store nothing
        const int cc = ok[k] ? c[k] : 0;
        bc[k] = (size_t)b * D + cc;
        xv[k] = to_f32(x[bc[k]]);
        dtv[k] = to_f32(dt[bc[k]]);
        hv[k] = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(h_in + bc[k] * N + 4 * q[k]));
        av[k] = *reinterpret_cast<const float4*>(A + (size_t)cc * N + 4 * q[k]);
    }
    // B and C of this batch row: the state quad of item k is q[k] = threadIdx.x % NQ for all k
    const int qq = threadIdx.x % NQ;
    if constexpr (VEC_BC) {
        const float4 b4 = *reinterpret_cast<const float4*>((const float*)Bm + (size_t)b * N + 4 * qq);
        const float4 c4 = *reinterpret_cast<const float4*>((const float*)Cm + (size_t)b * N + 4 * qq);
        bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
        cv[0] = c4.x; cv[1] = c4.y; cv[2] = c4.z; cv[3] = c4.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bv[i] = to_f32(Bm[(size_t)b * N + 4 * qq + i]);
            cv[i] = to_f32(Cm[(size_t)b * N + 4 * qq + i]);
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const float dtx = dtv[k] * xv[k];
        f4v hn;
        hn.x = fmaf(exp2_fast(dtv[k] * av[k].x * kLog2e), hv[k].x, dtx * bv[0]);
        hn.y = fmaf(exp2_fast(dtv[k] * av[k].y * kLog2e), hv[k].y, dtx * bv[1]);
        hn.z = fmaf(exp2_fast(dtv[k] * av[k].z * kLog2e), hv[k].z, dtx * bv[2]);
        hn.w = fmaf(exp2_fast(dtv[k] * av[k].w * kLog2e), hv[k].w, dtx * bv[3]);
        float p = cv[0] * hn.x + cv[1] * hn.y + cv[2] * hn.z + cv[3] * hn.w;
#pragma unroll
        for (int m = 1; m < NQ; m <<= 1) p += xor_lanes(p, m);   // all lanes take part
        if (ok[k]) {
            __builtin_nontemporal_store(hn, reinterpret_cast<f4v*>(h_out + bc[k] * N + 4 * q[k]));
            if (q[k] == 0) {
                const float dv = Dskip ? Dskip[c[k]] : 0.0f;
                store_out(&y[bc[k]], fmaf(dv, xv[k], p));
            }
        }
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
    const int n_cg = (int)((D + 63) / 64);
    const int n_wg = (int)(batch * n_cg);
#define MB_SCAN_LAUNCH(NW)                                                                    \
    hipLaunchKernelGGL((k_m1_scan<NW, IO>), dim3(n_wg), dim3(64 * NW), 0, stream,             \
                       (const IO*)x, (const IO*)dt, A, (const IO*)B, (const IO*)C, Dskip, h0, \
                       (IO*)y, h_out, (int)L, (int)D, (int)N, n_cg)
    if (N <= 4)
        MB_SCAN_LAUNCH(1);
    else if (N <= 8)
        MB_SCAN_LAUNCH(2);
    else if (N <= 16)
        MB_SCAN_LAUNCH(4);
    else if (N <= 32)
        MB_SCAN_LAUNCH(8);
    else
        MB_SCAN_LAUNCH(16);
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
    const bool vec_bc = sizeof(IO) == 4 && ((((uintptr_t)B | (uintptr_t)C) & 15) == 0);
#define MB_STEP_Q(NQ)                                                                         \
    do {                                                                                     \
        const dim3 grid((unsigned)((D * NQ + 511) / 512), (unsigned)batch);                  \
        if (vec_bc)                                                                          \
            hipLaunchKernelGGL((k_m1_step_q<NQ, IO, true, 2>), grid, dim3(256), 0, stream,   \
                               (const IO*)x, (const IO*)dt, A, (const IO*)B, (const IO*)C,   \
                               Dskip, h_in, h_out, (IO*)y, (int)D);                          \
        else                                                                                 \
            hipLaunchKernelGGL((k_m1_step_q<NQ, IO, false, 2>), grid, dim3(256), 0, stream,  \
                               (const IO*)x, (const IO*)dt, A, (const IO*)B, (const IO*)C,   \
                               Dskip, h_in, h_out, (IO*)y, (int)D);                          \
    } while (0)
    if (aligned && N == 16 && batch <= 65535)
        MB_STEP_Q(4);
    else if (aligned && N == 8 && batch <= 65535)
        MB_STEP_Q(2);
    else if (aligned && N == 4 && batch <= 65535)
        MB_STEP_Q(1);
    else if (aligned && N == 32 && batch <= 65535)
        MB_STEP_Q(8);
    else if (aligned && N == 64 && batch <= 65535)
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
    if (batch * ((D + 63) / 64) > INT32_MAX) return MB_ERR_SHAPE;
    // one batch row is addressed with 32-bit byte offsets (tile padding included)
    if ((L + 16) * D * 4 >= ((int64_t)1 << 31) || (L + 16) * N * 4 >= ((int64_t)1 << 31)) return MB_ERR_SHAPE;
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
