// ssd.hip -- chunkwise SSD family for gfx950: Mamba-2 scalar-decay SSD,
// Mamba-3 SISO exponential-trapezoidal SSD with data-dependent rotations, and
// Mamba-3 MIMO rank R.
//
// One formulation covers all three (TorchMamba README, Math notes M2 / M3 SISO
// / MIMO; mamba3-minimal README, Two-SSD Decomposition).  A chunk holds QT time
// steps x R ranks = 64 rows.  Inside a chunk, with chunk-local cumulative
// log-decay cum_t (cum_{-1} = 0), the contribution of step s to the state at
// step tau >= s is
//     w(tau, s) = gamma_s e^{cum_tau - cum_s} + [s < tau] beta_{s+1} e^{cum_tau - cum_{s+1}}
// (Mamba-2: gamma = 1, beta = 0), and step s = -1 (the previous chunk's last
// step, whose own gamma term already sits in the carried state) enters through
// its beta term only.  Pre-shifting B and x by one step is the two-SSD
// decomposition; keeping both passes in one mask is the "1SS @ band" form, so
// the scores C~ B~^T, the decay factors and the output contraction are shared.
// Per chunk, with H the state entering the chunk (physical frame):
//     Y   = (M o S) X + diag(e^{cum}) C~ H,      S = C~ B~^T (rows x (R + rows))
//     H' = e^{cum_last} H + B~^T diag(w(last, .)) X
// Rotations use chunk-local angles Phi_t = sum_{u<=t in chunk} theta_u, so B~ of
// the previous step is unrotated; the carried state is rotated back by
// R(-Phi_last) at the end of every chunk, which keeps it in the physical frame
// and keeps every angle small (no large accumulated angles in fp32).
//
// Kernels
//   k_scores  one workgroup per (batch, chunk, group-or-head): S = C~ B~^T with
//             fp32 MFMA 16x16x4, written to the caller's workspace.  Mamba-2
//             shares S across the heads of a group; Mamba-3 rotates per head.
//   k_walk    one workgroup per (batch, head, 16-column slice of P): walks the
//             chunks in order with the 128x16 state slice held in MFMA
//             accumulators, builds M o S in LDS and runs the three contractions
//             on fp32 MFMA.  No chunk state is ever written to HBM.
#include "mb_internal.h"

namespace mb {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;    // rows per chunk (time steps x ranks)
constexpr int kW = 16;       // state / output columns per walk workgroup
constexpr int kNMax = 128;   // largest supported state size
constexpr int kThreads = 256;

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp_e(float v) { return exp2_fast(v * kLog2e); }

// sin / cos of an angle in radians through the hardware units, which take the
// argument in revolutions; the fraction of a revolution is taken first so the
// argument stays in [-0.5, 0.5].
__device__ __forceinline__ void sincos_rev(float phi, float* s, float* c) {
    float r = phi * 0.15915494309189535f;
    r = r - rintf(r);
    *s = __builtin_amdgcn_sinf(r);
    *c = __builtin_amdgcn_cosf(r);
}

template <int R, bool TRAP>
struct Geo {
    static constexpr int QT = kRows / R;                 // time steps per chunk
    static constexpr int EXTRA = TRAP ? R : 0;           // previous-step rows
    static constexpr int KC = kRows + EXTRA;             // columns of S
    static constexpr int KP = (KC + 3) / 4 * 4;          // padded to the MFMA K step
    static constexpr int KT = (KC + 15) / 16 * 16;       // padded to 16-wide tiles
    static constexpr int MS = KP + 2;                    // LDS row stride of M (= 2 mod 4)
};

struct Args {
    const void* X;
    const float* ld;
    const void* B;
    const void* C;
    const float* beta;
    const float* gamma;
    const float* theta;
    const float* h0;
    void* Y;
    float* h_out;
    float* S;        // workspace: scores
    int L, H, P, G, N, nch;
};

// Column j of a chunk's score matrix -> local time step s (-1 = previous step)
// and rank r; returns false for padding columns.
template <int R, bool TRAP>
__device__ __forceinline__ bool col_of(int j, int* s, int* r) {
    using G = Geo<R, TRAP>;
    if (j >= G::KC) return false;
    int jj = j - G::EXTRA;
    if (jj < 0) {
        *s = -1;
        *r = jj + R;
    } else {
        *s = jj / R;
        *r = jj % R;
    }
    return true;
}

// Offset of element n of the B/C row for (global step tg, rank r).
template <int R, bool GROUPED>
__device__ __forceinline__ size_t bc_off(const Args& a, int b, int tg, int hg, int n, int r) {
    if (GROUPED)   // (batch, L, G, N)
        return (((size_t)b * a.L + tg) * a.G + hg) * a.N + n;
    return ((((size_t)b * a.L + tg) * a.H + hg) * a.N + n) * R + r;   // (batch, L, H, N, R)
}

// Offset of X/Y element (global step tg, rank r, column p) of head h.
template <int R>
__device__ __forceinline__ size_t x_off(const Args& a, int b, int tg, int h, int p, int r) {
    return ((((size_t)b * a.L + tg) * a.H + h) * a.P + p) * R + r;
}

// Chunk-local rotation angles Phi[t][k] for local steps t in [0, QT): theta is
// staged into `phi` and prefix-summed along t in place (zero past the end).
template <int QT>
__device__ void stage_angles(const Args& a, int b, int h, int t0g, float* phi /*[QT][64]*/) {
    const int K = a.N / 2;
    for (int e = threadIdx.x; e < QT * 64; e += kThreads) {
        int t = e / 64, k = e % 64;
        int tg = t0g + t;
        float v = 0.0f;
        if (k < K && tg < a.L) v = a.theta[(((size_t)b * a.L + tg) * a.H + h) * K + k];
        phi[e] = v;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        float acc = 0.0f;
        for (int t = 0; t < QT; ++t) {
            acc += phi[t * 64 + threadIdx.x];
            phi[t * 64 + threadIdx.x] = acc;
        }
    }
    __syncthreads();
}

// Stage rotated rows into LDS.  Rows are indexed by "row slot" q: the caller
// maps q to (local step s, rank r); s = -1 means the previous chunk's last
// step (global t0g - 1), which is never rotated.  dst[q * stride + n].
template <int R, bool ROT, bool GROUPED, typename IO>
__device__ void stage_rows(const Args& a, const IO* src, int b, int hg, int t0g, int nslots,
                           int first_s, float* dst, int stride, const float* phi,
                           const float* scale /*per local step, may be null*/) {
    const int N = a.N;
    const int per_step = N * R;
    const int total = nslots * N;   // nslots = steps * R
    for (int e = threadIdx.x; e < total; e += kThreads) {
        // memory order within a step: GROUPED -> n; otherwise (n, r)
        int step_i = e / per_step;
        int rem = e % per_step;
        int n = GROUPED ? rem : rem / R;
        int r = GROUPED ? 0 : rem % R;
        int s = first_s + step_i;
        int tg = t0g + s;
        int q = step_i * R + r;
        float v = 0.0f, w = 0.0f;
        if (tg >= 0 && tg < a.L) {
            v = to_f32(src[bc_off<R, GROUPED>(a, b, tg, hg, n, r)]);
            if (ROT && s >= 0) {
                // partner element of the rotation pair
                int np = n ^ 1;
                w = to_f32(src[bc_off<R, GROUPED>(a, b, tg, hg, np, r)]);
                float sn, cs;
                sincos_rev(phi[s * 64 + (n >> 1)], &sn, &cs);
                // (v0, v1) -> (c v0 - s v1, s v0 + c v1)
                v = (n & 1) ? fmaf(sn, w, cs * v) : fmaf(-sn, w, cs * v);
            }
            if (scale && s >= 0) v *= scale[s];
        }
        dst[q * stride + n] = v;
    }
}

// ---------------------------------------------------------------------------
// Scores S = C~ B~^T per (batch, chunk, group-or-head)
// ---------------------------------------------------------------------------
template <int R, bool TRAP, bool ROT, bool GROUPED, typename IO>
__global__ __launch_bounds__(kThreads) void k_scores(Args a) {
    using Gm = Geo<R, TRAP>;
    constexpr int QT = Gm::QT;
    constexpr int SB = kNMax + 2;    // LDS stride (= 2 mod 4)
    __shared__ float sC[kRows * SB];
    __shared__ float sB[Gm::KT * SB];
    __shared__ float sphi[ROT ? QT * 64 : 1];

    const int c = blockIdx.x, hs = blockIdx.y, b = blockIdx.z;
    // hs indexes heads for rotated/per-head layouts and groups for Mamba-2
    const int h = hs;
    const int hg = (GROUPED && TRAP) ? hs / (a.H / a.G) : hs;   // source row of B/C
    const int t0g = c * QT;
    if (ROT) stage_angles<QT>(a, b, h, t0g, sphi);
    stage_rows<R, ROT, GROUPED, IO>(a, (const IO*)a.C, b, hg, t0g, kRows, 0, sC, SB, sphi, nullptr);
    stage_rows<R, ROT, GROUPED, IO>(a, (const IO*)a.B, b, hg, t0g, Gm::KC, TRAP ? -1 : 0, sB, SB,
                                    sphi, nullptr);
    // zero the padding rows of B~ so padding columns of S are zero
    for (int e = threadIdx.x; e < (Gm::KT - Gm::KC) * kNMax; e += kThreads)
        sB[(Gm::KC + e / kNMax) * SB + e % kNMax] = 0.0f;
    __syncthreads();

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int li = lane % 16, lk = lane / 16;
    constexpr int CT = Gm::KT / 16;               // column tiles
    float* Sout = a.S + (((size_t)b * a.nch + c) * gridDim.y + hs) * (size_t)(kRows * Gm::KC);
    for (int tile = wave; tile < 4 * CT; tile += 4) {
        const int rt = tile / CT, ct = tile % CT;
        floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        const float* pa = sC + (rt * 16 + li) * SB + lk;
        const float* pb = sB + (ct * 16 + li) * SB + lk;
        for (int n = 0; n < a.N; n += 4) acc = mfma4(pa[n], pb[n], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int i = rt * 16 + lk * 4 + r, j = ct * 16 + li;
            if (j < Gm::KC) Sout[i * Gm::KC + j] = acc[r];
        }
    }
}

// ---------------------------------------------------------------------------
// Chunk walk
// ---------------------------------------------------------------------------
template <int R, bool TRAP, bool ROT, bool GROUPED, typename IO>
__global__ __launch_bounds__(kThreads) void k_walk(Args a) {
    using Gm = Geo<R, TRAP>;
    constexpr int QT = Gm::QT;
    constexpr int KP = Gm::KP;
    constexpr int MS = Gm::MS;
    constexpr int SC = kNMax + 2;    // stride of C rows (A operand, = 2 mod 4)
    constexpr int SBW = kNMax + 16;  // stride of B rows (read transposed, = 16 mod 32)

    __shared__ float sM[kRows * MS];
    __shared__ float sX[KP * kW];
    __shared__ float sXd[KP * kW];
    __shared__ float sB[KP * SBW];
    __shared__ float sC[kRows * SC];
    __shared__ float sH[kNMax * kW];
    __shared__ float sphi[ROT ? QT * 64 : 1];
    __shared__ float s_cum[QT + 1];     // s_cum[t + 1] = cum_t, s_cum[0] = 0
    __shared__ float s_gam[QT];
    __shared__ float s_bet[QT + 1];     // s_bet[t] = beta_t, s_bet[QT] = 0
    __shared__ float s_din[QT];
    __shared__ float s_wend[KP];

    const int p0 = blockIdx.x * kW, h = blockIdx.y, b = blockIdx.z;
    const int hg = GROUPED ? h / (a.H / a.G) : h;
    const int hs = TRAP ? h : hg;               // index of this head's scores
    const int nS = TRAP ? a.H : a.G;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int li = lane % 16, lk = lane / 16;
    const size_t sh_off = (size_t)(b * a.H + h) * a.N * a.P;   // state (batch, H, N, P)

    // state accumulators: wave w owns rows n in [32w, 32w + 32) of the slice
    floatx4 acc_h[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int n = 32 * wave + 16 * tt + 4 * lk + r;
            acc_h[tt][r] = (a.h0 && n < a.N) ? a.h0[sh_off + (size_t)n * a.P + p0 + li] : 0.0f;
        }
    for (int e = tid; e < kNMax * kW; e += kThreads) {
        int n = e / kW, p = e % kW;
        sH[e] = (a.h0 && n < a.N) ? a.h0[sh_off + (size_t)n * a.P + p0 + p] : 0.0f;
    }

    for (int c = 0; c < a.nch; ++c) {
        const int t0g = c * QT;
        // ---- per-step scalars and chunk-local cumulative decay -------------
        if (wave == 0) {
            float ldv = 0.0f;
            if (lane < QT && t0g + lane < a.L)
                ldv = a.ld[((size_t)b * a.L + t0g + lane) * a.H + h];
            // inclusive scan across the wave (QT <= 64)
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                float o = __shfl_up(ldv, d, 64);
                if (lane >= d) ldv += o;
            }
            if (lane < QT) s_cum[lane + 1] = ldv;
            if (lane == 0) s_cum[0] = 0.0f;
        } else if (TRAP && wave == 1) {
            if (lane < QT) {
                int tg = t0g + lane;
                bool ok = tg < a.L;
                size_t o = ((size_t)b * a.L + tg) * a.H + h;
                s_gam[lane] = ok ? a.gamma[o] : 0.0f;
                s_bet[lane] = ok ? a.beta[o] : 0.0f;
            }
            if (lane == 0) s_bet[QT] = 0.0f;
        }
        if (ROT) stage_angles<QT>(a, b, h, t0g, sphi);   // contains barriers
        else __syncthreads();
        // din_t = e^{cum_t};  w_end for every column
        if (tid < QT) s_din[tid] = exp_e(s_cum[tid + 1]);
        const float cum_last = s_cum[QT];
        for (int j = tid; j < KP; j += kThreads) {
            int s, r;
            float w = 0.0f;
            if (col_of<R, TRAP>(j, &s, &r)) {
                if (!TRAP) {
                    w = exp_e(cum_last - s_cum[s + 1]);
                } else {
                    if (s >= 0) w = s_gam[s] * exp_e(cum_last - s_cum[s + 1]);
                    if (s < QT - 1) w += s_bet[s + 1] * exp_e(cum_last - s_cum[s + 2]);
                }
            }
            s_wend[j] = w;
        }
        __syncthreads();
        // ---- stage C~ (scaled by din), B~, X, weighted X, and M o S ---------
        stage_rows<R, ROT, GROUPED, IO>(a, (const IO*)a.C, b, hg, t0g, kRows, 0, sC, SC, sphi, s_din);
        stage_rows<R, ROT, GROUPED, IO>(a, (const IO*)a.B, b, hg, t0g, Gm::KC, TRAP ? -1 : 0, sB,
                                        SBW, sphi, nullptr);
        for (int e = tid; e < (KP - Gm::KC) * kNMax; e += kThreads)
            sB[(Gm::KC + e / kNMax) * SBW + e % kNMax] = 0.0f;
        for (int e = tid; e < KP * kW; e += kThreads) {
            int j = e / kW, p = e % kW;
            int s, r;
            float v = 0.0f;
            if (col_of<R, TRAP>(j, &s, &r)) {
                int tg = t0g + s;
                if (tg >= 0 && tg < a.L) v = to_f32(((const IO*)a.X)[x_off<R>(a, b, tg, h, p0 + p, r)]);
            }
            sX[e] = v;
            sXd[e] = v * s_wend[j];
        }
        {
            const float* Sin = a.S + (((size_t)b * a.nch + c) * nS + hs) * (size_t)(kRows * Gm::KC);
            for (int e = tid; e < kRows * KP; e += kThreads) {
                int i = e / KP, j = e % KP;
                int s, r;
                float v = 0.0f;
                if (col_of<R, TRAP>(j, &s, &r)) {
                    const int tau = i / R;
                    if (s <= tau) {
                        float w;
                        if (!TRAP) {
                            w = exp_e(s_cum[tau + 1] - s_cum[s + 1]);
                        } else {
                            w = 0.0f;
                            if (s >= 0) w = s_gam[s] * exp_e(s_cum[tau + 1] - s_cum[s + 1]);
                            if (s < tau) w += s_bet[s + 1] * exp_e(s_cum[tau + 1] - s_cum[s + 2]);
                        }
                        v = Sin[i * Gm::KC + j] * w;
                    }
                }
                sM[i * MS + j] = v;
            }
        }
        __syncthreads();

        // ---- Y = (M o S) X + C~' H  (rows 16w .. 16w+15) ---------------------
        floatx4 acc_y = {0.0f, 0.0f, 0.0f, 0.0f};
        {
            const int rmax = 16 * wave + 15;
            int kend = Gm::EXTRA + (rmax / R + 1) * R;   // columns with s <= tau(rmax)
            kend = (kend + 3) / 4 * 4;
            if (kend > KP) kend = KP;
            const float* pa = sM + (16 * wave + li) * MS + lk;
            const float* pb = sX + lk * kW + li;
            for (int k = 0; k < kend; k += 4) acc_y = mfma4(pa[k], pb[k * kW], acc_y);
            const float* pc = sC + (16 * wave + li) * SC + lk;
            const float* ph = sH + lk * kW + li;
            for (int n = 0; n < a.N; n += 4) acc_y = mfma4(pc[n], ph[n * kW], acc_y);
        }
        // ---- H' = e^{cum_last} H + B~^T (w_end o X) ---------------------------
        {
            const float tot = exp_e(cum_last);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int n0 = 32 * wave + 16 * tt;
                if (n0 < a.N) {
                    floatx4 acc = acc_h[tt] * tot;
                    const float* pa = sB + lk * SBW + n0 + li;
                    const float* pb = sXd + lk * kW + li;
                    for (int k = 0; k < KP; k += 4) acc = mfma4(pa[k * SBW], pb[k * kW], acc);
                    acc_h[tt] = acc;
                }
            }
        }
        // ---- write Y ----------------------------------------------------------
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int i = 16 * wave + 4 * lk + r;
            int tg = t0g + i / R;
            if (tg < a.L) store_out(&((IO*)a.Y)[x_off<R>(a, b, tg, h, p0 + li, i % R)], acc_y[r]);
        }
        __syncthreads();   // everyone is done with sH / sphi of this chunk
        // ---- rotate the state back to the physical frame and publish it -------
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int n0 = 32 * wave + 16 * tt + 4 * lk;
            if (ROT && n0 < a.N) {
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    float sn, cs;
                    sincos_rev(sphi[(QT - 1) * 64 + (n0 >> 1) + pr], &sn, &cs);
                    float v0 = acc_h[tt][2 * pr], v1 = acc_h[tt][2 * pr + 1];
                    // R(-phi): (c v0 + s v1, -s v0 + c v1)
                    acc_h[tt][2 * pr] = fmaf(sn, v1, cs * v0);
                    acc_h[tt][2 * pr + 1] = fmaf(-sn, v0, cs * v1);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sH[(n0 + r) * kW + li] = acc_h[tt][r];
        }
        __syncthreads();
    }
    if (a.h_out) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int n = 32 * wave + 16 * tt + 4 * lk + r;
                if (n < a.N) a.h_out[sh_off + (size_t)n * a.P + p0 + li] = acc_h[tt][r];
            }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int R, bool TRAP>
size_t scores_bytes(int64_t batch, int64_t L, int64_t nS) {
    using Gm = Geo<R, TRAP>;
    int64_t nch = (L + Gm::QT - 1) / Gm::QT;
    return (size_t)(batch * nch * nS) * (size_t)(kRows * Gm::KC) * sizeof(float);
}

template <int R, bool TRAP, bool ROT, bool GROUPED, typename IO>
mb_status launch(Args a, int64_t batch, hipStream_t stream) {
    using Gm = Geo<R, TRAP>;
    a.nch = (a.L + Gm::QT - 1) / Gm::QT;
    const int nS = TRAP ? a.H : a.G;
    hipLaunchKernelGGL((k_scores<R, TRAP, ROT, GROUPED, IO>), dim3(a.nch, nS, (unsigned)batch),
                       dim3(kThreads), 0, stream, a);
    mb_status st = check_launch();
    if (st != MB_OK) return st;
    hipLaunchKernelGGL((k_walk<R, TRAP, ROT, GROUPED, IO>), dim3(a.P / kW, a.H, (unsigned)batch),
                       dim3(kThreads), 0, stream, a);
    return check_launch();
}

template <int R, bool TRAP, bool GROUPED>
mb_status dispatch(Args a, int64_t batch, mb_dtype dtype, hipStream_t stream) {
    const bool rot = a.theta != nullptr;
    if (dtype == MB_F32)
        return rot ? launch<R, TRAP, true, GROUPED, float>(a, batch, stream)
                   : launch<R, TRAP, false, GROUPED, float>(a, batch, stream);
    return rot ? launch<R, TRAP, true, GROUPED, bf16>(a, batch, stream)
               : launch<R, TRAP, false, GROUPED, bf16>(a, batch, stream);
}

bool dims_ok(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N) {
    if (batch < 0 || L < 0 || H < 1 || P < 1 || N < 1) return false;
    if (N > kNMax || N % 4 != 0 || P % kW != 0) return false;
    if (batch > 65535 || H > 65535 || L > INT32_MAX / 2) return false;
    return true;
}

size_t ws_needed(mb_op op, int64_t batch, int64_t L, int64_t H, int64_t G, int64_t R) {
    switch (op) {
        case MB_OP_SSD_CHUNKED: return scores_bytes<1, false>(batch, L, G);
        case MB_OP_TRAP_SSD: return scores_bytes<1, true>(batch, L, H);
        case MB_OP_MIMO_SSD:
            switch (R) {
                case 1: return scores_bytes<1, true>(batch, L, H);
                case 2: return scores_bytes<2, true>(batch, L, H);
                case 4: return scores_bytes<4, true>(batch, L, H);
                case 8: return scores_bytes<8, true>(batch, L, H);
                case 16: return scores_bytes<16, true>(batch, L, H);
                default: return 0;
            }
        default: return 0;
    }
}

mb_status check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return MB_OK;
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255)) return MB_ERR_WORKSPACE;
    return MB_OK;
}

}  // namespace
}  // namespace mb

using namespace mb;

extern "C" size_t mb_workspace_size(mb_op op, int64_t batch, int64_t L, int64_t H, int64_t P,
                                    int64_t G, int64_t N, int64_t R, int64_t chunk) {
    (void)chunk;
    if (op == MB_OP_SELECTIVE_SCAN || op == MB_OP_SSM_STEP) return 0;
    if (!dims_ok(batch, L, H, P, N)) return 0;
    if (op == MB_OP_SSD_CHUNKED && (G < 1 || H % G)) return 0;
    return ws_needed(op, batch, L, H, G, R);
}

static mb_status ssd_common_checks(const void* X, const float* logdecay, const void* B,
                                   const void* C, const float* h0, void* Y, float* h_out,
                                   const float* beta, const float* gamma, const float* theta,
                                   int64_t batch, int64_t L, int64_t H, int64_t P, int64_t nBC,
                                   int64_t N, int64_t R, mb_dtype dtype, int64_t chunk,
                                   bool trap) {
    if (!dtype_ok(dtype)) return MB_ERR_DTYPE;
    if (!dims_ok(batch, L, H, P, N)) return MB_ERR_SHAPE;
    if (chunk != 0 && chunk != kRows) return MB_ERR_SHAPE;
    if (theta && (N % 2)) return MB_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const size_t n_x = (size_t)(batch * L * H * P * R);
    const size_t n_bc = (size_t)(batch * L * nBC * N * R);
    const size_t n_s = (size_t)(batch * L * H);
    const size_t n_h = (size_t)(batch * H * N * P);
    if (n_x && (!X || !Y || !logdecay || !B || !C)) return MB_ERR_NULL;
    if (trap && n_x && (!beta || !gamma)) return MB_ERR_NULL;
    const Span ins[] = {{X, n_x * es}, {B, n_bc * es}, {C, n_bc * es}, {logdecay, n_s * 4},
                        {beta, trap && beta ? n_s * 4 : 0}, {gamma, trap && gamma ? n_s * 4 : 0},
                        {theta, theta ? n_s * (size_t)(N / 2) * 4 : 0}, {h0, h0 ? n_h * 4 : 0}};
    if (overlaps_any(Y, n_x * es, ins, 8)) return MB_ERR_ALIAS;
    if (h_out) {
        if (overlaps_any(h_out, n_h * 4, ins, 7)) return MB_ERR_ALIAS;
        if (h0 && h0 != h_out && overlaps(h_out, n_h * 4, h0, n_h * 4)) return MB_ERR_ALIAS;
        if (overlaps(h_out, n_h * 4, Y, n_x * es)) return MB_ERR_ALIAS;
    }
    return MB_OK;
}

extern "C" mb_status mb_ssd_chunked(const void* X, const float* logdecay, const void* B,
                                    const void* C, const float* h0, void* Y, float* h_out,
                                    int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G,
                                    int64_t N, int64_t chunk, mb_dtype dtype, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
    if (G < 1 || H < 1 || H % G) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, nullptr, nullptr, nullptr,
                                     batch, L, H, P, G, N, 1, dtype, chunk, false);
    if (st != MB_OK) return st;
    const size_t need = ws_needed(MB_OP_SSD_CHUNKED, batch, L, H, G, 1);
    if (L > 0 && batch > 0 && (st = check_ws(ws, ws_bytes, need)) != MB_OK) return st;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    Args a{X, logdecay, B, C, nullptr, nullptr, nullptr, h0, Y, h_out, (float*)ws,
           (int)L, (int)H, (int)P, (int)G, (int)N, 0};
    return dispatch<1, false, true>(a, batch, dtype, stream);
}

extern "C" mb_status mb_trap_ssd(const void* X, const float* logdecay, const void* B,
                                 const void* C, const float* beta, const float* gamma,
                                 const float* theta, const float* h0, void* Y, float* h_out,
                                 int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G,
                                 int64_t N, int64_t chunk, mb_dtype dtype, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
    if (G < 1 || H < 1 || H % G) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, beta, gamma, theta, batch,
                                     L, H, P, G, N, 1, dtype, chunk, true);
    if (st != MB_OK) return st;
    const size_t need = ws_needed(MB_OP_TRAP_SSD, batch, L, H, G, 1);
    if (L > 0 && batch > 0 && (st = check_ws(ws, ws_bytes, need)) != MB_OK) return st;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    Args a{X, logdecay, B, C, beta, gamma, theta, h0, Y, h_out, (float*)ws,
           (int)L, (int)H, (int)P, (int)G, (int)N, 0};
    return dispatch<1, true, true>(a, batch, dtype, stream);
}

extern "C" mb_status mb_mimo_ssd(const void* X, const float* logdecay, const void* B,
                                 const void* C, const float* beta, const float* gamma,
                                 const float* theta, const float* h0, void* Y, float* h_out,
                                 int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                 int64_t R, int64_t chunk, mb_dtype dtype, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
    if (R != 1 && R != 2 && R != 4 && R != 8 && R != 16) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, beta, gamma, theta, batch,
                                     L, H, P, H, N, R, dtype, chunk, true);
    if (st != MB_OK) return st;
    const size_t need = ws_needed(MB_OP_MIMO_SSD, batch, L, H, 1, R);
    if (L > 0 && batch > 0 && (st = check_ws(ws, ws_bytes, need)) != MB_OK) return st;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    Args a{X, logdecay, B, C, beta, gamma, theta, h0, Y, h_out, (float*)ws,
           (int)L, (int)H, (int)P, (int)H, (int)N, 0};
    switch (R) {
        case 1: return dispatch<1, true, false>(a, batch, dtype, stream);
        case 2: return dispatch<2, true, false>(a, batch, dtype, stream);
        case 4: return dispatch<4, true, false>(a, batch, dtype, stream);
        case 8: return dispatch<8, true, false>(a, batch, dtype, stream);
        default: return dispatch<16, true, false>(a, batch, dtype, stream);
    }
}
