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
//     Y   = (w o S) X + diag(e^{cum}) C~ H,      S = C~ B~^T (rows x (R + rows))
//     H'  = e^{cum_last} H + B~^T diag(w(last, .)) X
// Rotations use chunk-local angles Phi_t = sum_{u<=t in chunk} theta_u, so B~ of
// the previous step is unrotated; the carried state is rotated back by
// R(-Phi_last) at the end of every chunk, which keeps it in the physical frame
// and keeps every angle small (no large accumulated angles in fp32).
//
// Kernels
//   k_scores  one workgroup per (batch, chunk, group-or-head): S = C~ B~^T on
//             fp32 MFMA 16x16x4 from LDS-staged rows, written to the caller's
//             workspace with a row stride padded to a multiple of 4.  Mamba-2
//             shares S across the heads of a group and the walk applies each
//             head's decay mask; for Mamba-3 (rotation per head) the trapezoid
//             weights w are applied here and the walk reads w o S directly.
//   k_walk    one workgroup (4 waves) per (batch, head, 16-column slice of P):
//             walks the chunks in order with the N x 16 state slice held in
//             MFMA accumulators.  Every wave loads the MFMA operands it needs
//             (its 16 rows of w o S and of C~, its 32 state rows of B~) straight
//             into registers one chunk ahead; only X, the weighted X, the state
//             and the angles go through LDS (double-buffered by chunk parity,
//             one barrier per chunk).  No chunk state is written to HBM.
// All global reads go through buffer resources that cover one batch row of a
// tensor, so reads before the first or after the last step return zero in
// hardware and the hot loops carry no bounds branches.
#include "mb_internal.h"

namespace mb {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------------------
// buffer resources: raw buffers (stride 0) whose size is the byte length of one
// batch row of a tensor; an offset at or past the size (negative offsets wrap
// to large unsigned values) reads as zero.
// ---------------------------------------------------------------------------
struct Buf {
    __amdgpu_buffer_rsrc_t r;
};

__device__ __forceinline__ Buf make_buf(const void* base, size_t bytes) {
    Buf b;
    b.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
    return b;
}

template <typename T>
__device__ __forceinline__ float bload(const Buf& b, int e);
template <>
__device__ __forceinline__ float bload<float>(const Buf& b, int e) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(b.r, e * 4, 0, 0));
}
template <>
__device__ __forceinline__ float bload<bf16>(const Buf& b, int e) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(b.r, e * 2, 0, 0) << 16);
}

template <typename T>
__device__ __forceinline__ float4 bload4(const Buf& b, int e);
template <>
__device__ __forceinline__ float4 bload4<float>(const Buf& b, int e) {
    uintx4 u = __builtin_amdgcn_raw_buffer_load_b128(b.r, e * 4, 0, 0);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w));
}
template <>
__device__ __forceinline__ float4 bload4<bf16>(const Buf& b, int e) {
    uintx2 u = __builtin_amdgcn_raw_buffer_load_b64(b.r, e * 2, 0, 0);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

template <int R, bool TRAP>
struct Geo {
    static constexpr int QT = kRows / R;                 // time steps per chunk
    static constexpr int EXTRA = TRAP ? R : 0;           // previous-step rows
    static constexpr int KC = kRows + EXTRA;             // columns of S
    static constexpr int KP = (KC + 3) / 4 * 4;          // padded to the MFMA K step (row stride of S)
    static constexpr int KS = KP / 4;                    // MFMA K steps over the columns
    static constexpr int KT = (KC + 15) / 16 * 16;       // padded to 16-wide tiles
    static constexpr int QS = QT / 4;                    // steps per angle-prefix segment
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
    float* S;        // workspace: scores (Mamba-2) or weighted scores (Mamba-3)
    int L, H, P, G, N, nch;
};

// Column j of a chunk's score matrix -> local time step s (-1 = previous step)
// and rank r; false for padding columns.
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

// Per-batch-row views of the inputs.  B/C: element (step t, n, rank r) at
//   t * bc_step + bc_head + n * R + r   with bc_step = G*N (grouped layout,
//   R == 1) or H*N*R (per-head layout), bc_head = g*N or h*N*R.
// X/Y: element (step t, p, r) at t * x_step + h*P*R + p*R + r, x_step = H*P*R.
template <int R, bool GROUPED, typename IO>
struct Views {
    Buf B, C, X, ld, gam, bet, th;
    int bc_step, bc_head, x_step, x_head;
    __device__ Views(const Args& a, int b, int h, int hg) {
        bc_step = GROUPED ? a.G * a.N : a.H * a.N * R;
        bc_head = GROUPED ? hg * a.N : hg * a.N * R;
        x_step = a.H * a.P * R;
        x_head = h * a.P * R;
        const size_t nbc = (size_t)a.L * bc_step;
        B = make_buf((const IO*)a.B + (size_t)b * nbc, nbc * sizeof(IO));
        C = make_buf((const IO*)a.C + (size_t)b * nbc, nbc * sizeof(IO));
        const size_t nx = (size_t)a.L * x_step;
        X = make_buf((const IO*)a.X + (size_t)b * nx, nx * sizeof(IO));
        const size_t ns = (size_t)a.L * a.H;
        ld = make_buf(a.ld + (size_t)b * ns, ns * 4);
        gam = make_buf(a.gamma ? a.gamma + (size_t)b * ns : a.ld, a.gamma ? ns * 4 : 0);
        bet = make_buf(a.beta ? a.beta + (size_t)b * ns : a.ld, a.beta ? ns * 4 : 0);
        const size_t nt = ns * (size_t)(a.N / 2);
        th = make_buf(a.theta ? a.theta + (size_t)b * nt : a.ld, a.theta ? nt * 4 : 0);
    }
};

// ---------------------------------------------------------------------------
// chunk-local rotation angles Phi[t][k] = sum_{u <= t} theta_u[k], t in [0, QT).
// Thread (k = 16 * wave + lane / 4, seg = lane % 4) owns steps
// [seg*QS, seg*QS + QS) of pair k: it prefix-sums them, takes the totals of the
// earlier segments from its quad and writes complete prefixes.
// ---------------------------------------------------------------------------
template <int QT, bool GROUPED_UNUSED = false>
__device__ __forceinline__ void angles_load(const Buf& th, int K, int H, int h, int t0g, float* v) {
    constexpr int QS = QT / 4;
    const int lane = threadIdx.x % 64;
    const int k = 16 * (threadIdx.x / 64) + lane / 4, seg = lane % 4;
    const int kk = k < K ? k : 0;
    const int base = ((t0g + seg * QS) * H + h) * K + kk;
#pragma unroll
    for (int i = 0; i < QS; ++i) {
        float x = bload<float>(th, base + i * H * K);
        v[i] = k < K ? x : 0.0f;
    }
}

template <int QT>
__device__ __forceinline__ void angles_store(const float* v, float* phi) {
    constexpr int QS = QT / 4;
    const int lane = threadIdx.x % 64;
    const int k = 16 * (threadIdx.x / 64) + lane / 4, seg = lane % 4;
    float acc[QS];
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < QS; ++i) {
        run += v[i];
        acc[i] = run;
    }
    // exclusive prefix of the segment totals within the quad
    const float t1 = __shfl_up(run, 1, 4);
    const float s1 = seg >= 1 ? t1 : 0.0f;
    const float incl1 = run + s1;                  // inclusive over 2
    const float t2 = __shfl_up(incl1, 2, 4);
    const float off = s1 + (seg >= 2 ? t2 : 0.0f);
#pragma unroll
    for (int i = 0; i < QS; ++i) phi[(seg * QS + i) * 64 + k] = acc[i] + off;
}

// ---------------------------------------------------------------------------
// Stage B or C rows of local steps [first_s, first_s + NSTEPS) into
// dst[((s - first_s) * R + r) * stride + n], rotated by the chunk-local angle of
// step s (step -1 is never rotated), zero outside the sequence and for n >= N.
// Work unit: U consecutive values of one step, holding whole rotation pairs
// (n, n+1) for every rank.  All loads of a thread are issued before use.
// ---------------------------------------------------------------------------
template <int NP, int R, int NSTEPS, bool ROT, typename IO>
__device__ __forceinline__ void stage_bc(const Buf& src, int bc_step, int bc_head, int N,
                                         int t0g, int first_s, float* dst, int stride,
                                         const float* phi) {
    constexpr int U = (2 * R > 8) ? 2 * R : 8;
    constexpr int UPS = NP * R / U;                  // units per step
    constexpr int NU = NSTEPS * UPS;
    constexpr int IT = (NU + kThreads - 1) / kThreads;
    float v[IT][U];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int u = threadIdx.x + it * kThreads;
        const int uu = u < NU ? u : 0;
        const int si = uu / UPS, f = (uu % UPS) * U;
        const int e = (t0g + first_s + si) * bc_step + bc_head + f;
        const bool okn = f / R < N && u < NU;
#pragma unroll
        for (int q = 0; q < U; q += 4) {
            float4 w4 = bload4<IO>(src, e + q);
            v[it][q] = okn ? w4.x : 0.0f;
            v[it][q + 1] = okn ? w4.y : 0.0f;
            v[it][q + 2] = okn ? w4.z : 0.0f;
            v[it][q + 3] = okn ? w4.w : 0.0f;
        }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int u = threadIdx.x + it * kThreads;
        if (u >= NU) continue;
        const int si = u / UPS, f = (u % UPS) * U;
        const int s = first_s + si;
        if (ROT && s >= 0) {
#pragma unroll
            for (int q = 0; q < U; ++q) {
                if (((q / R) & 1) == 0) {
                    const int k = ((f + q) / R) >> 1;
                    float sn, cs;
                    sincos_rev(phi[s * 64 + k], &sn, &cs);
                    const float v0 = v[it][q], v1 = v[it][q + R];
                    v[it][q] = fmaf(-sn, v1, cs * v0);
                    v[it][q + R] = fmaf(sn, v0, cs * v1);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int flat = f + q;
            dst[(si * R + flat % R) * stride + flat / R] = v[it][q];
        }
    }
}

__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        float o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// ---------------------------------------------------------------------------
// Scores per (batch, chunk, group-or-head)
// ---------------------------------------------------------------------------
template <int NP, int R, bool TRAP, bool ROT, bool GROUPED, typename IO>
__global__ __launch_bounds__(kThreads) void k_scores(Args a) {
    using Gm = Geo<R, TRAP>;
    constexpr int QT = Gm::QT;
    constexpr int SB = NP + 2;    // LDS row stride (= 2 mod 4: conflict-free MFMA reads)
    __shared__ float sC[kRows * SB];
    __shared__ float sB[Gm::KT * SB];
    __shared__ float sPhi[ROT ? QT * 64 : 1];
    __shared__ float s_cum[QT + 1];
    __shared__ float s_gam[QT];
    __shared__ float s_bet[QT + 1];

    const int c = blockIdx.x, hs = blockIdx.y, b = blockIdx.z;
    const int hg = (GROUPED && TRAP) ? hs / (a.H / a.G) : hs;
    const int t0g = c * QT;
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform per wave
    const Views<R, GROUPED, IO> vw(a, b, hs, hg);
    if (ROT) {
        float th[Gm::QS];
        angles_load<QT>(vw.th, a.N / 2, a.H, hs, t0g, th);
        angles_store<QT>(th, sPhi);
    }
    if (TRAP && wave == 0) {
        const int o = (t0g + lane) * a.H + hs;
        const bool in = lane < QT;
        const float ldv = in ? bload<float>(vw.ld, o) : 0.0f;
        const float cum = wave_incl_scan(ldv, lane);
        if (in) {
            s_cum[lane + 1] = cum;
            s_gam[lane] = bload<float>(vw.gam, o);
            s_bet[lane] = bload<float>(vw.bet, o);
        }
        if (lane == 0) {
            s_cum[0] = 0.0f;
            s_bet[QT] = 0.0f;
        }
    }
    for (int e = tid; e < (Gm::KT - Gm::KC) * NP; e += kThreads)
        sB[(Gm::KC + e / NP) * SB + e % NP] = 0.0f;
    __syncthreads();
    stage_bc<NP, R, QT, ROT, IO>(vw.C, vw.bc_step, vw.bc_head, a.N, t0g, 0, sC, SB, sPhi);
    stage_bc<NP, R, QT + (TRAP ? 1 : 0), ROT, IO>(vw.B, vw.bc_step, vw.bc_head, a.N, t0g,
                                                   TRAP ? -1 : 0, sB, SB, sPhi);
    __syncthreads();

    const int li = lane % 16, lk = lane / 16;
    constexpr int CT = Gm::KT / 16;
    float* Sout = a.S + (((size_t)b * a.nch + c) * gridDim.y + hs) * (size_t)(kRows * Gm::KP);
    for (int tile = wave; tile < 4 * CT; tile += 4) {
        const int rt = tile / CT, ct = tile % CT;
        floatx4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
        const float* pa = sC + (rt * 16 + li) * SB + lk;
        const float* pb = sB + (ct * 16 + li) * SB + lk;
#pragma unroll
        for (int n = 0; n < NP; n += 8) {
            acc0 = mfma4(pa[n], pb[n], acc0);
            acc1 = mfma4(pa[n + 4], pb[n + 4], acc1);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = rt * 16 + lk * 4 + r, j = ct * 16 + li;
            if (j >= Gm::KP) continue;
            float v = 0.0f;
            int s, rk;
            if (col_of<R, TRAP>(j, &s, &rk)) {
                v = acc0[r] + acc1[r];
                if (TRAP) {
                    const int tau = i / R;
                    float w = 0.0f;
                    if (s <= tau) {
                        if (s >= 0) w = s_gam[s] * exp_e(s_cum[tau + 1] - s_cum[s + 1]);
                        if (s < tau) w += s_bet[s + 1] * exp_e(s_cum[tau + 1] - s_cum[s + 2]);
                    }
                    v *= w;
                }
            }
            Sout[i * Gm::KP + j] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Chunk walk
// ---------------------------------------------------------------------------
// Uniform part of the element offset of B row j = 4s + lk (lk < 4): the step of
// row j, relative to the chunk's first step, times the step stride, plus the
// rank where it does not depend on lk.
template <int R, bool TRAP>
__device__ __forceinline__ int brow_uniform(int s, int step) {
    if (R == 1) return 4 * s * step;
    if (R == 2) return 2 * s * step;
    return (4 * s / R) * step + (4 * s) % R;
}
// Lane part of the same offset (everything that depends on lk and n).
template <int R, bool TRAP>
__device__ __forceinline__ int brow_lane(int lk, int n, int step, int head) {
    constexpr int E = TRAP ? 1 : 0;   // previous-step rows are one step back
    if (R == 1) return (lk - E) * step + head + n;
    if (R == 2) return (lk / 2 - E) * step + head + 2 * n + lk % 2;
    return -E * step + head + n * R + lk;
}

template <int NP, int R, bool TRAP>
struct WalkRegs {
    static constexpr int KS = Geo<R, TRAP>::KS;
    float m[KS];        // row 16w+li of (w o) S, columns 4s + lk
    float bb[2][KS];    // B rows 4s + lk, state row n = 32w + 16tt + li
    float cc[NP / 4];   // C row 16w + li, n = lk * NP/4 + s
};

template <int NP, int R, bool TRAP, bool ROT, bool GROUPED, typename IO, bool FULLN>
__global__ __launch_bounds__(kThreads) void k_walk(Args a) {
    using Gm = Geo<R, TRAP>;
    constexpr int QT = Gm::QT;
    constexpr int KP = Gm::KP;
    constexpr int KS = Gm::KS;
    constexpr int NQ = NP / 4;                    // state rows per lane quarter in C~ H
    constexpr int SHP = NP * kW + 4 * kW;         // state slice + a 16-float skew per quarter
    constexpr int XU = KP * 4;                    // float4 units of the staged X block
    constexpr int XR = (XU + kThreads - 1) / kThreads;

    __shared__ float sX[2][KP * kW];
    __shared__ float sXd[2][KP * kW];
    __shared__ float sH[2][SHP];
    __shared__ float sPhi[2][ROT ? QT * 64 : 1];
    __shared__ float s_cum[2][QT + 1];

    const int p0 = blockIdx.x * kW, h = blockIdx.y, b = blockIdx.z;
    const int hg = GROUPED ? h / (a.H / a.G) : h;
    const int hs = TRAP ? h : hg;
    const int nS = TRAP ? a.H : a.G;
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // uniform per wave
    const int li = lane % 16, lk = lane / 16;
    const size_t sh_off = (size_t)(b * a.H + h) * a.N * a.P;
    const Views<R, GROUPED, IO> vw(a, b, h, hg);
    constexpr bool fullN = FULLN;   // N == NP: no state rows to mask

    auto hidx = [](int n, int p) { return n * kW + p + (n / NQ) * kW; };

    // ---- lane constants of the operand loads ----------------------------------
    // S (or w o S): row 16w + li, column 4s + lk of chunk c's block
    const Buf Sbuf = make_buf(a.S + ((size_t)b * a.nch * nS + hs) * (size_t)(kRows * KP),
                              (size_t)a.nch * nS * kRows * KP * 4);
    const int s_lane = (16 * wave + li) * KP + lk;
    const int s_chunk = nS * kRows * KP;
    // B: two state rows per lane
    int b_lane[2];
    bool b_ok[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int n = 32 * wave + 16 * tt + li;
        b_ok[tt] = n < a.N;
        b_lane[tt] = brow_lane<R, TRAP>(lk, b_ok[tt] ? n : 0, vw.bc_step, vw.bc_head);
    }
    // C: row i = 16w + li (step i / R, rank i % R), state rows lk*NQ + s
    const int c_row = 16 * wave + li;
    const int c_lane = (c_row / R) * vw.bc_step + vw.bc_head + lk * NQ * R + c_row % R;
    const int c_nlim = a.N - lk * NQ;    // valid s < c_nlim

    // (w o) S rows and B~ columns of chunk c
    auto load_mb = [&](int c, WalkRegs<NP, R, TRAP>& o) {
        const int t0g = c * QT;
        const int sb = c * s_chunk + s_lane;
#pragma unroll
        for (int s = 0; s < KS; ++s) o.m[s] = bload<float>(Sbuf, sb + 4 * s);
        const int cb = t0g * vw.bc_step;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int s = 0; s < KS; ++s)
                o.bb[tt][s] = bload<IO>(vw.B, cb + b_lane[tt] + brow_uniform<R, TRAP>(s, vw.bc_step));
        }
        if (!fullN) {   // state rows past N (uniform, small N only)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int s = 0; s < KS; ++s) o.bb[tt][s] = b_ok[tt] ? o.bb[tt][s] : 0.0f;
        }
    };
    // C~ row of chunk c
    auto load_c = [&](int c, WalkRegs<NP, R, TRAP>& o) {
        const int cb = c * QT * vw.bc_step;
        if (R == 1) {
#pragma unroll
            for (int s = 0; s < NQ; s += 4) {
                const float4 w4 = bload4<IO>(vw.C, cb + c_lane + s);
                o.cc[s] = w4.x;
                o.cc[s + 1] = w4.y;
                o.cc[s + 2] = w4.z;
                o.cc[s + 3] = w4.w;
            }
        } else {
#pragma unroll
            for (int s = 0; s < NQ; ++s) o.cc[s] = bload<IO>(vw.C, cb + c_lane + s * R);
        }
        if (!fullN) {
#pragma unroll
            for (int s = 0; s < NQ; ++s) o.cc[s] = s < c_nlim ? o.cc[s] : 0.0f;
        }
    };

    // ---- X block, step scalars and angles of chunk c -> LDS buffer c & 1 ------
    float4 xr[XR];
    float th[ROT ? Gm::QS : 1];
    float sc_ld, sc_gam, sc_bet;
    auto load_stage = [&](int c) {
        const int t0g = c * QT;
#pragma unroll
        for (int q = 0; q < XR; ++q) {
            const int u = tid + q * kThreads;
            const int si = u / (4 * R), f = (u % (4 * R)) * 4;
            const int s = si - (TRAP ? 1 : 0);
            const int j0 = Gm::EXTRA + s * R;
            float4 v = bload4<IO>(vw.X, (t0g + s) * vw.x_step + vw.x_head + p0 * R + f);
            const bool ok = u < XU && j0 + R <= Gm::KC;
            xr[q] = ok ? v : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        if (ROT) angles_load<QT>(vw.th, a.N / 2, a.H, h, t0g, th);
        const bool in = lane < QT && t0g + lane < a.L;
        const size_t o = ((size_t)b * a.L + (in ? t0g + lane : 0)) * a.H + h;
        sc_ld = in ? a.ld[o] : 0.0f;
        sc_gam = (TRAP && in) ? a.gamma[o] : 0.0f;
        sc_bet = (TRAP && in) ? a.beta[o] : 0.0f;
    };
    auto store_stage = [&](int c) {
        const int buf = c & 1;
        const float cum = wave_incl_scan(sc_ld, lane);
        const float cum_last = __shfl(cum, QT - 1, 64);
        const float e = exp_e(cum_last - cum);
        const float wg = TRAP ? sc_gam * e : e;
        const float wb = TRAP ? sc_bet * e : 0.0f;
        if (wave == 0) {
            if (lane < QT) s_cum[buf][lane + 1] = cum;
            if (lane == 0) s_cum[buf][0] = 0.0f;
        }
#pragma unroll
        for (int q = 0; q < XR; ++q) {
            const int u = tid + q * kThreads;
            const int si = u / (4 * R), f = (u % (4 * R)) * 4;
            const int s = si - (TRAP ? 1 : 0);
            // weight of step s in the chunk-end state
            const float w_g = __shfl(wg, s < 0 ? 0 : (s < 64 ? s : 63), 64);
            const float w_b = __shfl(wb, s + 1 < 64 ? s + 1 : 63, 64);
            const float w = (s >= 0 ? w_g : 0.0f) + (s + 1 < QT ? w_b : 0.0f);
            if (u < XU) {
                const float vv[4] = {xr[q].x, xr[q].y, xr[q].z, xr[q].w};
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int flat = f + e4;               // (p, r) with r innermost
                    const int j = Gm::EXTRA + s * R + flat % R;
                    const int p = flat / R;
                    if (j < KP) {
                        sX[buf][j * kW + p] = vv[e4];
                        sXd[buf][j * kW + p] = vv[e4] * w;
                    }
                }
            }
        }
        if (ROT) angles_store<QT>(th, sPhi[buf]);
    };

    // ---- state ------------------------------------------------------------
    floatx4 acc_h[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = 32 * wave + 16 * tt + 4 * lk + r;
            acc_h[tt][r] = (a.h0 && n < a.N) ? a.h0[sh_off + (size_t)n * a.P + p0 + li] : 0.0f;
        }
    for (int e = tid; e < NP * kW; e += kThreads) {
        const int n = e / kW, p = e % kW;
        sH[0][hidx(n, p)] = (a.h0 && n < a.N) ? a.h0[sh_off + (size_t)n * a.P + p0 + p] : 0.0f;
    }

    WalkRegs<NP, R, TRAP> cur;
    load_mb(0, cur);
    load_c(0, cur);
    load_stage(0);
    store_stage(0);

    for (int c = 0; c < a.nch; ++c) {
        const int buf = c & 1;
        const int t0g = c * QT;
        __syncthreads();
        const bool more = c + 1 < a.nch;
        if (more) load_stage(c + 1);
        const float* phi = sPhi[buf];
        const float cum_last = s_cum[buf][QT];
        const float tot = exp_e(cum_last);

        // ---- Y_intra = (w o S) X and H' = e^{cum_last} H + B~^T (w_end o X) ---------
        floatx4 acc_y = {0.0f, 0.0f, 0.0f, 0.0f};
        floatx4 hacc0 = acc_h[0] * tot, hacc1 = acc_h[1] * tot;
        {
            const int tau_row = (16 * wave + li) / R;      // this lane's row, for the Mamba-2 mask
            const float cum_row = s_cum[buf][tau_row + 1];
            const int kend = Gm::EXTRA + ((16 * wave + 15) / R + 1) * R;
            const float* px = sX[buf] + lk * kW + li;
            const float* pxd = sXd[buf] + lk * kW + li;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if (4 * s < kend) {
                    float av = cur.m[s];
                    if (!TRAP) {
                        // R == 1: column j is step j; causal decay mask, branch-free
                        const int j = 4 * s + lk;
                        const float dec = exp_e(fminf(cum_row - s_cum[buf][j + 1], 0.0f));
                        av = (j <= tau_row) ? av * dec : 0.0f;
                    }
                    acc_y = mfma4(av, px[4 * s * kW], acc_y);
                }
                const float xd = pxd[4 * s * kW];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    // state rows past N have zero B~ and stay zero
                    float bv = cur.bb[tt][s];
                    if (ROT) {
                        const int n = 32 * wave + 16 * tt + li;
                        int st = 0, rk;
                        const bool col = col_of<R, TRAP>(4 * s + lk, &st, &rk);
                        const float partner = __shfl_xor(bv, 1, 64);
                        const bool rot = col && st >= 0;
                        float sn, cs;
                        sincos_rev(phi[(rot ? st : 0) * 64 + (n >> 1)], &sn, &cs);
                        const float sgn = (n & 1) ? sn : -sn;
                        const float rv = fmaf(sgn, partner, cs * bv);
                        bv = rot ? rv : bv;
                    }
                    if (tt == 0)
                        hacc0 = mfma4(bv, xd, hacc0);
                    else
                        hacc1 = mfma4(bv, xd, hacc1);
                }
            }
        }
        acc_h[0] = hacc0;
        acc_h[1] = hacc1;
        // the next chunk's S and B~ go into the registers just freed; they have the
        // C~ H product, the epilogue and the barrier to arrive
        if (more) load_mb(c + 1, cur);
        // ---- Y_state = C~ H  (H = state entering the chunk, from sH[buf]) ----------
        floatx4 acc_s0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc_s1 = {0.0f, 0.0f, 0.0f, 0.0f};
        {
            const int tau = c_row / R;
            if (ROT) {
#pragma unroll
                for (int s = 0; s < NQ; s += 2) {
                    const int k = (lk * NQ + s) >> 1;
                    float sn, cs;
                    sincos_rev(phi[tau * 64 + k], &sn, &cs);
                    const float v0 = cur.cc[s], v1 = cur.cc[s + 1];
                    cur.cc[s] = fmaf(-sn, v1, cs * v0);
                    cur.cc[s + 1] = fmaf(sn, v0, cs * v1);
                }
            }
            const float* ph = sH[buf] + hidx(lk * NQ, li);
#pragma unroll
            for (int s = 0; s < NQ; s += 2) {
                acc_s0 = mfma4(cur.cc[s], ph[s * kW], acc_s0);
                acc_s1 = mfma4(cur.cc[s + 1], ph[(s + 1) * kW], acc_s1);
            }
        }
        // the next chunk's C~ rows: needed only at its C~ H product
        if (more) load_c(c + 1, cur);
        // ---- write Y = Y_intra + e^{cum_tau} Y_state ---------------------------------
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * wave + 4 * lk + r;
            const int tau = i / R;
            const int tg = t0g + tau;
            const float y = fmaf(exp_e(s_cum[buf][tau + 1]), acc_s0[r] + acc_s1[r], acc_y[r]);
            if (tg < a.L)
                store_out(&((IO*)a.Y)[(((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P * R +
                                      (size_t)(p0 + li) * R + i % R], y);
        }
        // ---- rotate the state back to the physical frame and publish it ----------
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int n0 = 32 * wave + 16 * tt + 4 * lk;
            if (ROT && n0 < a.N) {
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    float sn, cs;
                    sincos_rev(phi[(QT - 1) * 64 + (n0 >> 1) + pr], &sn, &cs);
                    const float v0 = acc_h[tt][2 * pr], v1 = acc_h[tt][2 * pr + 1];
                    // R(-phi): (c v0 + s v1, -s v0 + c v1)
                    acc_h[tt][2 * pr] = fmaf(sn, v1, cs * v0);
                    acc_h[tt][2 * pr + 1] = fmaf(-sn, v0, cs * v1);
                }
            }
            if (n0 < NP) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sH[buf ^ 1][hidx(n0 + r, li)] = acc_h[tt][r];
            }
        }
        if (more) store_stage(c + 1);
    }
    if (a.h_out) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = 32 * wave + 16 * tt + 4 * lk + r;
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
    return (size_t)(batch * nch * nS) * (size_t)(kRows * Gm::KP) * sizeof(float);
}

template <int NP, int R, bool TRAP, bool ROT, bool GROUPED, typename IO>
mb_status launch(Args a, int64_t batch, hipStream_t stream) {
    using Gm = Geo<R, TRAP>;
    a.nch = (a.L + Gm::QT - 1) / Gm::QT;
    const int nS = TRAP ? a.H : a.G;
    hipLaunchKernelGGL((k_scores<NP, R, TRAP, ROT, GROUPED, IO>), dim3(a.nch, nS, (unsigned)batch),
                       dim3(kThreads), 0, stream, a);
    mb_status st = check_launch();
    if (st != MB_OK) return st;
    if (a.N == NP)
        hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, true>),
                           dim3(a.P / kW, a.H, (unsigned)batch), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false>),
                           dim3(a.P / kW, a.H, (unsigned)batch), dim3(kThreads), 0, stream, a);
    return check_launch();
}

template <int R, bool TRAP, bool ROT, bool GROUPED, typename IO>
mb_status launch_np(Args a, int64_t batch, hipStream_t stream) {
    if (a.N <= 64) return launch<64, R, TRAP, ROT, GROUPED, IO>(a, batch, stream);
    return launch<128, R, TRAP, ROT, GROUPED, IO>(a, batch, stream);
}

template <int R, bool TRAP, bool GROUPED>
mb_status dispatch(Args a, int64_t batch, mb_dtype dtype, hipStream_t stream) {
    const bool rot = a.theta != nullptr;
    if (dtype == MB_F32)
        return rot ? launch_np<R, TRAP, true, GROUPED, float>(a, batch, stream)
                   : launch_np<R, TRAP, false, GROUPED, float>(a, batch, stream);
    return rot ? launch_np<R, TRAP, true, GROUPED, bf16>(a, batch, stream)
               : launch_np<R, TRAP, false, GROUPED, bf16>(a, batch, stream);
}

bool dims_ok(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R = 1) {
    if (batch < 0 || L < 0 || H < 1 || P < 1 || N < 1) return false;
    if (N > kNMax || N % 4 != 0 || P % kW != 0) return false;
    if (batch > 65535 || H > 65535 || L > INT32_MAX / 2) return false;
    // one batch row of any tensor is addressed with 32-bit byte offsets
    const int64_t row = L * H * (P > N ? P : N) * R * 4;
    if (row >= (int64_t)1 << 31) return false;
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
    if (!dims_ok(batch, L, H, P, N, R)) return MB_ERR_SHAPE;
    if (chunk != 0 && chunk != kRows) return MB_ERR_SHAPE;
    if (theta && (N % 2)) return MB_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const size_t n_x = (size_t)(batch * L * H * P * R);
    const size_t n_bc = (size_t)(batch * L * nBC * N * R);
    const size_t n_s = (size_t)(batch * L * H);
    const size_t n_h = (size_t)(batch * H * N * P);
    if (n_x && (!X || !Y || !logdecay || !B || !C)) return MB_ERR_NULL;
    if (((uintptr_t)X | (uintptr_t)Y | (uintptr_t)B | (uintptr_t)C) & 15) return MB_ERR_ALIGN;
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
