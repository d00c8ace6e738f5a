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
//     Y   = (w o S) X + diag(e^{cum}) C~ H,      S = C~ B~^T (rows x (rows + R))
//     H'  = e^{cum_last} H + B~^T diag(w(last, .)) X
// The full pass of the trapezoid folds the previous step's term into the state
// first, H+ = alpha_0 H + beta_0 B_{-1}^T x_{-1}, after which it decays with the
// chunk like the state: Y = (w o S) X + diag(e^{cum - cum_0}) C~ H+ with S only
// over the chunk's own rows, and H' = e^{cum_last - cum_0} H+ + B~^T diag(w) X.
// Rotations use chunk-local angles Phi_t = sum_{u<=t in chunk} theta_u, so B~ of
// the previous step is unrotated; the carried state is rotated back by
// R(-Phi_last) at the end of every chunk, which keeps it in the physical frame
// and keeps every angle small (no large accumulated angles in fp32).
//
// Sequence segments.  The state entering segment s of the sequence is
//     H_in(s+1) = e^{sum ld over s} R(-sum theta over s) H_in(s) + H_loc(s),
// where H_loc(s) is segment s walked from a zero state: the (decay, state) pair
// composition of a linear recurrence.  A state-only pass computes H_loc, the
// total log-decay and the total angle of every segment but the last; the full
// pass then starts every segment from its combined entering state, so all
// segments of a sequence run in parallel.
//
// Kernels
//   k_scores  (Mamba-2 only) one workgroup per (batch, chunk, group):
//             S = C B^T on fp32 MFMA, shared by the heads of the group.
//   k_walk_m2s  (Mamba-2, fp32 full pass) the same walk with the roles split:
//             four matrix waves hold the state and do every product, four
//             staging waves copy B and C into LDS and stage X and the masked
//             scores of the next chunk.
//   k_walk_bfs  (Mamba-2, bf16 full pass) the same split on the bf16 matrix
//             instruction; k_walk_bf is its state-only pass.
//   k_seg_state  (Mamba-2, fp32 state-only pass) each segment's local end
//             state as one weighted product over its steps, without a walk;
//             k_seg_trap the same for SISO (trapezoid weights, rotations).
//   k_pad     zero-padded copies for Mamba-2 shapes outside the walks' tiles.
//   k_walk    one workgroup (8 waves) per (batch, head, segment, 64 state
//             columns), walking the segment's chunks in order.  Per chunk the
//             workgroup stages B~ and C~ (rotated once, for all columns), X and
//             the chunk-end-weighted X (transposed) and the masked score matrix
//             in LDS; waves w and w+4 own state columns 16w..16w+15, each for
//             half of the N rows, as MFMA accumulators.  For Mamba-3 the scores C~ B~^T are computed in
//             the walk (they are per head).  The state rows are permuted inside
//             the accumulator tiles so that the accumulators are directly the
//             operand of the next chunk's C~ H product: the state never leaves
//             registers.
//             Two variants carry the Mamba-3 block's ends for SISO and every
//             MIMO rank (mamba3-minimal README, Architecture): EPI (full
//             pass) loads X and the gate z at the chunk's start and stores
//             (y + D_h x) SiLU(z); BCN (both passes) turns each raw B, C row
//             in the prefetch registers into row / rms(row) * weight + bias_h
//             (one DPP sum over the row's wave) before the rotations.  PRO
//             (Mamba-2 state-only pass of the layer) convolves x as it stages
//             it.
// All global reads go through buffer resources that cover one batch row of a
// tensor, so reads before the first or after the last step return zero in
// hardware and the hot loops carry no bounds branches.
#include <mutex>

#include "mb_internal.h"

namespace mb {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;      // rows per chunk (time steps x ranks)
constexpr int kPG = 64;        // state / output columns per walk workgroup
constexpr int kNMax = 128;     // largest supported state size
constexpr int kThreads = 256;

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp_e(float v) { return exp2_fast(v * kLog2e); }

// a compile-time int carried by a lambda argument
template <int V>
struct Par {
    static constexpr int value = V;
};

// bf16 matrix instruction: 16 x 16 x 32, fp32 accumulation.  Lane l supplies
// A[l % 16][8 (l / 16) + q] and B[8 (l / 16) + q][l % 16], q = 0..7, as four
// registers of bf16 pairs; the accumulator layout is that of the fp32 16 x 16
// instruction.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mfma_bf(uintx4 a, uintx4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// two fp32 values rounded to nearest-even bf16, packed (lo in the low half)
__device__ __forceinline__ uint32_t pack_bf(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){lo, hi}, bf16x2));
}

// Wait until at most N vector memory operations of this wave are outstanding
// (s_waitcnt vmcnt(N), other counters unconstrained).
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));
}

// sin / cos of an angle in radians through the hardware units, which take the
// argument in revolutions; the fraction of a revolution is taken first so the
// argument stays in [-0.5, 0.5].
__device__ __forceinline__ void sincos_rev(float phi, float* s, float* c) {
    float r = phi * 0.15915494309189535f;
    r = r - rintf(r);
    *s = __builtin_amdgcn_sinf(r);
    *c = __builtin_amdgcn_cosf(r);
}

// inclusive prefix sum over the 64 lanes with DPP row shifts and broadcasts
__device__ __forceinline__ float wave_scan_dpp(float v) {
#define MB_DPP(ctrl, rmask) \
    __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rmask, 0xf, false))
    v += MB_DPP(0x111, 0xf);   // row_shr:1
    v += MB_DPP(0x112, 0xf);   // row_shr:2
    v += MB_DPP(0x114, 0xf);   // row_shr:4
    v += MB_DPP(0x118, 0xf);   // row_shr:8
    v += MB_DPP(0x142, 0xa);   // row_bcast:15 into rows 1 and 3
    v += MB_DPP(0x143, 0xc);   // row_bcast:31 into rows 2 and 3
#undef MB_DPP
    return v;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// A chunk's decay factors e^{cum_i - cum_t} (i >= t) may be taken as
// e^{cum_i - cum_31} e^{cum_31 - cum_t} when neither factor can leave the fp32
// range: every |cum_i - cum_31| is at most the sum of |ld| over steps 0..31 or
// over 32..63, so both sums at most 80 suffice.  ld: step `lane`'s log-decay
// (zero past the chunk); the result is the same on every lane.
__device__ __forceinline__ bool decay_factors_safe(float ld) {
    const float sa = wave_scan_dpp(fabsf(ld));
    const float lo = readlane_f(sa, 31), all = readlane_f(sa, 63);
    return fmaxf(lo, all - lo) <= 80.0f;
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


// CNT contiguous elements starting at element e, widened to fp32.
template <typename IO, int CNT>
struct VecLoad;
template <int CNT>
struct VecLoad<float, CNT> {
    static __device__ __forceinline__ void run(const Buf& b, int e, float* o) {
        if constexpr (CNT == 1) {
            o[0] = bload<float>(b, e);
        } else if constexpr (CNT == 2) {
            const uintx2 u = __builtin_amdgcn_raw_buffer_load_b64(b.r, e * 4, 0, 0);
            o[0] = __uint_as_float(u.x);
            o[1] = __uint_as_float(u.y);
        } else {
            static_assert(CNT % 4 == 0, "fp32 vector loads take 1, 2 or 4k elements");
#pragma unroll
            for (int q = 0; q < CNT; q += 4) {
                const uintx4 u = __builtin_amdgcn_raw_buffer_load_b128(b.r, (e + q) * 4, 0, 0);
                o[q] = __uint_as_float(u.x);
                o[q + 1] = __uint_as_float(u.y);
                o[q + 2] = __uint_as_float(u.z);
                o[q + 3] = __uint_as_float(u.w);
            }
        }
    }
};
template <int CNT>
struct VecLoad<bf16, CNT> {
    static __device__ __forceinline__ void run(const Buf& b, int e, float* o) {
        if constexpr (CNT == 1) {
            o[0] = bload<bf16>(b, e);
        } else if constexpr (CNT == 2) {
            const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(b.r, e * 2, 0, 0);
            o[0] = __uint_as_float(u << 16);
            o[1] = __uint_as_float(u & 0xffff0000u);
        } else {
            static_assert(CNT % 4 == 0, "bf16 vector loads take 1, 2 or 4k elements");
#pragma unroll
            for (int q = 0; q < CNT; q += 4) {
                const uintx2 u = __builtin_amdgcn_raw_buffer_load_b64(b.r, (e + q) * 2, 0, 0);
                o[q] = __uint_as_float(u.x << 16);
                o[q + 1] = __uint_as_float(u.x & 0xffff0000u);
                o[q + 2] = __uint_as_float(u.y << 16);
                o[q + 3] = __uint_as_float(u.y & 0xffff0000u);
            }
        }
    }
};

template <int R, bool TRAP>
struct Geo {
    static constexpr int QT = kRows / R;                  // time steps per chunk
    static constexpr int QS = QT / 4;                     // steps per staging quarter
    static constexpr int EXTRA = TRAP ? R : 0;            // previous-step rows j = 64 .. 64+EXTRA-1
    static constexpr int JX = (EXTRA + 3) / 4;            // MFMA K steps over them
    static constexpr int JC = kRows + 4 * JX;             // columns of X^T / M in use
    static constexpr int JP = (JC % 8 == 0) ? JC + 4 : JC + 8;   // LDS row stride (4 mod 8)
    static constexpr int BR = TRAP ? kRows + 16 : kRows;  // staged B~ rows (zero padded)
    static constexpr int PR = (R + 3) / 4;                // previous-step ranks per staging thread
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
    const void* X_prev;   // trapezoid: the token before the call (NULL: zeros)
    const void* B_prev;
    void* Y;
    float* h_out;
    float* S;        // Mamba-2 scores, (batch, chunk, group, 64, 64)
    bf16* BT;        // Mamba-2 with bf16 inputs: B^T per chunk, (batch, chunk, group, NP, 64)
    float* seg_h;    // local end states of segments 0..nseg-2, (batch, H, nseg-1, N, P)
    float* seg_ld;   // their total log-decay, (batch, H, nseg-1)
    float* seg_rev;  // their total angle per pair in revolutions mod 1, (batch, H, nseg-1, N/2)
    int L, H, P, G, N, nch, nseg, cps, npg;
    // SISO output epilogue (NULL: none): Y = (S^T C~ + Dh[h] X) SiLU(Zg)
    const float* Dh;  // (H)
    const void* Zg;   // (batch, L, H, P), the dtype of X
    // SISO BCNorm + bias prologue on B and C (bcn != 0): each row scaled by
    // 1/sqrt(mean over N of its squares + eps), times the per-state weight
    // (NULL: ones), plus the head's bias (NULL: zeros)
    const float* nwB;    // (N)
    const float* nwC;    // (N)
    const float* biasB;  // (H, N)
    const float* biasC;  // (H, N)
    float eps;
    int bcn;
    // Mamba-2 block (pro != 0): the scan's inputs come from the block's raw
    // projected channels xBC = (x | B | C) by the causal convolution over time
    // (K taps, the last on the current step; the K - 1 rows before the call
    // from xh) and SiLU, and dt' = softplus(dt + dt_bias).  k_scores convolves
    // B and C (to Bw, Cw) and writes dt' and the log-decay dt' A (to dtp, and
    // to ld, which the walks read); the walks convolve x themselves (X then
    // points at xBC, rows cin apart) and apply dt' to the masked scores and the
    // chunk-end weights rather than to x, with Dskip on the diagonal of the
    // masked scores (the skip term on the convolved x)
    const void* Xr;       // xBC (batch, L, cin), the dtype of X
    const float* cw;      // (cin, K)
    const float* cbias;   // (cin) or NULL
    const void* xh;       // (batch, K - 1, cin) or NULL
    const float* dtr;     // raw dt (batch, L, H)
    const float* dtbias;  // (H) or NULL
    const float* Ah;      // (H)
    float* dtp;           // dt' (batch, L, H), workspace
    void* Bw;             // convolved B, C (batch, L, G, N), the dtype of X, workspace
    void* Cw;
    int cin, K, pro;
    // output side of the Mamba-2 layer run as two passes (prologue pass, then the
    // walk on its X = x dt'): the skip term takes x = X / dt', dt' (batch, L, H)
    // here; NULL: the skip term takes X
    const float* skip_dt;
};

// softplus(v) = max(v, 0) + log(1 + e^-|v|)
__device__ __forceinline__ float softplus_acc(float v) {
    return fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v)));
}
// SiLU(v) = v / (1 + e^-v) through the hardware exp2 and reciprocal (about
// 1e-7 relative)
__device__ __forceinline__ float silu_acc(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-v * kLog2e));
}

// Right-aligned taps of a channel's causal convolution (the last tap on the
// current step) and its bias; zeros outside 0 <= channel < cin.
__device__ __forceinline__ void conv_taps(const Args& a, int ch, bool ok, float* w4, float* cb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int k = kk - (4 - a.K);
        w4[kk] = (ok && k >= 0) ? a.cw[(size_t)ch * a.K + k] : 0.0f;
    }
    *cb = (ok && a.cbias) ? a.cbias[ch] : 0.0f;
}

// a raw input of the history before the call: step t < 0 of channel ch (zero
// without a history or before it)
template <typename IO>
__device__ __forceinline__ float hist_in(const Args& a, int b, int t, int ch) {
    const int r = t + a.K - 1;
    if (!a.xh || r < 0) return 0.0f;
    return to_f32(((const IO*)a.xh)[((size_t)b * (a.K - 1) + r) * a.cin + ch]);
}

// four consecutive elements of an fp32 or bf16 tensor, as fp32
template <typename IO>
__device__ __forceinline__ void load4(const void* p, size_t e, float* o) {
    if constexpr (sizeof(IO) == 4) {
        const float4 v = *(const float4*)((const float*)p + e);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else {
        const uint2 u = *(const uint2*)((const bf16*)p + e);
        o[0] = __uint_as_float(u.x << 16);
        o[1] = __uint_as_float(u.x & 0xffff0000u);
        o[2] = __uint_as_float(u.y << 16);
        o[3] = __uint_as_float(u.y & 0xffff0000u);
    }
}

// Per-batch-row views of the inputs.  B/C: element (step t, n, rank r) at
//   t * bc_step + bc_head + n * R + r   with bc_step = G*N (grouped layout,
//   R == 1) or H*N*R (per-head layout), bc_head = g*N or h*N*R.
// X/Y: element (step t, p, r) at t * x_step + h*P*R + p*R + r, x_step = H*P*R.
template <int R, bool GROUPED, typename IO>
struct Views {
    Buf B, C, X, ld, gam, bet, th, Bp, Xp;
    int bc_step, bc_head, x_step, x_head;
    bool has_prev;
    __device__ Views(const Args& a, int b, int h, int hg) {
        bc_step = GROUPED ? a.G * a.N : a.H * a.N * R;
        bc_head = GROUPED ? hg * a.N : hg * a.N * R;
        x_step = a.pro ? a.cin : a.H * a.P * R;   // block prologue: X is the x part of xBC
        x_head = h * a.P * R;
        const size_t nbc = (size_t)a.L * bc_step;
        B = make_buf((const IO*)a.B + (size_t)b * nbc, nbc * sizeof(IO));
        C = make_buf((const IO*)a.C + (size_t)b * nbc, nbc * sizeof(IO));
        const size_t nx = (size_t)a.L * x_step;
        X = make_buf((const IO*)a.X + (size_t)b * nx, nx * sizeof(IO));
        // the token before the call: one step of B and X, same element offsets
        // as a row of B / X without the step term
        has_prev = a.B_prev != nullptr;
        Bp = make_buf(has_prev ? (const IO*)a.B_prev + (size_t)b * bc_step : (const IO*)a.B,
                      has_prev ? (size_t)bc_step * sizeof(IO) : 0);
        Xp = make_buf(has_prev ? (const IO*)a.X_prev + (size_t)b * x_step : (const IO*)a.X,
                      has_prev ? (size_t)x_step * sizeof(IO) : 0);
        const size_t ns = (size_t)a.L * a.H;
        ld = make_buf(a.ld + (size_t)b * ns, ns * 4);
        gam = make_buf(a.gamma ? a.gamma + (size_t)b * ns : a.ld, a.gamma ? ns * 4 : 0);
        bet = make_buf(a.beta ? a.beta + (size_t)b * ns : a.ld, a.beta ? ns * 4 : 0);
        const size_t nt = ns * (size_t)(a.N / 2);
        th = make_buf(a.theta ? a.theta + (size_t)b * nt : a.ld, a.theta ? nt * 4 : 0);
    }
};

// ---------------------------------------------------------------------------
// Mamba-2 scores S = C B^T per (batch, chunk, group): 64 x 64, contraction over
// the state.  Only the causal blocks (column block <= row block) are computed;
// the walk never reads the others.  Stored in blocks of 8 columns: element
// (i, j) at (j / 8) * 512 + i * 8 + j % 8, so a row's 8 columns of one block
// are 32 contiguous bytes.
// ---------------------------------------------------------------------------
template <int NP, typename IO, bool PRO = false>
__global__ __launch_bounds__(kThreads) void k_scores(Args a) {
    constexpr int SB = NP + 4;
    constexpr int NQ = NP / 4;
    __shared__ __attribute__((aligned(16))) float sC[kRows * SB];
    __shared__ __attribute__((aligned(16))) float sB[kRows * SB];
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int t0g = c * kRows;
    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const Views<1, true, IO> vw(a, b, 0, g);
    if constexpr (PRO) {
        // block prologue: thread (role, n) convolves channel n of B (role 0) or C
        // (role 1) over the chunk's rows, a sliding window of three raw inputs in
        // registers, and writes the activated value to LDS and to the workspace
        // (rounded to the dtype the walks read; the scores use the same values)
        if (tid < 2 * NP) {
            const int role = tid / NP, n = tid % NP;
            const bool ok = n < a.N;
            const int ch = a.H * a.P + (role * a.G + g) * a.N + n;
            float w4[4], cbv;
            conv_taps(a, ch, ok, w4, &cbv);
            const size_t nrow = (size_t)a.L * a.cin;
            const Buf xr = make_buf((const IO*)a.Xr + (size_t)b * nrow, nrow * sizeof(IO));
            float win[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int t = t0g - 3 + j;
                win[j] = !ok ? 0.0f : (t >= 0 ? bload<IO>(xr, t * a.cin + ch) : hist_in<IO>(a, b, t, ch));
            }
            float* dst = role ? sC : sB;
            IO* gdst = (IO*)(role ? a.Cw : a.Bw);
            // all of the chunk's raw inputs in flight at once
            float xall[kRows];
#pragma unroll
            for (int r = 0; r < kRows; ++r) xall[r] = ok ? bload<IO>(xr, (t0g + r) * a.cin + ch) : 0.0f;
#pragma unroll
            for (int r0 = 0; r0 < kRows; r0 += 16) {
                const float* xv = xall + r0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = t0g + r0 + r;
                    const float pre = fmaf(w4[3], xv[r], fmaf(w4[2], win[2], fmaf(w4[1], win[1], fmaf(w4[0], win[0], cbv))));
                    win[0] = win[1];
                    win[1] = win[2];
                    win[2] = xv[r];
                    float v = (ok && t < a.L) ? silu_acc(pre) : 0.0f;
                    if constexpr (sizeof(IO) == 2) v = to_f32(f32_to_bf16(v));
                    dst[(r0 + r) * SB + n] = v;
                    if (ok && t < a.L) store_out(&gdst[(((size_t)b * a.L + t) * a.G + g) * a.N + n], v);
                }
            }
        }
        // dt' and the log-decay of the chunk's steps for the group's heads
        const int HG = a.H / a.G;
        for (int e = tid; e < kRows * HG; e += kThreads) {
            const int t = t0g + e / HG, hh = g * HG + e % HG;
            if (t < a.L) {
                const size_t o = ((size_t)b * a.L + t) * a.H + hh;
                const float d = softplus_acc(a.dtr[o] + (a.dtbias ? a.dtbias[hh] : 0.0f));
                a.dtp[o] = d;
                ((float*)a.ld)[o] = d * a.Ah[hh];
            }
        }
    } else {
        const int row = tid / 4, q = tid % 4;
        float vb[NQ], vc[NQ];
        const int e = (t0g + row) * vw.bc_step + vw.bc_head + q * NQ;
        VecLoad<IO, NQ>::run(vw.B, e, vb);
        VecLoad<IO, NQ>::run(vw.C, e, vc);
#pragma unroll
        for (int i = 0; i < NQ; i += 4) {
            const bool ok = q * NQ + i < a.N;   // N is a multiple of 4
            float4 fb = ok ? make_float4(vb[i], vb[i + 1], vb[i + 2], vb[i + 3]) : make_float4(0, 0, 0, 0);
            float4 fc = ok ? make_float4(vc[i], vc[i + 1], vc[i + 2], vc[i + 3]) : make_float4(0, 0, 0, 0);
            *(float4*)&sB[row * SB + q * NQ + i] = fb;
            *(float4*)&sC[row * SB + q * NQ + i] = fc;
        }
    }
    __syncthreads();
    if constexpr (sizeof(IO) == 2) {
        // bf16 inputs: also store this chunk's B transposed, rows n (zero at n >= N),
        // 64 steps each, for the walk's state update
        bf16* bt = a.BT + (((size_t)b * a.nch + c) * a.G + g) * (size_t)(NP * kRows);
        for (int e = tid; e < NP * 8; e += kThreads) {
            const int n = e % NP, blk = e / NP;
            uint32_t u[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                u[q] = pack_bf(sB[(8 * blk + 2 * q) * SB + n], sB[(8 * blk + 2 * q + 1) * SB + n]);
            *(uint4*)(bt + n * kRows + 8 * blk) = make_uint4(u[0], u[1], u[2], u[3]);
        }
    }
    const int li = lane % 16, lk = lane / 16;
    float* Sout = a.S + (((size_t)b * a.nch + c) * a.G + g) * (size_t)(kRows * kRows);
    const int it = wave;
    for (int jt = 0; jt <= it; ++jt) {
        floatx4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
        const float* pa = sC + (16 * it + li) * SB + NQ * lk;
        const float* pb = sB + (16 * jt + li) * SB + NQ * lk;
#pragma unroll
        for (int q = 0; q < NQ; q += 4) {
            const float4 av = *(const float4*)(pa + q);
            const float4 bv = *(const float4*)(pb + q);
            acc0 = mfma4(av.x, bv.x, acc0);
            acc1 = mfma4(av.y, bv.y, acc1);
            acc0 = mfma4(av.z, bv.z, acc0);
            acc1 = mfma4(av.w, bv.w, acc1);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sout[((16 * jt + li) / 8) * (kRows * 8) + (16 * it + 4 * lk + r) * 8 + (li % 8)] = acc0[r] + acc1[r];
    }
}

// ---------------------------------------------------------------------------
// Chunk walk.  SO = state only (the segment pre-pass).
//
// Eight waves, two per SIMD.  Waves w and w + 4 own state columns
// p = p0 + 16 (w % 4) + li; wave w holds state rows n < NP/2, wave w + 4 rows
// n >= NP/2, each in NT2 = NP/32 accumulator tiles.  Tile t, register r of lane
// (li, lk) of half nh is row
//     n(t, r) = (NP/2) nh + (NP/8) lk + NT2 r + t,
// i.e. lane group lk owns NP/8 consecutive rows.  Read as the A operand of
// Y^T = H^T C~^T, the accumulators are a K-slice of consecutive rows per lane
// group, matching contiguous 16-byte reads of C~: the state never leaves
// registers.  Rotation pairs (2k, 2k + 1) sit in tiles (t, t + 1) of one lane.
// The two halves' partial outputs are summed through LDS.
// ---------------------------------------------------------------------------
constexpr int kWalkThreads = 512;

template <int NP>
__device__ __forceinline__ int state_row(int t, int r, int lk, int nh) {
    return (NP / 2) * nh + (NP / 8) * lk + (NP / 32) * r + t;
}

// Causal score tiles (row block << 4 | column block) of the trapezoid per wave,
// three per SIMD on SIMDs 0 and 1 and two on SIMDs 2 and 3 (waves w and w + 4
// share SIMD w); -1 ends a list.
__constant__ int kTrapTiles[8][2] = {{0x33, 0x00}, {0x32, 0x11}, {0x22, -1}, {0x20, -1},
                                     {0x30, -1}, {0x31, -1}, {0x21, -1}, {0x10, -1}};

template <int NP, int R, bool TRAP, bool ROT, bool GROUPED, typename IO, bool SO, bool EPI = false,
          bool BCN = false, bool PRO = false>
__global__ __launch_bounds__(kWalkThreads, SO ? 4 : 2) void k_walk(Args a) {
    static_assert(!PRO || (!TRAP && R == 1 && SO), "the block prologue here: the Mamba-2 state-only pass");
    static_assert(!EPI || !SO, "the output epilogue is a full-pass feature");
    static_assert(!BCN || TRAP, "the B / C prologue is a Mamba-3 feature");
    using Gm = Geo<R, TRAP>;
    constexpr int QT = Gm::QT, EXTRA = Gm::EXTRA, JX = Gm::JX;
    constexpr int JC = Gm::JC, JP = Gm::JP;
    constexpr int NT2 = NP / 32;    // state tiles per wave
    constexpr int KQ = NP / 4;      // contraction slice over the state per lane group (scores)
    constexpr int NSG = QT < 8 ? QT : 8;       // step groups (one per wave) of the B / C / angle staging
    constexpr int QSG = QT / NSG;              // steps per group
    constexpr int PRG = (R + NSG - 1) / NSG;   // previous-step ranks per staging thread
    constexpr int NXG = QT < 8 ? QT : 8;       // step groups of the X staging
    constexpr int QXG = QT / NXG;
    constexpr int PRX = (R + NXG - 1) / NXG;
    constexpr bool FULL = !SO;
    constexpr int BS = NP + 4;      // LDS row stride of B~ / C~ (4 mod 32 floats)
    // R >= 4: output tiles are computed as Y = C~ H (a lane holds four rows of one
    // column: the four ranks of a step, stored as one 16-byte piece); otherwise as
    // Y^T = H^T C~^T (a lane holds four columns of one row)
    constexpr bool YROW = R >= 4;

    __shared__ __attribute__((aligned(16))) float sB[Gm::BR * BS];
    // float offset of element (row j, state n) of sB / sC
    auto bcx = [](int j, int n) { return j * BS + n; };
    __shared__ __attribute__((aligned(16))) float sC[FULL ? kRows * BS : 4];
    __shared__ __attribute__((aligned(16))) float sXT[FULL ? kPG * JP : 4];
    __shared__ __attribute__((aligned(16))) float sXdT[kPG * JP];
    __shared__ __attribute__((aligned(16))) float sM[FULL ? kRows * JP : 4];
    __shared__ __attribute__((aligned(16))) float sYp[FULL ? 4 * 4 * 64 * 4 : 4];
    __shared__ float s_cum[QT + 1];
    __shared__ float s_gam[TRAP ? QT : 1];
    __shared__ float s_bet[TRAP ? QT + 1 : 1];
    __shared__ float s_dc[ROT ? NP / 2 : 1];
    __shared__ float s_ds[ROT ? NP / 2 : 1];
    __shared__ float s_tht[ROT ? 8 * 64 : 1];   // per step group: chunk-local angle totals per pair

    // ---- workgroup -> (batch, segment, head, column group) ------------------
    // Workgroups of one (batch, segment) share B and C; ids i, i+8, i+16, ... run
    // on one XCD, so they are given the heads of one (batch, segment).
    const int nsegL = SO ? a.nseg - 1 : a.nseg;
    const int gsize = a.H * a.npg;
    const int ngroups = (int)(gridDim.x / gsize);
    const int id = blockIdx.x;
    const int full = ngroups / 8 * 8 * gsize;
    int grp, wi;
    if (id < full) {
        const int x = id % 8, k = id / 8;
        grp = x + 8 * (k / gsize);
        wi = k % gsize;
    } else {
        grp = id / gsize;
        wi = id % gsize;
    }
    const int b = grp / nsegL, seg = grp % nsegL;
    const int h = wi / a.npg, pg = wi % a.npg;
    const int hg = GROUPED ? h / (a.H / a.G) : h;
    const int p0 = pg * kPG;
    const int c_begin = seg * a.cps;
    const int c_end = min(a.nch, c_begin + a.cps);

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int pw = wave & 3, nh = wave >> 2;
    const int li = lane % 16, lk = lane / 16;
    const int pw_n = (min(kPG, a.P - p0)) / 16;
    const bool active = pw < pw_n;   // uniform
    const int pcol = p0 + 16 * pw + li;
    const Views<R, GROUPED, IO> vw(a, b, h, hg);
    const size_t sh_off = (size_t)(b * a.H + h) * a.N * a.P;

    // staging roles: (sk, ssg) = rotation pair (lane) and step group (wave) for
    // B / C / angles; (xpl, xtq) = state column and step group for X.  Lanes run
    // along the row, so loads are contiguous and LDS writes hit distinct banks.
    const int sk = tid % 64, ssg = tid / 64;
    const bool k_in = sk < NP / 2 && ssg < NSG;
    const bool k_ok = k_in && 2 * sk < a.N;
    const int xpl = tid % 64, xtq = tid / 64;
    const bool x_in = xtq < NXG;
    const bool x_ok = x_in && p0 + xpl < a.P;
    const int si = tid / 8, sq = tid % 8;   // Mamba-2 score staging: row, 8-column block
    // BCNorm + bias: this lane's states (2 sk, 2 sk + 1)
    float nwb[2] = {1.0f, 1.0f}, nbb[2] = {0.0f, 0.0f}, nwc[2] = {1.0f, 1.0f}, nbc[2] = {0.0f, 0.0f};
    if constexpr (BCN) if (k_ok) {
        const int n = 2 * sk;
        if (a.nwB) { nwb[0] = a.nwB[n]; nwb[1] = a.nwB[n + 1]; }
        if (a.biasB) { nbb[0] = a.biasB[(size_t)h * a.N + n]; nbb[1] = a.biasB[(size_t)h * a.N + n + 1]; }
        if constexpr (FULL) {
            if (a.nwC) { nwc[0] = a.nwC[n]; nwc[1] = a.nwC[n + 1]; }
            if (a.biasC) { nbc[0] = a.biasC[(size_t)h * a.N + n]; nbc[1] = a.biasC[(size_t)h * a.N + n + 1]; }
        }
    }

    // ---- one-time zero fill of padding that staging never writes ------------
    if constexpr (TRAP) {
        for (int e = tid; e < (Gm::BR - kRows - EXTRA) * BS; e += kWalkThreads)
            sB[(kRows + EXTRA) * BS + e] = 0.0f;
    }
    if constexpr (JC > kRows + EXTRA) {
        constexpr int PADC = JC > kRows + EXTRA ? JC - kRows - EXTRA : 1;
        for (int e = tid; e < kPG * PADC; e += kWalkThreads) {
            const int row = e / PADC, col = kRows + EXTRA + e % PADC;
            if constexpr (FULL) sXT[row * JP + col] = 0.0f;
            sXdT[row * JP + col] = 0.0f;
        }
    }

    // ---- prefetch registers -------------------------------------------------
    struct Pre {
        float b[QSG][2 * R];          // B pair (2sk, 2sk+1) x ranks, steps ssg*QSG + i
        float bp[2 * PRG];            // previous step, ranks ssg*PRG + q
        float c[FULL ? QSG : 1][2 * R];
        float th[ROT ? QSG : 1];
        float x[QXG][R];              // X column p0 + xpl, steps xtq*QXG + i
        float xp[PRX];                // previous step, ranks xtq*PRX + q
        float xh[PRO ? 3 : 1];        // block prologue: raw x of the three steps before the group
        float dtp;                    // block prologue: dt' of step `lane`
        float sc[(FULL && !TRAP) ? 8 : 1];   // Mamba-2 score row si, columns 8 sq ..
        float ld, gam, bet;           // step `lane` of the chunk
        float ldn, betn;              // step `lane` + 1 (trapezoid only)
    };
    const Buf Sbuf = (FULL && !TRAP)
        ? make_buf(a.S + (size_t)b * a.nch * a.G * (kRows * kRows), (size_t)a.nch * a.G * kRows * kRows * 4)
        : make_buf(a.ld, 0);
    // block prologue: dt' per (step, head), and this lane's x column's taps
    const Buf dtpb = PRO ? make_buf(a.dtp + (size_t)b * a.L * a.H, (size_t)a.L * a.H * 4) : make_buf(a.ld, 0);
    float cw4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cwb = 0.0f;
    if constexpr (PRO) conv_taps(a, h * a.P + p0 + xpl, x_ok, cw4, &cwb);

    // FIRST: the chunk may be the call's first, whose previous step is the given
    // previous token (only the prefetch before the loop; the loop's prefetches
    // never are, and stay free of the selection)
    auto prefetch = [&](int c, Pre& p, auto first_tag) {
        constexpr bool FIRST = decltype(first_tag)::value != 0;
        const int t0g = c * QT;
        if (k_ok) {
#pragma unroll
            for (int i = 0; i < QSG; ++i) {
                const int e = (t0g + ssg * QSG + i) * vw.bc_step + vw.bc_head + 2 * sk * R;
                VecLoad<IO, 2 * R>::run(vw.B, e, p.b[i]);
                if constexpr (FULL) VecLoad<IO, 2 * R>::run(vw.C, e, p.c[i]);
            }
            if constexpr (TRAP) if (ssg * PRG < R) {
                // the previous step; before the call's first step it is the given
                // previous token (or zeros: a negative offset reads zero)
                const bool first = FIRST && t0g == 0 && vw.has_prev;
                const int e = (first ? 0 : (t0g - 1) * vw.bc_step) + vw.bc_head + 2 * sk * R + ssg * PRG;
                VecLoad<IO, PRG>::run(first ? vw.Bp : vw.B, e, p.bp);
                VecLoad<IO, PRG>::run(first ? vw.Bp : vw.B, e + R, p.bp + PRG);
            }
            if constexpr (ROT) {
#pragma unroll
                for (int i = 0; i < QSG; ++i)
                    p.th[i] = bload<float>(vw.th, ((t0g + ssg * QSG + i) * a.H + h) * (a.N / 2) + sk);
            }
        }
        if (x_ok) {
#pragma unroll
            for (int i = 0; i < QXG; ++i)
                VecLoad<IO, R>::run(vw.X, (t0g + xtq * QXG + i) * vw.x_step + vw.x_head + (p0 + xpl) * R,
                                    p.x[i]);
            if constexpr (PRO) {
                // the convolution window before the group; before the call, the history
                const int ch = h * a.P + p0 + xpl;
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int t = t0g + xtq * QXG - 3 + j;
                    p.xh[j] = (FIRST && t < 0) ? hist_in<IO>(a, b, t, ch) : bload<IO>(vw.X, t * vw.x_step + ch);
                }
            }
            if constexpr (TRAP) if (xtq * PRX < R) {
                const bool first = FIRST && t0g == 0 && vw.has_prev;
                VecLoad<IO, PRX>::run(first ? vw.Xp : vw.X,
                                      (first ? 0 : (t0g - 1) * vw.x_step) + vw.x_head + (p0 + xpl) * R + xtq * PRX,
                                      p.xp);
            }
        }
        if constexpr (FULL && !TRAP) if (8 * sq <= si) {
            const int e = (c * a.G + hg) * (kRows * kRows) + sq * (kRows * 8) + si * 8;
            VecLoad<float, 8>::run(Sbuf, e, p.sc);
        }
        const int o = (t0g + lane) * a.H + h;
        p.ld = lane < QT ? bload<float>(vw.ld, o) : 0.0f;
        if constexpr (PRO) p.dtp = lane < QT ? bload<float>(dtpb, o) : 0.0f;
        if constexpr (TRAP) {
            p.gam = lane < QT ? bload<float>(vw.gam, o) : 0.0f;
            p.bet = lane < QT ? bload<float>(vw.bet, o) : 0.0f;
            p.ldn = lane + 1 < QT ? bload<float>(vw.ld, o + a.H) : 0.0f;
            p.betn = lane + 1 < QT ? bload<float>(vw.bet, o + a.H) : 0.0f;
        }
    };

    // chunk-local angle prefix within this thread's step group, and the group
    // total for the other groups (read by the next stage, after a barrier)
    auto angle_prefix = [&](Pre& p) {
        if constexpr (ROT) {
            float run = 0.0f;
#pragma unroll
            for (int i = 0; i < QSG; ++i) {
                run += k_ok ? p.th[i] : 0.0f;
                p.th[i] = run;
            }
            if (ssg < NSG) s_tht[ssg * 64 + sk] = run;
        }
    };

    float seg_acc = 0.0f;   // SO: total log-decay of the segment
    float rev_acc = 0.0f;   // SO: total angle of pair sk (last step group), revolutions mod 1
    float cum_last = 0.0f;
    float cum0 = 0.0f;      // trapezoid: log-decay of the chunk's first step

    // ---- staging of one chunk from the prefetch registers into LDS ----------
    auto stage = [&](const Pre& p, int t0g_stage) {
        const float cum = wave_scan_dpp(p.ld);   // lanes >= QT add zero
        cum_last = readlane_f(cum, QT - 1);
        // chunk-end weights of step `lane` and of the previous step (the full
        // pass adds the previous step's term to the state at the start of the
        // chunk, with weight beta_0; the state-only pass at the end, decayed)
        float wl, wprev = 0.0f;
        if constexpr (TRAP) {
            const float cum_n = cum + p.ldn;       // cumulative log-decay of step `lane` + 1
            wl = p.gam * exp_e(cum_last - cum) + (lane + 1 < QT ? p.betn * exp_e(cum_last - cum_n) : 0.0f);
            cum0 = readlane_f(cum, 0);
            wprev = readlane_f(p.bet, 0) * (SO ? exp_e(cum_last - cum0) : 1.0f);
        } else {
            wl = exp_e(cum_last - cum);
        }
        if (wave == 0) {
            if (lane < QT) {
                s_cum[lane + 1] = TRAP ? cum - cum0 : cum;   // trapezoid: relative to step 0
                if constexpr (TRAP) {
                    s_gam[lane] = p.gam;
                    s_bet[lane] = p.bet;
                }
            }
            if (lane == 0) {
                s_cum[0] = 0.0f;
                if constexpr (TRAP) s_bet[QT] = 0.0f;
            }
        }
        // angles: this thread's local prefix (made before the barrier) plus the
        // totals of the earlier step groups
        float phi[ROT ? QSG : 1];
        if constexpr (ROT) {
            float off = 0.0f;
            for (int g = 0; g < ssg && g < NSG; ++g) off += s_tht[g * 64 + sk];
#pragma unroll
            for (int i = 0; i < QSG; ++i) phi[i] = p.th[i] + off;
            if (ssg == NSG - 1 && k_in) {
                float sn, cs;
                sincos_rev(phi[QSG - 1], &sn, &cs);
                s_dc[sk] = k_ok ? cs : 1.0f;
                s_ds[sk] = k_ok ? sn : 0.0f;
                if constexpr (SO) {
                    rev_acc += phi[QSG - 1] * 0.15915494309189535f;
                    rev_acc -= rintf(rev_acc);
                }
            }
        }
        // B~, C~ rows (t R + r), columns (2 sk, 2 sk + 1)
        if (k_in) {
#pragma unroll
            for (int i = 0; i < QSG; ++i) {
                const int t = ssg * QSG + i;
                float cs = 1.0f, sn = 0.0f;
                if constexpr (ROT) sincos_rev(phi[i], &sn, &cs);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float b0 = p.b[i][r], b1 = p.b[i][R + r];
                    float2 vb = make_float2(fmaf(-sn, b1, cs * b0), fmaf(sn, b0, cs * b1));
                    if (!k_ok) vb = make_float2(0.0f, 0.0f);
                    *(float2*)&sB[(t * R + r) * BS + 2 * sk] = vb;
                    if constexpr (FULL) {
                        const float c0 = p.c[i][r], c1 = p.c[i][R + r];
                        float2 vc = make_float2(fmaf(-sn, c1, cs * c0), fmaf(sn, c0, cs * c1));
                        if (!k_ok) vc = make_float2(0.0f, 0.0f);
                        *(float2*)&sC[(t * R + r) * BS + 2 * sk] = vc;
                    }
                }
            }
            if constexpr (TRAP) if (ssg * PRG < R) {
#pragma unroll
                for (int q = 0; q < PRG; ++q) {
                    const int r = ssg * PRG + q;
                    if (r < R) {
                        float2 vb = make_float2(p.bp[q], p.bp[PRG + q]);
                        if (!k_ok) vb = make_float2(0.0f, 0.0f);
                        *(float2*)&sB[(kRows + r) * BS + 2 * sk] = vb;
                    }
                }
            }
        }
        // X^T and the chunk-end-weighted X^T: rows xpl, columns (t R + r)
        if (x_in) {
            float xv[QXG * R], xd[QXG * R];
            float win[3] = {PRO ? p.xh[0] : 0.0f, PRO ? p.xh[1] : 0.0f, PRO ? p.xh[2] : 0.0f};
#pragma unroll
            for (int i = 0; i < QXG; ++i) {
                float w = readlane_f(wl, xtq * QXG + i);   // xtq is the wave index
                if constexpr (PRO) w *= readlane_f(p.dtp, xtq * QXG + i);   // dt' with the weight
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float v = x_ok ? p.x[i][r] : 0.0f;
                    if constexpr (PRO) {
                        // convolved, activated x (zero past the sequence)
                        const float pre = fmaf(cw4[3], v, fmaf(cw4[2], win[2], fmaf(cw4[1], win[1], fmaf(cw4[0], win[0], cwb))));
                        win[0] = win[1];
                        win[1] = win[2];
                        win[2] = v;
                        v = (x_ok && t0g_stage + xtq * QXG + i < a.L) ? silu_acc(pre) : 0.0f;
                    }
                    xv[i * R + r] = v;
                    xd[i * R + r] = v * w;
                }
            }
            const int j0 = xtq * QXG * R;
#pragma unroll
            for (int q = 0; q < QXG * R; q += 4) {
                if constexpr (FULL) *(float4*)&sXT[xpl * JP + j0 + q] = make_float4(xv[q], xv[q + 1], xv[q + 2], xv[q + 3]);
                *(float4*)&sXdT[xpl * JP + j0 + q] = make_float4(xd[q], xd[q + 1], xd[q + 2], xd[q + 3]);
            }
            if constexpr (TRAP) if (xtq * PRX < R) {
#pragma unroll
                for (int q = 0; q < PRX; ++q) {
                    const int r = xtq * PRX + q;
                    if (r < R) {
                        const float v = x_ok ? p.xp[q] : 0.0f;
                        if constexpr (FULL) sXT[xpl * JP + kRows + r] = v;
                        sXdT[xpl * JP + kRows + r] = v * wprev;
                    }
                }
            }
        }
        // Mamba-2: masked scores M[i][j] = S[i][j] e^{cum_i - cum_j}, j <= i
        if constexpr (FULL && !TRAP) {
            const float cum_i = __shfl(cum, si, 64);
            float mv[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int j = 8 * sq + q;
                const float cum_j = __shfl(cum, j, 64);
                const bool ok = j <= si;
                const float e = exp_e(ok ? cum_i - cum_j : 0.0f);
                mv[q] = ok ? p.sc[q] * e : 0.0f;
            }
            *(float4*)&sM[si * JP + 8 * sq] = make_float4(mv[0], mv[1], mv[2], mv[3]);
            *(float4*)&sM[si * JP + 8 * sq + 4] = make_float4(mv[4], mv[5], mv[6], mv[7]);
        }
    };

    // ---- state ----------------------------------------------------------------
    floatx4 acc_h[NT2];
#pragma unroll
    for (int t = 0; t < NT2; ++t) acc_h[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (FULL) if (active) {
        if (a.h0) {
#pragma unroll
            for (int t = 0; t < NT2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = state_row<NP>(t, r, lk, nh);
                    acc_h[t][r] = n < a.N ? a.h0[sh_off + (size_t)n * a.P + pcol] : 0.0f;
                }
        }
        // entering state of this segment: compose the earlier segments
        for (int s2 = 0; s2 < seg; ++s2) {
            const size_t u = (size_t)(b * a.H + h) * (a.nseg - 1) + s2;
            const float d = exp_e(a.seg_ld[u]);
            if constexpr (ROT) {
#pragma unroll
                for (int t = 0; t < NT2; t += 2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int n = state_row<NP>(t, r, lk, nh);
                        const float rev = n < a.N ? a.seg_rev[u * (a.N / 2) + n / 2] : 0.0f;
                        const float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
                        const float v0 = acc_h[t][r], v1 = acc_h[t + 1][r];
                        acc_h[t][r] = fmaf(sn, v1, cs * v0);
                        acc_h[t + 1][r] = fmaf(-sn, v0, cs * v1);
                    }
            }
#pragma unroll
            for (int t = 0; t < NT2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = state_row<NP>(t, r, lk, nh);
                    const float hl = n < a.N ? a.seg_h[(u * a.N + n) * a.P + pcol] : 0.0f;
                    acc_h[t][r] = fmaf(d, acc_h[t][r], hl);
                }
        }
    }

    // BCNorm + bias on the raw rows, before the rotations: a row (one step and
    // rank) lies on lanes sk of its step group's wave, pair sk on lane sk; lanes
    // past N add zero to the sum of squares, and staging zeroes what they hold.
    // Every rank of a step is its own row; the head's bias is the same for all.
    auto bc_prologue = [&](Pre& p) {
        if constexpr (BCN) if (ssg < NSG) {   // wave-uniform
            const float rN = 1.0f / (float)a.N;
            auto norm = [&](float& v0, float& v1, const float* w, const float* bi) {
                const float sq2 = k_ok ? fmaf(v0, v0, v1 * v1) : 0.0f;
                const float inv = rsqrtf(fmaf(readlane_f(wave_scan_dpp(sq2), 63), rN, a.eps));
                v0 = fmaf(v0 * inv, w[0], bi[0]);
                v1 = fmaf(v1 * inv, w[1], bi[1]);
            };
#pragma unroll
            for (int i = 0; i < QSG; ++i)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    norm(p.b[i][r], p.b[i][R + r], nwb, nbb);
                    if constexpr (FULL) norm(p.c[i][r], p.c[i][R + r], nwc, nbc);
                }
            if (ssg * PRG < R) {
#pragma unroll
                for (int q = 0; q < PRG; ++q)
                    if (ssg * PRG + q < R) norm(p.bp[q], p.bp[PRG + q], nwb, nbb);   // wave-uniform
            }
        }
    };

    Pre pre;
    if (c_begin < c_end) {
        prefetch(c_begin, pre, Par<1>{});
        angle_prefix(pre);
    }

    for (int c = c_begin; c < c_end; ++c) {
        const int t0g = c * QT;
        __syncthreads();                 // the previous chunk's LDS reads are done
        bc_prologue(pre);
        stage(pre, t0g);
        if constexpr (SO) {
            if (c + 1 < c_end) prefetch(c + 1, pre, Par<0>{});
        }
        __syncthreads();
        if constexpr (SO) seg_acc += cum_last;

        // ---- trapezoid: H+ = alpha_0 H + beta_0 B_{-1}^T x_{-1} (the previous
        // step's beta term, which then decays with the chunk like the state) -----
        if constexpr (TRAP && FULL) if (active) {
            const float a0 = exp_e(cum0);
#pragma unroll
            for (int t = 0; t < NT2; ++t) acc_h[t] *= a0;
            const int nb = (NP / 2) * nh + NT2 * li;   // first state row of this lane's tiles
#pragma unroll
            for (int e = 0; e < JX; ++e) {
                const int j = kRows + 4 * e + lk;
                const float xd = sXdT[(16 * pw + li) * JP + j];
                if constexpr (NT2 == 4) {
                    const float4 bv = *(const float4*)(sB + bcx(j, nb));
                    acc_h[0] = mfma4(bv.x, xd, acc_h[0]);
                    acc_h[1] = mfma4(bv.y, xd, acc_h[1]);
                    acc_h[2] = mfma4(bv.z, xd, acc_h[2]);
                    acc_h[3] = mfma4(bv.w, xd, acc_h[3]);
                } else {
                    const float2 bv = *(const float2*)(sB + bcx(j, nb));
                    acc_h[0] = mfma4(bv.x, xd, acc_h[0]);
                    acc_h[1] = mfma4(bv.y, xd, acc_h[1]);
                }
            }
        }

        if constexpr (FULL) {
            floatx4 acc_y[4];
            // output epilogue: X and z of this lane's outputs load now, under the
            // chunk's matrix work, rather than in front of the store (one rank: four
            // columns of a step; rank rows: four ranks of a step and column; rank 2:
            // four columns of one rank of a step, R elements apart)
            float ex[4][4] = {}, ez[4][4] = {};
            if constexpr (EPI) {
                if (active && nh == 0) {
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int i0 = YROW ? 16 * it + 4 * lk : 16 * it + li;
                        const int tg = t0g + i0 / R;
                        if (tg < a.L) {
                            const size_t e = YROW
                                ? (((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P * R + (size_t)(p0 + 16 * pw + li) * R + i0 % R
                                : (((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P * R + (size_t)(p0 + 16 * pw + 4 * lk) * R + i0 % R;
                            if constexpr (YROW || R == 1) {
                                if (a.Dh) load4<IO>(a.X, e, ex[it]);
                                if (a.Zg) load4<IO>(a.Zg, e, ez[it]);
                            } else {
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    if (a.Dh) ex[it][r] = to_f32(((const IO*)a.X)[e + (size_t)r * R]);
                                    if (a.Zg) ez[it][r] = to_f32(((const IO*)a.Zg)[e + (size_t)r * R]);
                                }
                            }
                        }
                    }
                }
            }
            // (y + Dh x) SiLU(z) of the four outputs of tile it
            auto epilogue = [&](float* yv, int it) __attribute__((always_inline)) {
                if constexpr (EPI) {
                    const float dh = a.Dh ? a.Dh[h] : 0.0f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = fmaf(dh, ex[it][r], yv[r]);
                        const float sg = ez[it][r] * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-ez[it][r] * kLog2e));
                        yv[r] = a.Zg ? v * sg : v;
                    }
                }
            };
            // The two waves of a SIMD (same column group, other state half) take the
            // score tiles and the state part in opposite orders, so that one
            // wave's vector work on the score weights meets the other's matrix
            // instructions.
            auto score_tiles = [&]() __attribute__((always_inline)) {
                // ---- Mamba-3: weighted scores M = w o (C~ B~^T) -> LDS ---------------
                if constexpr (TRAP) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int code = kTrapTiles[wave][q];
                        if (code < 0) break;
                        const int it = code >> 4, jt = code & 15;
                        floatx4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
                        const float* pa = sC + (16 * it + li) * BS + KQ * lk;
                        const float* pb = sB + (16 * jt + li) * BS + KQ * lk;
#pragma unroll
                        for (int n = 0; n < KQ; n += 4) {
                            const float4 av = *(const float4*)(pa + n);
                            const float4 bv = *(const float4*)(pb + n);
                            s0 = mfma4(av.x, bv.x, s0);
                            s1 = mfma4(av.y, bv.y, s1);
                            s0 = mfma4(av.z, bv.z, s0);
                            s1 = mfma4(av.w, bv.w, s1);
                        }
                        const int j = 16 * jt + li;
                        const bool colv = jt < 4 || j - kRows < EXTRA;
                        const int sj = jt < 4 ? j / R : -1;       // step of column j
                        const float cum_s = s_cum[sj + 1];
                        const float cum_s1 = s_cum[min(sj + 2, QT)];
                        const float gam_s = s_gam[sj < 0 ? 0 : sj];
                        const float bet_s1 = s_bet[sj + 1];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = 16 * it + 4 * lk + r;
                            const int tau = i / R;
                            const float cum_t = s_cum[tau + 1];
                            const bool vg = colv && sj >= 0 && sj <= tau;
                            const bool vb = colv && sj < tau;
                            const float eg = exp_e(vg ? cum_t - cum_s : 0.0f);
                            const float eb = exp_e(vb ? cum_t - cum_s1 : 0.0f);
                            const float w = (vg ? gam_s * eg : 0.0f) + (vb ? bet_s1 * eb : 0.0f);
                            if (j < JC) sM[i * JP + j] = (s0[r] + s1[r]) * w;
                        }
                    }
                }
            };
            auto state_part = [&]() __attribute__((always_inline)) {
                // ---- partial Y^T = H^T C~^T over this wave's state rows ---------------
                if (active) {
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        floatx4 y0 = {0.0f, 0.0f, 0.0f, 0.0f}, y1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int q4 = 0; q4 < NP / 32; ++q4) {
                            // columns 4 q4 .. 4 q4 + 3 of the lane group's slice: s = NT2 r + t
                            const float4 cv = *(const float4*)(sC + bcx(16 * it + li, (NP / 2) * nh + (NP / 8) * lk + 4 * q4));
                            const float cvs[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int s = 4 * q4 + e;
                                const int t = s % NT2, r = s / NT2;
                                if (e % 2 == 0)
                                    y0 = YROW ? mfma4(cvs[e], acc_h[t][r], y0) : mfma4(acc_h[t][r], cvs[e], y0);
                                else
                                    y1 = YROW ? mfma4(cvs[e], acc_h[t][r], y1) : mfma4(acc_h[t][r], cvs[e], y1);
                            }
                        }
                        // the state part carries the row decay e^{cum_i}; the intra part does not
                        acc_y[it] = (y0 + y1) * exp_e(s_cum[(16 * it + (YROW ? 4 * lk : li)) / R + 1]);
                    }
                }
            };
            if (nh == 0) {
                state_part();
                score_tiles();
            } else {
                score_tiles();
                state_part();
            }
            // the next chunk's operands load while the rest of this chunk computes
            if (c + 1 < c_end) prefetch(c + 1, pre, Par<0>{});
            if constexpr (TRAP) __syncthreads();   // M complete
            // ---- partial Y^T += X^T M^T over half of the column blocks ------------
            if (active) {
                const float* px = sXT + (16 * pw + li) * JP + 4 * lk;
#pragma unroll
                for (int jh = 0; jh < 2; ++jh) {
                    const int jt = 2 * nh + jh;
                    const float4 xv = *(const float4*)(px + 16 * jt);
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        if (it < jt) continue;
                        const float4 mv = *(const float4*)(sM + (16 * it + li) * JP + 16 * jt + 4 * lk);
                        if constexpr (YROW) {
                            acc_y[it] = mfma4(mv.x, xv.x, acc_y[it]);
                            acc_y[it] = mfma4(mv.y, xv.y, acc_y[it]);
                            acc_y[it] = mfma4(mv.z, xv.z, acc_y[it]);
                            acc_y[it] = mfma4(mv.w, xv.w, acc_y[it]);
                        } else {
                            acc_y[it] = mfma4(xv.x, mv.x, acc_y[it]);
                            acc_y[it] = mfma4(xv.y, mv.y, acc_y[it]);
                            acc_y[it] = mfma4(xv.z, mv.z, acc_y[it]);
                            acc_y[it] = mfma4(xv.w, mv.w, acc_y[it]);
                        }
                    }
                }
            }
            // ---- H' = e^{cum_last} H + B~^T Xd over this wave's rows ------------------
            // (trapezoid: H is already H+, decayed through step 0)
            if (active) {
                const float tot = exp_e(cum_last - cum0);
#pragma unroll
                for (int t = 0; t < NT2; ++t) acc_h[t] *= tot;
            }
            if (active) {
                // exchange: the upper half writes its partial sums, the lower half adds them
                if (nh == 1) {
#pragma unroll
                    for (int it = 0; it < 4; ++it)
                        *(floatx4*)&sYp[((pw * 4 + it) * 64 + lane) * 4] = acc_y[it];
                }
            }
            __syncthreads();
            if (active && nh == 0) {
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const floatx4 o = *(const floatx4*)&sYp[((pw * 4 + it) * 64 + lane) * 4];
                    const floatx4 y = acc_y[it] + o;
                    if constexpr (YROW) {
                        // lane holds Y[i = 16 it + 4 lk + r][p = p0 + 16 pw + li]: ranks
                        // rk .. rk + 3 of step tg
                        const int i0 = 16 * it + 4 * lk;
                        const int tg = t0g + i0 / R, rk = i0 % R;
                        if (tg < a.L) {
                            IO* yrow = (IO*)a.Y + (((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P * R;
                            const size_t e = (size_t)(p0 + 16 * pw + li) * R + rk;
                            float yv[4] = {y[0], y[1], y[2], y[3]};
                            epilogue(yv, it);
                            if constexpr (sizeof(IO) == 4) {
                                *(float4*)((float*)yrow + e) = make_float4(yv[0], yv[1], yv[2], yv[3]);
                            } else {
                                const uint32_t u0 = f32_to_bf16(yv[0]) | ((uint32_t)f32_to_bf16(yv[1]) << 16);
                                const uint32_t u1 = f32_to_bf16(yv[2]) | ((uint32_t)f32_to_bf16(yv[3]) << 16);
                                *(uint2*)((bf16*)yrow + e) = make_uint2(u0, u1);
                            }
                        }
                        continue;
                    }
                    // lane holds Y[i = 16 it + li][p = p0 + 16 pw + 4 lk + r]
                    const int i = 16 * it + li;
                    const int tg = t0g + i / R;
                    if (tg < a.L) {
                        const int pp = p0 + 16 * pw + 4 * lk;
                        IO* yrow = (IO*)a.Y + (((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P * R;
                        if (R == 1) {
                            float yv[4] = {y[0], y[1], y[2], y[3]};
                            epilogue(yv, it);   // gated output of the same elements
                            if constexpr (sizeof(IO) == 4) {
                                *(float4*)((float*)yrow + pp) = make_float4(yv[0], yv[1], yv[2], yv[3]);
                            } else {
                                const uint32_t u0 = f32_to_bf16(yv[0]) | ((uint32_t)f32_to_bf16(yv[1]) << 16);
                                const uint32_t u1 = f32_to_bf16(yv[2]) | ((uint32_t)f32_to_bf16(yv[3]) << 16);
                                *(uint2*)((bf16*)yrow + pp) = make_uint2(u0, u1);
                            }
                        } else {
                            float yv[4] = {y[0], y[1], y[2], y[3]};
                            epilogue(yv, it);
#pragma unroll
                            for (int r = 0; r < 4; ++r) store_out(&yrow[(size_t)(pp + r) * R + i % R], yv[r]);
                        }
                    }
                }
            }
        } else {
            if (active) {
                const float tot = exp_e(cum_last);
#pragma unroll
                for (int t = 0; t < NT2; ++t) acc_h[t] *= tot;
            }
        }

        // ---- H' += B~^T Xd over this wave's rows, then back to the physical frame --
        if (active) {
            const float* pxd = sXdT + (16 * pw + li) * JP + 16 * lk;
            const int nb = (NP / 2) * nh + NT2 * li;   // first state row of this lane's tiles
#pragma unroll
            for (int sq4 = 0; sq4 < 4; ++sq4) {
                const float4 xd = *(const float4*)(pxd + 4 * sq4);
                const float xds[4] = {xd.x, xd.y, xd.z, xd.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * lk + 4 * sq4 + e;
                    if constexpr (NT2 == 4) {
                        const float4 bv = *(const float4*)(sB + bcx(j, nb));
                        acc_h[0] = mfma4(bv.x, xds[e], acc_h[0]);
                        acc_h[1] = mfma4(bv.y, xds[e], acc_h[1]);
                        acc_h[2] = mfma4(bv.z, xds[e], acc_h[2]);
                        acc_h[3] = mfma4(bv.w, xds[e], acc_h[3]);
                    } else {
                        const float2 bv = *(const float2*)(sB + bcx(j, nb));
                        acc_h[0] = mfma4(bv.x, xds[e], acc_h[0]);
                        acc_h[1] = mfma4(bv.y, xds[e], acc_h[1]);
                    }
                }
            }
            // state-only pass: the previous step's beta term, decayed to the chunk end
            if constexpr (SO) {
#pragma unroll
                for (int e = 0; e < JX; ++e) {
                    const int j = kRows + 4 * e + lk;
                    const float xd = sXdT[(16 * pw + li) * JP + j];
                    if constexpr (NT2 == 4) {
                        const float4 bv = *(const float4*)(sB + bcx(j, nb));
                        acc_h[0] = mfma4(bv.x, xd, acc_h[0]);
                        acc_h[1] = mfma4(bv.y, xd, acc_h[1]);
                        acc_h[2] = mfma4(bv.z, xd, acc_h[2]);
                        acc_h[3] = mfma4(bv.w, xd, acc_h[3]);
                    } else {
                        const float2 bv = *(const float2*)(sB + bcx(j, nb));
                        acc_h[0] = mfma4(bv.x, xd, acc_h[0]);
                        acc_h[1] = mfma4(bv.y, xd, acc_h[1]);
                    }
                }
            }
            if constexpr (ROT) {
#pragma unroll
                for (int t = 0; t < NT2; t += 2)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int k = state_row<NP>(t, r, lk, nh) >> 1;
                        const float cs = s_dc[k], sn = s_ds[k];
                        const float v0 = acc_h[t][r], v1 = acc_h[t + 1][r];
                        // R(-phi): (c v0 + s v1, -s v0 + c v1)
                        acc_h[t][r] = fmaf(sn, v1, cs * v0);
                        acc_h[t + 1][r] = fmaf(-sn, v0, cs * v1);
                    }
            }
        }
        if (c + 1 < c_end) angle_prefix(pre);
    }

    // ---- outputs of the walk ------------------------------------------------------
    if constexpr (SO) {
        const size_t u = (size_t)(b * a.H + h) * (a.nseg - 1) + seg;
        if (active) {
#pragma unroll
            for (int t = 0; t < NT2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = state_row<NP>(t, r, lk, nh);
                    if (n < a.N) a.seg_h[(u * a.N + n) * a.P + pcol] = acc_h[t][r];
                }
        }
        if (pg == 0) {
            if (tid == 0) a.seg_ld[u] = seg_acc;
            if (ROT && ssg == NSG - 1 && k_ok) a.seg_rev[u * (a.N / 2) + sk] = rev_acc;
        }
    } else {
        if (a.h_out && seg == a.nseg - 1 && active) {
#pragma unroll
            for (int t = 0; t < NT2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = state_row<NP>(t, r, lk, nh);
                    if (n < a.N) a.h_out[sh_off + (size_t)n * a.P + pcol] = acc_h[t][r];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Mamba-2 fp32 walk (full pass), wave-specialised.  Waves 0-3 (one per SIMD)
// are the matrix waves: wave w owns state columns p0 + 16 w .. + 15 for all NP
// state rows (NT = NP/16 accumulator tiles; tile t, register r of lane
// (li, lk) is row (NP/4) lk + (NP/16) r + t) and does every matrix product of
// the chunk for those columns, so the output needs no exchange.  Waves 4-7 are
// the staging waves: they copy B and C into LDS by LDS DMA, load X, the scores
// and the log-decay of the next chunk into registers and stage X^T, the
// chunk-end-weighted X^T and the masked scores.  Per chunk c, three phases
// separated by workgroup barriers:
//   1. matrix: Y^T = H^T C^T x e^{cum}      staging: B(c) -> LDS; loads for c+1
//   2. matrix: Y^T += X^T M^T, store Y(c)   staging: C(c+1) -> LDS (in flight
//                                            until the end of phase 3)
//   3. matrix: H = e^{cum_last} H + B^T Xd  staging: X^T, Xd^T, M, cum of c+1
// Each buffer is written in the phase after its last reader, so single LDS
// buffers suffice (Xd^T and cum, read in phase 3, are double-buffered).  Every
// copy and load of the staging waves is issued unconditionally (offsets past a
// buffer read zeros), so their vmcnt waits are exact.
// ---------------------------------------------------------------------------
template <int NP, bool EPI = false, bool PRO = false>
__global__ __launch_bounds__(kWalkThreads) void k_walk_m2s(Args a) {
    static_assert(!PRO || EPI, "the block's walk stores through the output side");
    constexpr int JP = kRows + 4;   // LDS row stride of X^T / Xd^T / M (4 mod 32)
    constexpr int NT = NP / 16;     // state tiles per matrix wave
    constexpr int NDMA = kRows * NP / 256 / 4;   // 16-byte copies per staging wave for B or C
    constexpr uint32_t kOut = 0x80000000u;       // byte offset past any buffer: reads zero

    __shared__ __attribute__((aligned(16))) float sB[kRows * NP];
    __shared__ __attribute__((aligned(16))) float sC[kRows * NP];
    __shared__ __attribute__((aligned(16))) float sXT[kPG * JP];
    __shared__ __attribute__((aligned(16))) float sXdT[2][kPG * JP];
    __shared__ __attribute__((aligned(16))) float sM[kRows * JP];
    __shared__ float s_cum[2][kRows + 1];
    __shared__ __attribute__((aligned(16))) float s_bc[4][PRO ? 3 : 2][kRows];   // per staging wave: cum, wl (, dt')

    // float offset of element (row j, state n) of sB / sC: 16-byte column
    // groups of row j XOR-swizzled by j % 8 (conflict-free operand reads)
    auto bcx = [](int j, int n) { return j * NP + ((((n >> 2) ^ (j & 7))) << 2) + (n & 3); };

    // ---- workgroup -> (batch, segment, head, column group), as k_walk ------------
    const int gsize = a.H * a.npg;
    const int ngroups = (int)(gridDim.x / gsize);
    const int id = blockIdx.x;
    const int full = ngroups / 8 * 8 * gsize;
    int grp, wi;
    if (id < full) {
        const int x = id % 8, k = id / 8;
        grp = x + 8 * (k / gsize);
        wi = k % gsize;
    } else {
        grp = id / gsize;
        wi = id % gsize;
    }
    const int b = grp / a.nseg, seg = grp % a.nseg;
    const int h = wi / a.npg, pg = wi % a.npg;
    const int hg = h / (a.H / a.G);
    const int p0 = pg * kPG;
    const int c_begin = seg * a.cps;
    const int c_end = min(a.nch, c_begin + a.cps);

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const bool mma = wave < 4;         // uniform
    const int pw = wave & 3;           // matrix wave: column block; staging wave: step block
    const int li = lane % 16, lk = lane / 16;
    const int pw_n = (min(kPG, a.P - p0)) / 16;
    const bool active = mma && pw < pw_n;   // uniform
    const int pcol = p0 + 16 * pw + li;
    const Views<1, true, float> vw(a, b, h, hg);
    const size_t sh_off = (size_t)(b * a.H + h) * a.N * a.P;
    const Buf Sbuf = make_buf(a.S + (size_t)b * a.nch * a.G * (kRows * kRows),
                              (size_t)a.nch * a.G * kRows * kRows * 4);
    auto srow = [](int t, int r, int lk_) { return (NP / 4) * lk_ + (NP / 16) * r + t; };

    // ---- staging waves -----------------------------------------------------------
    // LDS DMA of the 64 rows of B or C of chunk c: staging wave pw moves 1 KB per
    // instruction, lane l filling the 16 bytes at dst + 256 q + 4 l (a swizzled
    // position) from the matching global column group; groups at or past N read
    // zero.
    auto dma_rows = [&](const Buf& src, float* dst, int c) {
        const int t0g = c * kRows;
#pragma unroll
        for (int m = 0; m < NDMA; ++m) {
            const int q = pw + 4 * m;
            const int f = 256 * q + 4 * lane;
            const int j = f / NP, gp = (f % NP) >> 2;
            const int g = gp ^ (j & 7);
            const uint32_t off = (uint32_t)(((t0g + j) * vw.bc_step + vw.bc_head + 4 * g) * 4) | (4 * g < a.N ? 0u : kOut);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                src.r, (__attribute__((address_space(3))) void*)(dst + 256 * q), 16, off, 0, 0, 0);
        }
    };
    // registers of the next chunk: X column p0 + lane at steps 16 pw + i; score row
    // `lane`, columns 16 pw .. 16 pw + 15; log-decay of step `lane`
    float px[16], psc[16], pld = 0.0f;
    // block prologue: raw x of the three steps before the block, dt' of step `lane`
    float pxh[3] = {0.0f, 0.0f, 0.0f}, pdt = 0.0f;
    // offsets of lanes without a value get the top bit set (past any buffer);
    // kept as arithmetic so that the loads stay one straight block
    const uint32_t xbad = p0 + lane < a.P ? 0u : kOut;
    const uint32_t sbad = 16 * pw <= lane ? 0u : kOut;   // score rows before the block: masked
    const Buf dtpb = PRO ? make_buf(a.dtp + (size_t)b * a.L * a.H, (size_t)a.L * a.H * 4) : make_buf(a.ld, 0);
    float cw4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cwb = 0.0f;
    if constexpr (PRO) if (!mma) conv_taps(a, h * a.P + p0 + lane, p0 + lane < a.P, cw4, &cwb);
    auto prefetch = [&](int c) {
        const int t0g = c * kRows;
        const uint32_t xo = (uint32_t)(((t0g + 16 * pw) * vw.x_step + vw.x_head + p0 + lane) * 4);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            px[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                vw.X.r, (xo + (uint32_t)(i * vw.x_step * 4)) | xbad, 0, 0));
        if constexpr (PRO) {
            const int ch = h * a.P + p0 + lane;
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int t = t0g + 16 * pw - 3 + j;
                pxh[j] = t < 0 ? (p0 + lane < a.P ? hist_in<float>(a, b, t, ch) : 0.0f)
                               : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                     vw.X.r, (uint32_t)((t * vw.x_step + ch) * 4) | xbad, 0, 0));
            }
            pdt = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                dtpb.r, (uint32_t)(((t0g + lane) * a.H + h) * 4), 0, 0));
        }
        // blocked score layout: columns 8 (2 pw + q) .. + 7 of row `lane`
        const uint32_t so = (uint32_t)(((c * a.G + hg) * (kRows * kRows) + (2 * pw) * (kRows * 8) + lane * 8) * 4);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const uintx4 u = __builtin_amdgcn_raw_buffer_load_b128(
                    Sbuf.r, (so + (uint32_t)(q * kRows * 8 * 4 + v * 16)) | sbad, 0, 0);
                psc[8 * q + 4 * v] = __uint_as_float(u.x);
                psc[8 * q + 4 * v + 1] = __uint_as_float(u.y);
                psc[8 * q + 4 * v + 2] = __uint_as_float(u.z);
                psc[8 * q + 4 * v + 3] = __uint_as_float(u.w);
            }
        pld = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            vw.ld.r, (uint32_t)(((t0g + lane) * a.H + h) * 4), 0, 0));
    };
    auto stage = [&](int c) {
        const float cum = wave_scan_dpp(pld);
        const float cum_last = readlane_f(cum, kRows - 1);
        const float wl = exp_e(cum_last - cum);   // chunk-end weight of step `lane`
        if (pw == 0) {
            s_cum[c & 1][lane + 1] = cum;
            if (lane == 0) s_cum[c & 1][0] = 0.0f;
        }
        // the masked scores' decay e^{cum_i - cum_t} as e^{cum_i - cum_m} e^{cum_m - cum_t}
        // around the middle step m when neither factor can overflow, else directly
        const float cmid = readlane_f(cum, 31);
        const bool fact = decay_factors_safe(pld);
        // the 16 steps of this wave's block, broadcast through the wave's own LDS
        // slots (cheaper than one readlane per value): cum, or the column factor
        s_bc[pw][0][lane] = fact ? exp_e(cmid - cum) : cum;
        s_bc[pw][1][lane] = wl;
        if constexpr (PRO) s_bc[pw][2][lane] = pdt;
        float cumv[16], wlv[16], dtv[16];
#pragma unroll
        for (int q = 0; q < 16; q += 4) {
            const float4 u = *(const float4*)&s_bc[pw][0][16 * pw + q];
            const float4 v = *(const float4*)&s_bc[pw][1][16 * pw + q];
            cumv[q] = u.x; cumv[q + 1] = u.y; cumv[q + 2] = u.z; cumv[q + 3] = u.w;
            wlv[q] = v.x; wlv[q + 1] = v.y; wlv[q + 2] = v.z; wlv[q + 3] = v.w;
            if constexpr (PRO) {
                const float4 d = *(const float4*)&s_bc[pw][2][16 * pw + q];
                dtv[q] = d.x; dtv[q + 1] = d.y; dtv[q + 2] = d.z; dtv[q + 3] = d.w;
            }
        }
        float* xd = sXdT[c & 1];
        float xv[16], xw[16], mv[16];
        if constexpr (PRO) {
            // block prologue: convolved, activated x (zero past the sequence); dt'
            // goes to the chunk-end weights and the masked scores, the skip term
            // to the scores' diagonal
            float win[3] = {pxh[0], pxh[1], pxh[2]};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = 16 * pw + i;
                const float pre = fmaf(cw4[3], px[i], fmaf(cw4[2], win[2], fmaf(cw4[1], win[1], fmaf(cw4[0], win[0], cwb))));
                win[0] = win[1];
                win[1] = win[2];
                win[2] = px[i];
                const float xc = (p0 + lane < a.P && c * kRows + t < a.L) ? silu_acc(pre) : 0.0f;
                xv[i] = xc;
                xw[i] = xc * (wlv[i] * dtv[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                xv[i] = px[i];
                xw[i] = px[i] * wlv[i];
            }
        }
        float ev[16];
        if (fact) {
            const float er = exp_e(cum - cmid);
#pragma unroll
            for (int i = 0; i < 16; ++i) ev[i] = er * cumv[i];
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) ev[i] = exp_e(16 * pw + i <= lane ? cum - cumv[i] : 0.0f);
        }
        const float dh = (PRO && a.Dh) ? a.Dh[h] : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * pw + i;
            if constexpr (PRO) {
                mv[i] = t <= lane ? fmaf(psc[i] * ev[i], dtv[i], t == lane ? dh : 0.0f) : 0.0f;
            } else {
                mv[i] = t <= lane ? psc[i] * ev[i] : 0.0f;
            }
        }
        // X^T[p][t] for p = p0 + lane (rows of X^T are columns of X); M[lane][t]
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            *(float4*)&sXT[lane * JP + 16 * pw + i] = make_float4(xv[i], xv[i + 1], xv[i + 2], xv[i + 3]);
            *(float4*)&xd[lane * JP + 16 * pw + i] = make_float4(xw[i], xw[i + 1], xw[i + 2], xw[i + 3]);
            *(float4*)&sM[lane * JP + 16 * pw + i] = make_float4(mv[i], mv[i + 1], mv[i + 2], mv[i + 3]);
        }
    };

    // ---- matrix waves: entering state (h0 and the earlier segments) -----------------
    floatx4 acc_h[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc_h[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (active) {
        if (a.h0) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = srow(t, r, lk);
                    acc_h[t][r] = n < a.N ? a.h0[sh_off + (size_t)n * a.P + pcol] : 0.0f;
                }
        }
        for (int s2 = 0; s2 < seg; ++s2) {
            const size_t u = (size_t)(b * a.H + h) * (a.nseg - 1) + s2;
            const float d = exp_e(a.seg_ld[u]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = srow(t, r, lk);
                    const float hl = n < a.N ? a.seg_h[(u * a.N + n) * a.P + pcol] : 0.0f;
                    acc_h[t][r] = fmaf(d, acc_h[t][r], hl);
                }
        }
    }

    // ---- first chunk ------------------------------------------------------------
    if (!mma && c_begin < c_end) {
        dma_rows(vw.C, sC, c_begin);
        prefetch(c_begin);
        vm_wait<0>();
        stage(c_begin);
    }
    __syncthreads();

    // The two roles run separate loops with the same three barriers per chunk.
    if (mma) {
        for (int c = c_begin; c < c_end; ++c) {
            const int t0g = c * kRows;
            // output side: X and z of this lane's outputs load now, under the
            // chunk's matrix work (four columns of a step per tile)
            float ex[4][4] = {}, ez[4][4] = {};
            if constexpr (EPI) {
                if (active) {
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int tg = t0g + 16 * it + li;
                        if (tg < a.L) {
                            const size_t e = (((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P + p0 + 16 * pw + 4 * lk;
                            if (!PRO && a.Dh) load4<float>(a.X, e, ex[it]);
                            if (a.Zg) load4<float>(a.Zg, e, ez[it]);
                        }
                    }
                }
            }
            // ---- phase 1: Y^T = H^T C^T, scaled by e^{cum} per row ------------------------
            floatx4 acc_y[4];
            if (active) {
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    floatx4 y4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y4[e] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int q4 = 0; q4 < NP / 16; ++q4) {
                        // state rows (NP/4) lk + 4 q4 .. + 3 of this lane group: s = NT r + t
                        const float4 cv = *(const float4*)(sC + bcx(16 * it + li, (NP / 4) * lk + 4 * q4));
                        const float cvs[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int s = 4 * q4 + e;
                            const int t = s % NT, r = s / NT;
                            y4[e] = mfma4(acc_h[t][r], cvs[e], y4[e]);
                        }
                    }
                    acc_y[it] = ((y4[0] + y4[1]) + (y4[2] + y4[3])) * exp_e(s_cum[c & 1][16 * it + li + 1]);
                }
            }
            __syncthreads();
            // ---- phase 2: Y^T += X^T M^T; store Y(c) -----------------------------------------
            if (active) {
                const float* pxr = sXT + (16 * pw + li) * JP + 4 * lk;
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const float4 xv = *(const float4*)(pxr + 16 * jt);
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        if (it < jt) continue;
                        const float4 mv = *(const float4*)(sM + (16 * it + li) * JP + 16 * jt + 4 * lk);
                        acc_y[it] = mfma4(xv.x, mv.x, acc_y[it]);
                        acc_y[it] = mfma4(xv.y, mv.y, acc_y[it]);
                        acc_y[it] = mfma4(xv.z, mv.z, acc_y[it]);
                        acc_y[it] = mfma4(xv.w, mv.w, acc_y[it]);
                    }
                }
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    // lane holds Y[i = 16 it + li][p = p0 + 16 pw + 4 lk + r]
                    const int tg = t0g + 16 * it + li;
                    if (tg < a.L) {
                        float yv[4] = {acc_y[it][0], acc_y[it][1], acc_y[it][2], acc_y[it][3]};
                        if constexpr (EPI) {
                            // (y + Dh x) SiLU(z) (block prologue: the skip term is already in y)
                            const float dh = (!PRO && a.Dh) ? a.Dh[h] : 0.0f;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float v = fmaf(dh, ex[it][r], yv[r]);
                                const float sg = ez[it][r] * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-ez[it][r] * kLog2e));
                                yv[r] = a.Zg ? v * sg : v;
                            }
                        }
                        float* yrow = (float*)a.Y + (((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P;
                        *(float4*)(yrow + p0 + 16 * pw + 4 * lk) = make_float4(yv[0], yv[1], yv[2], yv[3]);
                    }
                }
            }
            __syncthreads();
            // ---- phase 3: H = e^{cum_last} H + B^T Xd ------------------------------------------
            if (active) {
                const float tot = exp_e(s_cum[c & 1][kRows]);   // decay over this chunk
#pragma unroll
                for (int t = 0; t < NT; ++t) acc_h[t] *= tot;
                const float* pxd = sXdT[c & 1] + (16 * pw + li) * JP + 16 * lk;
                const int nb = (NP / 4) * (li / 4) + (NP / 16) * (li % 4);   // this lane's first row
#pragma unroll
                for (int sq4 = 0; sq4 < 4; ++sq4) {
                    const float4 xd = *(const float4*)(pxd + 4 * sq4);
                    const float xds[4] = {xd.x, xd.y, xd.z, xd.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 16 * lk + 4 * sq4 + e;
#pragma unroll
                        for (int g4 = 0; g4 < NT / 4; ++g4) {
                            const float4 bv = *(const float4*)(sB + bcx(j, nb + 4 * g4));
                            acc_h[4 * g4 + 0] = mfma4(bv.x, xds[e], acc_h[4 * g4 + 0]);
                            acc_h[4 * g4 + 1] = mfma4(bv.y, xds[e], acc_h[4 * g4 + 1]);
                            acc_h[4 * g4 + 2] = mfma4(bv.z, xds[e], acc_h[4 * g4 + 2]);
                            acc_h[4 * g4 + 3] = mfma4(bv.w, xds[e], acc_h[4 * g4 + 3]);
                        }
                    }
                }
            }
            __syncthreads();
        }
    } else {
        for (int c = c_begin; c < c_end; ++c) {
            // phase 1: B(c) -> LDS (read in phase 3); the registers of chunk c + 1
            // (past the segment: unused; past the sequence: zeros)
            dma_rows(vw.B, sB, c);
            prefetch(c + 1);
            __syncthreads();
            // phase 2: C(c + 1) -> LDS (C(c) was last read in phase 1).  The barrier
            // closing phase 2 has no fence, so it does not wait for this copy: it
            // lands during phases 2 and 3 and is waited for before the barrier
            // closing phase 3 (phase 2 writes nothing else the matrix waves read
            // before then; the empty asm keeps the compiler from moving LDS
            // accesses across the barrier)
            dma_rows(vw.C, sC, c + 1);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            // phase 3: stage c + 1
            if (c + 1 < c_end) stage(c + 1);
            vm_wait<0>();
            __syncthreads();
        }
    }

    if (a.h_out && seg == a.nseg - 1 && active) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = srow(t, r, lk);
                if (n < a.N) a.h_out[sh_off + (size_t)n * a.P + pcol] = acc_h[t][r];
            }
    }
}

// ---------------------------------------------------------------------------
// Mamba-2 state-only pass with bf16 inputs on the bf16 matrix instruction: the
// local end state of every sequence segment but the last, for the full pass
// (k_walk_bfs) to compose.  Four waves, one workgroup per (batch, segment,
// head, 64 columns); wave w owns state columns p0 + 16 w .. + 15 for all NP
// state rows in NT = NP/16 fp32 accumulator tiles.  Tile t, register r of lane
// (li, lk) holds state row
//     n = 32 (t / 2) + 8 lk + 4 (t % 2) + r
// (the layout k_walk_bfs uses).  Per chunk:
//   H = e^{cum_last} H + B^T Xd            (Xd = X weighted to the chunk end)
// B^T (a transposed copy that k_scores writes) comes into double-buffered LDS
// by LDS DMA; X is loaded straight into operand registers (the eight steps of
// a lane group per register quad).  One workgroup barrier per chunk: every
// buffer a chunk reads is written before that chunk's barrier and rewritten
// only after the next one.
// ---------------------------------------------------------------------------
constexpr int kBfThreads = 256;

// A value the compiler cannot see through: per-load offsets built from it by
// uniform adds are not hoisted out of the chunk loop as one register each.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// XOR swizzles of the 16-byte pieces of an LDS row, chosen so that the operand
// reads (16 rows, one piece each, per lane group) hit distinct banks
template <int NP>
__device__ __forceinline__ int swz_c(int i) {   // C: rows i of NP/8 pieces
    return NP == 128 ? (i & 15) : ((i & 7) ^ ((i >> 3) & 1));
}
__device__ __forceinline__ int swz_m(int i) { return (i & 7) ^ ((i >> 3) & 1); }   // M: 8 pieces
__device__ __forceinline__ int swz_bt(int n) {   // B^T: rows n of 8 pieces, read as 16 state rows
    return ((n & 3) | (((n >> 3) & 1) << 2)) ^ ((n >> 4) & 1);
}

template <int NP>
__global__ __launch_bounds__(kBfThreads, 2) void k_walk_bf(Args a) {
    constexpr int NT = NP / 16;      // state tiles per wave
    constexpr int NDMA = NP / 32;    // 1 KB copies per wave for B^T
    constexpr int CB = kRows * NP;   // bf16 elements of one B^T buffer

    // Double buffers as separate objects, and the chunk loop unrolled by two so
    // that every access names its buffer at compile time: the compiler then sees
    // that a copy into one buffer cannot alias reads of the other, and does not
    // wait for the copies of the next chunk before reading this one.
    __shared__ __attribute__((aligned(16))) bf16 sBT0[CB];
    __shared__ __attribute__((aligned(16))) bf16 sBT1[CB];

    // ---- workgroup -> (batch, segment, head, column group), as k_walk ------------
    const int nsegL = a.nseg - 1;
    const int gsize = a.H * a.npg;
    const int ngroups = (int)(gridDim.x / gsize);
    const int id = blockIdx.x;
    const int full = ngroups / 8 * 8 * gsize;
    int grp, wi;
    if (id < full) {
        const int x = id % 8, k = id / 8;
        grp = x + 8 * (k / gsize);
        wi = k % gsize;
    } else {
        grp = id / gsize;
        wi = id % gsize;
    }
    const int b = grp / nsegL, seg = grp % nsegL;
    const int h = wi / a.npg, pg = wi % a.npg;
    const int hg = h / (a.H / a.G);
    const int p0 = pg * kPG;
    const int c_begin = seg * a.cps;
    const int c_end = min(a.nch, c_begin + a.cps);

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int li = lane % 16, lk = lane / 16;
    const bool active = 16 * wave < a.P - p0;   // uniform (P is a multiple of 16)
    const int pcol = p0 + 16 * wave + li;
    const Views<1, true, bf16> vw(a, b, h, hg);
    const size_t bt_rows = (size_t)a.nch * a.G * (NP * kRows);
    const Buf BTbuf = make_buf(a.BT + (size_t)b * bt_rows, bt_rows * 2);
    // state row of tile t, row rho of the tile (rho = 4 lk + r in the accumulators)
    auto srow = [](int t, int rho) { return 32 * (t >> 1) + 8 * (rho >> 2) + 4 * (t & 1) + (rho & 3); };

    // ---- LDS DMA of B^T of chunk c into buffer PB: wave w moves pieces
    // 64 (w + 4 m) + lane; piece m is row n0 + 32 m of the same swizzled column
    // group --------------------------------------------------------------------------
    auto dma_bt = [&](int c, auto par) {
        constexpr int PB = decltype(par)::value;
        bf16* dst;
        if constexpr (PB) dst = sBT1;
        else dst = sBT0;
        const int gi0 = 64 * wave + lane;
        const int n0 = gi0 / 8, g = (gi0 % 8) ^ swz_bt(n0);
        const uint32_t base = opaque((uint32_t)((((c * a.G + hg) * NP + n0) * kRows + 8 * g) * 2));
#pragma unroll
        for (int m = 0; m < NDMA; ++m) {
            const int q = wave + 4 * m;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                BTbuf.r, (__attribute__((address_space(3))) void*)(dst + 512 * q), 16,
                base + (uint32_t)(m * 32 * kRows * 2), 0, 0, 0);
        }
    };

    // ---- prefetch registers -------------------------------------------------------
    uint32_t px[16];     // X[32 k + 8 lk + q][pcol] (k = q / 8): raw bf16 bits
    float pld = 0.0f;    // log-decay of step `lane`
    const uint32_t xlane = (uint32_t)(((8 * lk) * vw.x_step + vw.x_head + pcol) * 2);
    auto prefetch = [&](int c) {
        const int t0g = c * kRows;
        if (active) {
            // the whole offset goes in the vector operand: the range check that
            // turns steps past the sequence into zeros does not see the scalar one
            const uint32_t xo = opaque((uint32_t)(t0g * vw.x_step * 2) + xlane);
#pragma unroll
            for (int q = 0; q < 16; ++q)
                px[q] = __builtin_amdgcn_raw_buffer_load_b16(
                    vw.X.r, xo + (uint32_t)((32 * (q / 8) + q % 8) * vw.x_step * 2), 0, 0);
        }
        pld = bload<float>(vw.ld, (t0g + lane) * a.H + h);
    };

    floatx4 acc_h[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc_h[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    if (c_begin < c_end) {
        dma_bt(c_begin, Par<0>{});
        prefetch(c_begin);
    }
    float seg_acc = 0.0f;   // total log-decay of the segment

    // one chunk; its operands sit in buffer PB, the next chunk's go to 1 - PB
    auto chunk = [&](int c, auto par) __attribute__((always_inline)) {
        constexpr int PB = decltype(par)::value;
        vm_wait<0>();   // this wave's copies and loads of chunk c
        const float cum = wave_scan_dpp(pld);
        const float cum_last = readlane_f(cum, kRows - 1);
        seg_acc += cum_last;
        const float wl = exp_e(cum_last - cum);   // chunk-end weight of step `lane`
        // Xd: X weighted to the chunk end (steps 32 k + 8 lk + q)
        uintx4 xd[2];
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                const uint32_t lo = px[8 * k + 2 * q2] & 0xffffu, hi = px[8 * k + 2 * q2 + 1] & 0xffffu;
                const int t = 32 * k + 8 * lk + 2 * q2;
                const float w0 = __shfl(wl, t, 64), w1 = __shfl(wl, t + 1, 64);
                xd[k][q2] = pack_bf(__uint_as_float(lo << 16) * w0, __uint_as_float(hi << 16) * w1);
            }
        __syncthreads();
        if (c + 1 < c_end) {
            dma_bt(c + 1, Par<1 - PB>{});
            prefetch(c + 1);
        }
        if (active) {
            // H = e^{cum_last} H + B^T Xd
            const bf16* btb;
            if constexpr (PB) btb = sBT1;
            else btb = sBT0;
            const float tot = exp_e(cum_last);
#pragma unroll
            for (int t = 0; t < NT; ++t) acc_h[t] *= tot;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int n = srow(t, li);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const uintx4 bv = *(const uintx4*)&btb[n * kRows + 8 * ((4 * k + lk) ^ swz_bt(n))];
                    acc_h[t] = mfma_bf(bv, xd[k], acc_h[t]);
                }
            }
        }
    };
    for (int c = c_begin; c < c_end; c += 2) {
        chunk(c, Par<0>{});
        if (c + 1 < c_end) chunk(c + 1, Par<1>{});
    }
    vm_wait<0>();

    // ---- the segment's local end state and total log-decay --------------------------
    const size_t u = (size_t)(b * a.H + h) * (a.nseg - 1) + seg;
    if (active) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = srow(t, 4 * lk + r);
                if (n < a.N) a.seg_h[(u * a.N + n) * a.P + pcol] = acc_h[t][r];
            }
    }
    if (pg == 0 && tid == 0) a.seg_ld[u] = seg_acc;
}

// ---------------------------------------------------------------------------
// Mamba-2 walk with bf16 inputs (full pass), wave-specialised as k_walk_m2s.
// Waves 0-3 are the matrix waves: wave w owns state columns p0 + 16 w .. + 15
// for all NP state rows (the accumulator layout of k_walk_bf) and does every
// product of the chunk for them on the bf16 matrix instruction.  Waves 4-7 are
// the staging waves: they copy C and the transposed B into LDS by LDS DMA, load
// X, the scores and the log-decay of the next chunk into registers, and stage
// X^T, the chunk-end-weighted Xd^T and the masked scores M as bf16 rows in LDS.
// The matrix waves read every operand with 16-byte LDS reads and never wait on
// the decay scan, the exponentials or global memory.  Per chunk c, three phases
// separated by workgroup barriers:
//   1. matrix: Y^T = H^T C^T x e^{cum}       staging: B^T(c) -> LDS; loads for c+1
//   2. matrix: Y^T += X^T M^T, store Y(c)    staging: C(c+1) -> LDS (in flight
//                                             until the end of phase 3)
//   3. matrix: H = e^{cum_last} H + B^T Xd   staging: X^T, Xd^T, M, cum of c+1
// Xd^T and cum are double-buffered, the other buffers single: each is written
// in the phase after its last reader.  The matrix waves only read LDS, and use
// every value they read within the phase, so their barriers carry no wait:
// their stores of Y drain while the next phase runs.  The staging waves issue
// the loads of chunk c + 2 right after staging c + 1, so a whole chunk covers
// their latency; their barriers wait only for the copies the next phase reads
// (exact vmcnt counts: the loads and copies are issued unconditionally).
// ---------------------------------------------------------------------------
template <int NP, bool EPI = false>
__global__ __launch_bounds__(kWalkThreads, 4) void k_walk_bfs(Args a) {
    constexpr int NT = NP / 16;      // state tiles per matrix wave
    constexpr int KB = NP / 32;      // 32-row blocks of the output contraction
    constexpr int GPR = NP / 8;      // 16-byte pieces per row of C
    constexpr int NDMA = NP / 32;    // 1 KB copies per staging wave for C or B^T
    constexpr int CB = kRows * NP;   // bf16 elements of the C or B^T buffer
    constexpr int MB = kRows * kRows;
    constexpr uint32_t kOut = 0x80000000u;   // byte offset past any buffer: reads zero

    __shared__ __attribute__((aligned(16))) bf16 sC[CB];
    __shared__ __attribute__((aligned(16))) bf16 sBT[CB];
    __shared__ __attribute__((aligned(16))) bf16 sXT[kPG * kRows];
    __shared__ __attribute__((aligned(16))) bf16 sXdT[2][kPG * kRows];
    __shared__ __attribute__((aligned(16))) bf16 sM[MB];
    __shared__ float s_cum[2][kRows + 1];
    __shared__ __attribute__((aligned(16))) float s_bc[4][2][kRows];   // per staging wave: cum, wl

    // ---- workgroup -> (batch, segment, head, column group), as k_walk ------------
    const int gsize = a.H * a.npg;
    const int ngroups = (int)(gridDim.x / gsize);
    const int id = blockIdx.x;
    const int full = ngroups / 8 * 8 * gsize;
    int grp, wi;
    if (id < full) {
        const int x = id % 8, k = id / 8;
        grp = x + 8 * (k / gsize);
        wi = k % gsize;
    } else {
        grp = id / gsize;
        wi = id % gsize;
    }
    const int b = grp / a.nseg, seg = grp % a.nseg;
    const int h = wi / a.npg, pg = wi % a.npg;
    const int hg = h / (a.H / a.G);
    const int p0 = pg * kPG;
    const int c_begin = seg * a.cps;
    const int c_end = min(a.nch, c_begin + a.cps);

    const int tid = threadIdx.x, lane = tid % 64;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const bool mma = wave < 4;         // uniform
    const int pw = wave & 3;           // matrix wave: column block; staging wave: step block
    const int li = lane % 16, lk = lane / 16;
    const int pw_n = min(kPG, a.P - p0) / 16;
    const bool active = mma && pw < pw_n;   // uniform
    const int pcol = p0 + 16 * pw + li;
    const Views<1, true, bf16> vw(a, b, h, hg);
    const size_t sh_off = (size_t)(b * a.H + h) * a.N * a.P;
    const size_t bt_rows = (size_t)a.nch * a.G * (NP * kRows);
    const Buf BTbuf = make_buf(a.BT + (size_t)b * bt_rows, bt_rows * 2);
    const Buf Sbuf = make_buf(a.S + (size_t)b * a.nch * a.G * MB, (size_t)a.nch * a.G * MB * 4);
    // state row of tile t, row rho of the tile (rho = 4 lk + r in the accumulators)
    auto srow = [](int t, int rho) { return 32 * (t >> 1) + 8 * (rho >> 2) + 4 * (t & 1) + (rho & 3); };

    // ---- staging waves ------------------------------------------------------------
    // LDS DMA of C and B^T of chunk c (the k_walk_bf copies, staging wave pw
    // moving pieces 64 (pw + 4 m) + lane)
    auto dma_c = [&](int c) {
        const int t0g = c * kRows;
        const int gi0 = 64 * pw + lane;
        const int i0 = gi0 / GPR, g = (gi0 % GPR) ^ swz_c<NP>(i0);
        const uint32_t base = opaque((uint32_t)(((t0g + i0) * vw.bc_step + vw.bc_head + 8 * g) * 2) |
                                     (8 * g < a.N ? 0u : kOut));
#pragma unroll
        for (int m = 0; m < NDMA; ++m) {
            const int q = pw + 4 * m;
            const uint32_t off = base + (uint32_t)(m * (256 / GPR) * vw.bc_step * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vw.C.r, (__attribute__((address_space(3))) void*)(sC + 512 * q), 16, off, 0, 0, 0);
        }
    };
    auto dma_bt = [&](int c) {
        const int gi0 = 64 * pw + lane;
        const int n0 = gi0 / 8, g = (gi0 % 8) ^ swz_bt(n0);
        const uint32_t base = opaque((uint32_t)((((c * a.G + hg) * NP + n0) * kRows + 8 * g) * 2));
#pragma unroll
        for (int m = 0; m < NDMA; ++m) {
            const int q = pw + 4 * m;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                BTbuf.r, (__attribute__((address_space(3))) void*)(sBT + 512 * q), 16,
                base + (uint32_t)(m * 32 * kRows * 2), 0, 0, 0);
        }
    };
    // registers of the next chunk: X column p0 + lane at steps 16 pw + i (raw bf16
    // bits); score row `lane`, columns 16 pw .. + 15; log-decay of step `lane`.
    // Lanes without a value read past the buffer (zeros), so the loads stay one
    // straight block and the waits stay exact.
    uint32_t px[16];
    float psc[16], pld = 0.0f;
    constexpr int kPf = 16 + 4 + 1;   // vector memory operations of one prefetch
    const uint32_t xbad = p0 + lane < a.P ? 0u : kOut;
    const uint32_t sbad = 16 * pw <= lane ? 0u : kOut;   // score rows before the block: masked
    auto prefetch = [&](int c) {
        const int t0g = c * kRows;
        const uint32_t xo = opaque((uint32_t)(((t0g + 16 * pw) * vw.x_step + vw.x_head + p0 + lane) * 2));
#pragma unroll
        for (int i = 0; i < 16; ++i)
            px[i] = __builtin_amdgcn_raw_buffer_load_b16(vw.X.r, (xo + (uint32_t)(i * vw.x_step * 2)) | xbad, 0, 0);
        // blocked score layout: columns 8 (2 pw + q) .. + 7 of row `lane`
        const uint32_t so = (uint32_t)(((c * a.G + hg) * MB + (2 * pw) * (kRows * 8) + lane * 8) * 4);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const uintx4 u = __builtin_amdgcn_raw_buffer_load_b128(
                    Sbuf.r, (so + (uint32_t)(q * kRows * 8 * 4 + v * 16)) | sbad, 0, 0);
                psc[8 * q + 4 * v] = __uint_as_float(u.x);
                psc[8 * q + 4 * v + 1] = __uint_as_float(u.y);
                psc[8 * q + 4 * v + 2] = __uint_as_float(u.z);
                psc[8 * q + 4 * v + 3] = __uint_as_float(u.w);
            }
        pld = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            vw.ld.r, (uint32_t)(((t0g + lane) * a.H + h) * 4), 0, 0));
    };
    // X^T, Xd^T and M rows of chunk c: row `lane` (X column p0 + lane, score row
    // `lane`), 16-byte pieces 2 pw and 2 pw + 1 (steps / columns 16 pw .. + 15)
    auto stage = [&](int c) {
        const float cum = wave_scan_dpp(pld);
        const float cum_last = readlane_f(cum, kRows - 1);
        const float wl = exp_e(cum_last - cum);   // chunk-end weight of step `lane`
        if (pw == 0) {
            s_cum[c & 1][lane + 1] = cum;
            if (lane == 0) s_cum[c & 1][0] = 0.0f;
        }
        // the 16 steps of this wave's block, broadcast through the wave's own LDS slots
        s_bc[pw][0][lane] = cum;
        s_bc[pw][1][lane] = wl;
        float cumv[16], wlv[16];
#pragma unroll
        for (int q = 0; q < 16; q += 4) {
            const float4 u = *(const float4*)&s_bc[pw][0][16 * pw + q];
            const float4 v = *(const float4*)&s_bc[pw][1][16 * pw + q];
            cumv[q] = u.x; cumv[q + 1] = u.y; cumv[q + 2] = u.z; cumv[q + 3] = u.w;
            wlv[q] = v.x; wlv[q + 1] = v.y; wlv[q + 2] = v.z; wlv[q + 3] = v.w;
        }
        uint32_t xv[8], xw[8], mv[8];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const uint32_t lo = px[i] & 0xffffu, hi = px[i + 1] & 0xffffu;
            xv[i / 2] = lo | (hi << 16);
            xw[i / 2] = pack_bf(__uint_as_float(lo << 16) * wlv[i], __uint_as_float(hi << 16) * wlv[i + 1]);
            const int t = 16 * pw + i;
            const float e0 = exp_e(t <= lane ? cum - cumv[i] : 0.0f);
            const float e1 = exp_e(t + 1 <= lane ? cum - cumv[i + 1] : 0.0f);
            mv[i / 2] = pack_bf(t <= lane ? psc[i] * e0 : 0.0f, t + 1 <= lane ? psc[i + 1] * e1 : 0.0f);
        }
        bf16* xd = sXdT[c & 1];
        const int sw = swz_m(lane);
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
            const int o = lane * kRows + 8 * ((2 * pw + g2) ^ sw);
            *(uint4*)&sXT[o] = make_uint4(xv[4 * g2], xv[4 * g2 + 1], xv[4 * g2 + 2], xv[4 * g2 + 3]);
            *(uint4*)&xd[o] = make_uint4(xw[4 * g2], xw[4 * g2 + 1], xw[4 * g2 + 2], xw[4 * g2 + 3]);
            *(uint4*)&sM[o] = make_uint4(mv[4 * g2], mv[4 * g2 + 1], mv[4 * g2 + 2], mv[4 * g2 + 3]);
        }
    };

    // ---- matrix waves: entering state (h0 and the earlier segments) -----------------
    floatx4 acc_h[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc_h[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (active) {
        if (a.h0) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = srow(t, 4 * lk + r);
                    acc_h[t][r] = n < a.N ? a.h0[sh_off + (size_t)n * a.P + pcol] : 0.0f;
                }
        }
        for (int s2 = 0; s2 < seg; ++s2) {
            const size_t u = (size_t)(b * a.H + h) * (a.nseg - 1) + s2;
            const float d = exp_e(a.seg_ld[u]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = srow(t, 4 * lk + r);
                    const float hl = n < a.N ? a.seg_h[(u * a.N + n) * a.P + pcol] : 0.0f;
                    acc_h[t][r] = fmaf(d, acc_h[t][r], hl);
                }
        }
    }

    // A barrier with no wait for this wave's memory operations; the empty asm
    // keeps the compiler from moving LDS accesses across it.
    auto bare_barrier = []() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // A barrier after this wave's LDS writes have landed and at most kPf vector
    // memory operations (the loads of a prefetch) are outstanding.
    auto stage_barrier = []() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((kPf & 15) | (7 << 4) | (0 << 8) | ((kPf >> 4) << 14));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // ---- first chunk ------------------------------------------------------------
    if (mma) {
        __syncthreads();
    } else {
        dma_c(c_begin);
        prefetch(c_begin);
        vm_wait<0>();
        if (c_begin < c_end) stage(c_begin);
        prefetch(c_begin + 1);
        stage_barrier();
    }

    // The two roles run separate loops with the same three barriers per chunk.
    if (mma) {
        const int pr = 16 * pw + li;   // this lane's row of X^T and Xd^T
        for (int c = c_begin; c < c_end; ++c) {
            const int t0g = c * kRows;
            // output side: X and z of this lane's outputs, loaded now under the
            // chunk's products and held as packed bf16 (two registers per four values)
            uint2 rx[4] = {}, rz[4] = {};
            if constexpr (EPI) {
                if (active) {
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const int tg = t0g + 16 * it + li;
                        if (tg < a.L) {
                            const size_t e = (((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P + p0 + 16 * pw + 4 * lk;
                            if (a.Dh) rx[it] = *(const uint2*)((const bf16*)a.X + e);
                            if (a.Zg) rz[it] = *(const uint2*)((const bf16*)a.Zg + e);
                        }
                    }
                }
            }
            // ---- phase 1: Y^T = H^T C^T, scaled by e^{cum} per step ---------------------
            floatx4 acc_y[4];
            if (active) {
                // H^T as bf16 operand: rows 32 k + 8 lk .. + 7 from tiles 2k, 2k + 1
                uintx4 hb[KB];
#pragma unroll
                for (int k = 0; k < KB; ++k)
                    hb[k] = uintx4{pack_bf(acc_h[2 * k][0], acc_h[2 * k][1]), pack_bf(acc_h[2 * k][2], acc_h[2 * k][3]),
                                   pack_bf(acc_h[2 * k + 1][0], acc_h[2 * k + 1][1]),
                                   pack_bf(acc_h[2 * k + 1][2], acc_h[2 * k + 1][3])};
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int i = 16 * it + li;
                    floatx4 y0 = {0.0f, 0.0f, 0.0f, 0.0f}, y1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < KB; ++k) {
                        const uintx4 cv = *(const uintx4*)&sC[i * NP + 8 * ((4 * k + lk) ^ swz_c<NP>(i))];
                        if (k % 2 == 0) y0 = mfma_bf(hb[k], cv, y0);
                        else y1 = mfma_bf(hb[k], cv, y1);
                    }
                    acc_y[it] = (y0 + y1) * exp_e(s_cum[c & 1][i + 1]);
                }
            }
            bare_barrier();
            // ---- phase 2: Y^T += X^T M^T; store Y(c) -------------------------------------
            if (active) {
                uintx4 xo[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) xo[k] = *(const uintx4*)&sXT[pr * kRows + 8 * ((4 * k + lk) ^ swz_m(pr))];
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int i = 16 * it + li;
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        if (32 * k > 16 * it + 15) continue;   // above the diagonal
                        const uintx4 mv = *(const uintx4*)&sM[i * kRows + 8 * ((4 * k + lk) ^ swz_m(i))];
                        acc_y[it] = mfma_bf(xo[k], mv, acc_y[it]);
                    }
                }
                // lane holds Y[t0 + 16 it + li][p0 + 16 w + 4 lk + r]
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int tg = t0g + 16 * it + li;
                    if (tg < a.L) {
                        float yv[4] = {acc_y[it][0], acc_y[it][1], acc_y[it][2], acc_y[it][3]};
                        if constexpr (EPI) {
                            // (y + Dh x) SiLU(z); the two-pass Mamba-2 layer takes x = X / dt'
                            float dh = a.Dh ? a.Dh[h] : 0.0f;
                            if (a.skip_dt) dh /= a.skip_dt[((size_t)b * a.L + tg) * a.H + h];
                            const float ex[4] = {__uint_as_float(rx[it].x << 16), __uint_as_float(rx[it].x & 0xffff0000u),
                                                 __uint_as_float(rx[it].y << 16), __uint_as_float(rx[it].y & 0xffff0000u)};
                            const float ez[4] = {__uint_as_float(rz[it].x << 16), __uint_as_float(rz[it].x & 0xffff0000u),
                                                 __uint_as_float(rz[it].y << 16), __uint_as_float(rz[it].y & 0xffff0000u)};
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const float v = fmaf(dh, ex[r], yv[r]);
                                const float sg = ez[r] * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-ez[r] * kLog2e));
                                yv[r] = a.Zg ? v * sg : v;
                            }
                        }
                        bf16* yrow = (bf16*)a.Y + (((size_t)b * a.L + tg) * a.H + h) * (size_t)a.P;
                        *(uint2*)(yrow + p0 + 16 * pw + 4 * lk) =
                            make_uint2(pack_bf(yv[0], yv[1]), pack_bf(yv[2], yv[3]));
                    }
                }
            }
            bare_barrier();
            // ---- phase 3: H = e^{cum_last} H + B^T Xd -------------------------------------
            if (active) {
                const float tot = exp_e(s_cum[c & 1][kRows]);   // decay over this chunk
#pragma unroll
                for (int t = 0; t < NT; ++t) acc_h[t] *= tot;
                const bf16* xdb = sXdT[c & 1];
                uintx4 xd[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) xd[k] = *(const uintx4*)&xdb[pr * kRows + 8 * ((4 * k + lk) ^ swz_m(pr))];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int n = srow(t, li);
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const uintx4 bv = *(const uintx4*)&sBT[n * kRows + 8 * ((4 * k + lk) ^ swz_bt(n))];
                        acc_h[t] = mfma_bf(bv, xd[k], acc_h[t]);
                    }
                }
            }
            bare_barrier();
        }
    } else {
        // outstanding on entry to chunk c: the loads of chunk c + 1
        for (int c = c_begin; c < c_end; ++c) {
            // phase 1: B^T(c) -> LDS (read in phase 3)
            dma_bt(c);
            bare_barrier();
            // phase 2: C(c + 1) -> LDS (C(c) was last read in phase 1); B^T(c) and
            // the loads of c + 1 have landed before the barrier, C(c + 1) before the
            // one closing phase 3
            dma_c(c + 1);
            vm_wait<NDMA>();
            bare_barrier();
            // phase 3: stage c + 1, then the loads of c + 2 (past the segment:
            // unused; past the sequence: zeros)
            if (c + 1 < c_end) stage(c + 1);
            prefetch(c + 2);
            stage_barrier();
        }
        vm_wait<0>();   // no copy into LDS may be in flight when the wave ends
    }

    if (a.h_out && seg == a.nseg - 1 && active) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = srow(t, 4 * lk + r);
                if (n < a.N) a.h_out[sh_off + (size_t)n * a.P + pcol] = acc_h[t][r];
            }
    }
}

// ---------------------------------------------------------------------------
// k_seg_state: the Mamba-2 state-only pass with fp32 inputs.  H_loc(s), the
// state that h_t = e^{ld_t} h_{t-1} + B_t x_t^T reaches at the end of segment
// s from zero, is one weighted product over the segment's steps,
//     H_loc(s) = sum_t B_t^T (e^{D_t} x_t),   D_t = sum of ld over the later steps of s,
// the chunk-state term of the chunkwise form (TorchMamba README, Math notes
// M2) with the whole segment as the chunk.  It runs as a plain contraction:
// no chunk staging and no barriers until the end, in work items small enough
// to spread evenly over the compute units.
//  - One workgroup of 4 waves per (batch, segment, head, 64 state rows, 64
//    columns); wave k takes the k-th quarter of the segment's steps for the
//    whole 64 x 64 block (4 x 4 accumulator tiles), and the four partial
//    blocks are summed through LDS at the end, each wave storing 16 rows.
//  - Operands go from global memory (B comes mostly from L2: the heads of a
//    group share it) straight into the operand registers of the 16 x 16 x 4
//    instruction.  Row i of accumulator tile j is state n0 + 4 i + j and
//    column i of tile q is column p0 + 4 i + q, so in K step ks of a block at
//    step t0 lane (i, k) supplies B[t][n0 + 4 i + j] for the four tiles j
//    with one 16-byte load, and the weighted X[t][p0 + 4 i + q] likewise,
//    t = t0 + 4 ks + k (the 16 lanes of a group read 256 contiguous bytes);
//    each operand feeds four products.  The next block of 8 steps is loaded
//    while the current one is multiplied.
//  - Blocks go from the quarter's end backwards: a step's weight is
//    e^{S + T - cum}, cum the block's inclusive prefix sum of ld (DPP scan),
//    T its total and S the total of the steps after the block in the segment,
//    so every weight is at most 1 for decaying states and the first quarter's S
//    ends as the segment's total log-decay.
// ---------------------------------------------------------------------------
constexpr int kSegThreads = 256;
constexpr int kSegStep = 8;    // steps per block

template <int NP>
__global__ __launch_bounds__(kSegThreads, 3) void k_seg_state(Args a) {
    constexpr int NH = NP / 64;                 // 64-row blocks of the state
    constexpr uint32_t kOut = 0x80000000u;      // byte offset past any buffer: reads zero
    const int nsegL = a.nseg - 1;
    const int npt = (a.P + 63) / 64;
    const int gsize = a.H * NH * npt;
    const int ngroups = (int)(gridDim.x / gsize);
    // ids i, i + 8, ... run on one XCD: give them the heads of one (batch, segment)
    const int id = blockIdx.x;
    const int full = ngroups / 8 * 8 * gsize;
    int grp, wi;
    if (id < full) {
        const int x = id % 8, k = id / 8;
        grp = x + 8 * (k / gsize);
        wi = k % gsize;
    } else {
        grp = id / gsize;
        wi = id % gsize;
    }
    const int b = grp / nsegL, seg = grp % nsegL;
    const int h = wi / (NH * npt), nb = (wi / npt) % NH, pt = wi % npt;
    const int g = h / (a.H / a.G);
    const int n0 = 64 * nb, p0 = 64 * pt;
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int li = lane % 16, lk = lane / 16;
    // Segments before the last hold cps whole chunks inside the sequence
    // ((nseg - 1) cps < nch), so a quarter is 2 cps blocks of 8 steps, all in
    // range; the step of K step ks goes into the scalar offset.
    constexpr int KS = kSegStep / 4;   // K steps per block
    const int seg_t0 = seg * a.cps * kRows;
    const int q_t0 = seg_t0 + wave * a.cps * 16;
    const int nblk = a.cps * 16 / kSegStep;

    // one batch row of each input
    const Buf bB = make_buf((const float*)a.B + (size_t)b * a.L * a.G * a.N, (size_t)a.L * a.G * a.N * 4);
    const Buf bX = make_buf((const float*)a.X + (size_t)b * a.L * a.H * a.P, (size_t)a.L * a.H * a.P * 4);
    const float* ldb = a.ld + (size_t)b * a.L * a.H + h;
    const Buf bL = make_buf(a.ld + (size_t)b * a.L * a.H, (size_t)a.L * a.H * 4);

    // byte offsets of this lane's four operands at step 0 (or past the buffer;
    // N and P are multiples of 4, so the four are in range or out together)
    const uint32_t ob = n0 + 4 * li < a.N ? (uint32_t)(g * a.N + n0 + 4 * li) * 4u : kOut;
    const uint32_t ox = p0 + 4 * li < a.P ? (uint32_t)(h * a.P + p0 + 4 * li) * 4u : kOut;
    const uint32_t sb = (uint32_t)a.G * a.N * 4u, sx = (uint32_t)a.H * a.P * 4u;

    // Every load is issued unconditionally (a block before the quarter's
    // first reads zeros: all its offsets past the buffers), so the compiler's
    // waits on the memory counter stay exact and the next block's loads stay
    // in flight while the current one is multiplied.
    float vb[2][4 * KS], vx[2][4 * KS], vl[2];
    auto load = [&](int slot, int kb) __attribute__((always_inline)) {
        const uint32_t kill = kb >= 0 ? 0u : kOut;
        const int t0 = q_t0 + kb * kSegStep;
        const uint32_t tk = (uint32_t)(t0 + lk);
        const uint32_t vbo = (ob + tk * sb) | kill, vxo = (ox + tk * sx) | kill;
        // the block's log-decay first, then its operands, in this order at this
        // point of the program: a wait for one slot then never covers the
        // loads of the other
        const uint32_t lo = lane < kSegStep ? ((uint32_t)((t0 + lane) * a.H + h) * 4u) | kill : kOut;
        __builtin_amdgcn_sched_barrier(0);
        vl[slot] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bL.r, (int)lo, 0, 0));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uintx4 ub = __builtin_amdgcn_raw_buffer_load_b128(bB.r, (int)vbo, (int)(4 * ks * sb), 0);
            const uintx4 ux = __builtin_amdgcn_raw_buffer_load_b128(bX.r, (int)vxo, (int)(4 * ks * sx), 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vb[slot][4 * ks + j] = __uint_as_float(ub[j]);
                vx[slot][4 * ks + j] = __uint_as_float(ux[j]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j][q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float S = 0.0f;   // the log-decay of the segment's steps after the current block
    auto step = [&](int slot) __attribute__((always_inline)) {
        const float cum = wave_scan_dpp(vl[slot]);   // lanes past the block add zero
        const float T = readlane_f(cum, 63);
        const float wl = exp_e(S + (T - cum));
        S += T;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float w = __shfl(wl, 4 * ks + lk, 64);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float xw = vx[slot][4 * ks + q] * w;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j][q] = mfma4(vb[slot][4 * ks + j], xw, acc[j][q]);
            }
        }
    };
    // blocks from the last to the first, two per iteration (the register
    // slots alternate, so no copies); the first block's loads fly while the
    // quarters' total log-decays are summed (lane l takes steps l, l + 64, ...)
    // and exchanged: S starts as the total of the later quarters
    int kb = nblk - 1;
    load(0, kb);
    __shared__ float s_tot[4];
    {
        const int q_t1 = q_t0 + nblk * kSegStep;
        float T = 0.0f;
        for (int t0 = q_t0; t0 < q_t1; t0 += 256) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 64 * i + lane;
                v[i] = t < q_t1 ? ldb[(size_t)t * a.H] : 0.0f;
            }
            T += (v[0] + v[1]) + (v[2] + v[3]);
        }
        T = readlane_f(wave_scan_dpp(T), 63);
        if (lane == 0) s_tot[wave] = T;
    }
    __syncthreads();
    for (int k = 3; k > wave; --k) S += s_tot[k];
    for (; kb >= 1; kb -= 2) {
        load(1, kb - 1);
        step(0);
        load(0, kb - 2);
        step(1);
    }
    if (kb == 0) step(0);

    // sum the quarters: wave v parks the 12 tiles of the other waves' rows
    // (tile (j, q) belongs to wave j), then each wave adds its 4 tiles
    __shared__ __attribute__((aligned(16))) floatx4 red[4 * 12 * 64];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j == wave) continue;
        const int base = wave * 12 + 4 * (j < wave ? j : j - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) red[(base + q) * 64 + lane] = acc[j][q];
    }
    __syncthreads();
    const size_t u = (size_t)(b * a.H + h) * nsegL + seg;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j != wave) continue;
        floatx4 s[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s[q] = acc[j][q];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (v != j) s[q] += red[(v * 12 + 4 * (j < v ? j : j - 1) + q) * 64 + lane];
        }
        // tile row 4 lk + r is state n0 + 16 lk + 4 r + j; columns p0 + 4 li + q
        const int p = p0 + 4 * li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = n0 + 16 * lk + 4 * r + j;
            if (n < a.N && p < a.P)
                *(float4*)&a.seg_h[(u * a.N + n) * a.P + p] = make_float4(s[0][r], s[1][r], s[2][r], s[3][r]);
        }
    }
    if (nb == 0 && pt == 0 && wave == 0 && lane == 0) a.seg_ld[u] = S;
}

// ---------------------------------------------------------------------------
// k_seg_trap: the Mamba-3 SISO state-only pass (rank 1, fp32, B and C without
// the block prologue), as k_seg_state with the trapezoid's two terms and the
// rotations.  In the frame of the last step of quarter k (steps q0 .. q1 - 1),
// step t contributes
//     R(-Th_t) B_t (w_t x_t)^T,   w_t = gamma_t e^{D_t} + [t + 1 < q1] beta_{t+1} e^{D_t - ld_{t+1}},
// D_t and Th_t the log-decay and the angle of each state pair over the
// quarter's steps after t (TorchMamba README, Math notes M3 SISO: after step t
// the state decays and turns by the later steps' factors, and step t's x
// enters once with gamma_t and once, a step later, with beta_{t+1}).  The
// step before the quarter contributes its beta term,
// R(-Th_{q0-1}) B_{q0-1} (beta_{q0} e^{D_{q0}} x_{q0-1})^T.  A quarter's block
// is then carried to the segment's end by the later quarters' total decay and
// angles, e^{S} R(-Th), and the four are summed; the quarters' totals also
// give the segment's log-decay and angles.
//  - Layout, loads and reduction as k_seg_state; B's operands are turned by
//    their pairs' angles, a pair being tiles 2 m and 2 m + 1 of one lane.
//  - Per block of 4 steps (8 without angles), lane (k, h) of a wave sums the
//    angles of pair k of its 64 rows over steps 2h, 2h + 1, in revolutions,
//    and writes the cos and sin of every (step, pair) to LDS for the operand
//    lanes.
// ---------------------------------------------------------------------------
template <int NP, bool GROUPED, bool ROT>
__global__ __launch_bounds__(kSegThreads, 3) void k_seg_trap(Args a) {
    constexpr int NH = NP / 64;                 // 64-row blocks of the state
    constexpr uint32_t kOut = 0x80000000u;      // byte offset past any buffer: reads zero
    constexpr int KS = ROT ? 1 : 2;             // K steps per block (fewer registers with the angles)
    constexpr int SPB = 4 * KS;                 // steps per block
    constexpr int APL = SPB / 2;                // angles staged per lane and block
    constexpr float kInv2Pi = 0.15915494309189535f;
    constexpr int RS = 34;                      // LDS row stride (float2) of the cos / sin table
    const int nsegL = a.nseg - 1;
    const int npt = (a.P + 63) / 64;
    const int gsize = a.H * NH * npt;
    const int ngroups = (int)(gridDim.x / gsize);
    // ids i, i + 8, ... run on one XCD: give them the heads of one (batch, segment)
    const int id = blockIdx.x;
    const int full = ngroups / 8 * 8 * gsize;
    int grp, wi;
    if (id < full) {
        const int x = id % 8, k = id / 8;
        grp = x + 8 * (k / gsize);
        wi = k % gsize;
    } else {
        grp = id / gsize;
        wi = id % gsize;
    }
    const int b = grp / nsegL, seg = grp % nsegL;
    const int h = wi / (NH * npt), nb = (wi / npt) % NH, pt = wi % npt;
    const int hg = GROUPED ? h / (a.H / a.G) : h;
    const int n0 = 64 * nb, p0 = 64 * pt;
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int li = lane % 16, lk = lane / 16;
    // segments before the last: cps whole chunks of 64 steps inside the sequence
    const int q0 = seg * a.cps * kRows + wave * a.cps * 16;
    const int q1 = q0 + a.cps * 16;
    const int nblk = a.cps * 16 / SPB;
    const int NP2 = a.N / 2;

    // one batch row of each input; B rows (step) are G N (grouped) or H N apart
    const int bc_step = GROUPED ? a.G * a.N : a.H * a.N;
    const int x_step = a.H * a.P;
    const Buf bB = make_buf((const float*)a.B + (size_t)b * a.L * bc_step, (size_t)a.L * bc_step * 4);
    const Buf bX = make_buf((const float*)a.X + (size_t)b * a.L * x_step, (size_t)a.L * x_step * 4);
    const size_t so = (size_t)b * a.L * a.H + h;   // (batch, step 0, head) of the per-head inputs
    const float* ldp = a.ld + so;
    const float* btp = a.beta + so;
    const size_t nsh = (size_t)a.L * a.H;
    const Buf bL = make_buf(a.ld + (size_t)b * nsh, nsh * 4);
    const Buf bG = make_buf(a.gamma + (size_t)b * nsh, nsh * 4);
    const Buf bE = make_buf(a.beta + (size_t)b * nsh, nsh * 4);
    const Buf bT = make_buf(ROT ? a.theta + (size_t)b * nsh * NP2 : a.ld, ROT ? nsh * NP2 * 4 : 0);

    // operand layout as k_seg_state: row i of tile j is state n0 + 4 i + j
    // (so a rotation pair is tiles 2 m, 2 m + 1 of one lane), column i of tile
    // q is p0 + 4 i + q; one 16-byte load per operand and K step
    const uint32_t ob = n0 + 4 * li < a.N ? (uint32_t)(hg * a.N + n0 + 4 * li) * 4u : kOut;
    const uint32_t ox = p0 + 4 * li < a.P ? (uint32_t)(h * a.P + p0 + 4 * li) * 4u : kOut;
    const uint32_t sb = (uint32_t)bc_step * 4u, sx = (uint32_t)x_step * 4u;
    const int kk = lane % 32, hf = lane / 32;   // angle staging: pair kk of the 64 rows, steps 4 hf ..
    const int pk = n0 / 2 + kk;
    const bool pk_ok = pk < NP2;
    // pairs past N read zeros (a mask the compiler cannot turn into branches)
    const uint32_t pk_kill = opaque(pk_ok ? 0u : kOut);

    // the LDS of the final sum; during the walk its start holds each wave's
    // cos / sin tables of two blocks (4 steps x 32 pairs each)
    __shared__ __attribute__((aligned(16))) floatx4 red[4 * 12 * 64];
    __shared__ float s_S[4];
    __shared__ float s_A[ROT ? 4 * 32 : 1];
    float2* rot = (float2*)red + wave * 2 * SPB * RS;

    float vb[2][4 * KS], vx[2][4 * KS];
    float sld[2], sgm[2], sbn[2], sldn[2];   // step t0 + lane: ld, gamma; step t0 + lane + 1: beta, ld
    float sth[2][APL];                        // angles of pair pk at steps t0 + APL hf + i
    // Every load is a buffer load issued unconditionally (a block before the
    // quarter's first reads zeros: all its offsets past the buffers), in a
    // fixed order at a fixed point of the program, so the compiler's waits on
    // the memory counter never cover loads issued after the ones it needs.
    // A block's operands are loaded one block ahead of its products, its
    // per-step inputs (log-decay, gamma, the next step's beta and log-decay,
    // the angles) two blocks ahead of its staging.
    auto load_ops = [&](int slot, int kb) __attribute__((always_inline)) {
        const uint32_t kill = kb >= 0 ? 0u : kOut;
        const uint32_t tk = (uint32_t)(q0 + kb * SPB + lk);
        const uint32_t vbo = (ob + tk * sb) | kill, vxo = (ox + tk * sx) | kill;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uintx4 ub = __builtin_amdgcn_raw_buffer_load_b128(bB.r, (int)vbo, (int)(4 * ks * sb), 0);
            const uintx4 ux = __builtin_amdgcn_raw_buffer_load_b128(bX.r, (int)vxo, (int)(4 * ks * sx), 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vb[slot][4 * ks + j] = __uint_as_float(ub[j]);
                vx[slot][4 * ks + j] = __uint_as_float(ux[j]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto load_par = [&](int slot, int kb) __attribute__((always_inline)) {
        const uint32_t kill = kb >= 0 ? 0u : kOut;
        const int t0 = q0 + kb * SPB;
        const int tu = t0 + lane;
        const bool in = lane < SPB, nx = in && tu + 1 < q1;
        const uint32_t o0 = in ? ((uint32_t)(tu * a.H + h) * 4u) | kill : kOut;
        const uint32_t o1 = nx ? ((uint32_t)((tu + 1) * a.H + h) * 4u) | kill : kOut;
        __builtin_amdgcn_sched_barrier(0);
        sld[slot] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bL.r, (int)o0, 0, 0));
        sgm[slot] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bG.r, (int)o0, 0, 0));
        sldn[slot] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bL.r, (int)o1, 0, 0));
        sbn[slot] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bE.r, (int)o1, 0, 0));
        if constexpr (ROT) {
#pragma unroll
            for (int i = 0; i < APL; ++i) {
                const uint32_t ot = ((uint32_t)(((t0 + APL * hf + i) * a.H + h) * NP2 + pk) * 4u) | kill | pk_kill;
                sth[slot][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bT.r, (int)ot, 0, 0));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[j][q] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    float S = 0.0f;      // log-decay of the quarter's steps after the current block
    float arev = 0.0f;   // angle of pair pk over those steps, revolutions mod 1
    // B's operands of this lane's two state pairs (tiles 0, 1 and 2, 3) turned
    // by the pairs' angles: cs = (cos, sin, cos, sin)
    auto turn = [&](float* v, float4 cs) __attribute__((always_inline)) {
        const float b0 = v[0], b1 = v[1], b2 = v[2], b3 = v[3];
        v[0] = fmaf(cs.y, b1, cs.x * b0);
        v[1] = fmaf(-cs.y, b0, cs.x * b1);
        v[2] = fmaf(cs.w, b3, cs.z * b2);
        v[3] = fmaf(-cs.w, b2, cs.z * b3);
    };
    // Staging of a block (its weights, and the cos / sin of its steps and
    // pairs into table slot `slot`) and its products are separate, so a block
    // is staged right after the products of the block before it are issued.
    float wl[2];
    auto stage = [&](int slot) __attribute__((always_inline)) {
        const float cum = wave_scan_dpp(sld[slot]);   // lanes past the block add zero
        const float T = readlane_f(cum, 63);
        const float D = S + (T - cum);                 // after step t0 + lane
        wl[slot] = sgm[slot] * exp_e(D) + sbn[slot] * exp_e(D - sldn[slot]);
        S += T;
        if constexpr (ROT) {
            // suffix sums over this lane's steps (revolutions), then the other half's total
            float suf[APL], ht = 0.0f;
#pragma unroll
            for (int i = APL - 1; i >= 0; --i) {
                suf[i] = ht;
                ht += sth[slot][i] * kInv2Pi;
            }
            const float other = __shfl_xor(ht, 32, 64);
            const float base = arev + (hf == 0 ? other : 0.0f);
#pragma unroll
            for (int i = 0; i < APL; ++i) {
                float r = base + suf[i];
                r -= rintf(r);
                rot[(slot * SPB + APL * hf + i) * RS + kk] =
                    make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
            }
            arev += ht + other;
            arev -= rintf(arev);
        }
    };
    auto mult = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float w = __shfl(wl[slot], 4 * ks + lk, 64);
            float bh[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bh[j] = vb[slot][4 * ks + j];
            if constexpr (ROT) turn(bh, *(const float4*)&rot[(slot * SPB + 4 * ks + lk) * RS + 2 * li]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float xw = vx[slot][4 * ks + q] * w;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j][q] = mfma4(bh[j], xw, acc[j][q]);
            }
        }
    };
    // blocks from the quarter's last to its first (register and table slots
    // alternate)
    // (blocks before the first read zeros: their staging leaves S and the
    // angle unchanged)
    int kb = nblk - 1;
    load_ops(0, kb);
    load_par(0, kb);
    load_par(1, kb - 1);
    stage(0);
    load_par(0, kb - 2);
    for (; kb >= 1; kb -= 2) {
        load_ops(1, kb - 1);
        mult(0);
        stage(1);
        load_par(1, kb - 3);
        load_ops(0, kb - 2);
        mult(1);
        stage(0);
        load_par(0, kb - 4);
    }
    if (kb == 0) mult(0);

    // the step before the quarter (before the call's first step: the given
    // previous token, or zeros), on lane group 0 of one more K step
    {
        const int tp = q0 - 1;
        const bool given = tp < 0 && a.B_prev != nullptr;
        const Buf bBp = make_buf(given ? (const float*)a.B_prev + (size_t)b * bc_step : (const float*)a.B,
                                 given ? (size_t)bc_step * 4 : 0);
        const Buf bXp = make_buf(given ? (const float*)a.X_prev + (size_t)b * x_step : (const float*)a.X,
                                 given ? (size_t)x_step * 4 : 0);
        float pb[4], px[4];
        {
            const bool on = lk == 0;
            const uint32_t offb = on ? (tp >= 0 ? ob + (uint32_t)tp * sb : ob) : kOut;
            const uint32_t offx = on ? (tp >= 0 ? ox + (uint32_t)tp * sx : ox) : kOut;
            const uintx4 ub = __builtin_amdgcn_raw_buffer_load_b128(tp >= 0 ? bB.r : bBp.r, (int)offb, 0, 0);
            const uintx4 ux = __builtin_amdgcn_raw_buffer_load_b128(tp >= 0 ? bX.r : bXp.r, (int)offx, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pb[j] = __uint_as_float(ub[j]);
                px[j] = __uint_as_float(ux[j]);
            }
        }
        const float wp = btp[(size_t)q0 * a.H] * exp_e(S - ldp[(size_t)q0 * a.H]);
        if constexpr (ROT) {
            // the quarter's total angle of this lane's pairs 2 li, 2 li + 1, from
            // their staging lanes
            const float r0 = __shfl(arev, 2 * li, 64), r1 = __shfl(arev, 2 * li + 1, 64);
            turn(pb, make_float4(__builtin_amdgcn_cosf(r0), __builtin_amdgcn_sinf(r0), __builtin_amdgcn_cosf(r1),
                                 __builtin_amdgcn_sinf(r1)));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float xw = px[q] * wp;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j][q] = mfma4(pb[j], xw, acc[j][q]);
        }
    }

    // the later quarters' totals carry this block to the segment's end
    if (lane == 0) s_S[wave] = S;
    if constexpr (ROT) if (lane < 32) s_A[wave * 32 + lane] = arev;
    __syncthreads();
    float Sl = 0.0f;
    for (int k = 3; k > wave; --k) Sl += s_S[k];
    const float dS = exp_e(Sl);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            // tile rows 4 lk + r of tiles 2 m, 2 m + 1: states n0 + 16 lk + 4 r + 2 m,
            // + 1, pair 8 lk + 2 r + m of the block
            float cs = 1.0f, sn = 0.0f;
            if constexpr (ROT) {
                float rv = 0.0f;
                for (int k = 3; k > wave; --k) rv += s_A[k * 32 + 8 * lk + 2 * r + m];
                rv -= rintf(rv);
                cs = __builtin_amdgcn_cosf(rv);
                sn = __builtin_amdgcn_sinf(rv);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float v0 = acc[2 * m][q][r], v1 = acc[2 * m + 1][q][r];
                acc[2 * m][q][r] = dS * fmaf(sn, v1, cs * v0);
                acc[2 * m + 1][q][r] = dS * fmaf(-sn, v0, cs * v1);
            }
        }
    }
    // sum the quarters (as k_seg_state)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j == wave) continue;
        const int base = wave * 12 + 4 * (j < wave ? j : j - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) red[(base + q) * 64 + lane] = acc[j][q];
    }
    __syncthreads();
    const size_t u = (size_t)(b * a.H + h) * nsegL + seg;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j != wave) continue;
        floatx4 s[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s[q] = acc[j][q];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (v != j) s[q] += red[(v * 12 + 4 * (j < v ? j : j - 1) + q) * 64 + lane];
        }
        // tile row 4 lk + r is state n0 + 16 lk + 4 r + j; columns p0 + 4 li + q
        const int p = p0 + 4 * li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = n0 + 16 * lk + 4 * r + j;
            if (n < a.N && p < a.P)
                *(float4*)&a.seg_h[(u * a.N + n) * a.P + p] = make_float4(s[0][r], s[1][r], s[2][r], s[3][r]);
        }
    }
    if (pt == 0 && wave == 0) {
        if (nb == 0 && lane == 0) a.seg_ld[u] = S + Sl;
        if constexpr (ROT) if (lane < 32 && pk_ok) {
            float r = 0.0f;
            for (int k = 3; k >= 0; --k) r += s_A[k * 32 + lane];
            a.seg_rev[u * NP2 + pk] = r - rintf(r);
        }
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Plan {
    int64_t nch, nseg, cps, npg;
    size_t off_bt, off_seg_h, off_seg_ld, off_seg_rev, bytes;
};

inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Chunks, segments and workspace for a problem (depends on the sizes and the
// current device's compute-unit count only, so mb_workspace_size agrees with a
// call on the same device).
Plan make_plan(bool trap, int64_t R, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G,
               int64_t N) {
    Plan p{};
    const int64_t QT = kRows / R;
    p.nch = (L + QT - 1) / QT;
    p.npg = (P + kPG - 1) / kPG;
    const int64_t units = batch * H * p.npg;
    // Segment count: minimise an estimate of the walk time on the device's
    // compute units, with one full-pass workgroup and two state-only workgroups
    // per unit, a state-only chunk costing about 0.45 of a full one and every
    // workgroup a start-up of about two chunks (both fitted to a sweep of the
    // segment count on MI355X); at least 4 chunks per segment.
    const int64_t cus = device_cu_count();
    int64_t best = 1;
    double best_cost = -1.0;
    for (int64_t ns = 1; ns <= 64; ++ns) {
        if (ns > 1 && p.nch / ns < 4) break;
        const int64_t cps = p.nch > 0 ? (p.nch + ns - 1) / ns : 1;
        const int64_t nse = p.nch > 0 ? (p.nch + cps - 1) / cps : 1;
        const double full_rounds = (double)((nse * units + cus - 1) / cus);
        const double so_rounds = (double)(((nse - 1) * units + 2 * cus - 1) / (2 * cus));
        const double cost = (full_rounds + 0.45 * so_rounds) * (double)(cps + 2);
        if (best_cost < 0.0 || cost < best_cost - 1e-9) {
            best_cost = cost;
            best = ns;
        }
    }
    p.cps = p.nch > 0 ? (p.nch + best - 1) / best : 1;
    p.nseg = p.nch > 0 ? (p.nch + p.cps - 1) / p.cps : 1;
    size_t off = 0;
    if (!trap) {
        // Mamba-2: scores, then the transposed B that the bf16 walk reads
        off = align256((size_t)(batch * p.nch * G) * kRows * kRows * 4);
        p.off_bt = off;
        off += align256((size_t)(batch * p.nch * G) * (N <= 64 ? 64 : 128) * kRows * 2);
    }
    p.off_seg_h = off;
    const size_t nsg = (size_t)(batch * H * (p.nseg - 1));
    off += align256(nsg * (size_t)(N * P) * 4);
    p.off_seg_ld = off;
    off += align256(nsg * 4);
    p.off_seg_rev = off;
    if (trap) off += align256(nsg * (size_t)(N / 2) * 4);
    p.bytes = (p.nseg > 1 || !trap) ? off : 0;
    return p;
}

template <int NP, int R, bool TRAP, bool ROT, bool GROUPED, typename IO>
mb_status launch(Args a, int64_t batch, const Plan& pl, char* ws, hipStream_t stream) {
    a.nch = (int)pl.nch;
    a.nseg = (int)pl.nseg;
    a.cps = (int)pl.cps;
    a.npg = (int)pl.npg;
    a.S = TRAP ? nullptr : (float*)ws;
    a.BT = TRAP ? nullptr : (bf16*)(ws + pl.off_bt);
    a.seg_h = (float*)(ws + pl.off_seg_h);
    a.seg_ld = (float*)(ws + pl.off_seg_ld);
    a.seg_rev = (float*)(ws + pl.off_seg_rev);
    if constexpr (!TRAP) {
        hipLaunchKernelGGL((k_scores<NP, IO>), dim3(a.nch, a.G, (unsigned)batch), dim3(kThreads), 0,
                           stream, a);
        mb_status st = check_launch();
        if (st != MB_OK) return st;
    }
    const int64_t per_seg = batch * a.H * a.npg;
    if constexpr (!TRAP && !ROT && sizeof(IO) == 2) {
        // bf16 inputs: the walk on the bf16 matrix instruction (16-byte copies of
        // C rows need N to be a multiple of 8)
        if (a.N % 8 == 0) {
            if (a.nseg > 1) {
                hipLaunchKernelGGL((k_walk_bf<NP>), dim3((unsigned)(per_seg * (a.nseg - 1))),
                                   dim3(kBfThreads), 0, stream, a);
                mb_status st = check_launch();
                if (st != MB_OK) return st;
            }
            if (a.Dh || a.Zg)
                hipLaunchKernelGGL((k_walk_bfs<NP, true>), dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads),
                                   0, stream, a);
            else
                hipLaunchKernelGGL((k_walk_bfs<NP>), dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads),
                                   0, stream, a);
            return check_launch();
        }
    }
    if (a.nseg > 1) {
        const dim3 g((unsigned)(per_seg * (a.nseg - 1)));
        if constexpr (!TRAP && !ROT && sizeof(IO) == 4) {
            // Mamba-2 with fp32 inputs: the segment states as plain products
            const int64_t nwg = batch * a.H * (NP / 64) * ((a.P + 63) / 64) * (a.nseg - 1);
            hipLaunchKernelGGL((k_seg_state<NP>), dim3((unsigned)nwg), dim3(kSegThreads), 0, stream, a);
        } else if constexpr (TRAP && R == 1 && sizeof(IO) == 4) {
            if (!a.bcn) {
                // SISO with fp32 inputs: the segment states as plain products
                const int64_t nwg = batch * a.H * (NP / 64) * ((a.P + 63) / 64) * (a.nseg - 1);
                hipLaunchKernelGGL((k_seg_trap<NP, GROUPED, ROT>), dim3((unsigned)nwg), dim3(kSegThreads), 0,
                                   stream, a);
            } else {
                hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, true, false, true>), g,
                                   dim3(kWalkThreads), 0, stream, a);
            }
        } else if constexpr (TRAP && (R == 1 || !GROUPED)) {
            if (a.bcn)
                hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, true, false, true>), g,
                                   dim3(kWalkThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, true>), g, dim3(kWalkThreads), 0,
                                   stream, a);
        } else {
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, true>), g, dim3(kWalkThreads), 0, stream,
                               a);
        }
        mb_status st = check_launch();
        if (st != MB_OK) return st;
    }
    if constexpr (!TRAP && !ROT && sizeof(IO) == 4) {
        if (a.Dh || a.Zg)
            hipLaunchKernelGGL((k_walk_m2s<NP, true>), dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((k_walk_m2s<NP>), dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads), 0,
                               stream, a);
    } else if constexpr (!TRAP && !ROT) {
        // bf16 Mamba-2 with N not a multiple of 8: the general walk
        if (a.Dh || a.Zg)
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false, true>),
                               dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false>),
                               dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads), 0, stream, a);
    }
    else if constexpr (R == 1 && TRAP) {
        const dim3 g((unsigned)(per_seg * a.nseg));
        const bool epi = a.Dh || a.Zg;
        if (a.bcn && epi)
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false, true, true>), g, dim3(kWalkThreads),
                               0, stream, a);
        else if (a.bcn)
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false, false, true>), g, dim3(kWalkThreads),
                               0, stream, a);
        else if (epi)
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false, true>),
                               dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false>),
                               dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads), 0, stream, a);
    } else if constexpr (TRAP && !GROUPED) {
        // MIMO with both ends of its block (the prologue always, the epilogue
        // when D or z is given)
        const dim3 g((unsigned)(per_seg * a.nseg));
        const bool epi = a.Dh || a.Zg;
        if (a.bcn && epi)
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false, true, true>), g, dim3(kWalkThreads),
                               0, stream, a);
        else if (a.bcn)
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false, false, true>), g, dim3(kWalkThreads),
                               0, stream, a);
        else
            hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false>), g, dim3(kWalkThreads), 0, stream, a);
    } else
        hipLaunchKernelGGL((k_walk<NP, R, TRAP, ROT, GROUPED, IO, false>),
                           dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads), 0, stream, a);
    return check_launch();
}

// The Mamba-2 layer around its scan: k_scores convolves B and C and computes
// dt' and the log-decay, then the walks convolve x themselves.
template <int NP, typename IO>
mb_status launch_block(Args a, int64_t batch, const Plan& pl, char* ws, hipStream_t stream) {
    a.nch = (int)pl.nch;
    a.nseg = (int)pl.nseg;
    a.cps = (int)pl.cps;
    a.npg = (int)pl.npg;
    a.S = (float*)ws;
    a.BT = (bf16*)(ws + pl.off_bt);
    a.seg_h = (float*)(ws + pl.off_seg_h);
    a.seg_ld = (float*)(ws + pl.off_seg_ld);
    a.seg_rev = (float*)(ws + pl.off_seg_rev);
    const int64_t per_seg = batch * a.H * a.npg;
    mb_status st;
    static_assert(sizeof(IO) == 4, "the one-pass layer is the fp32 path");
    {
        hipLaunchKernelGGL((k_scores<NP, IO, true>), dim3(a.nch, a.G, (unsigned)batch), dim3(kThreads), 0, stream, a);
        if ((st = check_launch()) != MB_OK) return st;
        if (a.nseg > 1) {
            hipLaunchKernelGGL((k_walk<NP, 1, false, false, true, float, true, false, false, true>),
                               dim3((unsigned)(per_seg * (a.nseg - 1))), dim3(kWalkThreads), 0, stream, a);
            if ((st = check_launch()) != MB_OK) return st;
        }
        hipLaunchKernelGGL((k_walk_m2s<NP, true, true>), dim3((unsigned)(per_seg * a.nseg)), dim3(kWalkThreads), 0,
                           stream, a);
    }
    return check_launch();
}

// workspace of the Mamba-2 layer: the SSD's, then the convolved B and C, dt'
// and the log-decay; bf16 (run as two passes) also X
struct BlockWs {
    size_t off_b, off_c, off_dtp, off_ld, off_x, bytes;
};
BlockWs block_ws(const Plan& pl, bool bf, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G,
                 int64_t N) {
    BlockWs w{};
    const size_t es = bf ? 2 : 4;
    size_t off = pl.bytes;
    w.off_b = off;
    off += align256((size_t)(batch * L * G * N) * es);
    w.off_c = off;
    off += align256((size_t)(batch * L * G * N) * es);
    w.off_dtp = off;
    off += align256((size_t)(batch * L * H) * 4);
    w.off_ld = off;
    off += align256((size_t)(batch * L * H) * 4);
    w.off_x = off;
    if (bf) off += align256((size_t)(batch * L * H * P) * es);
    w.bytes = off;
    return w;
}

template <int R, bool TRAP, bool ROT, bool GROUPED, typename IO>
mb_status launch_np(Args a, int64_t batch, const Plan& pl, char* ws, hipStream_t stream) {
    if (a.N <= 64) return launch<64, R, TRAP, ROT, GROUPED, IO>(a, batch, pl, ws, stream);
    return launch<128, R, TRAP, ROT, GROUPED, IO>(a, batch, pl, ws, stream);
}

template <int R, bool TRAP, bool GROUPED>
mb_status dispatch(Args a, int64_t batch, const Plan& pl, char* ws, mb_dtype dtype, hipStream_t stream) {
    const bool rot = a.theta != nullptr;
    if constexpr (!TRAP) {
        return dtype == MB_F32 ? launch_np<R, false, false, GROUPED, float>(a, batch, pl, ws, stream)
                               : launch_np<R, false, false, GROUPED, bf16>(a, batch, pl, ws, stream);
    }
    if (dtype == MB_F32)
        return rot ? launch_np<R, TRAP, true, GROUPED, float>(a, batch, pl, ws, stream)
                   : launch_np<R, TRAP, false, GROUPED, float>(a, batch, pl, ws, stream);
    return rot ? launch_np<R, TRAP, true, GROUPED, bf16>(a, batch, pl, ws, stream)
               : launch_np<R, TRAP, false, GROUPED, bf16>(a, batch, pl, ws, stream);
}

bool dims_ok(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R = 1) {
    if (batch < 0 || L < 0 || H < 1 || P < 1 || N < 1) return false;
    if (N > kNMax || N % 4 != 0 || P % 16 != 0) return false;
    if (batch > 65535 || H > 65535 || L > INT32_MAX / 2) return false;
    // one batch row of any tensor is addressed with 32-bit byte offsets
    const int64_t row = L * H * (P > N ? P : N) * R * 4;
    if (row >= (int64_t)1 << 31) return false;
    return true;
}

// Mamba-2 only: one batch row of the score workspace (a 64 x 64 fp32 block per
// chunk and group) is read through a buffer resource with 32-bit byte offsets.
bool m2_scores_ok(int64_t L, int64_t G) {
    const int64_t nch = (L + kRows - 1) / kRows;
    return nch * G * (int64_t)(kRows * kRows * 4) < ((int64_t)1 << 31);
}

Plan plan_for(mb_op op, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
              int64_t R) {
    return make_plan(op != MB_OP_SSD_CHUNKED, op == MB_OP_MIMO_SSD ? R : 1, batch, L, H, P,
                     op == MB_OP_SSD_CHUNKED ? G : H, N);
}

// Device scratch of the allocation-free Mamba-2 entry point: file-scope, one
// copy per device, alive until the process ends.  Host code never uses the
// array's name as an address: scratch_ptr() takes the device address of the
// current device's copy from the runtime, once per device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

mb_status scratch_ptr(char** out) {
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void* ptr[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_last_hip_error((int)e);
        return MB_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDev) return MB_ERR_HIP;
    std::lock_guard<std::mutex> lk(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_last_hip_error((int)e);
            return MB_ERR_HIP;
        }
        ptr[dev] = p;
    }
    *out = (char*)ptr[dev];
    return MB_OK;
}

mb_status check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return MB_OK;
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255)) return MB_ERR_WORKSPACE;
    return MB_OK;
}

// Mamba-2 shapes outside the tiles of the walks (P not a multiple of 16, N not
// a multiple of 4; e.g. P = 1, the Mamba-1 -> Mamba-2 reduction) run on the
// same kernels through zero-padded copies in the workspace: X, Y and z padded
// to P' columns, B and C to N' states, the state to N' x P'.  The added state
// rows see B = 0 and start at 0, the added columns see X = 0, and C = 0 on the
// added rows, so they add exact zeros to every sum and the result is that of
// the unpadded recurrence.
int64_t pad_p(int64_t P) { return (P + 15) / 16 * 16; }
int64_t pad_n(int64_t N) { return (N + 3) / 4 * 4; }
bool needs_pad(int64_t P, int64_t N) { return P % 16 != 0 || N % 4 != 0; }

// (rows, n_small, p_small) <-> (rows, n_big, p_big) copies of E-sized
// elements; PAD widens with zeros, !PAD takes the leading block back
template <typename E, bool PAD>
__global__ __launch_bounds__(256) void k_pad(const E* __restrict__ src, E* __restrict__ dst, int64_t rows,
                                             int n_small, int p_small, int n_big, int p_big) {
    const int64_t total = rows * (PAD ? (int64_t)n_big * p_big : (int64_t)n_small * p_small);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        if constexpr (PAD) {
            const int j = (int)(i % p_big);
            const int64_t q = i / p_big;
            const int k = (int)(q % n_big);
            const int64_t r = q / n_big;
            dst[i] = (j < p_small && k < n_small) ? src[(r * n_small + k) * p_small + j] : (E)0;
        } else {
            const int j = (int)(i % p_small);
            const int64_t q = i / p_small;
            const int k = (int)(q % n_small);
            const int64_t r = q / n_small;
            dst[i] = src[(r * n_big + k) * p_big + j];
        }
    }
}

mb_status pad_copy(bool pad, const void* src, void* dst, size_t es, int64_t rows, int64_t n_small, int64_t p_small,
                   int64_t n_big, int64_t p_big, hipStream_t stream) {
    const int64_t total = rows * (pad ? n_big * p_big : n_small * p_small);
    if (total == 0) return MB_OK;
    const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
    const int ns = (int)n_small, ps = (int)p_small, nb = (int)n_big, pb = (int)p_big;
    if (es == 2) {
        if (pad)
            hipLaunchKernelGGL((k_pad<uint16_t, true>), dim3(grid), dim3(256), 0, stream, (const uint16_t*)src,
                               (uint16_t*)dst, rows, ns, ps, nb, pb);
        else
            hipLaunchKernelGGL((k_pad<uint16_t, false>), dim3(grid), dim3(256), 0, stream, (const uint16_t*)src,
                               (uint16_t*)dst, rows, ns, ps, nb, pb);
    } else {
        if (pad)
            hipLaunchKernelGGL((k_pad<uint32_t, true>), dim3(grid), dim3(256), 0, stream, (const uint32_t*)src,
                               (uint32_t*)dst, rows, ns, ps, nb, pb);
        else
            hipLaunchKernelGGL((k_pad<uint32_t, false>), dim3(grid), dim3(256), 0, stream, (const uint32_t*)src,
                               (uint32_t*)dst, rows, ns, ps, nb, pb);
    }
    return check_launch();
}

// workspace of the Mamba-2 SSD: the plan's (at the padded sizes), then, for
// padded shapes, X, Y and z (P' columns), B and C (N' states) and one state;
// sized for 4-byte elements whatever the dtype
struct SsdWs {
    Plan pl;
    int64_t P2, N2;
    size_t off_x, off_y, off_z, off_b, off_c, off_h, bytes;
};
SsdWs ssd_ws(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N) {
    SsdWs w{};
    const bool pad = needs_pad(P, N);
    w.P2 = pad ? pad_p(P) : P;
    w.N2 = pad ? pad_n(N) : N;
    w.pl = plan_for(MB_OP_SSD_CHUNKED, batch, L, H, w.P2, G, w.N2, 1);
    size_t off = w.pl.bytes;
    if (pad) {
        const size_t nx = align256((size_t)(batch * L * H * w.P2) * 4);
        const size_t nbc = align256((size_t)(batch * L * G * w.N2) * 4);
        w.off_x = off;
        off += nx;
        w.off_y = off;
        off += nx;
        w.off_z = off;
        off += nx;
        w.off_b = off;
        off += nbc;
        w.off_c = off;
        off += nbc;
        w.off_h = off;
        off += align256((size_t)(batch * H * w.N2 * w.P2) * 4);
    }
    w.bytes = off;
    return w;
}

// the Mamba-2 SSD (with the output side when Dskip or z is given), after the
// caller's checks; batch > 0, L > 0
mb_status ssd_run(const void* X, const float* logdecay, const void* B, const void* C, const float* h0,
                  const float* Dskip, const void* z, void* Y, float* h_out, int64_t batch, int64_t L, int64_t H,
                  int64_t P, int64_t G, int64_t N, mb_dtype dtype, char* ws, size_t ws_bytes, hipStream_t stream) {
    const SsdWs w = ssd_ws(batch, L, H, P, G, N);
    mb_status st;
    if ((st = check_ws(ws, ws_bytes, w.bytes)) != MB_OK) return st;
    if (!needs_pad(P, N)) {
        Args a{X, logdecay, B, C, nullptr, nullptr, nullptr, h0, nullptr, nullptr, Y, h_out, nullptr,
               nullptr, nullptr, nullptr, nullptr, (int)L, (int)H, (int)P, (int)G, (int)N, 0, 0, 0, 0, Dskip, z};
        return dispatch<1, false, true>(a, batch, w.pl, ws, dtype, stream);
    }
    const size_t es = dtype_size(dtype);
    const int64_t P2 = w.P2, N2 = w.N2;
    void* Xp = ws + w.off_x;
    void* Yp = ws + w.off_y;
    void* zp = z ? (void*)(ws + w.off_z) : nullptr;
    const void* Bp = B;
    const void* Cp = C;
    float* hs = (float*)(ws + w.off_h);
    if ((st = pad_copy(true, X, Xp, es, batch * L * H, 1, P, 1, P2, stream)) != MB_OK) return st;
    if (z && (st = pad_copy(true, z, zp, es, batch * L * H, 1, P, 1, P2, stream)) != MB_OK) return st;
    if (N2 != N) {
        if ((st = pad_copy(true, B, ws + w.off_b, es, batch * L * G, 1, N, 1, N2, stream)) != MB_OK) return st;
        if ((st = pad_copy(true, C, ws + w.off_c, es, batch * L * G, 1, N, 1, N2, stream)) != MB_OK) return st;
        Bp = ws + w.off_b;
        Cp = ws + w.off_c;
    }
    if (h0 && (st = pad_copy(true, h0, hs, 4, batch * H, N, P, N2, P2, stream)) != MB_OK) return st;
    // one padded state serves as h0 and h_out (the walks allow them equal)
    Args a{Xp, logdecay, Bp, Cp, nullptr, nullptr, nullptr, h0 ? hs : nullptr, nullptr, nullptr, Yp,
           h_out ? hs : nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, (int)L, (int)H, (int)P2, (int)G,
           (int)N2, 0, 0, 0, 0, Dskip, zp};
    if ((st = dispatch<1, false, true>(a, batch, w.pl, ws, dtype, stream)) != MB_OK) return st;
    if ((st = pad_copy(false, Yp, Y, es, batch * L * H, 1, P, 1, P2, stream)) != MB_OK) return st;
    if (h_out) return pad_copy(false, hs, h_out, 4, batch * H, N, P, N2, P2, stream);
    return MB_OK;
}

}  // namespace
}  // namespace mb

using namespace mb;

extern "C" size_t mb_workspace_size(mb_op op, int64_t batch, int64_t L, int64_t H, int64_t P,
                                    int64_t G, int64_t N, int64_t R, int64_t chunk) {
    (void)chunk;
    if (op == MB_OP_SSM_STEP) return 0;
    // Mamba-1 scan: the sizes (batch, L, D, N) travel as (batch, L, H, N)
    if (op == MB_OP_SELECTIVE_SCAN) return m1_scan_workspace(batch, L, H, N);
    if (op == MB_OP_SSD_CHUNKED_BWD) return ssd_bwd_workspace(batch, L, H, P, G, N);
    if (op == MB_OP_TRAP_SSD_BWD) return trap_bwd_workspace(batch, L, H, P, G, N);
    if (op == MB_OP_MIMO_SSD_BWD) return mimo_bwd_workspace(batch, L, H, P, N, R);
    // Mamba-1 backward: the sizes (batch, L, D, N) travel as (batch, L, H, N)
    if (op == MB_OP_SELECTIVE_SCAN_BWD) return m1_bwd_workspace(batch, L, H, N);
    if (op == MB_OP_SSD_CHUNKED) {
        if (P < 1 || N < 1 || !dims_ok(batch, L, H, pad_p(P), pad_n(N))) return 0;
        if (G < 1 || H % G || !m2_scores_ok(L, G) || batch == 0 || L == 0) return 0;
        return ssd_ws(batch, L, H, P, G, N).bytes;
    }
    if (!dims_ok(batch, L, H, P, N)) return 0;
    const bool blk = op == MB_OP_SSD_BLOCK || op == MB_OP_SSD_BLOCK_BF16;
    if (blk && (G < 1 || H % G || !m2_scores_ok(L, G))) return 0;
    if (blk) {
        if (batch == 0 || L == 0) return 0;
        const Plan pl = plan_for(MB_OP_SSD_CHUNKED, batch, L, H, P, G, N, 1);
        return block_ws(pl, op == MB_OP_SSD_BLOCK_BF16, batch, L, H, P, G, N).bytes;
    }
    if (op == MB_OP_MIMO_SSD && R != 1 && R != 2 && R != 4 && R != 8 && R != 16) return 0;
    if (batch == 0 || L == 0) return 0;
    return plan_for(op, batch, L, H, P, G, N, R).bytes;
}

static mb_status ssd_common_checks(const void* X, const float* logdecay, const void* B,
                                   const void* C, const float* h0, void* Y, float* h_out,
                                   const float* beta, const float* gamma, const float* theta,
                                   const void* X_prev, const void* B_prev,
                                   int64_t batch, int64_t L, int64_t H, int64_t P, int64_t nBC,
                                   int64_t N, int64_t R, mb_dtype dtype, int64_t chunk,
                                   bool trap, bool pad = false) {
    if (!dtype_ok(dtype)) return MB_ERR_DTYPE;
    if (pad ? (P < 1 || N < 1 || !dims_ok(batch, L, H, pad_p(P), pad_n(N), R)) : !dims_ok(batch, L, H, P, N, R))
        return MB_ERR_SHAPE;
    if (chunk != 0 && chunk != kRows) return MB_ERR_SHAPE;
    if (theta && (N % 2)) return MB_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const size_t n_x = (size_t)(batch * L * H * P * R);
    const size_t n_bc = (size_t)(batch * L * nBC * N * R);
    const size_t n_s = (size_t)(batch * L * H);
    const size_t n_h = (size_t)(batch * H * N * P);
    if (n_x && (!X || !Y || !logdecay || !B || !C)) return MB_ERR_NULL;
    if ((X_prev == nullptr) != (B_prev == nullptr)) return MB_ERR_NULL;
    if (((uintptr_t)X | (uintptr_t)Y | (uintptr_t)B | (uintptr_t)C | (uintptr_t)X_prev |
         (uintptr_t)B_prev) & 15)
        return MB_ERR_ALIGN;
    if (trap && n_x && (!beta || !gamma)) return MB_ERR_NULL;
    const size_t n_xp = (size_t)(batch * H * P * R), n_bp = (size_t)(batch * nBC * N * R);
    const Span ins[] = {{X, n_x * es}, {B, n_bc * es}, {C, n_bc * es}, {logdecay, n_s * 4},
                        {beta, trap && beta ? n_s * 4 : 0}, {gamma, trap && gamma ? n_s * 4 : 0},
                        {theta, theta ? n_s * (size_t)(N / 2) * 4 : 0},
                        {X_prev, X_prev ? n_xp * es : 0}, {B_prev, B_prev ? n_bp * es : 0},
                        {h0, h0 ? n_h * 4 : 0}};
    if (overlaps_any(Y, n_x * es, ins, 10)) return MB_ERR_ALIAS;
    if (h_out) {
        if (overlaps_any(h_out, n_h * 4, ins, 9)) return MB_ERR_ALIAS;
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
    if (!m2_scores_ok(L, G)) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, batch, L, H, P, G, N, 1, dtype, chunk, false, true);
    if (st != MB_OK) return st;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    return ssd_run(X, logdecay, B, C, h0, nullptr, nullptr, Y, h_out, batch, L, H, P, G, N, dtype, (char*)ws,
                   ws_bytes, stream);
}

extern "C" mb_status mb_ssd_chunked_gated(const void* X, const float* logdecay, const void* B,
                                          const void* C, const float* h0, const float* Dskip, const void* z,
                                          void* Y, float* h_out, int64_t batch, int64_t L, int64_t H,
                                          int64_t P, int64_t G, int64_t N, int64_t chunk, mb_dtype dtype,
                                          void* ws, size_t ws_bytes, hipStream_t stream) {
    if (G < 1 || H < 1 || H % G) return MB_ERR_SHAPE;
    if (!m2_scores_ok(L, G)) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, batch, L, H, P, G, N, 1, dtype, chunk, false, true);
    if (st != MB_OK) return st;
    if (((uintptr_t)z & 15) || ((uintptr_t)Dskip & 3)) return MB_ERR_ALIGN;
    const size_t ny = (size_t)(batch * L * H * P) * dtype_size(dtype);
    if (overlaps(Y, ny, z, z ? ny : 0) || overlaps(Y, ny, Dskip, Dskip ? (size_t)H * 4 : 0)) return MB_ERR_ALIAS;
    if (h_out && (overlaps(h_out, (size_t)(batch * H * N * P) * 4, z, z ? ny : 0) ||
                  overlaps(h_out, (size_t)(batch * H * N * P) * 4, Dskip, Dskip ? (size_t)H * 4 : 0)))
        return MB_ERR_ALIAS;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    return ssd_run(X, logdecay, B, C, h0, Dskip, z, Y, h_out, batch, L, H, P, G, N, dtype, (char*)ws, ws_bytes,
                   stream);
}

extern "C" mb_status mb_ssd_block(const void* xBC, const float* conv_w, const float* conv_b,
                                  const void* x_hist, const float* dt, const float* dt_bias,
                                  const float* A, const float* Dskip, const void* z, const float* h0,
                                  void* Y, float* h_out, int64_t batch, int64_t L, int64_t H, int64_t P,
                                  int64_t G, int64_t N, int64_t K, mb_dtype dtype, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return MB_ERR_DTYPE;
    if (G < 1 || H < 1 || H % G || K < 1 || K > 4) return MB_ERR_SHAPE;
    if (!dims_ok(batch, L, H, P, N) || !m2_scores_ok(L, G)) return MB_ERR_SHAPE;
    if (dtype == MB_BF16 && N % 8) return MB_ERR_SHAPE;
    const int64_t cin = H * P + 2 * G * N;
    if ((L + 64) * cin * 4 >= ((int64_t)1 << 31)) return MB_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const size_t n_in = (size_t)(batch * L * cin), n_y = (size_t)(batch * L * H * P);
    const size_t n_s = (size_t)(batch * L * H), n_h = (size_t)(batch * H * N * P);
    if (n_y && (!xBC || !conv_w || !dt || !A || !Y)) return MB_ERR_NULL;
    if (((uintptr_t)Y | (uintptr_t)z | (uintptr_t)xBC | (uintptr_t)x_hist) & 15) return MB_ERR_ALIGN;
    if (((uintptr_t)conv_w | (uintptr_t)conv_b | (uintptr_t)dt | (uintptr_t)dt_bias | (uintptr_t)A |
         (uintptr_t)Dskip | (uintptr_t)h0 | (uintptr_t)h_out) & 3)
        return MB_ERR_ALIGN;
    const Span ins[] = {{xBC, n_in * es}, {conv_w, (size_t)(cin * K) * 4}, {conv_b, conv_b ? (size_t)cin * 4 : 0},
                        {x_hist, x_hist ? (size_t)(batch * (K - 1) * cin) * es : 0}, {dt, n_s * 4},
                        {dt_bias, dt_bias ? (size_t)H * 4 : 0}, {A, (size_t)H * 4},
                        {Dskip, Dskip ? (size_t)H * 4 : 0}, {z, z ? n_y * es : 0}, {h0, h0 ? n_h * 4 : 0}};
    if (overlaps_any(Y, n_y * es, ins, 10)) return MB_ERR_ALIAS;
    if (h_out) {
        if (overlaps_any(h_out, n_h * 4, ins, 9)) return MB_ERR_ALIAS;
        if (h0 && h0 != h_out && overlaps(h_out, n_h * 4, h0, n_h * 4)) return MB_ERR_ALIAS;
        if (overlaps(h_out, n_h * 4, Y, n_y * es)) return MB_ERR_ALIAS;
    }
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    const Plan pl = plan_for(MB_OP_SSD_CHUNKED, batch, L, H, P, G, N, 1);
    const BlockWs bw = block_ws(pl, dtype == MB_BF16, batch, L, H, P, G, N);
    mb_status st;
    if ((st = check_ws(ws, ws_bytes, bw.bytes)) != MB_OK) return st;
    if (overlaps_any(ws, bw.bytes, ins, 10) || overlaps(ws, bw.bytes, Y, n_y * es) ||
        (h_out && overlaps(ws, bw.bytes, h_out, n_h * 4)))
        return MB_ERR_ALIAS;
    char* w = (char*)ws;
    if (dtype == MB_BF16) {
        // bf16 as two passes, measured faster at the Mamba-2 block shape (0.19
        // against 0.26 ms): the bf16 walk is bound by latency per chunk, and
        // building X inside it costs more than the round trip of X.  The prologue
        // pass writes X, B, C, the log-decay and dt' into the workspace; the SSD runs
        // on them with the output side, its skip term on x = X / dt'.
        st = mb_ssd_prologue(xBC, conv_w, conv_b, x_hist, dt, dt_bias, A, w + bw.off_x, w + bw.off_b,
                             w + bw.off_c, (float*)(w + bw.off_ld), (float*)(w + bw.off_dtp), batch, L, H, P, G,
                             N, K, dtype, stream);
        if (st != MB_OK) return st;
        Args a2{w + bw.off_x, (const float*)(w + bw.off_ld), w + bw.off_b, w + bw.off_c, nullptr, nullptr,
                nullptr, h0, nullptr, nullptr, Y, h_out, nullptr, nullptr, nullptr, nullptr, nullptr, (int)L,
                (int)H, (int)P, (int)G, (int)N, 0, 0, 0, 0, Dskip, z};
        a2.skip_dt = (const float*)(w + bw.off_dtp);
        return dispatch<1, false, true>(a2, batch, pl, w, dtype, stream);
    }
    Args a{};
    a.X = xBC;
    a.ld = (const float*)(w + bw.off_ld);
    a.B = w + bw.off_b;
    a.C = w + bw.off_c;
    a.h0 = h0;
    a.Y = Y;
    a.h_out = h_out;
    a.L = (int)L; a.H = (int)H; a.P = (int)P; a.G = (int)G; a.N = (int)N;
    a.Dh = Dskip;
    a.Zg = z;
    a.eps = 0.0f;
    a.Xr = xBC;
    a.cw = conv_w;
    a.cbias = conv_b;
    a.xh = K > 1 ? x_hist : nullptr;
    a.dtr = dt;
    a.dtbias = dt_bias;
    a.Ah = A;
    a.dtp = (float*)(w + bw.off_dtp);
    a.Bw = w + bw.off_b;
    a.Cw = w + bw.off_c;
    a.cin = (int)cin;
    a.K = (int)K;
    a.pro = 1;
    return N <= 64 ? launch_block<64, float>(a, batch, pl, w, stream) : launch_block<128, float>(a, batch, pl, w, stream);
}

extern "C" mb_status mb_ssd_chunked_noalloc(const void* X, const float* logdecay, const void* B,
                                            const void* C, const float* h0, void* Y, float* h_out,
                                            int64_t batch, int64_t L, int64_t H, int64_t P,
                                            int64_t G, int64_t N, int64_t chunk, mb_dtype dtype,
                                            hipStream_t stream) {
    if (G < 1 || H < 1 || H % G) return MB_ERR_SHAPE;
    if (!m2_scores_ok(L, G)) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, nullptr, nullptr, nullptr,
                                     nullptr, nullptr, batch, L, H, P, G, N, 1, dtype, chunk, false, true);
    if (st != MB_OK) return st;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    if (ssd_ws(batch, L, H, P, G, N).bytes > kScratchBytes) return MB_ERR_WORKSPACE;
    char* ws = nullptr;
    if ((st = scratch_ptr(&ws)) != MB_OK) return st;
    return ssd_run(X, logdecay, B, C, h0, nullptr, nullptr, Y, h_out, batch, L, H, P, G, N, dtype, ws,
                   kScratchBytes, stream);
}

extern "C" mb_status mb_trap_ssd(const void* X, const float* logdecay, const void* B,
                                 const void* C, const float* beta, const float* gamma,
                                 const float* theta, const float* h0, const void* X_prev,
                                 const void* B_prev, void* Y, float* h_out, int64_t batch,
                                 int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                                 int64_t chunk, mb_dtype dtype, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    if (G < 1 || H < 1 || H % G) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, beta, gamma, theta, X_prev,
                                     B_prev, batch, L, H, P, G, N, 1, dtype, chunk, true);
    if (st != MB_OK) return st;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    const Plan pl = plan_for(MB_OP_TRAP_SSD, batch, L, H, P, G, N, 1);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != MB_OK) return st;
    Args a{X, logdecay, B, C, beta, gamma, theta, h0, X_prev, B_prev, Y, h_out, nullptr, nullptr,
           nullptr, nullptr, nullptr, (int)L, (int)H, (int)P, (int)G, (int)N, 0, 0, 0, 0};
    return dispatch<1, true, true>(a, batch, pl, (char*)ws, dtype, stream);
}

extern "C" mb_status mb_trap_ssd_gated(const void* X, const float* logdecay, const void* B,
                                       const void* C, const float* beta, const float* gamma,
                                       const float* theta, const float* h0, const void* X_prev,
                                       const void* B_prev, const float* Dskip, const void* z, void* Y,
                                       float* h_out, int64_t batch, int64_t L, int64_t H, int64_t P,
                                       int64_t G, int64_t N, int64_t chunk, mb_dtype dtype, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
    if (G < 1 || H < 1 || H % G) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, beta, gamma, theta, X_prev,
                                     B_prev, batch, L, H, P, G, N, 1, dtype, chunk, true);
    if (st != MB_OK) return st;
    if (((uintptr_t)z & 15) || ((uintptr_t)Dskip & 3)) return MB_ERR_ALIGN;
    const size_t ny = (size_t)(batch * L * H * P) * dtype_size(dtype);
    if (overlaps(Y, ny, z, z ? ny : 0) || overlaps(Y, ny, Dskip, Dskip ? (size_t)H * 4 : 0)) return MB_ERR_ALIAS;
    if (h_out && (overlaps(h_out, (size_t)(batch * H * N * P) * 4, z, z ? ny : 0) ||
                  overlaps(h_out, (size_t)(batch * H * N * P) * 4, Dskip, Dskip ? (size_t)H * 4 : 0)))
        return MB_ERR_ALIAS;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    const Plan pl = plan_for(MB_OP_TRAP_SSD, batch, L, H, P, G, N, 1);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != MB_OK) return st;
    Args a{X, logdecay, B, C, beta, gamma, theta, h0, X_prev, B_prev, Y, h_out, nullptr, nullptr,
           nullptr, nullptr, nullptr, (int)L, (int)H, (int)P, (int)G, (int)N, 0, 0, 0, 0, Dskip, z};
    return dispatch<1, true, true>(a, batch, pl, (char*)ws, dtype, stream);
}

extern "C" mb_status mb_trap_ssd_block(const void* X, const float* logdecay, const void* B,
                                       const void* C, const float* beta, const float* gamma,
                                       const float* theta, const float* h0, const void* X_prev,
                                       const void* B_prev, const float* normB_w, const float* normC_w,
                                       const float* biasB, const float* biasC, float eps,
                                       const float* Dskip, const void* z, void* Y, float* h_out,
                                       int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G,
                                       int64_t N, int64_t chunk, mb_dtype dtype, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
    if (G < 1 || H < 1 || H % G) return MB_ERR_SHAPE;
    if (!(eps > 0.0f) || !(eps < 3.0e38f)) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, beta, gamma, theta, X_prev,
                                     B_prev, batch, L, H, P, G, N, 1, dtype, chunk, true);
    if (st != MB_OK) return st;
    const float* pars[6] = {normB_w, normC_w, biasB, biasC, Dskip, nullptr};
    const size_t pbytes[6] = {(size_t)N * 4, (size_t)N * 4, (size_t)(H * N) * 4, (size_t)(H * N) * 4,
                              (size_t)H * 4, 0};
    if ((uintptr_t)z & 15) return MB_ERR_ALIGN;
    const size_t ny = (size_t)(batch * L * H * P) * dtype_size(dtype);
    const size_t nh = (size_t)(batch * H * N * P) * 4;
    if (overlaps(Y, ny, z, z ? ny : 0) || (h_out && overlaps(h_out, nh, z, z ? ny : 0))) return MB_ERR_ALIAS;
    for (int k = 0; k < 5; ++k) {
        if ((uintptr_t)pars[k] & 3) return MB_ERR_ALIGN;
        const size_t nb = pars[k] ? pbytes[k] : 0;
        if (overlaps(Y, ny, pars[k], nb) || (h_out && overlaps(h_out, nh, pars[k], nb))) return MB_ERR_ALIAS;
    }
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    const Plan pl = plan_for(MB_OP_TRAP_SSD, batch, L, H, P, G, N, 1);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != MB_OK) return st;
    Args a{X, logdecay, B, C, beta, gamma, theta, h0, X_prev, B_prev, Y, h_out, nullptr, nullptr,
           nullptr, nullptr, nullptr, (int)L, (int)H, (int)P, (int)G, (int)N, 0, 0, 0, 0, Dskip, z,
           normB_w, normC_w, biasB, biasC, eps, 1};
    return dispatch<1, true, true>(a, batch, pl, (char*)ws, dtype, stream);
}

extern "C" mb_status mb_mimo_ssd_block(const void* X, const float* logdecay, const void* B,
                                       const void* C, const float* beta, const float* gamma,
                                       const float* theta, const float* h0, const void* X_prev,
                                       const void* B_prev, const float* normB_w, const float* normC_w,
                                       const float* biasB, const float* biasC, float eps,
                                       const float* Dskip, const void* z, void* Y, float* h_out,
                                       int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                       int64_t R, int64_t chunk, mb_dtype dtype, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
    if (R != 1 && R != 2 && R != 4 && R != 8 && R != 16) return MB_ERR_SHAPE;
    if (!(eps > 0.0f) || !(eps < 3.0e38f)) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, beta, gamma, theta, X_prev,
                                     B_prev, batch, L, H, P, H, N, R, dtype, chunk, true);
    if (st != MB_OK) return st;
    const float* pars[5] = {normB_w, normC_w, biasB, biasC, Dskip};
    const size_t pbytes[5] = {(size_t)N * 4, (size_t)N * 4, (size_t)(H * N) * 4, (size_t)(H * N) * 4,
                              (size_t)H * 4};
    if ((uintptr_t)z & 15) return MB_ERR_ALIGN;
    const size_t ny = (size_t)(batch * L * H * P * R) * dtype_size(dtype);
    const size_t nh = (size_t)(batch * H * N * P) * 4;
    if (overlaps(Y, ny, z, z ? ny : 0) || (h_out && overlaps(h_out, nh, z, z ? ny : 0))) return MB_ERR_ALIAS;
    for (int k = 0; k < 5; ++k) {
        if ((uintptr_t)pars[k] & 3) return MB_ERR_ALIGN;
        const size_t nb = pars[k] ? pbytes[k] : 0;
        if (overlaps(Y, ny, pars[k], nb) || (h_out && overlaps(h_out, nh, pars[k], nb))) return MB_ERR_ALIAS;
    }
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    const Plan pl = plan_for(MB_OP_MIMO_SSD, batch, L, H, P, 1, N, R);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != MB_OK) return st;
    Args a{X, logdecay, B, C, beta, gamma, theta, h0, X_prev, B_prev, Y, h_out, nullptr, nullptr,
           nullptr, nullptr, nullptr, (int)L, (int)H, (int)P, (int)H, (int)N, 0, 0, 0, 0, Dskip, z,
           normB_w, normC_w, biasB, biasC, eps, 1};
    switch (R) {
        case 1: return dispatch<1, true, false>(a, batch, pl, (char*)ws, dtype, stream);
        case 2: return dispatch<2, true, false>(a, batch, pl, (char*)ws, dtype, stream);
        case 4: return dispatch<4, true, false>(a, batch, pl, (char*)ws, dtype, stream);
        case 8: return dispatch<8, true, false>(a, batch, pl, (char*)ws, dtype, stream);
        default: return dispatch<16, true, false>(a, batch, pl, (char*)ws, dtype, stream);
    }
}

extern "C" mb_status mb_mimo_ssd(const void* X, const float* logdecay, const void* B,
                                 const void* C, const float* beta, const float* gamma,
                                 const float* theta, const float* h0, const void* X_prev,
                                 const void* B_prev, void* Y, float* h_out, int64_t batch,
                                 int64_t L, int64_t H, int64_t P, int64_t N, int64_t R,
                                 int64_t chunk, mb_dtype dtype, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    if (R != 1 && R != 2 && R != 4 && R != 8 && R != 16) return MB_ERR_SHAPE;
    mb_status st = ssd_common_checks(X, logdecay, B, C, h0, Y, h_out, beta, gamma, theta, X_prev,
                                     B_prev, batch, L, H, P, H, N, R, dtype, chunk, true);
    if (st != MB_OK) return st;
    if (batch == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, batch * H * N * P, stream);
    const Plan pl = plan_for(MB_OP_MIMO_SSD, batch, L, H, P, 1, N, R);
    if ((st = check_ws(ws, ws_bytes, pl.bytes)) != MB_OK) return st;
    Args a{X, logdecay, B, C, beta, gamma, theta, h0, X_prev, B_prev, Y, h_out, nullptr, nullptr,
           nullptr, nullptr, nullptr, (int)L, (int)H, (int)P, (int)H, (int)N, 0, 0, 0, 0};
    char* w = (char*)ws;
    switch (R) {
        case 1: return dispatch<1, true, false>(a, batch, pl, w, dtype, stream);
        case 2: return dispatch<2, true, false>(a, batch, pl, w, dtype, stream);
        case 4: return dispatch<4, true, false>(a, batch, pl, w, dtype, stream);
        case 8: return dispatch<8, true, false>(a, batch, pl, w, dtype, stream);
        default: return dispatch<16, true, false>(a, batch, pl, w, dtype, stream);
    }
}
