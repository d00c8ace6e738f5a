// ssd_bwd.hip -- backward of the Mamba-2 scalar-decay SSD (fp32) for gfx950.
//
// The forward recurrence (TorchMamba README, Math notes M2), per batch b and
// head h with group g:
//     h_t = e^{ld_t} h_{t-1} + B_t X_t^T      (N x P),   Y_t = h_t^T C_t.
// Its vector-Jacobian product for dY and dh_out (back-propagation through time,
// the training mode listed on the mamba-rs page) is computed chunkwise.  A chunk
// holds Q = 64 steps; cum_j is the chunk-local inclusive sum of ld, Lam = cum_63.
// With Hc the state entering chunk c and Gc the adjoint of the state at its end
// (the gradient arriving from every later step and dh_out):
//     H_{c+1} = e^{Lam_c} H_c + U_c,     U_c = sum_j e^{Lam - cum_j} B_j X_j^T
//     G_{c-1} = e^{Lam_c} G_c + V_c,     V_c = sum_j e^{cum_j} C_j dY_j^T
// with H_0 = h0, G_last = dh_out and dh0 = G_{-1}.  Inside a chunk, with the
// causal decay mask W[i][j] = e^{cum_i - cum_j} [j <= i]:
//     dC = (dY X^T o W) B + diag(e^{cum}) dY H^T
//     dX = (C B^T o W)^T dY + diag(e^{Lam - cum}) B G
//     dB = (dY X^T o W)^T C + diag(e^{Lam - cum}) X G^T
// (dB and dC summed over the heads of a group).  The log-decay gradient follows
// from the same quantities: with dl_t = C_t . dC_t - X_t . dX_t (per head),
//     dlogdecay_t = sum_{tau >= t} dl_tau + <dh_out, h_out>,
// since <G_t, h_t> telescopes along the sequence.
//
// Kernels
//   k_bwd_local  (batch, chunk, group), heads in turn: U_c, V_c and Lam_c on
//                fp32 MFMA into the workspace.
//   k_bwd_pass   one thread per (batch, head, state element): the two chunk
//                recurrences, elementwise, in place (U_c -> H_c, V_c -> G_c), dh0,
//                and the partial sums of <dh_out, h_out>.
//   k_bwd_grad   (batch, chunk, group), heads in turn: dX, the suffix sums of
//                dl inside the chunk and the chunk's total, and dB, dC
//                accumulated over the group's heads, on fp32 MFMA.
//   k_bwd_ld     one wave per (batch, head, chunk): adds the later chunks' totals
//                and <dh_out, h_out>.
#include "mb_internal.h"

namespace mb {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;          // steps per chunk
constexpr int kBwdThreads = 256;
constexpr int kLQ = kQ + 4;     // LDS row stride of the 64 x 64 score tiles

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp_e(float v) { return exp2_fast(v * kLog2e); }

struct BwdArgs {
    const float* X;         // (batch, L, H, P)
    const float* ld;        // (batch, L, H)
    const float* B;         // (batch, L, G, N)
    const float* C;
    const float* h0;        // (batch, H, N, P) or NULL
    const float* dY;        // (batch, L, H, P)
    const float* dh_out;    // (batch, H, N, P) or NULL
    float* dX;
    float* dld;             // (batch, L, H)
    float* dB;              // (batch, L, G, N)
    float* dC;
    float* dh0;             // (batch, H, N, P) or NULL
    float* st;              // workspace: per (b, h, c) two N x P slots (H_c, G_c)
    float* lam;             // workspace: per (b, h, c) total log-decay of the chunk
    float* tot;             // workspace: per (b, h, c) the sum of dl over the chunk
    float* fin;             // workspace: per (b, h) partial sums of <dh_out, h_out>
    float* h_final;         // optional output: (batch, H, N, P) the final state
    int L, H, G, N, P, nch, nfin;
};

// Row stride (floats) of an LDS array of rows `w` wide: w + 4, so that rows
// four apart fall sixteen banks apart (column reads of four rows per lane group).
template <int W>
struct Ld {
    static constexpr int v = W + 4;
};

// Rows t0 .. t0 + 63 of a tensor with rows of W floats (row pitch `pitch`),
// held in registers between a load and an LDS store: float4 f = tid + T k of
// the 64 x W / 4, rows at or past L read as zero.  Loading one head's rows
// while the previous head computes hides the global latency.
template <int W, int T>
struct RowPref {
    static constexpr int V = W / 4;
    static constexpr int F = (kQ * V + T - 1) / T;
    float4 v[F];
    __device__ __forceinline__ void load(const float* src, size_t pitch, int t0, int L) {
#pragma unroll
        for (int k = 0; k < F; ++k) {
            const int f = threadIdx.x + T * k;
            const int j = f / V, v4 = f % V;
            v[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (f < kQ * V && t0 + j < L) v[k] = *(const float4*)(src + (size_t)(t0 + j) * pitch + 4 * v4);
        }
    }
    // to LDS rows of stride LDW, each row scaled by scale[j] when given
    __device__ __forceinline__ void store(float* dst, int LDW, const float* scale) const {
#pragma unroll
        for (int k = 0; k < F; ++k) {
            const int f = threadIdx.x + T * k;
            if (f >= kQ * V) continue;
            const int j = f / V, v4 = f % V;
            float4 x = v[k];
            if (scale) {
                const float s = scale[j];
                x.x *= s; x.y *= s; x.z *= s; x.w *= s;
            }
            *(float4*)(dst + j * LDW + 4 * v4) = x;
        }
    }
};

// Chunk-local cumulative log-decay by one wave from its lanes' log-decays (lane
// j: step t0 + j): s_cum[j], e^{Lam - cum_j} (s_we), e^{cum_j} (s_ws); returns Lam.
__device__ __forceinline__ float chunk_weights(float v, float* s_cum, float* s_we, float* s_ws) {
    const int lane = threadIdx.x % 64;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    const float lam = __shfl(v, 63, 64);
    if (s_cum) s_cum[lane] = v;
    s_we[lane] = exp_e(lam - v);
    s_ws[lane] = exp_e(v);
    return lam;
}

constexpr int kMma = 512;   // threads of the two matrix kernels: 8 waves, two per SIMD

// ---------------------------------------------------------------------------
// k_bwd_local: U_c = B^T diag(e^{Lam - cum}) X and V_c = C^T diag(e^{cum}) dY for
// every head of the group, and Lam_c.  Wave w owns the state row blocks
// w, w + 8, ... (16 rows each) of both, for all P columns.
// ---------------------------------------------------------------------------
template <int NN, int PP>
__global__ __launch_bounds__(kMma) void k_bwd_local(BwdArgs a) {
    constexpr int LB = Ld<NN>::v, LX = Ld<PP>::v;
    constexpr int NB = NN / 16, PB = PP / 16;
    constexpr int NBW = (NB + 7) / 8;        // row blocks per wave
    __shared__ __attribute__((aligned(16))) float sB[kQ * LB];
    __shared__ __attribute__((aligned(16))) float sC[kQ * LB];
    __shared__ __attribute__((aligned(16))) float sX[kQ * LX];
    __shared__ __attribute__((aligned(16))) float sD[kQ * LX];
    __shared__ float s_we[kQ], s_ws[kQ];

    const int g = blockIdx.x % a.G;
    const int c = (blockIdx.x / a.G) % a.nch;
    const int b = blockIdx.x / (a.G * a.nch);
    const int t0 = c * kQ;
    const int hpg = a.H / a.G;
    const int lane = threadIdx.x % 64, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int li = lane % 16, q = lane / 16;
    const size_t bc_pitch = (size_t)a.G * NN, x_pitch = (size_t)a.H * PP;
    const size_t NP = (size_t)NN * PP;
    {
        RowPref<NN, kMma> r;
        r.load(a.B + ((size_t)b * a.L * a.G + g) * NN, bc_pitch, t0, a.L);
        r.store(sB, LB, nullptr);
        r.load(a.C + ((size_t)b * a.L * a.G + g) * NN, bc_pitch, t0, a.L);
        r.store(sC, LB, nullptr);
    }
    RowPref<PP, kMma> px, pd;
    float ldv = 0.0f;
    auto prefetch = [&](int h) {
        px.load(a.X + ((size_t)b * a.L * a.H + h) * PP, x_pitch, t0, a.L);
        pd.load(a.dY + ((size_t)b * a.L * a.H + h) * PP, x_pitch, t0, a.L);
        if (wave == 0) ldv = t0 + lane < a.L ? a.ld[((size_t)b * a.L + t0 + lane) * a.H + h] : 0.0f;
    };
    prefetch(g * hpg);

    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        if (wave == 0) {
            const float lam = chunk_weights(ldv, nullptr, s_we, s_ws);
            if (lane == 0) a.lam[((size_t)b * a.H + h) * a.nch + c] = lam;
        }
        __syncthreads();   // weights ready; the previous head's reads of sX / sD done
        px.store(sX, LX, s_we);
        pd.store(sD, LX, s_ws);
        __syncthreads();
        if (hh + 1 < hpg) prefetch(h + 1);

        floatx4 accu[NBW][PB], accv[NBW][PB];
#pragma unroll
        for (int m = 0; m < NBW; ++m)
#pragma unroll
            for (int pb = 0; pb < PB; ++pb) {
                accu[m][pb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                accv[m][pb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
        for (int kg = 0; kg < kQ / 16; ++kg) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int j = 16 * kg + 4 * q + s;     // the step this lane supplies
                float xb[PB], db[PB];
#pragma unroll
                for (int pb = 0; pb < PB; ++pb) {
                    xb[pb] = sX[j * LX + 16 * pb + li];
                    db[pb] = sD[j * LX + 16 * pb + li];
                }
#pragma unroll
                for (int m = 0; m < NBW; ++m) {
                    const int nb = wave + 8 * m;
                    if (nb >= NB) continue;
                    const float bv = sB[j * LB + 16 * nb + li];
                    const float cv = sC[j * LB + 16 * nb + li];
#pragma unroll
                    for (int pb = 0; pb < PB; ++pb) {
                        accu[m][pb] = mfma4(bv, xb[pb], accu[m][pb]);
                        accv[m][pb] = mfma4(cv, db[pb], accv[m][pb]);
                    }
                }
            }
        }
        float* slot = a.st + (((size_t)b * a.H + h) * a.nch + c) * 2 * NP;
#pragma unroll
        for (int m = 0; m < NBW; ++m) {
            const int nb = wave + 8 * m;
            if (nb >= NB) continue;
#pragma unroll
            for (int pb = 0; pb < PB; ++pb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const size_t e = (size_t)(16 * nb + 4 * q + r) * PP + 16 * pb + li;
                    slot[e] = accu[m][pb][r];
                    slot[NP + e] = accv[m][pb][r];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// k_bwd_pass: the chunk recurrences, elementwise.  Thread e of (b, h) holds
// the four state elements 4 e .. 4 e + 3 (n P + p order).  Forward: slot 0 of
// chunk c becomes H_c (read U_c first); reverse: slot 1 becomes G_c.  Eight
// chunks are loaded ahead of their use.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads) void k_bwd_pass(BwdArgs a) {
    const int bh = blockIdx.y;
    const size_t NP = (size_t)a.N * a.P;
    const int e = blockIdx.x * kBwdThreads + threadIdx.x;
    const bool ok = 4 * (size_t)e < NP;
    const size_t ee = ok ? 4 * (size_t)e : 0;
    float* base = a.st + (size_t)bh * a.nch * 2 * NP;
    const float* lam = a.lam + (size_t)bh * a.nch;
    constexpr int KU = 8;
    const float4 z4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

    float4 hs = (ok && a.h0) ? *(const float4*)(a.h0 + (size_t)bh * NP + ee) : z4;
    for (int c0 = 0; c0 < a.nch; c0 += KU) {
        float4 u[KU];
        float d[KU];
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int c = c0 + k;
            u[k] = (ok && c < a.nch) ? *(const float4*)(base + (size_t)c * 2 * NP + ee) : z4;
            d[k] = c < a.nch ? exp_e(lam[c]) : 1.0f;
        }
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int c = c0 + k;
            if (ok && c < a.nch) *(float4*)(base + (size_t)c * 2 * NP + ee) = hs;
            hs.x = fmaf(d[k], hs.x, u[k].x);
            hs.y = fmaf(d[k], hs.y, u[k].y);
            hs.z = fmaf(d[k], hs.z, u[k].z);
            hs.w = fmaf(d[k], hs.w, u[k].w);
        }
    }
    if (ok && a.h_final) *(float4*)(a.h_final + (size_t)bh * NP + ee) = hs;
    const float4 dh = (ok && a.dh_out) ? *(const float4*)(a.dh_out + (size_t)bh * NP + ee) : z4;
    // partial sum of <dh_out, h_out> over this block
    {
        float v = (dh.x * hs.x + dh.y * hs.y) + (dh.z * hs.z + dh.w * hs.w);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        __shared__ float s_part[kBwdThreads / 64];
        if (threadIdx.x % 64 == 0) s_part[threadIdx.x / 64] = v;
        __syncthreads();
        if (threadIdx.x == 0)
            a.fin[(size_t)bh * a.nfin + blockIdx.x] = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
    }
    float4 gs = dh;
    for (int c1 = a.nch - 1; c1 >= 0; c1 -= KU) {
        float4 v[KU];
        float d[KU];
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int c = c1 - k;
            v[k] = (ok && c >= 0) ? *(const float4*)(base + ((size_t)c * 2 + 1) * NP + ee) : z4;
            d[k] = c >= 0 ? exp_e(lam[c]) : 1.0f;
        }
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int c = c1 - k;
            if (ok && c >= 0) *(float4*)(base + ((size_t)c * 2 + 1) * NP + ee) = gs;
            gs.x = fmaf(d[k], gs.x, v[k].x);
            gs.y = fmaf(d[k], gs.y, v[k].y);
            gs.z = fmaf(d[k], gs.z, v[k].z);
            gs.w = fmaf(d[k], gs.w, v[k].w);
        }
    }
    if (ok && a.dh0) *(float4*)(a.dh0 + (size_t)bh * NP + ee) = gs;
}

// ---------------------------------------------------------------------------
// k_bwd_grad: per chunk and group, heads in turn.  Waves w and w + 4 own the 16
// steps 16 w .. 16 w + 15 of the chunk for every output (dC, dX, dB rows), each
// for half of the output columns, so the causal parts balance across row
// blocks: dC sums over the earlier steps, dX and dB over the later ones.
//   once per chunk:  S = C B^T (lower block triangle) -> sS
//   per head:        W2 = (dY X^T) o W -> sW;  M = S o W -> sM
//                    dC_h = diag(e^{cum}) dY H^T + W2 B
//                    dX   = diag(e^{Lam - cum}) B G + M^T dY      (stored)
//                    dB  += diag(e^{Lam - cum}) X G^T + W2^T C
//                    dl   = rows of C . dC_h - X . dX              (stored)
//                    dC  += dC_h
// MFMA operands whose contraction index runs along an LDS row are read four at
// a time; the others (contraction down a column) one row each.  The next
// head's X, dY and log-decay load into registers during the products.
// ---------------------------------------------------------------------------
template <int NN, int PP>
__global__ __launch_bounds__(kMma) void k_bwd_grad(BwdArgs a) {
    constexpr int LB = Ld<NN>::v, LX = Ld<PP>::v;
    constexpr int NB = NN / 16, PB = PP / 16;
    constexpr int NBH = NB / 2, PBH = PB / 2;    // column tiles per half
    static_assert(NB % 2 == 0 && PB % 2 == 0, "column tiles split in halves");
    __shared__ __attribute__((aligned(16))) float sB[kQ * LB];
    __shared__ __attribute__((aligned(16))) float sC[kQ * LB];
    __shared__ __attribute__((aligned(16))) float sX[kQ * LX];
    __shared__ __attribute__((aligned(16))) float sD[kQ * LX];
    __shared__ __attribute__((aligned(16))) float sS[kQ * kLQ];
    __shared__ __attribute__((aligned(16))) float sW[kQ * kLQ];
    __shared__ __attribute__((aligned(16))) float sM[kQ * kLQ];
    __shared__ float s_cum[kQ], s_we[kQ], s_ws[kQ], s_dl[2][kQ];

    const int g = blockIdx.x % a.G;
    const int c = (blockIdx.x / a.G) % a.nch;
    const int b = blockIdx.x / (a.G * a.nch);
    const int t0 = c * kQ;
    const int hpg = a.H / a.G;
    const int lane = threadIdx.x % 64, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int rb = wave & 3, half = wave >> 2;
    const int li = lane % 16, q = lane / 16;
    const size_t bc_pitch = (size_t)a.G * NN, x_pitch = (size_t)a.H * PP;
    const size_t NP = (size_t)NN * PP;
    const int jrow = 16 * rb + 4 * q;            // first of the four rows of this lane's accumulators
    const int nb0 = half * NBH, pb0 = half * PBH;

    {
        RowPref<NN, kMma> r;
        r.load(a.B + ((size_t)b * a.L * a.G + g) * NN, bc_pitch, t0, a.L);
        r.store(sB, LB, nullptr);
        r.load(a.C + ((size_t)b * a.L * a.G + g) * NN, bc_pitch, t0, a.L);
        r.store(sC, LB, nullptr);
    }
    RowPref<PP, kMma> px, pd;
    float ldv = 0.0f;
    auto prefetch = [&](int h) {
        px.load(a.X + ((size_t)b * a.L * a.H + h) * PP, x_pitch, t0, a.L);
        pd.load(a.dY + ((size_t)b * a.L * a.H + h) * PP, x_pitch, t0, a.L);
        if (wave == 0) ldv = t0 + lane < a.L ? a.ld[((size_t)b * a.L + t0 + lane) * a.H + h] : 0.0f;
    };
    prefetch(g * hpg);
    __syncthreads();
    // S = C B^T, tiles (rb, jb <= rb), alternate tiles to the two halves
    for (int jb = half; jb <= rb; jb += 2) {
        floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kg = 0; kg < NB; ++kg) {
            const float4 av = *(const float4*)(sC + (16 * rb + li) * LB + 16 * kg + 4 * q);
            const float4 bv = *(const float4*)(sB + (16 * jb + li) * LB + 16 * kg + 4 * q);
            acc = mfma4(av.x, bv.x, acc);
            acc = mfma4(av.y, bv.y, acc);
            acc = mfma4(av.z, bv.z, acc);
            acc = mfma4(av.w, bv.w, acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[(jrow + r) * kLQ + 16 * jb + li] = acc[r];
    }

    floatx4 dBs[NBH], dCs[NBH];
#pragma unroll
    for (int k = 0; k < NBH; ++k) {
        dBs[k] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        dCs[k] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // by wave 0: the two halves' partial dl of a head's rows summed, the suffix
    // sums inside the chunk stored as dlogdecay (k_bwd_ld adds the rest) and the
    // chunk's total kept (lane l takes row 63 - l: a prefix over lanes is a
    // suffix over steps)
    auto store_dl = [&](int h) {
        const int j = 63 - lane, t = t0 + j;
        float v = t < a.L ? s_dl[0][j] + s_dl[1][j] : 0.0f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float u = __shfl_up(v, d, 64);
            if (lane >= d) v += u;
        }
        if (t < a.L) a.dld[((size_t)b * a.L + t) * a.H + h] = v;
        if (lane == 63) a.tot[((size_t)b * a.H + h) * a.nch + c] = v;
    };

    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        __syncthreads();   // A: the previous head's reads of sX, sD, sW, sM, weights done
        if (wave == 0) {
            if (hh > 0) store_dl(h - 1);
            chunk_weights(ldv, s_cum, s_we, s_ws);
        }
        px.store(sX, LX, nullptr);
        pd.store(sD, LX, nullptr);
        __syncthreads();   // B
        if (hh + 1 < hpg) prefetch(h + 1);

        // ---- W2 = (dY X^T) o W and M = S o W, tiles (rb, jb <= rb) ----------------
        float cum_r[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) cum_r[r] = s_cum[jrow + r];
        for (int jb = half; jb <= rb; jb += 2) {
            floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kg = 0; kg < PB; ++kg) {
                const float4 av = *(const float4*)(sD + (16 * rb + li) * LX + 16 * kg + 4 * q);
                const float4 bv = *(const float4*)(sX + (16 * jb + li) * LX + 16 * kg + 4 * q);
                acc = mfma4(av.x, bv.x, acc);
                acc = mfma4(av.y, bv.y, acc);
                acc = mfma4(av.z, bv.z, acc);
                acc = mfma4(av.w, bv.w, acc);
            }
            const int jc = 16 * jb + li;
            const float cj = s_cum[jc];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = jrow + r;
                const float w = jc <= i ? exp_e(cum_r[r] - cj) : 0.0f;
                sW[i * kLQ + jc] = acc[r] * w;
                sM[i * kLQ + jc] = sS[i * kLQ + jc] * w;
            }
        }
        __syncthreads();   // C

        const float* Hs = a.st + (((size_t)b * a.H + h) * a.nch + c) * 2 * NP;
        const float* Gs = Hs + NP;
        float we_r[4], ws_r[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            we_r[r] = s_we[jrow + r];
            ws_r[r] = s_ws[jrow + r];
        }

        // ---- dC_h = diag(e^{cum}) dY H^T + W2 B ------------------------------------
        floatx4 dCh[NBH];
#pragma unroll
        for (int k = 0; k < NBH; ++k) {
            const int nb = nb0 + k;
            floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kg = 0; kg < PB; ++kg) {
                const float4 av = *(const float4*)(sD + (16 * rb + li) * LX + 16 * kg + 4 * q);
                const float4 bv = *(const float4*)(Hs + (size_t)(16 * nb + li) * PP + 16 * kg + 4 * q);
                acc = mfma4(av.x, bv.x, acc);
                acc = mfma4(av.y, bv.y, acc);
                acc = mfma4(av.z, bv.z, acc);
                acc = mfma4(av.w, bv.w, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= ws_r[r];
            dCh[k] = acc;
        }
        for (int kg = 0; kg <= rb; ++kg) {
            const float4 av = *(const float4*)(sW + (16 * rb + li) * kLQ + 16 * kg + 4 * q);
            const float avs[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = 16 * kg + 4 * q + s;
#pragma unroll
                for (int k = 0; k < NBH; ++k) dCh[k] = mfma4(avs[s], sB[i * LB + 16 * (nb0 + k) + li], dCh[k]);
            }
        }

        // ---- dX = diag(e^{Lam - cum}) B G + M^T dY ---------------------------------
        floatx4 dXa[PBH];
#pragma unroll
        for (int k = 0; k < PBH; ++k) {
            const int pb = pb0 + k;
            floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kg = 0; kg < NB; ++kg) {
                // G is read down its columns: four rows of 16 consecutive columns
                // per instruction
                const float4 av = *(const float4*)(sB + (16 * rb + li) * LB + 16 * kg + 4 * q);
                const float* gc = Gs + (size_t)(16 * kg + 4 * q) * PP + 16 * pb + li;
                acc = mfma4(av.x, gc[0], acc);
                acc = mfma4(av.y, gc[PP], acc);
                acc = mfma4(av.z, gc[2 * PP], acc);
                acc = mfma4(av.w, gc[3 * PP], acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= we_r[r];
            dXa[k] = acc;
        }
        for (int kg = rb; kg < 4; ++kg) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = 16 * kg + 4 * q + s;
                const float mv = sM[i * kLQ + 16 * rb + li];
#pragma unroll
                for (int k = 0; k < PBH; ++k) dXa[k] = mfma4(mv, sD[i * LX + 16 * (pb0 + k) + li], dXa[k]);
            }
        }

        // ---- dB += diag(e^{Lam - cum}) X G^T + W2^T C --------------------------------
        {
            floatx4 dBh[NBH];
#pragma unroll
            for (int k = 0; k < NBH; ++k) {
                const int nb = nb0 + k;
                floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kg = 0; kg < PB; ++kg) {
                    const float4 av = *(const float4*)(sX + (16 * rb + li) * LX + 16 * kg + 4 * q);
                    const float4 bv = *(const float4*)(Gs + (size_t)(16 * nb + li) * PP + 16 * kg + 4 * q);
                    acc = mfma4(av.x, bv.x, acc);
                    acc = mfma4(av.y, bv.y, acc);
                    acc = mfma4(av.z, bv.z, acc);
                    acc = mfma4(av.w, bv.w, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= we_r[r];
                dBh[k] = acc;
            }
            for (int kg = rb; kg < 4; ++kg) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int i = 16 * kg + 4 * q + s;
                    const float wv = sW[i * kLQ + 16 * rb + li];
#pragma unroll
                    for (int k = 0; k < NBH; ++k) dBh[k] = mfma4(wv, sC[i * LB + 16 * (nb0 + k) + li], dBh[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < NBH; ++k) dBs[k] += dBh[k];
        }

        // ---- partial dl = C . dC_h - X . dX over this half's columns; store dX -------
        float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < NBH; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[r] = fmaf(sC[(jrow + r) * LB + 16 * (nb0 + k) + li], dCh[k][r], part[r]);
#pragma unroll
        for (int k = 0; k < PBH; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[r] = fmaf(-sX[(jrow + r) * LX + 16 * (pb0 + k) + li], dXa[k][r], part[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) part[r] += __shfl_xor(part[r], off, 16);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = t0 + jrow + r;
            if (li == 0) s_dl[half][jrow + r] = part[r];
            if (t < a.L) {
                float* dxr = a.dX + (((size_t)b * a.L + t) * a.H + h) * PP;
#pragma unroll
                for (int k = 0; k < PBH; ++k) dxr[16 * (pb0 + k) + li] = dXa[k][r];
            }
        }
#pragma unroll
        for (int k = 0; k < NBH; ++k) dCs[k] += dCh[k];
    }
    __syncthreads();
    if (wave == 0 && hpg > 0) store_dl(g * hpg + hpg - 1);

    // ---- the group's dB, dC, this half's columns --------------------------------------
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = t0 + jrow + r;
        if (t >= a.L) continue;
        float* dbr = a.dB + (((size_t)b * a.L + t) * a.G + g) * NN;
        float* dcr = a.dC + (((size_t)b * a.L + t) * a.G + g) * NN;
#pragma unroll
        for (int k = 0; k < NBH; ++k) {
            dbr[16 * (nb0 + k) + li] = dBs[k][r];
            dcr[16 * (nb0 + k) + li] = dCs[k][r];
        }
    }
}

// ---------------------------------------------------------------------------
// k_bwd_ld: one wave per (batch, head, chunk) adds to the chunk's in-chunk
// suffix sums the totals of every later chunk and <dh_out, h_out>.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_bwd_ld(BwdArgs a) {
    const int c = blockIdx.x % a.nch;
    const int bh = blockIdx.x / a.nch;
    const int b = bh / a.H, h = bh % a.H;
    const int lane = threadIdx.x;
    float off = 0.0f;
    for (int k = lane; k < a.nfin; k += 64) off += a.fin[(size_t)bh * a.nfin + k];
    for (int k = c + 1 + lane; k < a.nch; k += 64) off += a.tot[(size_t)bh * a.nch + k];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) off += __shfl_xor(off, d, 64);
    const int t = c * kQ + lane;
    if (t < a.L) a.dld[((size_t)b * a.L + t) * a.H + h] += off;
}

struct BwdPlan {
    int64_t nch, nfin;
    size_t off_lam, off_tot, off_fin, bytes;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

BwdPlan bwd_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N) {
    BwdPlan p{};
    p.nch = (L + kQ - 1) / kQ;
    p.nfin = (N * P / 4 + kBwdThreads - 1) / kBwdThreads;   // blocks of k_bwd_pass per (b, h)
    size_t off = align256((size_t)(batch * H * p.nch) * 2 * (size_t)(N * P) * 4);
    p.off_lam = off;
    off += align256((size_t)(batch * H * p.nch) * 4);
    p.off_tot = off;
    off += align256((size_t)(batch * H * p.nch) * 4);
    p.off_fin = off;
    off += align256((size_t)(batch * H * p.nfin) * 4);
    p.bytes = off;
    return p;
}

bool bwd_dims_ok(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N) {
    if (batch < 0 || L < 0 || H < 1 || G < 1 || H % G) return false;
    if (N != 64 && N != 128) return false;
    if (P != 32 && P != 64) return false;
    if (batch > INT32_MAX || L > INT32_MAX || H > 65535) return false;
    if (batch * H > 65535) return false;                     // grid y of the pass
    if (batch * ((L + kQ - 1) / kQ) * G > INT32_MAX) return false;
    if (batch * H * ((L + kQ - 1) / kQ) > INT32_MAX) return false;   // grid of k_bwd_ld
    return true;
}

template <int NN, int PP>
mb_status bwd_launch(const BwdArgs& a, int64_t batch, hipStream_t stream) {
    const unsigned nwg = (unsigned)(batch * a.nch * a.G);
    hipLaunchKernelGGL((k_bwd_local<NN, PP>), dim3(nwg), dim3(kMma), 0, stream, a);
    hipLaunchKernelGGL(k_bwd_pass, dim3((unsigned)a.nfin, (unsigned)(batch * a.H)), dim3(kBwdThreads), 0,
                       stream, a);
    hipLaunchKernelGGL((k_bwd_grad<NN, PP>), dim3(nwg), dim3(kMma), 0, stream, a);
    hipLaunchKernelGGL(k_bwd_ld, dim3((unsigned)(batch * a.H * a.nch)), dim3(64), 0, stream, a);
    return check_launch();
}

}  // namespace

size_t ssd_bwd_workspace(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N) {
    if (!bwd_dims_ok(batch, L, H, P, G, N) || batch == 0 || L == 0) return 0;
    return bwd_plan(batch, L, H, P, N).bytes;
}

}  // namespace mb

using namespace mb;

extern "C" mb_status mb_ssd_chunked_bwd(const float* X, const float* logdecay, const float* B,
                                        const float* C, const float* h0, const float* dY,
                                        const float* dh_out, float* dX, float* dlogdecay, float* dB,
                                        float* dC, float* dh0, int64_t batch, int64_t L, int64_t H,
                                        int64_t P, int64_t G, int64_t N, mb_dtype dtype, void* ws,
                                        size_t ws_bytes, hipStream_t stream)
{
    if (dtype != MB_F32) return MB_ERR_DTYPE;
    if (!bwd_dims_ok(batch, L, H, P, G, N)) return MB_ERR_SHAPE;
    const size_t n_x = (size_t)(batch * L * H * P), n_b = (size_t)(batch * L * G * N);
    const size_t n_l = (size_t)(batch * L * H), n_h = (size_t)(batch * H * N * P);
    if (n_x && (!X || !dY || !dX || !logdecay || !dlogdecay)) return MB_ERR_NULL;
    if (n_b && (!B || !C || !dB || !dC)) return MB_ERR_NULL;
    if ((((uintptr_t)X | (uintptr_t)B | (uintptr_t)C | (uintptr_t)dY | (uintptr_t)dX | (uintptr_t)dB |
          (uintptr_t)dC | (uintptr_t)h0 | (uintptr_t)dh_out | (uintptr_t)dh0) & 15))
        return MB_ERR_ALIGN;
    const Span ins[] = {{X, n_x * 4}, {logdecay, n_l * 4}, {B, n_b * 4}, {C, n_b * 4},
                        {h0, h0 ? n_h * 4 : 0}, {dY, n_x * 4}, {dh_out, dh_out ? n_h * 4 : 0}};
    const Span outs[] = {{dX, n_x * 4}, {dlogdecay, n_l * 4}, {dB, n_b * 4}, {dC, n_b * 4},
                         {dh0, dh0 ? n_h * 4 : 0}};
    for (int i = 0; i < 5; ++i) {
        if (overlaps_any(outs[i].p, outs[i].bytes, ins, 7)) return MB_ERR_ALIAS;
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes)) return MB_ERR_ALIAS;
    }
    if (batch == 0) return MB_OK;
    if (L == 0) return dh0 ? copy_state(dh_out, dh0, (int64_t)n_h, stream) : MB_OK;   // dh0 = dh_out
    const BwdPlan pl = bwd_plan(batch, L, H, P, N);
    if (!ws || ws_bytes < pl.bytes || ((uintptr_t)ws & 255)) return MB_ERR_WORKSPACE;
    if (overlaps_any(ws, pl.bytes, ins, 7) || overlaps_any(ws, pl.bytes, outs, 5)) return MB_ERR_ALIAS;
    char* w = (char*)ws;
    BwdArgs a{};
    a.X = X; a.ld = logdecay; a.B = B; a.C = C; a.h0 = h0; a.dY = dY; a.dh_out = dh_out;
    a.dX = dX; a.dld = dlogdecay; a.dB = dB; a.dC = dC; a.dh0 = dh0;
    a.st = (float*)w;
    a.lam = (float*)(w + pl.off_lam);
    a.tot = (float*)(w + pl.off_tot);
    a.fin = (float*)(w + pl.off_fin);
    a.L = (int)L; a.H = (int)H; a.G = (int)G; a.N = (int)N; a.P = (int)P;
    a.nch = (int)pl.nch; a.nfin = (int)pl.nfin;
    if (N == 128)
        return P == 64 ? bwd_launch<128, 64>(a, batch, stream) : bwd_launch<128, 32>(a, batch, stream);
    return P == 64 ? bwd_launch<64, 64>(a, batch, stream) : bwd_launch<64, 32>(a, batch, stream);
}

// ===========================================================================
// Backward of the Mamba-3 SISO recurrence (mb_trap_ssd_bwd), through the SSD
// backward above.  In the rotated frame the trapezoid step
//     S_t = e^{ld_t} S_{t-1} + beta_t Bt_{t-1} X_{t-1}^T + gamma_t Bt_t X_t^T
// is two SSD steps: pseudo-step 2t decays by e^{ld_t} and adds
// Bt_{t-1} (beta_t X_{t-1})^T with no output, pseudo-step 2t + 1 does not decay
// and adds Bt_t (gamma_t X_t)^T with the output Y_t = S^T Ct_t.  The SSD
// backward runs on that interleaved sequence (2L steps, every head its own
// group, per-head rotated B and C) from the rotated dh_out, and these kernels
// map its gradients back: dX, dbeta, dgamma from the two pseudo-steps, dB and dC
// rotated back to the physical frame and summed over the group's heads, and the
// angle gradient per pair (Bt0 dBt1 - Bt1 dBt0 + Ct0 dCt1 - Ct1 dCt0, plus the
// rotation of h_out at the last step) summed over later steps.
// ===========================================================================
namespace mb {
namespace {

struct TrapBwd {
    const float *X, *ld, *B, *C, *beta, *gamma, *theta, *Xp, *Bp, *dY, *dh_out;
    float *dX, *dld, *dB, *dC, *dbeta, *dgamma, *dtheta, *dXp, *dBp;
    // workspace
    float *X2, *dY2, *B2, *C2, *ld2;          // the interleaved inputs (2L steps)
    float *dX2, *dld2, *dB2, *dC2;            // their gradients
    float *Th, *dTh;                          // (batch, L, H, K) angles (as the fraction of a
                                              // revolution) and angle gradients
    float *seg, *hterm, *dh2, *hfin;          // segment sums, h_out term, rotated dh_out, final state
    int L, H, G, N, P, nseg, batch;
};

constexpr int kSeg = 64;   // steps per segment of the angle sums

// sin and cos of an angle given as the fraction of a revolution (|f| <= 0.5)
__device__ __forceinline__ void sincos_frac(float f, float* sn, float* cs) {
    *sn = __builtin_amdgcn_sinf(f);
    *cs = __builtin_amdgcn_cosf(f);
}

// sum of theta over each 64-step segment: one wave per (batch, head, segment),
// lane k = pair
__global__ __launch_bounds__(64) void k_tb_segsum(TrapBwd a, const float* v, float* out) {
    const int sg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, h = bh % a.H, K = a.N / 2, k = threadIdx.x;
    if (k >= K) return;
    float s = 0.0f;
    const int t1 = min(a.L, (sg + 1) * kSeg);
    for (int t = sg * kSeg; t < t1; ++t) s += v[(((size_t)b * a.L + t) * a.H + h) * K + k];
    out[((size_t)bh * a.nseg + sg) * K + k] = s;
}

// angles Theta_t (prefix sums of theta), the per-head rotated B and C of both
// pseudo-steps, and the angles for the mapping back
__global__ __launch_bounds__(64) void k_tb_prep_bc(TrapBwd a) {
    const int sg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G), K = a.N / 2, k = threadIdx.x;
    if (k >= K) return;
    // the cumulative angle reaches hundreds of radians: it is summed in fp64 and
    // kept as the fraction of a revolution
    double th = 0.0;
    if (a.theta)
        for (int s2 = 0; s2 < sg; ++s2) th += (double)a.seg[((size_t)bh * a.nseg + s2) * K + k];
    const size_t L2 = 2 * (size_t)a.L;
    auto row = [&](float* base, size_t t2) { return base + (((size_t)b * L2 + t2) * a.H + h) * a.N + 2 * k; };
    if (sg == 0) {
        // pseudo-step 0: the previous token, unrotated; no output
        const float2 bp = a.Bp ? *(const float2*)(a.Bp + ((size_t)b * a.G + g) * a.N + 2 * k) : make_float2(0.0f, 0.0f);
        *(float2*)row(a.B2, 0) = bp;
        *(float2*)row(a.C2, 0) = make_float2(0.0f, 0.0f);
    }
    const int t1 = min(a.L, (sg + 1) * kSeg);
    // the inputs are never written here: loads may run ahead of the stores
    const float* __restrict__ thv = a.theta;
    const float* __restrict__ Bv = a.B;
    const float* __restrict__ Cv = a.C;
    float* __restrict__ Tho = a.Th;
    constexpr int KB = 8;   // steps whose loads are issued before any of their stores
    for (int tb = sg * kSeg; tb < t1; tb += KB) {
        float thb[KB];
        float2 bvb[KB], cvb[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const int t = tb + j;
            const bool ok = t < t1;
            const size_t bth = ((size_t)b * a.L + (ok ? t : tb)) * a.H + h;
            const size_t o = (((size_t)b * a.L + (ok ? t : tb)) * a.G + g) * a.N + 2 * k;
            thb[j] = thv ? thv[bth * K + k] : 0.0f;
            bvb[j] = *(const float2*)(Bv + o);
            cvb[j] = *(const float2*)(Cv + o);
        }
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const int t = tb + j;
            if (t >= t1) break;
            const size_t bth = ((size_t)b * a.L + t) * a.H + h;
            th += (double)thb[j];
            const double r = th * 0.15915494309189535;
            const float f = (float)(r - rint(r));
            Tho[bth * K + k] = f;
            float sn, cs;
            sincos_frac(f, &sn, &cs);
            const float2 bv = bvb[j], cv = cvb[j];
            const float2 br = make_float2(cs * bv.x - sn * bv.y, sn * bv.x + cs * bv.y);
            const float2 cr = make_float2(cs * cv.x - sn * cv.y, sn * cv.x + cs * cv.y);
            *(float2*)row(a.B2, 2 * (size_t)t + 1) = br;
            *(float2*)row(a.C2, 2 * (size_t)t + 1) = cr;
            if (t + 1 < a.L) {
                *(float2*)row(a.B2, 2 * (size_t)t + 2) = br;
                *(float2*)row(a.C2, 2 * (size_t)t + 2) = make_float2(0.0f, 0.0f);
            }
        }
    }
}

// the interleaved X, dY and log-decay: one thread per (batch, step, head, 4 columns)
__global__ __launch_bounds__(256) void k_tb_prep_x(TrapBwd a) {
    const int P4 = a.P / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int b = blockIdx.y;
    if (i >= (int64_t)a.L * a.H * P4) return;
    const int p4 = (int)(i % P4);
    const int64_t th = i / P4;              // t * H + h
    const int h = (int)(th % a.H), t = (int)(th / a.H);
    const size_t bth = (size_t)b * a.L * a.H + th;
    const float4 z4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const float4 xt = *(const float4*)(a.X + bth * a.P + 4 * p4);
    const float4 xq = t > 0 ? *(const float4*)(a.X + (bth - a.H) * a.P + 4 * p4)
                            : (a.Xp ? *(const float4*)(a.Xp + ((size_t)b * a.H + h) * a.P + 4 * p4) : z4);
    const float be = a.beta[bth], ga = a.gamma[bth];
    const size_t r0 = ((size_t)b * 2 * a.L + 2 * (size_t)t) * a.H + h, r1 = r0 + a.H;
    *(float4*)(a.X2 + r0 * a.P + 4 * p4) = make_float4(be * xq.x, be * xq.y, be * xq.z, be * xq.w);
    *(float4*)(a.X2 + r1 * a.P + 4 * p4) = make_float4(ga * xt.x, ga * xt.y, ga * xt.z, ga * xt.w);
    *(float4*)(a.dY2 + r0 * a.P + 4 * p4) = z4;
    *(float4*)(a.dY2 + r1 * a.P + 4 * p4) = *(const float4*)(a.dY + bth * a.P + 4 * p4);
    if (p4 == 0) {
        a.ld2[r0] = a.ld[bth];
        a.ld2[r1] = 0.0f;
    }
}

// dh_out in the rotated frame, R(Theta_{L-1}) dh_out: one thread per (b, h, pair, column)
__global__ __launch_bounds__(256) void k_tb_rot_dh(TrapBwd a) {
    const int K = a.N / 2;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per = (int64_t)K * a.P;
    const int bh = blockIdx.y;
    if (i >= per) return;
    const int k = (int)(i / a.P), p = (int)(i % a.P);
    const int b = bh / a.H, h = bh % a.H;
    const float th = a.theta ? a.Th[(((size_t)b * a.L + a.L - 1) * a.H + h) * K + k] : 0.0f;
    float sn, cs;
    sincos_frac(th, &sn, &cs);
    const float* src = a.dh_out + (size_t)bh * a.N * a.P;
    float* dst = a.dh2 + (size_t)bh * a.N * a.P;
    const float v0 = src[(2 * k) * a.P + p], v1 = src[(2 * k + 1) * a.P + p];
    dst[(2 * k) * a.P + p] = cs * v0 - sn * v1;
    dst[(2 * k + 1) * a.P + p] = sn * v0 + cs * v1;
}

// dX, dgamma, dbeta, dlogdecay: one wave per four (batch, step, head) rows,
// 16 lanes per row, four columns per lane (P <= 64)
__global__ __launch_bounds__(64) void k_tb_post_x(TrapBwd a) {
    const int64_t rows = (int64_t)a.batch * a.L * a.H;
    const int64_t bth = (int64_t)blockIdx.x * 4 + threadIdx.x / 16;
    const int c4 = threadIdx.x % 16;
    const bool rok = bth < rows;
    const int64_t bthc = rok ? bth : 0;
    const int h = (int)(bthc % a.H);
    const int t = (int)((bthc / a.H) % a.L), b = (int)(bthc / ((int64_t)a.H * a.L));
    const bool ok = rok && 4 * c4 < a.P;
    const int p = 4 * c4;
    const size_t r0 = ((size_t)b * 2 * a.L + 2 * (size_t)t) * a.H + h, r1 = r0 + a.H, r2 = r1 + a.H;
    const float4 z4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto ld4 = [&](const float* base, size_t r, bool c) { return c ? *(const float4*)(base + r * a.P + p) : z4; };
    const float4 d1 = ld4(a.dX2, r1, ok);                        // d(gamma_t X_t)
    const float4 d0 = ld4(a.dX2, r0, ok);                        // d(beta_t X_{t-1})
    const float4 dn = ld4(a.dX2, r2, ok && t + 1 < a.L);          // d(beta_{t+1} X_t)
    const float4 xt = ld4(a.X, (size_t)bthc, ok);
    const float4 xq = t > 0 ? ld4(a.X, (size_t)bthc - a.H, ok)
                            : (a.Xp ? ld4(a.Xp, (size_t)b * a.H + h, ok) : z4);
    const float ga = rok ? a.gamma[bthc] : 0.0f, be = rok ? a.beta[bthc] : 0.0f;
    const float bn = (rok && t + 1 < a.L) ? a.beta[bthc + a.H] : 0.0f;
    if (ok) {
        *(float4*)(a.dX + (size_t)bthc * a.P + p) =
            make_float4(fmaf(ga, d1.x, bn * dn.x), fmaf(ga, d1.y, bn * dn.y), fmaf(ga, d1.z, bn * dn.z),
                        fmaf(ga, d1.w, bn * dn.w));
        if (t == 0 && a.dXp)
            *(float4*)(a.dXp + ((size_t)b * a.H + h) * a.P + p) = make_float4(be * d0.x, be * d0.y, be * d0.z, be * d0.w);
    }
    float sg = (xt.x * d1.x + xt.y * d1.y) + (xt.z * d1.z + xt.w * d1.w);
    float sb = (xq.x * d0.x + xq.y * d0.y) + (xq.z * d0.z + xq.w * d0.w);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) {
        sg += __shfl_xor(sg, off, 16);
        sb += __shfl_xor(sb, off, 16);
    }
    if (rok && c4 == 0) {
        a.dgamma[bthc] = sg;
        a.dbeta[bthc] = sb;
        a.dld[bthc] = a.dld2[r0];
    }
}

// dB, dC in the physical frame summed over the group's heads, the per-head angle
// gradient, and dB_prev: one wave per (batch, step, group), lane = pair
__global__ __launch_bounds__(64) void k_tb_post_bc(TrapBwd a) {
    const int64_t btg = blockIdx.x;
    const int g = (int)(btg % a.G);
    const int t = (int)((btg / a.G) % a.L), b = (int)(btg / ((int64_t)a.G * a.L));
    const int K = a.N / 2, k = threadIdx.x;
    if (k >= K) return;
    const int hpg = a.H / a.G;
    float2 db = make_float2(0.0f, 0.0f), dc = make_float2(0.0f, 0.0f), dbp = make_float2(0.0f, 0.0f);
    // the physical B, C of the step (shared by the group's heads); the rotated
    // ones are recomputed per head from the angle
    const size_t o = (((size_t)b * a.L + t) * a.G + g) * a.N + 2 * k;
    const float2 bp = *(const float2*)(a.B + o), cp = *(const float2*)(a.C + o);
    const float* __restrict__ dB2 = a.dB2;
    const float* __restrict__ dC2 = a.dC2;
    const float* __restrict__ Thv = a.Th;
#pragma unroll 4
    for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
        const size_t r0 = ((size_t)b * 2 * a.L + 2 * (size_t)t) * a.H + h, r1 = r0 + a.H, r2 = r1 + a.H;
        auto ld2 = [&](const float* base, size_t r) { return *(const float2*)(base + r * a.N + 2 * k); };
        float2 dbr = ld2(dB2, r1);
        if (t + 1 < a.L) {
            const float2 u = ld2(dB2, r2);
            dbr.x += u.x;
            dbr.y += u.y;
        }
        const float2 dcr = ld2(dC2, r1);
        const size_t bth = ((size_t)b * a.L + t) * a.H + h;
        const float th = a.theta ? Thv[bth * K + k] : 0.0f;
        float sn, cs;
        sincos_frac(th, &sn, &cs);
        if (a.theta) {
            const float2 br = make_float2(cs * bp.x - sn * bp.y, sn * bp.x + cs * bp.y);
            const float2 cr = make_float2(cs * cp.x - sn * cp.y, sn * cp.x + cs * cp.y);
            a.dTh[bth * K + k] = (br.x * dbr.y - br.y * dbr.x) + (cr.x * dcr.y - cr.y * dcr.x);
        }
        // R(-Theta): (cs v0 + sn v1, -sn v0 + cs v1)
        db.x += cs * dbr.x + sn * dbr.y;
        db.y += -sn * dbr.x + cs * dbr.y;
        dc.x += cs * dcr.x + sn * dcr.y;
        dc.y += -sn * dcr.x + cs * dcr.y;
        if (t == 0) {
            const float2 u = ld2(a.dB2, r0);   // step -1 is unrotated
            dbp.x += u.x;
            dbp.y += u.y;
        }
    }
    *(float2*)(a.dB + o) = db;
    *(float2*)(a.dC + o) = dc;
    if (t == 0 && a.dBp) *(float2*)(a.dBp + ((size_t)b * a.G + g) * a.N + 2 * k) = dbp;
}

// the rotation of h_out = R(-Theta_{L-1}) S: per (b, h, pair) sum over columns of
// dh_out0 o1 - dh_out1 o0; one wave per (batch, head), lane = pair
__global__ __launch_bounds__(64) void k_tb_hterm(TrapBwd a) {
    const int bh = blockIdx.x, K = a.N / 2, k = threadIdx.x;
    if (k >= K) return;
    const int b = bh / a.H, h = bh % a.H;
    const float th = a.Th[(((size_t)b * a.L + a.L - 1) * a.H + h) * K + k];
    float sn, cs;
    sincos_frac(th, &sn, &cs);
    const float* S = a.hfin + (size_t)bh * a.N * a.P;
    const float* dh = a.dh_out + (size_t)bh * a.N * a.P;
    float acc = 0.0f;
    for (int p = 0; p < a.P; ++p) {
        const float s0 = S[(2 * k) * a.P + p], s1 = S[(2 * k + 1) * a.P + p];
        const float o0 = cs * s0 + sn * s1, o1 = -sn * s0 + cs * s1;
        acc += dh[(2 * k) * a.P + p] * o1 - dh[(2 * k + 1) * a.P + p] * o0;
    }
    a.hterm[(size_t)bh * K + k] = acc;
}

// dtheta_t = sum_{tau >= t} dTheta_tau (+ the h_out term): one wave per (batch,
// head, segment), the later segments' sums added first
__global__ __launch_bounds__(64) void k_tb_theta(TrapBwd a) {
    const int sg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, h = bh % a.H, K = a.N / 2, k = threadIdx.x;
    if (k >= K) return;
    float acc = a.dh_out ? a.hterm[(size_t)bh * K + k] : 0.0f;
    for (int s2 = sg + 1; s2 < a.nseg; ++s2) acc += a.seg[((size_t)bh * a.nseg + s2) * K + k];
    const int t1 = min(a.L, (sg + 1) * kSeg);
    for (int t = t1 - 1; t >= sg * kSeg; --t) {
        const size_t i = (((size_t)b * a.L + t) * a.H + h) * K + k;
        acc += a.dTh[i];
        a.dtheta[i] = acc;
    }
}

struct TrapBwdPlan {
    BwdPlan ssd;
    size_t off_x2, off_dy2, off_b2, off_c2, off_ld2, off_dx2, off_dld2, off_db2, off_dc2, off_th, off_dth, off_seg,
        off_hterm, off_dh2, off_hfin, bytes;
};

TrapBwdPlan trap_bwd_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N) {
    TrapBwdPlan p{};
    p.ssd = bwd_plan(batch, 2 * L, H, P, N);
    size_t off = p.ssd.bytes;
    const size_t nx = (size_t)(batch * 2 * L * H * P) * 4, nb = (size_t)(batch * 2 * L * H * N) * 4;
    const size_t nl = (size_t)(batch * 2 * L * H) * 4, nth = (size_t)(batch * L * H * (N / 2)) * 4;
    const size_t nseg = (size_t)((L + kSeg - 1) / kSeg), nh = (size_t)(batch * H * N * P) * 4;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    p.off_x2 = take(nx); p.off_dy2 = take(nx); p.off_b2 = take(nb); p.off_c2 = take(nb); p.off_ld2 = take(nl);
    p.off_dx2 = take(nx); p.off_dld2 = take(nl); p.off_db2 = take(nb); p.off_dc2 = take(nb);
    p.off_th = take(nth); p.off_dth = take(nth);
    p.off_seg = take((size_t)(batch * H) * nseg * (N / 2) * 4);
    p.off_hterm = take((size_t)(batch * H * (N / 2)) * 4);
    p.off_dh2 = take(nh); p.off_hfin = take(nh);
    p.bytes = off;
    return p;
}

}  // namespace

size_t trap_bwd_workspace(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N) {
    if (!bwd_dims_ok(batch, 2 * L, H, P, H, N) || G < 1 || H % G || batch == 0 || L == 0) return 0;
    return trap_bwd_plan(batch, L, H, P, N).bytes;
}

}  // namespace mb

extern "C" mb_status mb_trap_ssd_bwd(const float* X, const float* logdecay, const float* B, const float* C,
                                     const float* beta, const float* gamma, const float* theta, const float* h0,
                                     const float* X_prev, const float* B_prev, const float* dY,
                                     const float* dh_out, float* dX, float* dlogdecay, float* dB, float* dC,
                                     float* dbeta, float* dgamma, float* dtheta, float* dh0, float* dX_prev,
                                     float* dB_prev, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G,
                                     int64_t N, mb_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (dtype != MB_F32) return MB_ERR_DTYPE;
    if (G < 1 || H % G || !bwd_dims_ok(batch, 2 * L, H, P, H, N)) return MB_ERR_SHAPE;
    if (batch * L * H > INT32_MAX || batch * L * G > INT32_MAX) return MB_ERR_SHAPE;
    const size_t n_x = (size_t)(batch * L * H * P), n_b = (size_t)(batch * L * G * N);
    const size_t n_l = (size_t)(batch * L * H), n_h = (size_t)(batch * H * N * P);
    const size_t n_th = (size_t)(batch * L * H * (N / 2));
    const size_t n_xp = (size_t)(batch * H * P), n_bp = (size_t)(batch * G * N);
    if (n_x && (!X || !dY || !dX || !logdecay || !dlogdecay || !beta || !gamma || !dbeta || !dgamma))
        return MB_ERR_NULL;
    if (n_b && (!B || !C || !dB || !dC)) return MB_ERR_NULL;
    if (theta && n_th && !dtheta) return MB_ERR_NULL;
    if ((X_prev == nullptr) != (B_prev == nullptr)) return MB_ERR_NULL;
    if (((uintptr_t)X | (uintptr_t)B | (uintptr_t)C | (uintptr_t)dY | (uintptr_t)dX | (uintptr_t)dB |
         (uintptr_t)dC | (uintptr_t)h0 | (uintptr_t)dh_out | (uintptr_t)dh0 | (uintptr_t)X_prev |
         (uintptr_t)B_prev | (uintptr_t)dB_prev) & 15)
        return MB_ERR_ALIGN;
    const Span ins[] = {{X, n_x * 4}, {logdecay, n_l * 4}, {B, n_b * 4}, {C, n_b * 4}, {beta, n_l * 4},
                        {gamma, n_l * 4}, {theta, theta ? n_th * 4 : 0}, {h0, h0 ? n_h * 4 : 0},
                        {X_prev, X_prev ? n_xp * 4 : 0}, {B_prev, B_prev ? n_bp * 4 : 0}, {dY, n_x * 4},
                        {dh_out, dh_out ? n_h * 4 : 0}};
    const Span outs[] = {{dX, n_x * 4}, {dlogdecay, n_l * 4}, {dB, n_b * 4}, {dC, n_b * 4}, {dbeta, n_l * 4},
                         {dgamma, n_l * 4}, {dtheta, theta && dtheta ? n_th * 4 : 0}, {dh0, dh0 ? n_h * 4 : 0},
                         {dX_prev, dX_prev ? n_xp * 4 : 0}, {dB_prev, dB_prev ? n_bp * 4 : 0}};
    for (int i = 0; i < 10; ++i) {
        if (overlaps_any(outs[i].p, outs[i].bytes, ins, 12)) return MB_ERR_ALIAS;
        for (int j = i + 1; j < 10; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes)) return MB_ERR_ALIAS;
    }
    if (batch == 0) return MB_OK;
    if (L == 0) {
        // no steps: dh0 = dh_out; the previous token gets nothing
        mb_status st = dh0 ? copy_state(dh_out, dh0, (int64_t)n_h, stream) : MB_OK;
        if (st == MB_OK && dX_prev) st = copy_state(nullptr, dX_prev, (int64_t)n_xp, stream);
        if (st == MB_OK && dB_prev) st = copy_state(nullptr, dB_prev, (int64_t)n_bp, stream);
        return st;
    }
    const TrapBwdPlan pl = trap_bwd_plan(batch, L, H, P, N);
    if (!ws || ws_bytes < pl.bytes || ((uintptr_t)ws & 255)) return MB_ERR_WORKSPACE;
    if (overlaps_any(ws, pl.bytes, ins, 12) || overlaps_any(ws, pl.bytes, outs, 10)) return MB_ERR_ALIAS;
    char* w = (char*)ws;
    TrapBwd t{};
    t.X = X; t.ld = logdecay; t.B = B; t.C = C; t.beta = beta; t.gamma = gamma; t.theta = theta;
    t.Xp = X_prev; t.Bp = B_prev; t.dY = dY; t.dh_out = dh_out;
    t.dX = dX; t.dld = dlogdecay; t.dB = dB; t.dC = dC; t.dbeta = dbeta; t.dgamma = dgamma; t.dtheta = dtheta;
    t.dXp = dX_prev; t.dBp = dB_prev;
    t.X2 = (float*)(w + pl.off_x2); t.dY2 = (float*)(w + pl.off_dy2); t.B2 = (float*)(w + pl.off_b2);
    t.C2 = (float*)(w + pl.off_c2); t.ld2 = (float*)(w + pl.off_ld2); t.dX2 = (float*)(w + pl.off_dx2);
    t.dld2 = (float*)(w + pl.off_dld2); t.dB2 = (float*)(w + pl.off_db2); t.dC2 = (float*)(w + pl.off_dc2);
    t.Th = (float*)(w + pl.off_th); t.dTh = (float*)(w + pl.off_dth); t.seg = (float*)(w + pl.off_seg);
    t.hterm = (float*)(w + pl.off_hterm); t.dh2 = (float*)(w + pl.off_dh2); t.hfin = (float*)(w + pl.off_hfin);
    t.L = (int)L; t.H = (int)H; t.G = (int)G; t.N = (int)N; t.P = (int)P;
    t.nseg = (int)((L + kSeg - 1) / kSeg);
    t.batch = (int)batch;
    const unsigned nseg_all = (unsigned)(batch * H * t.nseg);
    // 1. angles, rotated and interleaved inputs
    if (theta) hipLaunchKernelGGL(k_tb_segsum, dim3(nseg_all), dim3(64), 0, stream, t, theta, t.seg);
    hipLaunchKernelGGL(k_tb_prep_bc, dim3(nseg_all), dim3(64), 0, stream, t);
    hipLaunchKernelGGL(k_tb_prep_x, dim3((unsigned)((L * H * (P / 4) + 255) / 256), (unsigned)batch), dim3(256), 0,
                       stream, t);
    if (dh_out)
        hipLaunchKernelGGL(k_tb_rot_dh, dim3((unsigned)(((N / 2) * P + 255) / 256), (unsigned)(batch * H)),
                           dim3(256), 0, stream, t);
    // 2. the SSD backward over the 2L pseudo-steps, every head its own group
    BwdArgs a{};
    a.X = t.X2; a.ld = t.ld2; a.B = t.B2; a.C = t.C2; a.h0 = h0; a.dY = t.dY2; a.dh_out = dh_out ? t.dh2 : nullptr;
    a.dX = t.dX2; a.dld = t.dld2; a.dB = t.dB2; a.dC = t.dC2; a.dh0 = dh0;
    a.st = (float*)w;
    a.lam = (float*)(w + pl.ssd.off_lam);
    a.tot = (float*)(w + pl.ssd.off_tot);
    a.fin = (float*)(w + pl.ssd.off_fin);
    a.h_final = t.hfin;
    a.L = (int)(2 * L); a.H = (int)H; a.G = (int)H; a.N = (int)N; a.P = (int)P;
    a.nch = (int)pl.ssd.nch; a.nfin = (int)pl.ssd.nfin;
    mb_status st;
    if (N == 128)
        st = P == 64 ? bwd_launch<128, 64>(a, batch, stream) : bwd_launch<128, 32>(a, batch, stream);
    else
        st = P == 64 ? bwd_launch<64, 64>(a, batch, stream) : bwd_launch<64, 32>(a, batch, stream);
    if (st != MB_OK) return st;
    // 3. back to the inputs
    hipLaunchKernelGGL(k_tb_post_x, dim3((unsigned)((batch * L * H + 3) / 4)), dim3(64), 0, stream, t);
    hipLaunchKernelGGL(k_tb_post_bc, dim3((unsigned)(batch * L * G)), dim3(64), 0, stream, t);
    if (theta) {
        if (dh_out) hipLaunchKernelGGL(k_tb_hterm, dim3((unsigned)(batch * H)), dim3(64), 0, stream, t);
        hipLaunchKernelGGL(k_tb_segsum, dim3(nseg_all), dim3(64), 0, stream, t, (const float*)t.dTh, t.seg);
        hipLaunchKernelGGL(k_tb_theta, dim3(nseg_all), dim3(64), 0, stream, t);
    }
    return check_launch();
}

// ===========================================================================
// Backward of the Mamba-3 MIMO recurrence (mb_mimo_ssd_bwd), the same way: with
// rank R a step becomes RS = 3R - 1 rows of a plain SSD, in order
//   rows 0 .. R-1      beta terms:  Bt_{t-1,r}, beta_t X_{t-1,r}   (row 0 decays by e^{ld_t})
//   rows R .. 2R-1     gamma terms: Bt_{t,r},   gamma_t X_{t,r}    (row 2R-1 also outputs rank 0)
//   rows 2R .. 3R-2    outputs of ranks 1 .. R-1 (no input)
// so every output of step t follows all of its inputs.  B, C are per head (no
// groups) with the rank innermost: (batch, L, H, N, R); X, dY (batch, L, H, P, R).
// ===========================================================================
namespace mb {
namespace {

struct MimoBwd {
    const float *X, *ld, *B, *C, *beta, *gamma, *theta, *Xp, *Bp, *dY, *dh_out;
    float *dX, *dld, *dB, *dC, *dbeta, *dgamma, *dtheta, *dXp, *dBp;
    float *X2, *dY2, *B2, *C2, *ld2, *dX2, *dld2, *dB2, *dC2;
    float *Th, *dTh, *seg, *hterm, *dh2, *hfin;
    int L, H, N, P, R, RS, nseg, batch;
};

// TrapBwd view of the fields the shared angle kernels use
TrapBwd as_trap(const MimoBwd& m) {
    TrapBwd t{};
    t.theta = m.theta; t.dh_out = m.dh_out; t.dtheta = m.dtheta;
    t.Th = m.Th; t.dTh = m.dTh; t.seg = m.seg; t.hterm = m.hterm; t.dh2 = m.dh2; t.hfin = m.hfin;
    t.L = m.L; t.H = m.H; t.G = m.H; t.N = m.N; t.P = m.P; t.nseg = m.nseg; t.batch = m.batch;
    return t;
}

// angles and the rotated per-rank B, C rows of every row of a step: one wave per
// (batch, head, segment), lane = pair
template <int R>
__global__ __launch_bounds__(64) void k_mb_prep_bc(MimoBwd a) {
    const int sg = blockIdx.x % a.nseg, bh = blockIdx.x / a.nseg;
    const int b = bh / a.H, h = bh % a.H, K = a.N / 2, k = threadIdx.x, RS = a.RS;
    if (k >= K) return;
    double th = 0.0;
    if (a.theta)
        for (int s2 = 0; s2 < sg; ++s2) th += (double)a.seg[((size_t)bh * a.nseg + s2) * K + k];
    const size_t L2 = (size_t)RS * a.L;
    auto row = [&](float* base, size_t t2) { return base + (((size_t)b * L2 + t2) * a.H + h) * a.N + 2 * k; };
    const float2 z2 = make_float2(0.0f, 0.0f);
    if (sg == 0)
        for (int r = 0; r < R; ++r) {
            // step 0's beta rows: the previous token, unrotated
            const float* bp = a.Bp ? a.Bp + ((size_t)b * a.H + h) * a.N * R : nullptr;
            *(float2*)row(a.B2, r) = bp ? make_float2(bp[(2 * k) * R + r], bp[(2 * k + 1) * R + r]) : z2;
        }
    const float* __restrict__ thv = a.theta;
    const float* __restrict__ Bv = a.B;
    const float* __restrict__ Cv = a.C;
    const int t1 = min(a.L, (sg + 1) * kSeg);
    constexpr int KB = R <= 4 ? 4 : 1;   // steps whose loads are issued before any of their stores
    for (int tb = sg * kSeg; tb < t1; tb += KB) {
      // the pairs' R ranks of B and C of KB steps, contiguous (rank innermost)
      float thb[KB], bq0[KB][R], bq1[KB][R], cq0[KB][R], cq1[KB][R];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int t = tb + j < t1 ? tb + j : tb;
        const size_t bth = ((size_t)b * a.L + t) * a.H + h;
        thb[j] = thv ? thv[bth * K + k] : 0.0f;
        const float* bs = Bv + bth * a.N * R;
        const float* cs_ = Cv + bth * a.N * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            bq0[j][r] = bs[(2 * k) * R + r];
            bq1[j][r] = bs[(2 * k + 1) * R + r];
            cq0[j][r] = cs_[(2 * k) * R + r];
            cq1[j][r] = cs_[(2 * k + 1) * R + r];
        }
      }
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int t = tb + j;
        if (t >= t1) break;
        const size_t bth = ((size_t)b * a.L + t) * a.H + h;
        th += (double)thb[j];
        const double rv = th * 0.15915494309189535;
        const float f = (float)(rv - rint(rv));
        a.Th[bth * K + k] = f;
        float sn, cs;
        sincos_frac(f, &sn, &cs);
        const size_t t0 = (size_t)RS * t;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float b0 = bq0[j][r], b1 = bq1[j][r], c0 = cq0[j][r], c1 = cq1[j][r];
            const float2 br = make_float2(cs * b0 - sn * b1, sn * b0 + cs * b1);
            const float2 cr = make_float2(cs * c0 - sn * c1, sn * c0 + cs * c1);
            *(float2*)row(a.B2, t0 + R + r) = br;                               // gamma row r
            if (t + 1 < a.L) *(float2*)row(a.B2, t0 + RS + r) = br;              // next step's beta row r
            *(float2*)row(a.C2, t0 + 2 * R - 1 + r) = cr;                       // output row of rank r
            *(float2*)row(a.C2, t0 + r) = z2;                                   // beta rows: no output
            if (r < R - 1) *(float2*)row(a.C2, t0 + R + r) = z2;                // gamma rows but the last
            if (r >= 1) *(float2*)row(a.B2, t0 + 2 * R - 1 + r) = z2;           // output-only rows: no input
        }
      }
    }
}

// the per-row X, dY and log-decay: one thread per (batch, step, head, column)
__global__ __launch_bounds__(256) void k_mb_prep_x(MimoBwd a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int b = blockIdx.y, R = a.R, RS = a.RS;
    if (i >= (int64_t)a.L * a.H * a.P) return;
    const int p = (int)(i % a.P);
    const int64_t th = i / a.P;
    const int h = (int)(th % a.H), t = (int)(th / a.H);
    const size_t bth = (size_t)b * a.L * a.H + th;
    const float be = a.beta[bth], ga = a.gamma[bth];
    const size_t rowbase = ((size_t)b * RS * a.L + (size_t)RS * t) * a.H + h;   // row (t, 0)
    auto at = [&](float* base, int j) { return base + (rowbase + (size_t)j * a.H) * a.P + p; };
    for (int r = 0; r < R; ++r) {
        const float xt = a.X[(bth * a.P + p) * R + r];
        const float xq = t > 0 ? a.X[((bth - a.H) * a.P + p) * R + r]
                               : (a.Xp ? a.Xp[(((size_t)b * a.H + h) * a.P + p) * R + r] : 0.0f);
        *at(a.X2, r) = be * xq;
        *at(a.X2, R + r) = ga * xt;
        *at(a.dY2, r) = 0.0f;
        if (r < R - 1) *at(a.dY2, R + r) = 0.0f;
        *at(a.dY2, 2 * R - 1 + r) = a.dY[(bth * a.P + p) * R + r];
        if (r >= 1) *at(a.X2, 2 * R - 1 + r) = 0.0f;
    }
    if (p == 0)
        for (int j = 0; j < RS; ++j) a.ld2[rowbase + (size_t)j * a.H] = j == 0 ? a.ld[bth] : 0.0f;
}

// dX, dgamma, dbeta, dlogdecay, dX_prev: one wave per (batch, step, head), lane = column
__global__ __launch_bounds__(64) void k_mb_post_x(MimoBwd a) {
    const int64_t bth = blockIdx.x;
    const int h = (int)(bth % a.H);
    const int t = (int)((bth / a.H) % a.L), b = (int)(bth / ((int64_t)a.H * a.L));
    const int p = threadIdx.x, R = a.R, RS = a.RS;
    const bool ok = p < a.P;
    const size_t rowbase = ((size_t)b * RS * a.L + (size_t)RS * t) * a.H + h;
    auto rowp = [&](int j) { return (rowbase + (size_t)j * a.H) * a.P + p; };
    const float ga = a.gamma[bth], be = a.beta[bth];
    const float bn = t + 1 < a.L ? a.beta[bth + a.H] : 0.0f;
    float sg = 0.0f, sb = 0.0f;
    for (int r = 0; r < R; ++r) {
        const float d1 = ok ? a.dX2[rowp(R + r)] : 0.0f;                     // d(gamma_t X_{t,r})
        const float d0 = ok ? a.dX2[rowp(r)] : 0.0f;                         // d(beta_t X_{t-1,r})
        const float dn = (ok && t + 1 < a.L) ? a.dX2[rowp(RS + r)] : 0.0f;   // d(beta_{t+1} X_{t,r})
        const float xt = ok ? a.X[(bth * a.P + p) * R + r] : 0.0f;
        const float xq = !ok ? 0.0f : t > 0 ? a.X[((bth - a.H) * a.P + p) * R + r]
                                           : (a.Xp ? a.Xp[(((size_t)b * a.H + h) * a.P + p) * R + r] : 0.0f);
        if (ok) a.dX[(bth * a.P + p) * R + r] = fmaf(ga, d1, bn * dn);
        if (ok && t == 0 && a.dXp) a.dXp[(((size_t)b * a.H + h) * a.P + p) * R + r] = be * d0;
        sg = fmaf(xt, d1, sg);
        sb = fmaf(xq, d0, sb);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        sg += __shfl_xor(sg, off, 64);
        sb += __shfl_xor(sb, off, 64);
    }
    if (p == 0) {
        a.dgamma[bth] = sg;
        a.dbeta[bth] = sb;
        a.dld[bth] = a.dld2[rowbase];
    }
}

// dB, dC per rank in the physical frame, the angle gradient summed over ranks,
// dB_prev: one wave per (batch, step, head), lane = pair
template <int R>
__global__ __launch_bounds__(64) void k_mb_post_bc(MimoBwd a) {
    const int64_t bth = blockIdx.x;
    const int h = (int)(bth % a.H);
    const int t = (int)((bth / a.H) % a.L), b = (int)(bth / ((int64_t)a.H * a.L));
    const int K = a.N / 2, k = threadIdx.x, RS = a.RS;
    if (k >= K) return;
    const size_t rowbase = ((size_t)b * RS * a.L + (size_t)RS * t) * a.H + h;
    auto ld2 = [&](const float* base, int j) {
        return *(const float2*)(base + (rowbase + (size_t)j * a.H) * a.N + 2 * k);
    };
    const float th = a.theta ? a.Th[bth * K + k] : 0.0f;
    float sn, cs;
    sincos_frac(th, &sn, &cs);
    float dth = 0.0f;
    const float* bs = a.B + bth * a.N * R;
    const float* cs_ = a.C + bth * a.N * R;
    // the pair's R ranks, loaded and stored whole (rank innermost)
    float bq0[R], bq1[R], cq0[R], cq1[R], ob0[R], ob1[R], oc0[R], oc1[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        bq0[r] = bs[(2 * k) * R + r];
        bq1[r] = bs[(2 * k + 1) * R + r];
        cq0[r] = cs_[(2 * k) * R + r];
        cq1[r] = cs_[(2 * k + 1) * R + r];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float2 dbr = ld2(a.dB2, R + r);
        if (t + 1 < a.L) {
            const float2 u = ld2(a.dB2, RS + r);
            dbr.x += u.x;
            dbr.y += u.y;
        }
        const float2 dcr = ld2(a.dC2, 2 * R - 1 + r);
        const float b0 = bq0[r], b1 = bq1[r], c0 = cq0[r], c1 = cq1[r];
        const float2 br = make_float2(cs * b0 - sn * b1, sn * b0 + cs * b1);
        const float2 cr = make_float2(cs * c0 - sn * c1, sn * c0 + cs * c1);
        dth += (br.x * dbr.y - br.y * dbr.x) + (cr.x * dcr.y - cr.y * dcr.x);
        ob0[r] = cs * dbr.x + sn * dbr.y;
        ob1[r] = -sn * dbr.x + cs * dbr.y;
        oc0[r] = cs * dcr.x + sn * dcr.y;
        oc1[r] = -sn * dcr.x + cs * dcr.y;
    }
    if (t == 0 && a.dBp) {
        float* dbp = a.dBp + ((size_t)b * a.H + h) * a.N * R;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float2 u = ld2(a.dB2, r);   // step 0's beta rows: unrotated
            dbp[(2 * k) * R + r] = u.x;
            dbp[(2 * k + 1) * R + r] = u.y;
        }
    }
    float* db = a.dB + bth * a.N * R;
    float* dc = a.dC + bth * a.N * R;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        db[(2 * k) * R + r] = ob0[r];
        db[(2 * k + 1) * R + r] = ob1[r];
        dc[(2 * k) * R + r] = oc0[r];
        dc[(2 * k + 1) * R + r] = oc1[r];
    }
    if (a.theta) a.dTh[bth * K + k] = dth;
}

struct MimoBwdPlan {
    BwdPlan ssd;
    size_t off_x2, off_dy2, off_b2, off_c2, off_ld2, off_dx2, off_dld2, off_db2, off_dc2, off_th, off_dth, off_seg,
        off_hterm, off_dh2, off_hfin, bytes;
};

MimoBwdPlan mimo_bwd_plan(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R) {
    MimoBwdPlan p{};
    const int64_t L2 = (3 * R - 1) * L;
    p.ssd = bwd_plan(batch, L2, H, P, N);
    size_t off = p.ssd.bytes;
    const size_t nx = (size_t)(batch * L2 * H * P) * 4, nb = (size_t)(batch * L2 * H * N) * 4;
    const size_t nl = (size_t)(batch * L2 * H) * 4, nth = (size_t)(batch * L * H * (N / 2)) * 4;
    const size_t nseg = (size_t)((L + kSeg - 1) / kSeg), nh = (size_t)(batch * H * N * P) * 4;
    auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
    p.off_x2 = take(nx); p.off_dy2 = take(nx); p.off_b2 = take(nb); p.off_c2 = take(nb); p.off_ld2 = take(nl);
    p.off_dx2 = take(nx); p.off_dld2 = take(nl); p.off_db2 = take(nb); p.off_dc2 = take(nb);
    p.off_th = take(nth); p.off_dth = take(nth);
    p.off_seg = take((size_t)(batch * H) * nseg * (N / 2) * 4);
    p.off_hterm = take((size_t)(batch * H * (N / 2)) * 4);
    p.off_dh2 = take(nh); p.off_hfin = take(nh);
    p.bytes = off;
    return p;
}

bool mimo_bwd_ok(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R) {
    if (R != 1 && R != 2 && R != 4 && R != 8 && R != 16) return false;
    if (!bwd_dims_ok(batch, (3 * R - 1) * L, H, P, H, N)) return false;
    if (batch * L * H > INT32_MAX) return false;
    return true;
}

}  // namespace

size_t mimo_bwd_workspace(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R) {
    if (!mimo_bwd_ok(batch, L, H, P, N, R) || batch == 0 || L == 0) return 0;
    return mimo_bwd_plan(batch, L, H, P, N, R).bytes;
}

}  // namespace mb

extern "C" mb_status mb_mimo_ssd_bwd(const float* X, const float* logdecay, const float* B, const float* C,
                                     const float* beta, const float* gamma, const float* theta, const float* h0,
                                     const float* X_prev, const float* B_prev, const float* dY,
                                     const float* dh_out, float* dX, float* dlogdecay, float* dB, float* dC,
                                     float* dbeta, float* dgamma, float* dtheta, float* dh0, float* dX_prev,
                                     float* dB_prev, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                                     int64_t R, mb_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (dtype != MB_F32) return MB_ERR_DTYPE;
    if (!mimo_bwd_ok(batch, L, H, P, N, R)) return MB_ERR_SHAPE;
    const size_t n_x = (size_t)(batch * L * H * P * R), n_b = (size_t)(batch * L * H * N * R);
    const size_t n_l = (size_t)(batch * L * H), n_h = (size_t)(batch * H * N * P);
    const size_t n_th = (size_t)(batch * L * H * (N / 2));
    const size_t n_xp = (size_t)(batch * H * P * R), n_bp = (size_t)(batch * H * N * R);
    if (n_x && (!X || !dY || !dX || !logdecay || !dlogdecay || !beta || !gamma || !dbeta || !dgamma))
        return MB_ERR_NULL;
    if (n_b && (!B || !C || !dB || !dC)) return MB_ERR_NULL;
    if (theta && n_th && !dtheta) return MB_ERR_NULL;
    if ((X_prev == nullptr) != (B_prev == nullptr)) return MB_ERR_NULL;
    if (((uintptr_t)h0 | (uintptr_t)dh_out | (uintptr_t)dh0) & 15) return MB_ERR_ALIGN;
    const Span ins[] = {{X, n_x * 4}, {logdecay, n_l * 4}, {B, n_b * 4}, {C, n_b * 4}, {beta, n_l * 4},
                        {gamma, n_l * 4}, {theta, theta ? n_th * 4 : 0}, {h0, h0 ? n_h * 4 : 0},
                        {X_prev, X_prev ? n_xp * 4 : 0}, {B_prev, B_prev ? n_bp * 4 : 0}, {dY, n_x * 4},
                        {dh_out, dh_out ? n_h * 4 : 0}};
    const Span outs[] = {{dX, n_x * 4}, {dlogdecay, n_l * 4}, {dB, n_b * 4}, {dC, n_b * 4}, {dbeta, n_l * 4},
                         {dgamma, n_l * 4}, {dtheta, theta && dtheta ? n_th * 4 : 0}, {dh0, dh0 ? n_h * 4 : 0},
                         {dX_prev, dX_prev ? n_xp * 4 : 0}, {dB_prev, dB_prev ? n_bp * 4 : 0}};
    for (int i = 0; i < 10; ++i) {
        if (overlaps_any(outs[i].p, outs[i].bytes, ins, 12)) return MB_ERR_ALIAS;
        for (int j = i + 1; j < 10; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes)) return MB_ERR_ALIAS;
    }
    if (batch == 0) return MB_OK;
    if (L == 0) {
        mb_status st = dh0 ? copy_state(dh_out, dh0, (int64_t)n_h, stream) : MB_OK;
        if (st == MB_OK && dX_prev) st = copy_state(nullptr, dX_prev, (int64_t)n_xp, stream);
        if (st == MB_OK && dB_prev) st = copy_state(nullptr, dB_prev, (int64_t)n_bp, stream);
        return st;
    }
    const MimoBwdPlan pl = mimo_bwd_plan(batch, L, H, P, N, R);
    if (!ws || ws_bytes < pl.bytes || ((uintptr_t)ws & 255)) return MB_ERR_WORKSPACE;
    if (overlaps_any(ws, pl.bytes, ins, 12) || overlaps_any(ws, pl.bytes, outs, 10)) return MB_ERR_ALIAS;
    char* w = (char*)ws;
    MimoBwd m{};
    m.X = X; m.ld = logdecay; m.B = B; m.C = C; m.beta = beta; m.gamma = gamma; m.theta = theta;
    m.Xp = X_prev; m.Bp = B_prev; m.dY = dY; m.dh_out = dh_out;
    m.dX = dX; m.dld = dlogdecay; m.dB = dB; m.dC = dC; m.dbeta = dbeta; m.dgamma = dgamma; m.dtheta = dtheta;
    m.dXp = dX_prev; m.dBp = dB_prev;
    m.X2 = (float*)(w + pl.off_x2); m.dY2 = (float*)(w + pl.off_dy2); m.B2 = (float*)(w + pl.off_b2);
    m.C2 = (float*)(w + pl.off_c2); m.ld2 = (float*)(w + pl.off_ld2); m.dX2 = (float*)(w + pl.off_dx2);
    m.dld2 = (float*)(w + pl.off_dld2); m.dB2 = (float*)(w + pl.off_db2); m.dC2 = (float*)(w + pl.off_dc2);
    m.Th = (float*)(w + pl.off_th); m.dTh = (float*)(w + pl.off_dth); m.seg = (float*)(w + pl.off_seg);
    m.hterm = (float*)(w + pl.off_hterm); m.dh2 = (float*)(w + pl.off_dh2); m.hfin = (float*)(w + pl.off_hfin);
    m.L = (int)L; m.H = (int)H; m.N = (int)N; m.P = (int)P; m.R = (int)R; m.RS = (int)(3 * R - 1);
    m.nseg = (int)((L + kSeg - 1) / kSeg);
    m.batch = (int)batch;
    const TrapBwd t = as_trap(m);
    const unsigned nseg_all = (unsigned)(batch * H * m.nseg);
    if (theta) hipLaunchKernelGGL(k_tb_segsum, dim3(nseg_all), dim3(64), 0, stream, t, theta, m.seg);
#define MB_MIMO_R(KERNEL, GRID)                                                                   \
    switch (R) {                                                                                  \
    case 1: hipLaunchKernelGGL((KERNEL<1>), GRID, dim3(64), 0, stream, m); break;                 \
    case 2: hipLaunchKernelGGL((KERNEL<2>), GRID, dim3(64), 0, stream, m); break;                 \
    case 4: hipLaunchKernelGGL((KERNEL<4>), GRID, dim3(64), 0, stream, m); break;                 \
    case 8: hipLaunchKernelGGL((KERNEL<8>), GRID, dim3(64), 0, stream, m); break;                 \
    default: hipLaunchKernelGGL((KERNEL<16>), GRID, dim3(64), 0, stream, m); break;               \
    }
    MB_MIMO_R(k_mb_prep_bc, dim3(nseg_all));
    hipLaunchKernelGGL(k_mb_prep_x, dim3((unsigned)((L * H * P + 255) / 256), (unsigned)batch), dim3(256), 0,
                       stream, m);
    if (dh_out)
        hipLaunchKernelGGL(k_tb_rot_dh, dim3((unsigned)(((N / 2) * P + 255) / 256), (unsigned)(batch * H)),
                           dim3(256), 0, stream, t);
    BwdArgs a{};
    a.X = m.X2; a.ld = m.ld2; a.B = m.B2; a.C = m.C2; a.h0 = h0; a.dY = m.dY2; a.dh_out = dh_out ? m.dh2 : nullptr;
    a.dX = m.dX2; a.dld = m.dld2; a.dB = m.dB2; a.dC = m.dC2; a.dh0 = dh0;
    a.st = (float*)w;
    a.lam = (float*)(w + pl.ssd.off_lam);
    a.tot = (float*)(w + pl.ssd.off_tot);
    a.fin = (float*)(w + pl.ssd.off_fin);
    a.h_final = m.hfin;
    a.L = (int)((3 * R - 1) * L); a.H = (int)H; a.G = (int)H; a.N = (int)N; a.P = (int)P;
    a.nch = (int)pl.ssd.nch; a.nfin = (int)pl.ssd.nfin;
    mb_status st;
    if (N == 128)
        st = P == 64 ? bwd_launch<128, 64>(a, batch, stream) : bwd_launch<128, 32>(a, batch, stream);
    else
        st = P == 64 ? bwd_launch<64, 64>(a, batch, stream) : bwd_launch<64, 32>(a, batch, stream);
    if (st != MB_OK) return st;
    hipLaunchKernelGGL(k_mb_post_x, dim3((unsigned)(batch * L * H)), dim3(64), 0, stream, m);
    MB_MIMO_R(k_mb_post_bc, dim3((unsigned)(batch * L * H)));
#undef MB_MIMO_R
    if (theta) {
        if (dh_out) hipLaunchKernelGGL(k_tb_hterm, dim3((unsigned)(batch * H)), dim3(64), 0, stream, t);
        hipLaunchKernelGGL(k_tb_segsum, dim3(nseg_all), dim3(64), 0, stream, t, (const float*)m.dTh, m.seg);
        hipLaunchKernelGGL(k_tb_theta, dim3(nseg_all), dim3(64), 0, stream, t);
    }
    return check_launch();
}
