// m1.hip -- Mamba-1 selective scan and single-token decode step for gfx950.
//
// Recurrence (TorchMamba README, Math notes M1; burn_mamba Mamba1 docs,
// selective_scan / selective_scan_step), exponential-Euler discretisation:
//     h_t[c,n] = exp(dt_t[c] A[c,n]) h_{t-1}[c,n] + dt_t[c] B_t[n] x_t[c]
//     y_t[c]   = sum_n C_t[n] h_t[c,n] + Dskip[c] x_t[c]
//
// Scans (layouts detailed at the kernels): every lane keeps several (channel,
// state) chains in registers and walks the whole sequence; one hardware exp2
// per (t, c, n) element.
//   k_m1_scan_w  fp32, N in {4, 8, 16, 32}: independent waves of 16 channels,
//                tiles copied into LDS by DMA, no barriers.
//   k_m1_scan    any other case: workgroups of 64 channels x ceil(N/4) waves,
//                partial sums over states reduced through LDS once per tile.
#include <algorithm>

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

// Scan layout for fp32 with N = 4 S, S in {1, 2, 4, 8}: one wave per (batch,
// 16 channels), nothing shared between waves and no barriers; a workgroup is
// four such waves (64 channels), so that its waves sit on the four SIMDs of one
// compute unit.  Lane l
// holds channel c0 + l / 4 and the S states n = S (l % 4) + s.  Tiles of T
// steps of dt and x (the wave's 16 channels) and of B and C (all N states) go
// global -> LDS by LDS DMA one tile ahead, into two separate buffers.  Per step
// a lane updates its S chains and sums C.h over them; the four lanes of a
// channel are summed per group of four steps by a two-stage exchange inside
// the quad, after which lane q holds step 4i + q, so one store writes four
// steps of the wave's 16 channels.  Every store is issued by the whole wave
// (lanes past D store to an offset that the buffer range check drops), so the
// number of memory operations issued after a tile's DMA is fixed and the wait
// for that DMA is exact.
constexpr int kScanT = 32;   // steps per tile

// one tile in LDS: dt[T][16], x[T][16], B[T][N], C[T][N], and with the block
// prologue / epilogue the gate z[T][16]
template <int S, bool Z = false, int T = kScanT>
struct ScanTile {
    float v[T * (32 + 8 * S + (Z ? 16 : 0))];
};

// The block prologue / epilogue of the fused scan (its extra inputs).
struct Fuse {
    const float* conv_w;    // (D, K), K <= 4
    const float* conv_b;    // (D) or NULL
    const float* x_hist;    // (batch, K-1, D) raw inputs before the call, or NULL
    const float* dt_bias;   // (D) or NULL
    const float* z;         // (batch, L, D) gate, or NULL
    int K;
    float* ck;              // checkpoint mode: (batch, ntiles, D, N) state entering every tile
};

// Sequence blocks (the cross-block carry of the scan).  The sequence is cut
// into nblk blocks of blk_tiles tiles.  The carry pass (MODE 1) runs blocks
// 0 .. nblk - 2 at once, each on its own: block 0 from h0, the others from
// zero, and writes per (batch, block) the block's end state and the sum of its
// step sizes.  Since the decay product of a block is exp(A sum dt), the pair
// (exp(A sdt_k), hloc_k) of block k composes with the state h entering it as
// exp(A sdt_k) h + hloc_k, and the scan pass (MODE 0) starts block j from the
// composition of blocks 0 .. j - 1.  nblk <= 1: the whole sequence in one
// block, no carry pass, no workspace.
struct Seq {
    int nblk, blk_tiles, units;   // units: batch x channel groups (workgroups per block)
    float* hblk;   // (batch, nblk, D, N): slot 0 = h0 (zeros when NULL), slot k + 1 = end of block k
    float* sdt;    // (batch, nblk, D): sum of dt over block k
};

// lane j's value of a quad, to every lane of the quad
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), J * 0x55, 0xF, 0xF, true));
}

// SiLU and softplus through the hardware exp2 / log2 / reciprocal
__device__ __forceinline__ float silu_f(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-v * kLog2e));
}
__device__ __forceinline__ float softplus_f(float v) {
    // max(v, 0) + log(1 + e^-|v|); below 1/16 the log1p series to u^5 (its
    // truncation is under 2e-7 relative), since forming 1 + u there would lose
    // the low bits of u
    // Both branches are computed and one is selected: no divergent branch.
    const float u = exp2_fast(-fabsf(v) * kLog2e);
    const float ser = u * (1.0f - u * (0.5f - u * (1.0f / 3.0f - u * (0.25f - 0.2f * u))));
    const float lg = __builtin_amdgcn_logf(1.0f + u) * 0.6931471805599453f;
    const float l = u < 0.0625f ? ser : lg;
    return fmaxf(v, 0.0f) + l;
}

// s_waitcnt vmcnt(N), other counters unconstrained
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) float lds_f;
typedef __attribute__((address_space(3))) const float lds_cf;
typedef float fv2 __attribute__((ext_vector_type(2)));
typedef float fv4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const fv2 lds_cf2;
typedef __attribute__((address_space(3))) const fv4 lds_cf4;

template <int S>
__device__ __forceinline__ void lds_row(lds_cf* p, float* o) {
    if constexpr (S == 1) {
        o[0] = p[0];
    } else if constexpr (S == 2) {
        const fv2 v = *(lds_cf2*)p;
        o[0] = v.x;
        o[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < S; i += 4) {
            const fv4 v = *(lds_cf4*)(p + i);
            o[i] = v.x;
            o[i + 1] = v.y;
            o[i + 2] = v.z;
            o[i + 3] = v.w;
        }
    }
}

template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// LDS DMA of W bytes per lane: lane l's piece lands at dst + W l bytes
template <int W>
__device__ __forceinline__ void dma_lds(const Buf& src, lds_f* dst, uint32_t off) {
    static_assert(W == 4 || W == 16, "copy width");
    if constexpr (W == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.r, (__attribute__((address_space(3))) void*)dst, 4, off, 0, 0, 0);
}

// MODE 0: the scan (y and the final state) over the whole sequence or over one
// sequence block; MODE 1: the carry pass (state only, no C, no y).
template <int S, bool V16, bool FUSED = false, bool CK = false, int MODE = 0, int T = kScanT>
__global__ __launch_bounds__(256) void k_m1_scan_w(
    const float* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ Bm, const float* __restrict__ Cm, const float* __restrict__ Dskip,
    const float* h0, float* y, float* h_out, int L, int D, int n_cg, Fuse fz = Fuse{}, Seq sq = Seq{})
{
    constexpr bool CARRY = MODE == 1;
    static_assert(!(CARRY && (FUSED || CK)), "the carry pass is a plain state-only scan");
    constexpr int N = 4 * S;
    constexpr int NG = T / 4;                   // groups of four steps per tile
    constexpr bool BC16 = (T * N) % 256 == 0;   // 16-byte copies for the B / C tile
    constexpr int XW = V16 ? 16 : 4;            // bytes per lane of a dt / x copy
    constexpr int BW = BC16 ? 16 : 4;
    constexpr int NDX = T * 16 * 4 / (64 * XW); // copies per dt / x tile
    constexpr int NDB = T * N * 4 / (64 * BW);  // copies per B / C tile
    constexpr int NDMA = CARRY ? 2 * NDX + NDB : (FUSED ? 3 : 2) * NDX + 2 * NDB;   // copies per tile
    constexpr int OX = T * 16, OB = 2 * T * 16, OC = 2 * T * 16 + T * N;   // offsets in a tile
    constexpr int OZ = OC + T * N;
    // three tile buffers, separate objects so that a copy into one never orders
    // the reads of another
    __shared__ __attribute__((aligned(16))) ScanTile<S, FUSED, T> tb0[4];
    __shared__ __attribute__((aligned(16))) ScanTile<S, FUSED, T> tb1[4];
    __shared__ __attribute__((aligned(16))) ScanTile<S, FUSED, T> tb2[4];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    lds_f* const p0 = (lds_f*)tb0[w].v;
    lds_f* const p1 = (lds_f*)tb1[w].v;
    lds_f* const p2 = (lds_f*)tb2[w].v;

    // workgroup -> (sequence block, batch, channel group); blocks are the slowest
    const bool blocks = sq.nblk > 1;
    const int ub = blocks ? (int)(blockIdx.x % sq.units) : (int)blockIdx.x;
    const int jb = blocks ? (int)(blockIdx.x / sq.units) : 0;
    const int b = ub / n_cg, c0 = (ub % n_cg) * 64 + 16 * w;
    const int lane = threadIdx.x % 64;
    const int cl = lane >> 2, q = lane & 3;
    const int c = c0 + cl;
    const bool cok = c < D;
    const size_t row = (size_t)L * D;
    const Buf bx = make_buf(x + (size_t)b * row, row * 4);
    const Buf bdt = make_buf(dt + (size_t)b * row, row * 4);
    const Buf bB = make_buf(Bm + (size_t)b * L * N, (size_t)L * N * 4);
    const Buf bC = make_buf(Cm + (size_t)b * L * N, (size_t)L * N * 4);
    // without y (checkpoint mode) the stores fall outside a zero-size buffer
    const Buf by = make_buf(y ? y + (size_t)b * row : x, y ? row * 4 : 0);
    // the gate: without one, its copies read zeros (the copy count stays fixed)
    const Buf bz = make_buf(FUSED && fz.z ? fz.z + (size_t)b * row : x, FUSED && fz.z ? row * 4 : 0);

    // byte offset of this lane's piece of a tile copy, relative to the tile's first
    // step.  Tiles at or past the end read zeros (offsets past the buffer).
    const uint32_t xo = V16 ? (uint32_t)(((lane >> 2) * D + c0 + 4 * (lane & 3)) * 4)
                            : (uint32_t)(((lane >> 4) * D + c0 + (lane & 15)) * 4);
    const uint32_t bo = (uint32_t)(BW * lane);
    // byte offset of this lane's output (step q of a group, channel c) relative
    // to the group's first step; channels past D store past the buffer
    const uint32_t yl = cok ? (uint32_t)(q * D + c) * 4u : 0x80000000u;
    // tiles of this wave's sequence block: kb0 .. kb1 - 1
    const int ntiles = (L + T - 1) / T;
    const int kb0 = blocks ? jb * sq.blk_tiles : 0;
    const int kb1 = blocks ? min(ntiles, kb0 + sq.blk_tiles) : ntiles;
    auto dma = [&](int k, lds_f* dst) __attribute__((always_inline)) {
        const int t0 = __builtin_amdgcn_readfirstlane(k * T);   // uniform: scalar offsets
        // copies of tiles past the block read zeros without touching memory (the
        // copy count stays fixed, so the waits stay exact)
        const uint32_t kill = k < kb1 ? 0u : 0x80000000u;
#pragma unroll
        for (int m = 0; m < NDX; ++m) {
            const uint32_t off = (xo + (uint32_t)((t0 + XW * m) * D) * 4u) | kill;   // XW steps per copy
            dma_lds<XW>(bdt, dst + 16 * XW * m, off);
            dma_lds<XW>(bx, dst + OX + 16 * XW * m, off);
            if constexpr (FUSED) dma_lds<XW>(bz, dst + OZ + 16 * XW * m, off);
        }
#pragma unroll
        for (int m = 0; m < NDB; ++m) {
            const uint32_t off = (bo + (uint32_t)(t0 * N + 16 * BW * m) * 4u) | kill;
            dma_lds<BW>(bB, dst + OB + 16 * BW * m, off);
            if constexpr (!CARRY) dma_lds<BW>(bC, dst + OC + 16 * BW * m, off);
        }
    };

    // the operands of four steps, read from LDS one group ahead of their use
    struct Grp {
        float dt[4], x[4], b[4][S], c[4][S];
        float xs;     // x of step 4i + q (skip term); fused: the gate z of that step
        float gate;   // fused: SiLU of the gate of step 4i + q (1 without a gate)
    };
    auto read_grp = [&](lds_cf* cur, int i, Grp& g) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 4 * i + j;
            g.dt[j] = cur[t * 16 + cl];
            g.x[j] = cur[OX + t * 16 + cl];
            lds_row<S>(cur + OB + t * N + S * q, g.b[j]);
            if constexpr (!CARRY) lds_row<S>(cur + OC + t * N + S * q, g.c[j]);
        }
        if constexpr (!CARRY) g.xs = cur[(FUSED ? OZ : OX) + (4 * i + q) * 16 + cl];
    };

    float A2[S], h[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = S * q + s;
        A2[s] = cok ? A[(size_t)c * N + n] * kLog2e : 0.0f;
        h[s] = (cok && h0 && (!blocks || (CARRY && jb == 0))) ? h0[((size_t)b * D + c) * N + n] : 0.0f;
    }
    // the state entering the block
    auto slot = [&](int k) __attribute__((always_inline)) {
        return sq.hblk + (((size_t)b * sq.nblk + k) * D + c) * N + S * q;
    };
    if (blocks && cok) {
        if constexpr (CARRY) {
            // block 0 keeps the initial state for the scan pass (h0 itself may
            // be overwritten by the scan pass as its h_out)
            if (jb == 0) {
#pragma unroll
                for (int s = 0; s < S; ++s) slot(0)[s] = h[s];
            }
        } else if (jb == 0) {
#pragma unroll
            for (int s = 0; s < S; ++s) h[s] = slot(0)[s];
        } else {
            // compose (exp(A sdt_k), hloc_k) over the blocks before this one
#pragma unroll
            for (int s = 0; s < S; ++s) h[s] = slot(1)[s];
            for (int k = 1; k < jb; ++k) {
                const float sd = sq.sdt[((size_t)b * sq.nblk + k) * D + c];
                const float* hl = slot(k + 1);
#pragma unroll
                for (int s = 0; s < S; ++s) h[s] = fmaf(exp2_fast(sd * A2[s]), h[s], hl[s]);
            }
        }
    }
    const float Dv = (cok && Dskip) ? Dskip[c] : 0.0f;
    float sdt_acc = 0.0f;   // carry pass: sum of this channel's step sizes over the block
    const bool lo = (q & 2) == 0, ev = (q & 1) == 0;

    // fused: the convolution taps (right-aligned to four), the biases and the
    // raw inputs of the three steps before the current group
    float cw[4] = {0.0f, 0.0f, 0.0f, 0.0f}, cbv = 0.0f, dtb = 0.0f, xw[3] = {0.0f, 0.0f, 0.0f};
    if constexpr (FUSED) {
        const int cc = cok ? c : 0;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int k = kk - (4 - fz.K);
            cw[kk] = k >= 0 ? fz.conv_w[(size_t)cc * fz.K + k] : 0.0f;
        }
        cbv = fz.conv_b ? fz.conv_b[cc] : 0.0f;
        dtb = fz.dt_bias ? fz.dt_bias[cc] : 0.0f;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int hk = j - 3 + (fz.K - 1);   // x_hist holds steps -(K-1) .. -1
            xw[j] = (fz.x_hist && hk >= 0 && cok) ? fz.x_hist[((size_t)b * (fz.K - 1) + hk) * D + c] : 0.0f;
        }
    }

    // fused: replace a group's raw x and dt by the convolved, activated input
    // and the step size; every lane forms the four convolution sums, applies
    // SiLU and softplus to its own step tg + q only and shares the results
    // within the quad.  xs becomes the activated input of step tg + q (skip
    // term) and gate SiLU(z) of that step.
    auto prologue = [&](Grp& g, int tg) __attribute__((always_inline)) {
        const float win[7] = {xw[0], xw[1], xw[2], g.x[0], g.x[1], g.x[2], g.x[3]};
        float pre[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            pre[j] = fmaf(cw[3], win[j + 3], fmaf(cw[2], win[j + 2], fmaf(cw[1], win[j + 1], fmaf(cw[0], win[j], cbv))));
        // element q of four, by two selects on the bits of q (a chained select on
        // q would be lowered to an indexed private array)
        auto own = [&](const float* v) __attribute__((always_inline)) {
            const float a = ev ? v[0] : v[1], bb = ev ? v[2] : v[3];
            return lo ? a : bb;
        };
        const float xq = silu_f(own(pre));
        // steps past the sequence keep the state: step size zero (a factor,
        // not a branch)
        const float dq = softplus_f(own(g.dt) + dtb) * (tg + q < L ? 1.0f : 0.0f);
        g.gate = fz.z ? silu_f(g.xs) : 1.0f;
        g.xs = xq;
        xw[0] = g.x[1]; xw[1] = g.x[2]; xw[2] = g.x[3];
        g.x[0] = quad_bcast<0>(xq); g.x[1] = quad_bcast<1>(xq);
        g.x[2] = quad_bcast<2>(xq); g.x[3] = quad_bcast<3>(xq);
        g.dt[0] = quad_bcast<0>(dq); g.dt[1] = quad_bcast<1>(dq);
        g.dt[2] = quad_bcast<2>(dq); g.dt[3] = quad_bcast<3>(dq);
    };

    Grp g;
    dma(kb0, p0);
    vm_wait<0>();         // the block's first tile (and the initial state) has arrived
    asm volatile("" ::: "memory");
    dma(kb0 + 1, p1);
    read_grp(p0, 0, g);
    if constexpr (FUSED) prologue(g, 0);

    // tile k: copies of tile k + 2 go out first; the operands of its groups are
    // read one group ahead, the last group reading the first of tile k + 1
    auto tile = [&](int k, lds_cf* cur, lds_f* nxt, lds_f* nxt2) __attribute__((always_inline)) {
        if constexpr (CK) {
            // the state entering tile k (issued before the copies of tile k + 2:
            // the waits below stay exact or conservative)
            if (cok) {
                float* dst = fz.ck + (((size_t)b * ntiles + k) * D + c) * N + S * q;
#pragma unroll
                for (int s = 0; s < S; ++s) dst[s] = h[s];
            }
        }
        dma(k + 2, nxt2);
        const int t0 = k * T;
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            Grp gn;
            if (i + 1 < NG) {
                read_grp(cur, i + 1, gn);
            } else {
                // tile k + 1's copies were followed by at most the previous
                // tile's stores, tile k + 2's copies and this tile's first NG - 1
                // stores (the carry pass stores nothing)
                vm_wait<CARRY ? NDMA : NDMA + NG - 1>();
                asm volatile("" ::: "memory");
                read_grp(nxt, 0, gn);
            }
            // keep the reads here, a whole group ahead of their use
            __builtin_amdgcn_sched_barrier(0);
            float xcv[4], dtev[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xcv[j] = g.x[j];
                dtev[j] = g.dt[j];
            }
            if constexpr (CARRY) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float dtv = dtev[j];
                    const float dtx = dtv * xcv[j];
#pragma unroll
                    for (int s = 0; s < S; ++s) h[s] = fmaf(exp2_fast(dtv * A2[s]), h[s], dtx * g.b[j][s]);
                    sdt_acc += dtv;
                }
                g = gn;
                continue;
            }
            float ps[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float dtv = dtev[j];
                const float dtx = dtv * xcv[j];
                float p = 0.0f;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    h[s] = fmaf(exp2_fast(dtv * A2[s]), h[s], dtx * g.b[j][s]);
                    p = fmaf(g.c[j][s], h[s], p);
                }
                ps[j] = p;
            }
            // sum over the quad: after the exchange lane q holds step 4i + q
            float k0 = lo ? ps[0] : ps[2], s0 = lo ? ps[2] : ps[0];
            float k1 = lo ? ps[1] : ps[3], s1 = lo ? ps[3] : ps[1];
            k0 += quad_swap<0x4E>(s0);
            k1 += quad_swap<0x4E>(s1);
            float kk = ev ? k0 : k1;
            const float ss = ev ? k1 : k0;
            kk += quad_swap<0xB1>(ss);
            if constexpr (FUSED)
                kk = fmaf(Dv, g.xs, kk) * g.gate;
            else
                kk = fmaf(Dv, g.xs, kk);
            // the lane's part of the offset is fixed; the group's step adds a
            // uniform term (steps past the sequence land past the buffer)
            const uint32_t off = yl + (uint32_t)((t0 + 4 * i) * D) * 4u;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(kk), by.r, off, 0, 0);
            // fused: the next group's prologue, a group ahead of its use, so that
            // its dependent chain overlaps this group's recurrence
            if constexpr (FUSED) prologue(gn, t0 + 4 * i + 4);
            g = gn;
        }
    };
    for (int k = kb0; k < kb1; k += 3) {
        tile(k, p0, p1, p2);
        if (k + 1 < kb1) tile(k + 1, p1, p2, p0);
        if (k + 2 < kb1) tile(k + 2, p2, p0, p1);
    }
    vm_wait<0>();   // no copy into LDS may be in flight when the wave ends
    if constexpr (CARRY) {
        if (cok) {
#pragma unroll
            for (int s = 0; s < S; ++s) slot(jb + 1)[s] = h[s];
            if (q == 0) sq.sdt[((size_t)b * sq.nblk + jb) * D + c] = sdt_acc;
        }
    } else if (h_out && cok && (!blocks || jb == sq.nblk - 1)) {
#pragma unroll
        for (int s = 0; s < S; ++s) h_out[((size_t)b * D + c) * N + S * q + s] = h[s];
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

// ---------------------------------------------------------------------------
// Backward of the Mamba-1 scan (fp32, N in {4, 8, 16}), the vector-Jacobian
// product of (y, h_out) for (dy, dh_out).  The lane layout of k_m1_scan_w: a
// wave holds 16 channels x 4 lanes, lane (cl, q) the states n = S q + s.  Tiles
// of 32 steps are walked last to first; each starts from the checkpointed state
// entering it (k_m1_scan_w in checkpoint mode), recomputes its 32 states in
// registers and runs the adjoint G back through them, with a_t = e^{dt_t A}:
//     G += C_t dy_t;   dB_t += G dt x;   dC_t += h_t dy_t;   U = sum_n G B_t
//     w = G a_t h_{t-1};   V = sum_n A w;   dA += dt w;   G *= a_t
//     dx_t = dt U + Dskip dy_t,   ddt_t = x U + V,   dDskip += dy x.
// U and V are summed over the quad by the forward's exchange (lane q then holds
// step 4i + q); dB and dC of four steps are summed over the wave's 16 channels
// by a halving butterfly (each exchange halves the values a lane keeps), over the
// workgroup's four waves in LDS once per tile, and over the workgroups by
// k_m1_bwd_reduce, in a fixed order (deterministic).
// ---------------------------------------------------------------------------
// a where the mask is all ones, b where it is zero (bitwise, so that a choice
// between two elements of a register array is never turned into an index)
__device__ __forceinline__ float bsel(uint32_t m, float a, float b) {
    return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}

struct M1Bwd {
    const float *x, *dt, *A, *B, *C, *Dskip, *dy, *dh_out, *ck;
    float *dx, *ddt, *dh0;
    float* pBC;   // (2, batch, n_cg, L, N) per-workgroup partial dB (0) and dC (1)
    float* pA;    // (batch, D, N) per-batch dA
    float* pD;    // (batch, D) per-batch dDskip
    int L, D, n_cg;
};

template <int S, bool V16>
__global__ __launch_bounds__(256) void k_m1_bwd(M1Bwd a) {
    constexpr int T = kScanT;
    constexpr int N = 4 * S;
    constexpr int NG = T / 4;
    constexpr bool BC16 = (T * N) % 256 == 0;
    constexpr int XW = V16 ? 16 : 4;
    constexpr int BW = BC16 ? 16 : 4;
    constexpr int NDX = T * 16 * 4 / (64 * XW);
    constexpr int NDB = T * N * 4 / (64 * BW);
    constexpr int OX = T * 16, OB = 2 * T * 16, OC = 2 * T * 16 + T * N, OZ = OC + T * N;
    constexpr int NV = 8 * S;                    // dB, dC values of four steps per lane
    __shared__ __attribute__((aligned(16))) ScanTile<S, true> tb0[4];
    __shared__ __attribute__((aligned(16))) ScanTile<S, true> tb1[4];
    __shared__ float sAcc[2][4][2][T][N];        // per tile parity and wave: dB, dC of the tile's steps
    constexpr int NFL = 2 * T * N / 256;         // flush stores per thread and tile

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    lds_f* const p0 = (lds_f*)tb0[w].v;
    lds_f* const p1 = (lds_f*)tb1[w].v;
    const int L = a.L, D = a.D;
    const int batch = gridDim.x / a.n_cg;
    const int b = blockIdx.x / a.n_cg, cg = blockIdx.x % a.n_cg, c0 = cg * 64 + 16 * w;
    const int lane = threadIdx.x % 64;
    const int cl = lane >> 2, q = lane & 3;
    const int c = c0 + cl;
    const bool cok = c < D;
    const size_t row = (size_t)L * D;
    const Buf bx = make_buf(a.x + (size_t)b * row, row * 4);
    const Buf bdt = make_buf(a.dt + (size_t)b * row, row * 4);
    const Buf bdy = make_buf(a.dy + (size_t)b * row, row * 4);
    const Buf bB = make_buf(a.B + (size_t)b * L * N, (size_t)L * N * 4);
    const Buf bC = make_buf(a.C + (size_t)b * L * N, (size_t)L * N * 4);
    const Buf bdx = make_buf(a.dx + (size_t)b * row, row * 4);
    const Buf bddt = make_buf(a.ddt + (size_t)b * row, row * 4);

    // tile copies as in k_m1_scan_w, with dy in the third stream
    const uint32_t xo = V16 ? (uint32_t)(((lane >> 2) * D + c0 + 4 * (lane & 3)) * 4)
                            : (uint32_t)(((lane >> 4) * D + c0 + (lane & 15)) * 4);
    const uint32_t bo = (uint32_t)(BW * lane);
    auto dma = [&](int k, lds_f* dst) __attribute__((always_inline)) {
        const int t0 = k * T;
#pragma unroll
        for (int m = 0; m < NDX; ++m) {
            const uint32_t off = xo + (uint32_t)((t0 + XW * m) * D) * 4u;
            dma_lds<XW>(bdt, dst + 16 * XW * m, off);
            dma_lds<XW>(bx, dst + OX + 16 * XW * m, off);
            dma_lds<XW>(bdy, dst + OZ + 16 * XW * m, off);
        }
#pragma unroll
        for (int m = 0; m < NDB; ++m) {
            const uint32_t off = bo + (uint32_t)(t0 * N + 16 * BW * m) * 4u;
            dma_lds<BW>(bB, dst + OB + 16 * BW * m, off);
            dma_lds<BW>(bC, dst + OC + 16 * BW * m, off);
        }
    };

    float A2[S], Ar[S], G[S], dA[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int n = S * q + s;
        Ar[s] = cok ? a.A[(size_t)c * N + n] : 0.0f;
        A2[s] = Ar[s] * kLog2e;
        G[s] = (cok && a.dh_out) ? a.dh_out[((size_t)b * D + c) * N + n] : 0.0f;
        dA[s] = 0.0f;
    }
    const float Dv = (cok && a.Dskip) ? a.Dskip[c] : 0.0f;
    float dDacc = 0.0f;
    const uint32_t mlo = (q & 2) == 0 ? ~0u : 0u, mev = (q & 1) == 0 ? ~0u : 0u;
    const int ntiles = (L + T - 1) / T;
    const float* ckb = a.ck + ((size_t)b * ntiles * D + (cok ? c : 0)) * N + S * q;
    float ckr[S];
    // one vector load (S consecutive floats)
    auto ld_ck = [&](int k) __attribute__((always_inline)) {
        const float* p = ckb + (size_t)k * D * N;
        if constexpr (S == 4) {
            const float4 v = *(const float4*)p;
            ckr[0] = v.x; ckr[1] = v.y; ckr[2] = v.z; ckr[3] = v.w;
        } else if constexpr (S == 2) {
            const float2 v = *(const float2*)p;
            ckr[0] = v.x; ckr[1] = v.y;
        } else {
            ckr[0] = p[0];
        }
    };

    auto tile = [&](int k, lds_cf* cur, lds_f* nxt, int par) __attribute__((always_inline)) {
        // tile k's copies were followed by at most one checkpoint load, the
        // previous tile's 2 NG stores of dx and ddt and its NFL partial-sum stores
        vm_wait<1 + 2 * NG + NFL>();
        asm volatile("" ::: "memory");
        float hst[S];
#pragma unroll
        for (int s = 0; s < S; ++s) hst[s] = ckr[s];
        if (k > 0) {
            dma(k - 1, nxt);
            ld_ck(k - 1);
        }
        const int t0 = k * T;
        // the tile's states, recomputed from the checkpoint
        float hs[T][S];
        {
            float h[S];
#pragma unroll
            for (int s = 0; s < S; ++s) h[s] = hst[s];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const float dtv = cur[t * 16 + cl];
                const float dtx = dtv * cur[OX + t * 16 + cl];
                float bb[S];
                lds_row<S>(cur + OB + t * N + S * q, bb);
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    h[s] = fmaf(exp2_fast(dtv * A2[s]), h[s], dtx * bb[s]);
                    hs[t][s] = h[s];
                }
            }
        }
        // the adjoint, back through the tile, four steps at a time
#pragma unroll
        for (int i = NG - 1; i >= 0; --i) {
            float U[4], V[4], vals[NV];
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                const int t = 4 * i + j;
                const float dtv = cur[t * 16 + cl];
                const float xv = cur[OX + t * 16 + cl];
                // lanes past the last channel read the next row's values: their dy
                // is zeroed so that they add nothing to the channel sums of dB, dC
                const float dyv = cok ? cur[OZ + t * 16 + cl] : 0.0f;
                const float dtx = dtv * xv;
                float bb[S], cc[S];
                lds_row<S>(cur + OB + t * N + S * q, bb);
                lds_row<S>(cur + OC + t * N + S * q, cc);
                float u = 0.0f, v = 0.0f;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    G[s] = fmaf(cc[s], dyv, G[s]);
                    vals[(j * S + s) * 2 + 0] = G[s] * dtx;
                    vals[(j * S + s) * 2 + 1] = hs[t][s] * dyv;
                    u = fmaf(G[s], bb[s], u);
                    const float av = exp2_fast(dtv * A2[s]);
                    const float hp = t > 0 ? hs[t > 0 ? t - 1 : 0][s] : hst[s];
                    const float wv = G[s] * av * hp;
                    v = fmaf(Ar[s], wv, v);
                    dA[s] = fmaf(dtv, wv, dA[s]);
                    G[s] *= av;
                }
                U[j] = u;
                V[j] = v;
            }
            // sums over the quad: lane q then holds step 4i + q
            auto quad_sum = [&](float p0, float p1, float p2, float p3) __attribute__((always_inline)) {
                float k0 = bsel(mlo, p0, p2), s0 = bsel(mlo, p2, p0);
                float k1 = bsel(mlo, p1, p3), s1 = bsel(mlo, p3, p1);
                k0 += quad_swap<0x4E>(s0);
                k1 += quad_swap<0x4E>(s1);
                const float kk = bsel(mev, k0, k1), ss = bsel(mev, k1, k0);
                return kk + quad_swap<0xB1>(ss);
            };
            const float Uq = quad_sum(U[0], U[1], U[2], U[3]), Vq = quad_sum(V[0], V[1], V[2], V[3]);
            const int tq = 4 * i + q;
            const float dtq = cur[tq * 16 + cl], xq = cur[OX + tq * 16 + cl], dyq = cur[OZ + tq * 16 + cl];
            dDacc = fmaf(dyq, xq, dDacc);
            const uint32_t off = cok ? (uint32_t)((t0 + tq) * D + c) * 4u : 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(fmaf(dtq, Uq, Dv * dyq)), bdx.r, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(fmaf(xq, Uq, Vq)), bddt.r, off, 0, 0);
            // dB, dC summed over the wave's 16 channels (lane bits 2..5)
            int base = 0;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int m = 4 << st;
                const uint32_t up = (lane & m) != 0 ? ~0u : 0u;
                const int half = (NV >> st) / 2;          // values kept after this exchange
                if constexpr (true) {
                    if (half >= 1) {
#pragma unroll
                        for (int e = 0; e < NV / 2; ++e) {
                            if (e < half) {
                                const float send = bsel(up, vals[e], vals[e + half]);
                                const float keep = bsel(up, vals[e + half], vals[e]);
                                vals[e] = keep + __shfl_xor(send, m, 64);
                            }
                        }
                        base += (lane & m) != 0 ? half : 0;
                    } else {
                        vals[0] += __shfl_xor(vals[0], m, 64);
                    }
                }
            }
            // the lane keeps cnt values, original indices base .. base + cnt - 1
            // (after a final plain exchange the lanes with bit 5 set hold copies)
            if (NV >= 16 || (lane & 32) == 0) {
#pragma unroll
                for (int e = 0; e < NV / 16 + (NV < 16 ? 1 : 0); ++e) {
                    const int idx = base + e;
                    const int kind = idx & 1, js = idx >> 1;
                    const int j = js / S, sidx = js % S;
                    sAcc[par][w][kind][4 * i + j][S * q + sidx] = vals[e];
                }
            }
        }
        // the tile's per-wave sums are in LDS; the other parity's were read
        // out by every wave before this barrier, so the next tile may write them
        __syncthreads();
#pragma unroll
        for (int f = 0; f < NFL; ++f) {
            const int e = threadIdx.x + 256 * f;
            const int kind = e / (T * N), t = (e / N) % T, n = e % N;
            if (t0 + t < L) {
                const float v = (sAcc[par][0][kind][t][n] + sAcc[par][1][kind][t][n]) +
                                (sAcc[par][2][kind][t][n] + sAcc[par][3][kind][t][n]);
                a.pBC[((((size_t)kind * batch + b) * a.n_cg + cg) * L + t0 + t) * N + n] = v;
            }
        }
    };

    ld_ck(ntiles - 1);
    dma(ntiles - 1, p0);
    vm_wait<0>();   // the first tile and its checkpoint
    for (int k = ntiles - 1; k >= 0; k -= 2) {
        tile(k, p0, p1, 0);
        if (k - 1 >= 0) tile(k - 1, p1, p0, 1);
    }
    vm_wait<0>();   // no copy into LDS may be in flight when the wave ends
    dDacc += __shfl_xor(dDacc, 1, 64);
    dDacc += __shfl_xor(dDacc, 2, 64);
    if (cok) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const size_t e = ((size_t)b * D + c) * N + S * q + s;
            if (a.dh0) a.dh0[e] = G[s];
            a.pA[e] = dA[s];
        }
        if (q == 0) a.pD[(size_t)b * D + c] = dDacc;
    }
}

// Sums of the backward's partials in a fixed order: dB, dC over the channel
// groups (job 0), dA over the batch (job 1), dDskip over the batch (job 2).
__global__ __launch_bounds__(256) void k_m1_bwd_reduce(M1Bwd a, float* dB, float* dC, float* dA, float* dD,
                                                      int batch, int N) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int job = blockIdx.y;
    if (job == 0) {
        const int64_t per = (int64_t)batch * a.L * N;
        if (i >= 2 * per) return;
        const int kind = (int)(i / per);
        const int64_t r = i % per;
        const int64_t b = r / ((int64_t)a.L * N), tn = r % ((int64_t)a.L * N);
        const float* src = a.pBC + (((size_t)kind * batch + b) * a.n_cg) * a.L * N + tn;
        float v = 0.0f;
        for (int g = 0; g < a.n_cg; ++g) v += src[(size_t)g * a.L * N];
        (kind ? dC : dB)[r] = v;
    } else if (job == 1) {
        const int64_t dn = (int64_t)a.D * N;
        if (i >= dn) return;
        float v = 0.0f;
        for (int b = 0; b < batch; ++b) v += a.pA[(size_t)b * dn + i];
        dA[i] = v;
    } else {
        if (i >= a.D || !dD) return;
        float v = 0.0f;
        for (int b = 0; b < batch; ++b) v += a.pD[(size_t)b * a.D + i];
        dD[i] = v;
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

constexpr int kScanTB = 16;   // steps per tile of the sequence-block scan

struct M1Plan {
    int nblk, blk_tiles;
    size_t off_sdt, bytes;
};

// Sequence blocks of the fp32 scan (N in {4, 8, 16}, the k_m1_scan_w layout).
// The carry pass repeats most of the scan's work without its output, so blocks
// pay only where batch x channel groups leave SIMDs idle: with workgroups of
// four waves for at least three quarters of the SIMDs the scan runs in one
// block; otherwise in enough blocks for about three workgroups (three waves
// per SIMD) on every compute unit, each block at least four tiles long.
// Measured on MI355X (fp32, N 16, D 1536, cache flushed): batch 1, L 16384:
// 1.007 ms in one block, 0.186 ms in 32; batch 4, L 4096: 0.269 -> 0.182 ms
// in 8; batch 8, L 2048 (192 workgroups): 0.153 ms in one block, 0.175 in 4.
// Depends on the sizes and the device's compute-unit count only, so
// mb_workspace_size agrees with the call on the same device.
M1Plan m1_plan(int64_t batch, int64_t L, int64_t D, int64_t N) {
    M1Plan p{1, 0, 0, 0};
    if ((N != 4 && N != 8 && N != 16) || batch <= 0 || L <= 0 || D <= 0) return p;
    const int64_t units = batch * ((D + 63) / 64);
    const int64_t ntiles = (L + kScanTB - 1) / kScanTB;
    const int64_t cus = device_cu_count();
    if (4 * units >= 3 * cus) return p;
    int64_t nb = std::min<int64_t>((3 * cus + units - 1) / units, ntiles / 4);
    if (nb <= 1) return p;
    const int64_t bt = (ntiles + nb - 1) / nb;
    nb = (ntiles + bt - 1) / bt;
    if (nb <= 1 || units * nb > INT32_MAX) return p;
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    p.nblk = (int)nb;
    p.blk_tiles = (int)bt;
    p.off_sdt = al((size_t)(batch * nb * D * N) * 4);
    p.bytes = p.off_sdt + al((size_t)(batch * nb * D) * 4);
    return p;
}

template <int S, bool V16>
mb_status launch_scan_blocks(const float* x, const float* dt, const float* A, const float* B,
                             const float* C, const float* Dskip, const float* h0, float* y,
                             float* h_out, int64_t batch, int64_t L, int64_t D, const M1Plan& pl,
                             char* ws, hipStream_t stream) {
    const int n_cg = (int)((D + 63) / 64);
    const int units = (int)(batch * n_cg);
    const Seq sq{pl.nblk, pl.blk_tiles, units, (float*)ws, (float*)(ws + pl.off_sdt)};
    hipLaunchKernelGGL((k_m1_scan_w<S, V16, false, false, 1, kScanTB>), dim3((unsigned)(units * (pl.nblk - 1))),
                       dim3(256), 0, stream, x, dt, A, B, C, Dskip, h0, nullptr, nullptr, (int)L, (int)D,
                       n_cg, Fuse{}, sq);
    mb_status st = check_launch();
    if (st != MB_OK) return st;
    hipLaunchKernelGGL((k_m1_scan_w<S, V16, false, false, 0, kScanTB>), dim3((unsigned)(units * pl.nblk)),
                       dim3(256), 0, stream, x, dt, A, B, C, Dskip, h0, y, h_out, (int)L, (int)D, n_cg,
                       Fuse{}, sq);
    return check_launch();
}

template <typename IO>
mb_status launch_scan(const void* x, const void* dt, const float* A, const void* B,
                      const void* C, const float* Dskip, const float* h0, void* y,
                      float* h_out, int64_t batch, int64_t L, int64_t D, int64_t N,
                      void* ws, size_t ws_bytes, hipStream_t stream)
{
    if constexpr (sizeof(IO) == 4) {
        // 16-byte LDS copies need 16-byte aligned rows
        const bool aligned = ((((uintptr_t)x | (uintptr_t)dt | (uintptr_t)B | (uintptr_t)C) & 15) == 0);
        if (aligned && (N == 4 || N == 8 || N == 16 || N == 32)) {
            const int n_cg = (int)((D + 63) / 64);
            const int n_wg = (int)(batch * n_cg);
            const bool v16 = D % 4 == 0;
            const M1Plan pl = m1_plan(batch, L, D, N);
            if (ws && pl.nblk > 1) {
                if (ws_bytes < pl.bytes || ((uintptr_t)ws & 255)) return MB_ERR_WORKSPACE;
#define MB_SCAN_B(S)                                                                                   \
    return v16 ? launch_scan_blocks<S, true>((const float*)x, (const float*)dt, A, (const float*)B,        \
                                             (const float*)C, Dskip, h0, (float*)y, h_out, batch, L, D, pl, \
                                             (char*)ws, stream)                                            \
               : launch_scan_blocks<S, false>((const float*)x, (const float*)dt, A, (const float*)B,       \
                                              (const float*)C, Dskip, h0, (float*)y, h_out, batch, L, D,    \
                                              pl, (char*)ws, stream)
                switch (N) {
                case 4: MB_SCAN_B(1);
                case 8: MB_SCAN_B(2);
                default: MB_SCAN_B(4);
                }
#undef MB_SCAN_B
            }
#define MB_SCAN_W(S)                                                                          \
    do {                                                                                     \
        if (v16)                                                                             \
            hipLaunchKernelGGL((k_m1_scan_w<S, true>), dim3(n_wg), dim3(256), 0, stream,       \
                               (const float*)x, (const float*)dt, A, (const float*)B,        \
                               (const float*)C, Dskip, h0, (float*)y, h_out, (int)L, (int)D, \
                               n_cg);                                                        \
        else                                                                                 \
            hipLaunchKernelGGL((k_m1_scan_w<S, false>), dim3(n_wg), dim3(256), 0, stream,     \
                               (const float*)x, (const float*)dt, A, (const float*)B,        \
                               (const float*)C, Dskip, h0, (float*)y, h_out, (int)L, (int)D, \
                               n_cg);                                                        \
    } while (0)
            switch (N) {
            case 4: MB_SCAN_W(1); break;
            case 8: MB_SCAN_W(2); break;
            case 16: MB_SCAN_W(4); break;
            default: MB_SCAN_W(8); break;
            }
#undef MB_SCAN_W
            return check_launch();
        }
    }
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
    // one (channel, state quad) item per thread: measured on MI355X at batch 256,
    // D 1536, N 16 after a last-level-cache flush, 11.4 us per call against 11.7
    // with two items per thread and 13.2 with four
#define MB_STEP_Q(NQ)                                                                         \
    do {                                                                                     \
        const dim3 grid((unsigned)((D * NQ + 255) / 256), (unsigned)batch);                  \
        if (vec_bc)                                                                          \
            hipLaunchKernelGGL((k_m1_step_q<NQ, IO, true, 1>), grid, dim3(256), 0, stream,   \
                               (const IO*)x, (const IO*)dt, A, (const IO*)B, (const IO*)C,   \
                               Dskip, h_in, h_out, (IO*)y, (int)D);                          \
        else                                                                                 \
            hipLaunchKernelGGL((k_m1_step_q<NQ, IO, false, 1>), grid, dim3(256), 0, stream,  \
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
                                       mb_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (!dtype_ok(dtype)) return MB_ERR_DTYPE;
    if (batch < 0 || L < 0 || D < 0 || N < 1 || N > 64) return MB_ERR_SHAPE;
    if (batch > INT32_MAX || L > INT32_MAX || D > INT32_MAX) return MB_ERR_SHAPE;
    const size_t es = dtype_size(dtype);
    const size_t n_x = (size_t)(batch * L * D), n_b = (size_t)(batch * L * N);
    const size_t n_h = (size_t)(batch * D * N);
    if (batch * ((D + 63) / 64) > INT32_MAX) return MB_ERR_SHAPE;
    // one batch row is addressed with 32-bit byte offsets (tile padding included)
    if ((L + 64) * D * 4 >= ((int64_t)1 << 31) || (L + 64) * N * 4 >= ((int64_t)1 << 31)) return MB_ERR_SHAPE;
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
    if (ws) {
        const size_t need = m1_plan(batch, L, D, N).bytes;
        if (need && (overlaps_any(ws, need, ins, 7) || overlaps(ws, need, y, n_x * es) ||
                     overlaps(ws, need, h_out, h_out ? n_h * 4 : 0)))
            return MB_ERR_ALIAS;
    }
    if (dtype == MB_F32)
        return launch_scan<float>(x, dt, A, B, C, Dskip, h0, y, h_out, batch, L, D, N, ws, ws_bytes, stream);
    return launch_scan<bf16>(x, dt, A, B, C, Dskip, h0, y, h_out, batch, L, D, N, nullptr, 0, stream);
}

extern "C" mb_status mb_selective_scan_fused(const float* x, const float* conv_w, const float* conv_b,
                                             const float* x_hist, const float* dt, const float* dt_bias,
                                             const float* A, const float* B, const float* C,
                                             const float* Dskip, const float* z, const float* h0, float* y,
                                             float* h_out, int64_t batch, int64_t L, int64_t D, int64_t N,
                                             int64_t K, mb_dtype dtype, hipStream_t stream)
{
    if (dtype != MB_F32) return MB_ERR_DTYPE;
    if (batch < 0 || L < 0 || D < 0 || K < 1 || K > 4) return MB_ERR_SHAPE;
    // three tiles of dt, x, z, B and C per wave fit the LDS up to N = 16
    if (N != 4 && N != 8 && N != 16) return MB_ERR_SHAPE;
    if (batch > INT32_MAX || L > INT32_MAX || D > INT32_MAX) return MB_ERR_SHAPE;
    const size_t n_x = (size_t)(batch * L * D), n_b = (size_t)(batch * L * N);
    const size_t n_h = (size_t)(batch * D * N);
    if (batch * ((D + 63) / 64) > INT32_MAX) return MB_ERR_SHAPE;
    if ((L + 64) * D * 4 >= ((int64_t)1 << 31) || (L + 64) * N * 4 >= ((int64_t)1 << 31)) return MB_ERR_SHAPE;
    if (n_x && (!x || !dt || !y)) return MB_ERR_NULL;
    if (n_b && (!B || !C)) return MB_ERR_NULL;
    if (D > 0 && (!A || !conv_w)) return MB_ERR_NULL;
    // the tiles are copied with 16-byte pieces of rows
    if (((uintptr_t)x | (uintptr_t)dt | (uintptr_t)B | (uintptr_t)C | (uintptr_t)z) & 15) return MB_ERR_ALIGN;
    const Span ins[] = {{x, n_x * 4}, {dt, n_x * 4}, {B, n_b * 4}, {C, n_b * 4},
                        {A, (size_t)(D * N) * 4}, {Dskip, Dskip ? (size_t)D * 4 : 0},
                        {conv_w, (size_t)(D * K) * 4}, {conv_b, conv_b ? (size_t)D * 4 : 0},
                        {dt_bias, dt_bias ? (size_t)D * 4 : 0}, {z, z ? n_x * 4 : 0},
                        {x_hist, x_hist ? (size_t)(batch * (K - 1) * D) * 4 : 0}, {h0, h0 ? n_h * 4 : 0}};
    if (overlaps_any(y, n_x * 4, ins, 12)) return MB_ERR_ALIAS;
    if (h_out) {
        if (overlaps_any(h_out, n_h * 4, ins, 11)) return MB_ERR_ALIAS;
        if (h0 && h0 != h_out && overlaps(h_out, n_h * 4, h0, n_h * 4)) return MB_ERR_ALIAS;
        if (overlaps(h_out, n_h * 4, y, n_x * 4)) return MB_ERR_ALIAS;
    }
    if (batch == 0 || D == 0) return MB_OK;
    if (L == 0) return copy_state(h0, h_out, (int64_t)n_h, stream);
    const Fuse fz{conv_w, conv_b, K > 1 ? x_hist : nullptr, dt_bias, z, (int)K};
    const int n_cg = (int)((D + 63) / 64);
    const int n_wg = (int)(batch * n_cg);
    const bool v16 = D % 4 == 0;
#define MB_SCAN_F(S)                                                                          \
    do {                                                                                     \
        if (v16)                                                                             \
            hipLaunchKernelGGL((k_m1_scan_w<S, true, true>), dim3(n_wg), dim3(256), 0, stream, \
                               x, dt, A, B, C, Dskip, h0, y, h_out, (int)L, (int)D, n_cg, fz);  \
        else                                                                                 \
            hipLaunchKernelGGL((k_m1_scan_w<S, false, true>), dim3(n_wg), dim3(256), 0, stream, \
                               x, dt, A, B, C, Dskip, h0, y, h_out, (int)L, (int)D, n_cg, fz);  \
    } while (0)
    switch (N) {
    case 4: MB_SCAN_F(1); break;
    case 8: MB_SCAN_F(2); break;
    default: MB_SCAN_F(4); break;
    }
#undef MB_SCAN_F
    return check_launch();
}

namespace mb {
namespace {
struct M1BwdPlan {
    size_t off_pbc, off_pa, off_pd, bytes;
};
M1BwdPlan m1_bwd_plan(int64_t batch, int64_t L, int64_t D, int64_t N) {
    M1BwdPlan p{};
    const int64_t ntiles = (L + kScanT - 1) / kScanT, n_cg = (D + 63) / 64;
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    size_t off = al((size_t)(batch * ntiles * D * N) * 4);                 // checkpoints
    p.off_pbc = off;
    off += al((size_t)(2 * batch * n_cg * L * N) * 4);
    p.off_pa = off;
    off += al((size_t)(batch * D * N) * 4);
    p.off_pd = off;
    off += al((size_t)(batch * D) * 4);
    p.bytes = off;
    return p;
}
bool m1_bwd_dims_ok(int64_t batch, int64_t L, int64_t D, int64_t N) {
    if (batch < 0 || L < 0 || D < 0) return false;
    if (N != 4 && N != 8 && N != 16) return false;
    if (batch > INT32_MAX || L > INT32_MAX || D > INT32_MAX) return false;
    if (batch * ((D + 63) / 64) > INT32_MAX) return false;
    if ((L + 64) * D * 4 >= ((int64_t)1 << 31) || (L + 64) * N * 4 >= ((int64_t)1 << 31)) return false;
    return true;
}
}  // namespace

size_t m1_scan_workspace(int64_t batch, int64_t L, int64_t D, int64_t N) {
    if (batch < 0 || L < 0 || D < 0 || N < 1 || N > 64) return 0;
    if (batch > INT32_MAX || L > INT32_MAX || D > INT32_MAX) return 0;
    if ((L + 64) * D * 4 >= ((int64_t)1 << 31) || (L + 64) * N * 4 >= ((int64_t)1 << 31)) return 0;
    return m1_plan(batch, L, D, N).bytes;
}

size_t m1_bwd_workspace(int64_t batch, int64_t L, int64_t D, int64_t N) {
    if (!m1_bwd_dims_ok(batch, L, D, N) || batch == 0 || L == 0 || D == 0) return 0;
    return m1_bwd_plan(batch, L, D, N).bytes;
}
}  // namespace mb

extern "C" mb_status mb_selective_scan_bwd(const float* x, const float* dt, const float* A, const float* B,
                                           const float* C, const float* Dskip, const float* h0,
                                           const float* dy, const float* dh_out, float* dx, float* ddt,
                                           float* dA, float* dB, float* dC, float* dD, float* dh0,
                                           int64_t batch, int64_t L, int64_t D, int64_t N, mb_dtype dtype,
                                           void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (dtype != MB_F32) return MB_ERR_DTYPE;
    if (!m1_bwd_dims_ok(batch, L, D, N)) return MB_ERR_SHAPE;
    const size_t n_x = (size_t)(batch * L * D), n_b = (size_t)(batch * L * N);
    const size_t n_h = (size_t)(batch * D * N), n_a = (size_t)(D * N);
    if (n_x && (!x || !dt || !dy || !dx || !ddt)) return MB_ERR_NULL;
    if (n_b && (!B || !C || !dB || !dC)) return MB_ERR_NULL;
    if (D > 0 && (!A || !dA)) return MB_ERR_NULL;
    // the tiles are copied with 16-byte pieces of rows
    if (((uintptr_t)x | (uintptr_t)dt | (uintptr_t)B | (uintptr_t)C | (uintptr_t)dy) & 15) return MB_ERR_ALIGN;
    const Span ins[] = {{x, n_x * 4}, {dt, n_x * 4}, {A, n_a * 4}, {B, n_b * 4}, {C, n_b * 4},
                        {Dskip, Dskip ? (size_t)D * 4 : 0}, {h0, h0 ? n_h * 4 : 0}, {dy, n_x * 4},
                        {dh_out, dh_out ? n_h * 4 : 0}};
    const Span outs[] = {{dx, n_x * 4}, {ddt, n_x * 4}, {dA, n_a * 4}, {dB, n_b * 4}, {dC, n_b * 4},
                         {dD, dD ? (size_t)D * 4 : 0}, {dh0, dh0 ? n_h * 4 : 0}};
    for (int i = 0; i < 7; ++i) {
        if (overlaps_any(outs[i].p, outs[i].bytes, ins, 9)) return MB_ERR_ALIAS;
        for (int j = i + 1; j < 7; ++j)
            if (overlaps(outs[i].p, outs[i].bytes, outs[j].p, outs[j].bytes)) return MB_ERR_ALIAS;
    }
    if (D == 0) return MB_OK;
    if (batch == 0 || L == 0) {
        // no steps: dA = dDskip = 0, dh0 = dh_out
        mb_status st = copy_state(nullptr, dA, (int64_t)n_a, stream);
        if (st == MB_OK && dD) st = copy_state(nullptr, dD, D, stream);
        if (st == MB_OK && dh0 && batch > 0) st = copy_state(dh_out, dh0, (int64_t)n_h, stream);
        return st;
    }
    const M1BwdPlan pl = m1_bwd_plan(batch, L, D, N);
    if (!ws || ws_bytes < pl.bytes || ((uintptr_t)ws & 255)) return MB_ERR_WORKSPACE;
    if (overlaps_any(ws, pl.bytes, ins, 9) || overlaps_any(ws, pl.bytes, outs, 7)) return MB_ERR_ALIAS;
    char* w = (char*)ws;
    const int n_cg = (int)((D + 63) / 64);
    const int n_wg = (int)(batch * n_cg);
    M1Bwd a{};
    a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.Dskip = Dskip; a.dy = dy; a.dh_out = dh_out;
    a.ck = (const float*)w;
    a.dx = dx; a.ddt = ddt; a.dh0 = dh0;
    a.pBC = (float*)(w + pl.off_pbc);
    a.pA = (float*)(w + pl.off_pa);
    a.pD = (float*)(w + pl.off_pd);
    a.L = (int)L; a.D = (int)D; a.n_cg = n_cg;
    Fuse ckf{};
    ckf.ck = (float*)w;
    const bool v16 = D % 4 == 0;
#define MB_M1_BWD(S)                                                                                   \
    do {                                                                                              \
        if (v16) {                                                                                    \
            hipLaunchKernelGGL((k_m1_scan_w<S, true, false, true>), dim3(n_wg), dim3(256), 0, stream, \
                               x, dt, A, B, C, nullptr, h0, nullptr, nullptr, (int)L, (int)D, n_cg, ckf); \
            hipLaunchKernelGGL((k_m1_bwd<S, true>), dim3(n_wg), dim3(256), 0, stream, a);             \
        } else {                                                                                      \
            hipLaunchKernelGGL((k_m1_scan_w<S, false, false, true>), dim3(n_wg), dim3(256), 0, stream,\
                               x, dt, A, B, C, nullptr, h0, nullptr, nullptr, (int)L, (int)D, n_cg, ckf); \
            hipLaunchKernelGGL((k_m1_bwd<S, false>), dim3(n_wg), dim3(256), 0, stream, a);            \
        }                                                                                             \
    } while (0)
    switch (N) {
    case 4: MB_M1_BWD(1); break;
    case 8: MB_M1_BWD(2); break;
    default: MB_M1_BWD(4); break;
    }
#undef MB_M1_BWD
    const int64_t most = std::max<int64_t>(2 * batch * L * N, D * N);
    hipLaunchKernelGGL(k_m1_bwd_reduce, dim3((unsigned)((most + 255) / 256), 3), dim3(256), 0, stream, a, dB, dC,
                       dA, dD, (int)batch, (int)N);
    return check_launch();
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
