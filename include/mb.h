/*
 * mb.h -- C ABI of libmb, the MI355X (gfx950) selective state-space scan
 * library.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer to contiguous row-major memory,
 *   last-named axis fastest, owned by the caller.  The library never keeps a
 *   pointer after the call returns and never allocates or frees memory.
 * - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued on
 *   it asynchronously; no entry point synchronises the host, so every call can
 *   be captured into a HIP graph.
 * - Arguments are validated before anything is enqueued.  On any error code
 *   other than MB_ERR_HIP nothing has been launched and no output was touched.
 *   MB_ERR_HIP reports a failed launch; mb_last_hip_error() gives its code.
 * - `dtype` selects the element type of the "activation" tensors named in each
 *   entry point (MB_F32 or MB_BF16).  Every other tensor is fp32.  Arithmetic is
 *   fp32 with fp32 accumulation; states are always fp32; a bf16 output is
 *   rounded to nearest-even.  (TorchMamba README, API notes: half-precision
 *   inputs compute in fp32, outputs take the input dtype, states stay fp32.)
 *   One exception: mb_ssd_chunked with MB_BF16 and N a multiple of 8 runs its
 *   matrix products on bf16 operands with fp32 accumulation.  The operands are
 *   the inputs and three rounded intermediates: a copy of the state (the
 *   carried state stays fp32), the masked scores and the chunk-end-weighted X.
 * - NaN or Inf inputs propagate to the outputs; they are not trapped.
 * - Outputs must not overlap inputs, except where an entry point says so.
 * - The chunked SSD entry points read X, B, C and write Y with 16-byte vector
 *   accesses: those four pointers must be 16-byte aligned (MB_ERR_ALIGN).
 * - A length-zero sequence is valid: the final state is h0 (or zeros) and no
 *   y is written.  A zero batch is a no-op.
 * - The library is re-entrant; its only global state is a per-device cache of
 *   the compute-unit count and of the static workspace's address
 *   (mb_ssd_chunked_noalloc), each filled once under a lock.
 */
#ifndef MB_H
#define MB_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MB_OK = 0,
    MB_ERR_NULL = 1,      /* a required pointer is NULL                         */
    MB_ERR_SHAPE = 2,     /* a size is negative, inconsistent or unsupported    */
    MB_ERR_DTYPE = 3,     /* dtype is not MB_F32 / MB_BF16                      */
    MB_ERR_WORKSPACE = 4, /* workspace missing, too small or misaligned        */
    MB_ERR_HIP = 5,       /* a HIP launch failed                               */
    MB_ERR_ALIAS = 6,     /* an output overlaps an input it may not overlap    */
    MB_ERR_ALIGN = 7      /* a tensor pointer is not 16-byte aligned           */
} mb_status;

typedef enum { MB_F32 = 0, MB_BF16 = 1 } mb_dtype;

typedef enum {
    MB_OP_SELECTIVE_SCAN = 0,
    MB_OP_SSM_STEP = 1,
    MB_OP_SSD_CHUNKED = 2,
    MB_OP_TRAP_SSD = 3,
    MB_OP_MIMO_SSD = 4,
    MB_OP_SSD_CHUNKED_BWD = 5,
    MB_OP_SELECTIVE_SCAN_BWD = 6,
    MB_OP_TRAP_SSD_BWD = 7,
    MB_OP_MIMO_SSD_BWD = 8,
    MB_OP_SSD_BLOCK = 9,        /* mb_ssd_block with MB_F32 */
    MB_OP_SSD_BLOCK_BF16 = 10   /* mb_ssd_block with MB_BF16 */
} mb_op;

/*
 * Mamba-1 selective scan (TorchMamba README, Models table row "Mamba-1 (S6)"
 * and Math notes M1; burn_mamba `struct Mamba1` docs, `selective_scan`).
 * For every batch b, channel c and state n, exponential-Euler discretisation:
 *     h_t[c,n] = exp(dt_t[c] * A[c,n]) * h_{t-1}[c,n] + dt_t[c] * B_t[n] * x_t[c]
 *     y_t[c]   = sum_n C_t[n] * h_t[c,n] + Dskip[c] * x_t[c]
 * h_{-1} = h0.  B and C are per (b, t) and shared by all channels.
 *   x, dt : (batch, L, D)     dtype     dt is the final positive step (no softplus)
 *   A     : (D, N)            fp32      used as given (not A_log)
 *   B, C  : (batch, L, N)     dtype
 *   Dskip : (D)               fp32      NULL = no skip term
 *   h0    : (batch, D, N)     fp32      NULL = zeros
 *   y     : (batch, L, D)     dtype     written
 *   h_out : (batch, D, N)     fp32      final state; NULL = not written; may equal h0
 * Supported: 1 <= N <= 64, and one batch row of x and of B addressed in
 * 32-bit offsets: (L + 64) * D * 4 < 2^31 and (L + 64) * N * 4 < 2^31
 * (MB_ERR_SHAPE otherwise); any batch >= 0.
 * ws / ws_bytes: optional device workspace for sequence blocks (the Math
 * notes M1 recurrence is time-varying and is computed as a scan; a scan splits
 * into blocks because the pair (decay product, state) of consecutive blocks
 * composes associatively: (P1, h1) then (P2, h2) is (P1 P2, P2 h1 + h2), and
 * a block's decay product is exp(A * sum of its dt)).  With ws != NULL of at
 * least mb_workspace_size(MB_OP_SELECTIVE_SCAN, batch, L, D, 1, 1, N) bytes,
 * 256-byte aligned (MB_ERR_WORKSPACE otherwise), the fp32 path with N in
 * {4, 8, 16} and 16-byte aligned x, dt, B, C cuts the sequence into as many
 * blocks as it takes to fill the device (the size is 0 when one block does):
 * a first pass computes every block's own (decay product, end state), a
 * second starts each block from the composition of the blocks before it.  The
 * result equals the one-block scan up to rounding.  ws = NULL (or bf16, other
 * N): the whole sequence in one block.  ws must not overlap any argument;
 * contents on entry are ignored.
 */
mb_status mb_selective_scan(const void* x, const void* dt, const float* A,
                            const void* B, const void* C, const float* Dskip,
                            const float* h0, void* y, float* h_out,
                            int64_t batch, int64_t L, int64_t D, int64_t N,
                            mb_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Mamba-1 single-token decode step (burn_mamba `struct Mamba1` docs,
 * `selective_scan_step`; mamba-rs Quick Start `mamba_step`).  One iteration
 * of the recurrence above for a batch of independent sequences:
 *     h[b,c,n] <- exp(dt[b,c] * A[c,n]) * h[b,c,n] + dt[b,c] * B[b,n] * x[b,c]
 *     y[b,c]    = sum_n C[b,n] * h[b,c,n] + Dskip[c] * x[b,c]
 *   x, dt : (batch, D)  dtype;   B, C : (batch, N)  dtype;   A : (D, N) fp32
 *   Dskip : (D) fp32 or NULL;    h_in, h_out : (batch, D, N) fp32
 *   y     : (batch, D)  dtype
 * h_out == h_in (in-place update, the decode use) is allowed; any other
 * overlap between h_out and h_in is MB_ERR_ALIAS.
 */
mb_status mb_ssm_step(const void* x, const void* dt, const float* A,
                      const void* B, const void* C, const float* Dskip,
                      const float* h_in, float* h_out, void* y,
                      int64_t batch, int64_t D, int64_t N,
                      mb_dtype dtype, hipStream_t stream);

/*
 * Mamba-1 selective scan with the block's prologue and epilogue fused around it
 * (TorchMamba README, Models table row Mamba-1, "conv1d + sequential selective
 * scan"; the Mamba block takes the softplus of dt plus a bias and gates the
 * output with SiLU(z)).  Per batch b, channel c, state n:
 *     xc_t  = SiLU(conv_b[c] + sum_{k<K} conv_w[c,k] * x_{t-K+1+k}[c])
 *     dt'_t = softplus(dt_t[c] + dt_bias[c])
 *     h_t   = exp(dt'_t * A[c,n]) * h_{t-1} + dt'_t * B_t[n] * xc_t
 *     y_t   = (sum_n C_t[n] h_t[n] + Dskip[c] * xc_t) * SiLU(z_t[c])
 * with SiLU(v) = v / (1 + e^-v), softplus(v) = log(1 + e^v); the inputs x_{-j}
 * before the call are x_hist (zeros when NULL), so a sequence split across
 * calls chains exactly with h0 = the previous h_out and x_hist = the previous
 * call's last K-1 raw inputs.
 *   x, dt, z, y : (batch, L, D) fp32   (raw x and dt; z NULL = no gate)
 *   conv_w      : (D, K) fp32, K in 1..4;   conv_b, dt_bias, Dskip : (D) or NULL
 *   x_hist      : (batch, K-1, D) fp32 or NULL
 *   A (D, N), B, C (batch, L, N), h0, h_out (batch, D, N): as mb_selective_scan
 * Supported: dtype MB_F32 (MB_ERR_DTYPE otherwise), N in {4, 8, 16}; x, dt, B, C
 * and z 16-byte aligned (MB_ERR_ALIGN).  No workspace.
 */
mb_status mb_selective_scan_fused(const float* x, const float* conv_w, const float* conv_b,
                                  const float* x_hist, const float* dt, const float* dt_bias,
                                  const float* A, const float* B, const float* C,
                                  const float* Dskip, const float* z, const float* h0, float* y,
                                  float* h_out, int64_t batch, int64_t L, int64_t D, int64_t N,
                                  int64_t K, mb_dtype dtype, hipStream_t stream);

/*
 * Mamba-2 scalar-decay SSD, chunkwise (TorchMamba README, Models table row
 * "Mamba-2 (SSD)" and Math notes M2: the dual form Y = (L o C B^T) X, computed
 * per chunk with the state carried between chunks).  Per batch b and head h,
 * with group g = h / (H/G):
 *     S_t = exp(logdecay_t[h]) * S_{t-1} + B_t[g] (outer) X_t[h]      (N x P)
 *     Y_t[h] = S_t^T C_t[g]
 * S_{-1} = h0.  Heads share B and C within a group (H % G == 0 required).
 *   X, Y      : (batch, L, H, P)  dtype
 *   logdecay  : (batch, L, H)     fp32   log of the per-step decay (<= 0 in use)
 *   B, C      : (batch, L, G, N)  dtype
 *   h0, h_out : (batch, H, N, P)  fp32   h0 NULL = zeros; h_out may equal h0
 * chunk: 0 selects the library's chunk length; otherwise must be 64.
 * ws / ws_bytes: device workspace of at least mb_workspace_size(MB_OP_SSD_CHUNKED, ...)
 * bytes, 256-byte aligned; contents on entry are ignored.
 * Supported: 1 <= N <= 128, P >= 1.  Shapes with P % 16 != 0 or N % 4 != 0
 * (e.g. P = 1, the Mamba-1 -> Mamba-2 reduction of the Math notes) run on the
 * same kernels through zero-padded copies in the workspace (P rounded up to a
 * multiple of 16, N to a multiple of 4): exact, at the cost of the copies.
 * With MB_BF16 and N % 8 == 0 (after that rounding) the products take bf16
 * operands (fp32 accumulation, fp32 state; see the dtype note at the top).
 */
mb_status mb_ssd_chunked(const void* X, const float* logdecay, const void* B,
                         const void* C, const float* h0, void* Y, float* h_out,
                         int64_t batch, int64_t L, int64_t H, int64_t P,
                         int64_t G, int64_t N, int64_t chunk, mb_dtype dtype,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * mb_ssd_chunked with the output side of the Mamba-2 block fused into its store
 * (TorchMamba README, API reference: Mamba2Block with psi = SiLU; the skip and
 * gate as in the Mamba-3 block, mamba3-minimal README, Architecture):
 *     Y_t = (S_t^T C_t + Dskip[h] X_t) * SiLU(z_t),   SiLU(v) = v / (1 + e^-v)
 * with X the scan's own input.  Dskip (H) fp32 or NULL (no skip term); z like X
 * (same dtype, 16-byte aligned) or NULL (no gate); with both NULL the result is
 * mb_ssd_chunked's.  Neither may overlap Y or h_out (MB_ERR_ALIAS); Dskip
 * 4-byte aligned.  Other arguments, limits, state and workspace as
 * mb_ssd_chunked.
 */
mb_status mb_ssd_chunked_gated(const void* X, const float* logdecay, const void* B,
                               const void* C, const float* h0, const float* Dskip, const void* z,
                               void* Y, float* h_out, int64_t batch, int64_t L, int64_t H,
                               int64_t P, int64_t G, int64_t N, int64_t chunk, mb_dtype dtype,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The Mamba-2 layer around its scan in one call: the block prologue of
 * mb_ssd_prologue (causal depthwise conv1d of K taps over the projected channels
 * xBC = (x | B | C), SiLU, dt' = softplus(dt + dt_bias), X = x dt', log-decay
 * dt' A) fused into the chunked SSD, and the output side
 *     Y_t = (S_t^T C_t + Dskip[h] x_t) * SiLU(z_t)
 * with x_t the convolved, activated x before dt' scales it (TorchMamba README,
 * API reference Mamba2Block: d_conv taps, psi = SiLU; Math notes M2).
 * With MB_F32, X, B and C never pass through memory as tensors of their own:
 * the scores kernel convolves B and C, the walks convolve x as they stage it.
 * With MB_BF16 the call runs as two passes (the prologue pass into the
 * workspace, then the SSD with the output side): the bf16 walk is bound by
 * latency per chunk, and measured faster so (0.19 against 0.26 ms at batch 4,
 * L 4096, H 24, P 64, N 128).
 *   xBC     : (batch, L, H*P + 2*G*N)  dtype   raw projected channels
 *   conv_w  : (H*P + 2*G*N, K) fp32; conv_b (H*P + 2*G*N) fp32 or NULL; K in 1..4
 *   x_hist  : (batch, K-1, H*P + 2*G*N) dtype, the raw rows before the call, or NULL (zeros)
 *   dt      : (batch, L, H) fp32 raw;  dt_bias (H) fp32 or NULL;  A (H) fp32
 *   Dskip   : (H) fp32 or NULL;  z : (batch, L, H, P) dtype or NULL (no gate)
 *   h0, h_out : (batch, H, N, P) fp32 as mb_ssd_chunked;  Y : (batch, L, H, P) dtype
 * A split sequence chains exactly with h0 = the previous h_out and x_hist = the
 * previous call's last K-1 rows of xBC.  ws: at least
 * mb_workspace_size(MB_OP_SSD_BLOCK or MB_OP_SSD_BLOCK_BF16, batch, L, H, P, G,
 * N) bytes, 256-byte aligned.  Limits as mb_ssd_chunked; with MB_BF16,
 * N % 8 == 0 (MB_ERR_SHAPE otherwise); xBC, x_hist, z and Y 16-byte aligned.
 */
mb_status mb_ssd_block(const void* xBC, const float* conv_w, const float* conv_b,
                       const void* x_hist, const float* dt, const float* dt_bias,
                       const float* A, const float* Dskip, const void* z, const float* h0,
                       void* Y, float* h_out, int64_t batch, int64_t L, int64_t H, int64_t P,
                       int64_t G, int64_t N, int64_t K, mb_dtype dtype, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * mb_ssd_chunked for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and limits, without ws / ws_bytes.  The
 * workspace is a static device buffer inside the library, one per device
 * (32 MiB, held from the first call on that device until the process ends);
 * the call allocates nothing.  The sizes must need at most 32 MiB of
 * workspace (mb_workspace_size(MB_OP_SSD_CHUNKED, ...) <= 33554432), else
 * MB_ERR_WORKSPACE and nothing is launched; the Mamba-2 block shape (batch 4,
 * L 4096, H 24, P 64, N 128, G 1) needs 21 MB.  Every call on one device
 * shares that buffer: calls that overlap in time on one device (different
 * streams, or host threads) race and give wrong results; calls ordered on one
 * stream are safe.  Nothing in the buffer needs clearing between calls.
 * MB_ERR_HIP if the buffer's address cannot be obtained.
 */
mb_status mb_ssd_chunked_noalloc(const void* X, const float* logdecay, const void* B,
                                 const void* C, const float* h0, void* Y, float* h_out,
                                 int64_t batch, int64_t L, int64_t H, int64_t P,
                                 int64_t G, int64_t N, int64_t chunk, mb_dtype dtype,
                                 hipStream_t stream);

/*
 * Mamba-3 SISO exponential-trapezoidal SSD with data-dependent rotations
 * (TorchMamba README, Models table row "Mamba-3 SISO" and Math notes M3 SISO;
 * mamba3-minimal README, "Two-SSD Decomposition").  Per batch b, head h:
 *     Theta_t = sum_{s<=t} theta_s                    (per pair k; restarts per call)
 *     B~_t = R(Theta_t) B_t,  C~_t = R(Theta_t) C_t   (consecutive pairs 2k, 2k+1)
 *     S_t = exp(logdecay_t) S_{t-1} + beta_t B~_{t-1} (x) X_{t-1} + gamma_t B~_t (x) X_t
 *     Y_t = S_t^T C~_t
 * with B~_{-1} = B_prev and X_{-1} = X_prev, the token before the call (zeros
 * when both are NULL; Theta restarts at 0 per call, so B~_{-1} is B_prev
 * unrotated).  R(phi) = [[cos, -sin], [sin, cos]].  A sequence split across
 * calls chains exactly when each call after the first gets h0 = the previous
 * call's h_out and X_prev, B_prev = the previous call's last X and B.
 *   X, Y                   : (batch, L, H, P)    dtype
 *   logdecay, beta, gamma  : (batch, L, H)       fp32 (alpha = exp(logdecay))
 *   B, C                   : (batch, L, G, N)    dtype
 *   theta                  : (batch, L, H, N/2)  fp32, or NULL for no rotation
 *   h0, h_out              : (batch, H, N, P)    fp32, in the PHYSICAL (unrotated)
 *                            frame: h_out = R(-Theta_{L-1}) S_{L-1}
 *   X_prev                 : (batch, H, P)       dtype, or NULL
 *   B_prev                 : (batch, G, N)       dtype, or NULL (with X_prev)
 * X_prev and B_prev are both given or both NULL; 16-byte aligned like X, B.
 * N must be even when theta != NULL.  Other limits as mb_ssd_chunked.
 */
mb_status mb_trap_ssd(const void* X, const float* logdecay, const void* B,
                      const void* C, const float* beta, const float* gamma,
                      const float* theta, const float* h0, const void* X_prev,
                      const void* B_prev, void* Y, float* h_out, int64_t batch,
                      int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                      int64_t chunk, mb_dtype dtype, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * mb_trap_ssd with the output epilogue of the Mamba-3 block fused into its
 * store (mamba3-minimal README, Architecture: the SSD output plus D x, then
 * gated by SiLU(z)):
 *     Y_t = (S_t^T C~_t + Dskip[h] X_t) * SiLU(z_t),   SiLU(v) = v / (1 + e^-v)
 * Dskip (H) fp32 or NULL (no skip term); z (batch, L, H, P) in the dtype of X,
 * or NULL (no gate).  Both NULL gives mb_trap_ssd.  Other arguments, the state
 * and the workspace as mb_trap_ssd; z must be 16-byte aligned (MB_ERR_ALIGN)
 * and must not overlap Y or h_out (MB_ERR_ALIAS).
 */
mb_status mb_trap_ssd_gated(const void* X, const float* logdecay, const void* B,
                            const void* C, const float* beta, const float* gamma,
                            const float* theta, const float* h0, const void* X_prev,
                            const void* B_prev, const float* Dskip, const void* z, void* Y,
                            float* h_out, int64_t batch, int64_t L, int64_t H, int64_t P,
                            int64_t G, int64_t N, int64_t chunk, mb_dtype dtype, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * The Mamba-2 block prologue in one pass (TorchMamba README, API reference:
 * Mamba2Block, d_conv taps and psi = SiLU; Math notes M1: exp-Euler, the input
 * scaled by dt and the decay exp(dt A)): from the block's projected channels
 * xBC = (x | B | C) and the raw dt it makes the inputs of mb_ssd_chunked,
 *     v_t[c]        = SiLU(conv_b[c] + sum_{k<K} conv_w[c][k] xBC_{t-K+1+k}[c])
 *     dt'_t[h]      = softplus(dt_t[h] + dt_bias[h])
 *     X_t[h][p]     = v_t[h P + p] dt'_t[h]
 *     B_t[g][n]     = v_t[H P + g N + n],   C_t[g][n] = v_t[H P + G N + g N + n]
 *     logdecay_t[h] = dt'_t[h] A[h]
 *   xBC      : (batch, L, H P + 2 G N) dtype, channel-last
 *   conv_w   : (H P + 2 G N, K) fp32;  conv_b: (H P + 2 G N) fp32 or NULL
 *   x_hist   : (batch, K-1, H P + 2 G N) dtype or NULL: the K-1 inputs before
 *              step 0 (zeros when NULL), so a split sequence chains exactly
 *   dt       : (batch, L, H) fp32;  dt_bias: (H) fp32 or NULL;  A: (H) fp32
 *   X        : (batch, L, H, P) dtype out;  B, C: (batch, L, G, N) dtype out
 *   logdecay : (batch, L, H) out;  dt_out: (batch, L, H) out (dt') or NULL
 * 1 <= K <= 4; P and N multiples of 4; H % G == 0; ceil(L / 16) <= 65535.
 * xBC, x_hist, X, B, C 16-byte aligned (MB_ERR_ALIGN); no output may overlap
 * an input or another output (MB_ERR_ALIAS).  dtype (MB_F32 or MB_BF16) is that
 * of the activations xBC, x_hist, X, B, C; the arithmetic is fp32 and the
 * bf16 outputs are rounded to nearest even once.
 */
mb_status mb_ssd_prologue(const void* xBC, const float* conv_w, const float* conv_b,
                          const void* x_hist, const float* dt, const float* dt_bias,
                          const float* A, void* X, void* B, void* C, float* logdecay,
                          float* dt_out, int64_t batch, int64_t L, int64_t H, int64_t P,
                          int64_t G, int64_t N, int64_t K, mb_dtype dtype, hipStream_t stream);

/*
 * The Mamba-3 SISO layer with both ends of the block fused into the scan
 * (mamba3-minimal README, Architecture: B and C pass a QK-style norm, then a
 * bias, then the rotations; TorchMamba README, Math notes M3 SISO: BCNorm and
 * bias take the place of the short convolution).  Before the rotations each
 * raw row of B and of C (one step, one group, N states) becomes
 *     B^_t[h][n] = B_t[g][n] / sqrt(mean_n' B_t[g][n']^2 + eps) * normB_w[n] + biasB[h][n]
 * (C likewise with normC_w, biasC), g the group of head h; the scan then runs
 * on the per-head rows B^, C^ exactly as mb_trap_ssd, and the output takes the
 * epilogue of mb_trap_ssd_gated.  B_prev (given with X_prev) is the previous
 * token's raw row and passes the same prologue.
 *   normB_w, normC_w : (N) fp32 or NULL (ones)
 *   biasB, biasC     : (H, N) fp32 or NULL (zeros)
 *   eps              : > 0 and finite (MB_ERR_SHAPE otherwise)
 *   Dskip, z         : as mb_trap_ssd_gated (NULL: no skip term / no gate)
 * The five parameter arrays must be 4-byte aligned (MB_ERR_ALIGN) and none of
 * them nor z may overlap Y or h_out (MB_ERR_ALIAS).  Other arguments, the
 * state and the workspace as mb_trap_ssd.
 */
mb_status mb_trap_ssd_block(const void* X, const float* logdecay, const void* B,
                            const void* C, const float* beta, const float* gamma,
                            const float* theta, const float* h0, const void* X_prev,
                            const void* B_prev, const float* normB_w, const float* normC_w,
                            const float* biasB, const float* biasC, float eps,
                            const float* Dskip, const void* z, void* Y, float* h_out,
                            int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                            int64_t chunk, mb_dtype dtype, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * Mamba-3 MIMO rank-R SSD (TorchMamba README, Models table row "Mamba-3 MIMO"
 * and Math notes MIMO: the rank-R update is a matrix product on one shared
 * (N, P) state).  As mb_trap_ssd, with every rank r of step t rotated by the
 * same Theta_t:
 *     S_t = exp(ld_t) S_{t-1} + beta_t sum_r B~_{t-1,r} (x) X_{t-1,r}
 *                             + gamma_t sum_r B~_{t,r} (x) X_{t,r}
 *     Y_{t,r} = S_t^T C~_{t,r}
 *   X, Y      : (batch, L, H, P, R)  dtype     (rank innermost)
 *   B, C      : (batch, L, H, N, R)  dtype     (per head, rank innermost)
 *   logdecay, beta, gamma, theta, h0, h_out : as mb_trap_ssd (state has no R axis)
 *   X_prev    : (batch, H, P, R)     dtype, or NULL   (the token before the call,
 *   B_prev    : (batch, H, N, R)     dtype, or NULL    as mb_trap_ssd)
 * Supported: R in {1, 2, 4, 8, 16}; other limits as mb_trap_ssd.
 */
mb_status mb_mimo_ssd(const void* X, const float* logdecay, const void* B,
                      const void* C, const float* beta, const float* gamma,
                      const float* theta, const float* h0, const void* X_prev,
                      const void* B_prev, void* Y, float* h_out, int64_t batch,
                      int64_t L, int64_t H, int64_t P, int64_t N, int64_t R,
                      int64_t chunk, mb_dtype dtype, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * The Mamba-3 MIMO layer with both ends of its block fused into the scan
 * (mamba3-minimal README, Architecture: QK-style norm, bias, rotations on B
 * and C; y + D x gated by SiLU(z); TorchMamba README, API reference: the MIMO
 * block takes the SISO block's parameters and the rank).  Every rank's raw row
 * of B and of C (one step, one head, one rank, N states) becomes
 *     B^_{t,r}[h][n] = B_{t,r}[h][n] / sqrt(mean_n' B_{t,r}[h][n']^2 + eps) * normB_w[n] + biasB[h][n]
 * (C likewise), the bias the same for every rank; the scan runs on B^, C^ as
 * mb_mimo_ssd; then per rank
 *     Y_{t,r} = (S_t^T C~_{t,r} + Dskip[h] X_{t,r}) * SiLU(z_{t,r}),  SiLU(v) = v / (1 + e^-v).
 * B_prev (with X_prev) is the previous token's raw rows and passes the prologue.
 *   z                : (batch, L, H, P, R) dtype, or NULL (no gate), 16-byte aligned
 *   Dskip            : (H) fp32 or NULL (no skip term)
 *   normB_w, normC_w, biasB, biasC, eps : as mb_trap_ssd_block
 * Supported: R in {1, 2, 4, 8, 16} (MB_ERR_SHAPE otherwise); other arguments, limits,
 * state and workspace as mb_mimo_ssd.
 */
mb_status mb_mimo_ssd_block(const void* X, const float* logdecay, const void* B,
                            const void* C, const float* beta, const float* gamma,
                            const float* theta, const float* h0, const void* X_prev,
                            const void* B_prev, const float* normB_w, const float* normC_w,
                            const float* biasB, const float* biasC, float eps,
                            const float* Dskip, const void* z, void* Y, float* h_out,
                            int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t R,
                            int64_t chunk, mb_dtype dtype, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * Decode step of the SSD family: one token per sequence, state in the physical
 * (unrotated) frame (TorchMamba README, Math notes M3 SISO and MIMO: plane
 * rotations compose additively, so the rotated-frame recurrence needs only the
 * token's angle increment and the unrotated B, C; Mamba-2, Math notes M2, is
 * beta = gamma = theta = NULL).  Per batch b and head h, group g = h / (H/G):
 *     S' = R(-theta) (exp(logdecay) S + beta sum_r Bp_r (outer) Xp_r)
 *          + gamma sum_r B_r (outer) X_r
 *     Y_r = S'^T C_r
 * R(phi) rotates consecutive state-row pairs (2k, 2k+1) by phi[k]; Bp, Xp are
 * the previous token's B and X.  The final state of mb_ssd_chunked,
 * mb_trap_ssd or mb_mimo_ssd (physical frame) continues exactly with this step,
 * passing that call's last B and X as B_prev, X_prev.
 *   X, X_prev, Y : (batch, H, P, R)   dtype   (R = 1: (batch, H, P))
 *   B, C, B_prev : (batch, G, N, R)   dtype   (MIMO: G = H, per head)
 *   logdecay, beta, gamma : (batch, H) fp32; beta NULL = 0, gamma NULL = 1
 *   theta        : (batch, H, N/2)  fp32 angle increments, or NULL (no rotation)
 *   h_in, h_out  : (batch, H, N, P) fp32; h_in NULL = zeros; h_out == h_in (in
 *                  place) is allowed
 * Every tensor pointer except logdecay, beta, gamma and theta must be 16-byte
 * aligned (MB_ERR_ALIGN): rows are read and written with 16-byte accesses.
 * X_prev and B_prev are both given or both NULL (NULL: zeros, the first token
 * of a sequence).  Supported: H % G == 0, P % 4 == 0 and P <= 1024, N even,
 * R in {1, 2, 4, 8, 16}.  No workspace.
 */
mb_status mb_ssd_step(const void* X, const float* logdecay, const void* B,
                      const void* C, const float* beta, const float* gamma,
                      const float* theta, const void* X_prev, const void* B_prev,
                      const float* h_in, float* h_out, void* Y, int64_t batch,
                      int64_t H, int64_t P, int64_t G, int64_t N, int64_t R,
                      mb_dtype dtype, hipStream_t stream);

/*
 * Backward of mb_selective_scan (fp32): the vector-Jacobian product of the
 * Mamba-1 scan (TorchMamba README, Math notes M1; trained by back-propagation
 * through time, as the mamba-rs page lists).  Given dy (gradient of the loss
 * with respect to y) and dh_out (with respect to h_out; NULL = zero), returns
 * the gradients of  sum dy . y + sum dh_out . h_out  with respect to x, dt, A,
 * B, C, Dskip and h0.  With a_t = exp(dt_t A) and G the adjoint of one
 * channel's state (G = dh_out, then per step from the last: G += C_t dy_t, ...,
 * G = a_t G):
 *     dx_t = dt_t sum_n G B_t + Dskip dy_t,  ddt_t = sum_n G (B_t x_t + A a_t h_{t-1}),
 *     dB_t = sum_c G dt_t x_t,  dC_t = sum_c h_t dy_t,
 *     dA = sum_{b,t} G dt_t a_t h_{t-1},  dDskip = sum_{b,t} dy_t x_t,  dh0 = G at the end.
 * The forward states are recomputed from per-32-step checkpoints in the
 * workspace; nothing of the forward call is needed.  Deterministic.
 *   x, dt, dy, dx, ddt : (batch, L, D)  fp32
 *   A, dA              : (D, N)         fp32
 *   B, C, dB, dC       : (batch, L, N)  fp32
 *   Dskip, dD          : (D)            fp32; Dskip NULL = no skip term; dD NULL = not wanted
 *   h0, dh_out, dh0    : (batch, D, N)  fp32; h0, dh_out NULL = zeros; dh0 NULL = not wanted
 * ws / ws_bytes: device workspace of at least
 * mb_workspace_size(MB_OP_SELECTIVE_SCAN_BWD, batch, L, D, <P ignored>, <G
 * ignored>, N, ...) bytes (D in the H argument), 256-byte aligned.
 * Supported: dtype MB_F32 (MB_ERR_DTYPE otherwise); N in {4, 8, 16}
 * (MB_ERR_SHAPE otherwise); x, dt, B, C, dy 16-byte aligned (MB_ERR_ALIGN).  No
 * output may overlap an input, another output or the workspace (MB_ERR_ALIAS).
 */
mb_status mb_selective_scan_bwd(const float* x, const float* dt, const float* A, const float* B,
                                const float* C, const float* Dskip, const float* h0,
                                const float* dy, const float* dh_out, float* dx, float* ddt,
                                float* dA, float* dB, float* dC, float* dD, float* dh0,
                                int64_t batch, int64_t L, int64_t D, int64_t N, mb_dtype dtype,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of mb_mimo_ssd (fp32): the vector-Jacobian product of the Mamba-3
 * MIMO recurrence (TorchMamba README, Math notes MIMO; trained by
 * back-propagation through time, as the mamba-rs page lists): the gradients of
 * sum dY . Y + sum dh_out . h_out  with respect to X, logdecay, B, C, beta,
 * gamma, theta, h0 and the previous token, as mb_trap_ssd_bwd with R ranks per
 * step (the adjoint takes the R output ranks; every rank has both trapezoid
 * terms; the angle gradient sums over the ranks of B and C).
 * Arguments as mb_mimo_ssd (X, dY, dX (batch, L, H, P, R); B, C, dB, dC
 * (batch, L, H, N, R); X_prev, dX_prev (batch, H, P, R); B_prev, dB_prev
 * (batch, H, N, R)), gradients shaped like their inputs; theta NULL = no
 * rotation (dtheta not written); X_prev, B_prev both given or both NULL; dh0,
 * dX_prev, dB_prev NULL = not wanted.
 * ws / ws_bytes: device workspace of at least
 * mb_workspace_size(MB_OP_MIMO_SSD_BWD, batch, L, H, P, <G ignored>, N, R, 0)
 * bytes, 256-byte aligned; it holds the sequence as (3R - 1) L rows of a plain
 * SSD (about 11 GB at batch 2, L 8192, H 16, P 64, N 128, R 4).
 * Supported: dtype MB_F32 (MB_ERR_DTYPE otherwise); N in {64, 128}, P in {32,
 * 64}, R in {1, 2, 4, 8, 16} (MB_ERR_SHAPE otherwise); h0, dh_out, dh0 16-byte aligned
 * (MB_ERR_ALIGN).  No output may overlap an input, another output or the
 * workspace (MB_ERR_ALIAS).
 */
mb_status mb_mimo_ssd_bwd(const float* X, const float* logdecay, const float* B, const float* C,
                          const float* beta, const float* gamma, const float* theta, const float* h0,
                          const float* X_prev, const float* B_prev, const float* dY,
                          const float* dh_out, float* dX, float* dlogdecay, float* dB, float* dC,
                          float* dbeta, float* dgamma, float* dtheta, float* dh0, float* dX_prev,
                          float* dB_prev, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                          int64_t R, mb_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of mb_trap_ssd (fp32): the vector-Jacobian product of the Mamba-3
 * SISO recurrence (TorchMamba README, Math notes M3 SISO; trained by
 * back-propagation through time, as the mamba-rs page lists).  Given dY and
 * dh_out (NULL = zero), returns the gradients of  sum dY . Y + sum dh_out . h_out
 * with respect to X, logdecay, B, C, beta, gamma, theta, h0 and the previous
 * token X_prev, B_prev.  In the rotated frame, with A the adjoint of the state
 * (A = R(Theta_{L-1}) dh_out at the end, since h_out = R(-Theta_{L-1}) S_{L-1}):
 *     A += Ct_t dY_t^T;  dgamma_t = X_t . A^T Bt_t;  dbeta_t = X_{t-1} . A^T Bt_{t-1};
 *     dX, dBt, dCt from both trapezoid terms;  dlogdecay_t = e^{ld_t} <A, S_{t-1}>;
 *     A = e^{ld_t} A
 * then dB_t = R(-Theta_t) dBt_t (likewise C, summed over the group's heads), and
 * dtheta_t = sum over steps >= t of the angle gradient of the rotations (and of
 * h_out at the last step).  dh0 is the adjoint before the first step.
 * Arguments as mb_trap_ssd, gradients shaped like their inputs; theta NULL = no
 * rotation (dtheta not written); X_prev, B_prev both given or both NULL;
 * dh0, dX_prev, dB_prev NULL = not wanted.
 * ws / ws_bytes: device workspace of at least
 * mb_workspace_size(MB_OP_TRAP_SSD_BWD, ...) bytes, 256-byte aligned.
 * Supported: dtype MB_F32 (MB_ERR_DTYPE otherwise); N in {64, 128}, P in
 * {32, 64} (MB_ERR_SHAPE otherwise); X, B, C, dY, dX, dB, dC, h0, dh_out, dh0,
 * X_prev, B_prev, dB_prev 16-byte aligned (MB_ERR_ALIGN).  No output may overlap
 * an input, another output or the workspace (MB_ERR_ALIAS).
 */
mb_status mb_trap_ssd_bwd(const float* X, const float* logdecay, const float* B, const float* C,
                          const float* beta, const float* gamma, const float* theta, const float* h0,
                          const float* X_prev, const float* B_prev, const float* dY,
                          const float* dh_out, float* dX, float* dlogdecay, float* dB, float* dC,
                          float* dbeta, float* dgamma, float* dtheta, float* dh0, float* dX_prev,
                          float* dB_prev, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G,
                          int64_t N, mb_dtype dtype, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward of mb_ssd_chunked (fp32): the vector-Jacobian product of the Mamba-2
 * SSD (TorchMamba README, Math notes M2; trained by back-propagation through
 * time, as the mamba-rs page lists).  Given dY (gradient of the loss with
 * respect to Y) and dh_out (with respect to h_out; NULL = zero), returns the
 * gradients of  sum dY . Y + sum dh_out . h_out  with respect to X, logdecay,
 * B, C and h0.  With h_t the forward state after step t and G_t its adjoint
 * (G_{L-1} = C_{L-1} dY_{L-1}^T + dh_out, G_{t-1} = e^{ld_t} G_t + C_{t-1} dY_{t-1}^T):
 *     dX_t = G_t^T B_t,  dB_t = sum_h G_t X_t,  dC_t = sum_h h_t dY_t,
 *     dlogdecay_t = e^{ld_t} <G_t, h_{t-1}>,  dh0 = e^{ld_0} G_0
 * (sums over the heads h of the group).  The forward states are recomputed
 * chunkwise; nothing of the forward call is needed.
 *   X, dY, dX           : (batch, L, H, P)  fp32
 *   logdecay, dlogdecay : (batch, L, H)     fp32
 *   B, C, dB, dC        : (batch, L, G, N)  fp32
 *   h0, dh_out, dh0     : (batch, H, N, P)  fp32; h0, dh_out NULL = zeros; dh0 NULL = not wanted
 * ws / ws_bytes: device workspace of at least
 * mb_workspace_size(MB_OP_SSD_CHUNKED_BWD, ...) bytes, 256-byte aligned (two
 * N x P states per (batch, head, 64-step chunk), plus small buffers).
 * Supported: dtype MB_F32 (MB_ERR_DTYPE otherwise); N in {64, 128}, P in
 * {32, 64} (MB_ERR_SHAPE otherwise); X, B, C, dY, dX, dB, dC, h0, dh_out, dh0
 * 16-byte aligned (MB_ERR_ALIGN).  No output may overlap an input, another output or the
 * workspace (MB_ERR_ALIAS).
 */
mb_status mb_ssd_chunked_bwd(const float* X, const float* logdecay, const float* B,
                             const float* C, const float* h0, const float* dY,
                             const float* dh_out, float* dX, float* dlogdecay, float* dB,
                             float* dC, float* dh0, int64_t batch, int64_t L, int64_t H,
                             int64_t P, int64_t G, int64_t N, mb_dtype dtype, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * Bytes of device workspace an entry point needs for the given sizes (0 if it
 * needs none).  Unused sizes are ignored: G for MB_OP_TRAP_SSD / MIMO, R for
 * the others.  Returns 0 for invalid sizes as well (the call itself reports
 * the error).  The Mamba-1 sequence blocks and the SSD segments are planned
 * for the current device's compute-unit count: query with the device current
 * that the call will run on (a call given less than its plan needs returns
 * MB_ERR_WORKSPACE).
 */
size_t mb_workspace_size(mb_op op, int64_t batch, int64_t L, int64_t H,
                         int64_t P, int64_t G, int64_t N, int64_t R,
                         int64_t chunk);

/* Static, NUL-terminated description of a status code. */
const char* mb_status_str(mb_status status);

/* The hipError_t of the most recent MB_ERR_HIP in this thread (0 if none). */
int mb_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int mb_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MB_H */
