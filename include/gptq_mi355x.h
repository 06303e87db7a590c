/*
 * gptq_mi355x.h -- C ABI of the MI355X (gfx950) GPTQ layer quantizer.
 *
 * The method: GPTQ layer-wise weight quantization as set out on the page
 * "GPTQ deep dive" (hncyxsy.com news 243429), section 3.1, four steps per
 * linear layer: (1) H = 2 X X^T + lambda I from the layer's calibration
 * inputs, (2) a Cholesky factorization standing in for repeated inversion,
 * (3) quantization of W column by column in blocks of 128 with error
 * compensation, (4) storing the integer weights with scale and zero-point.
 * The layer objective is min ||WX - W_qX||^2 ("LLM quantization principles:
 * GPTQ, AWQ, GGUF", 0539edu.com news 6111416, section 3.1).
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer (HBM) owned by the caller.  The
 *    library never allocates device memory: scratch space comes from a
 *    caller-provided workspace whose size the *_workspace_size queries give
 *    (gptq_quantize_layer_noalloc instead uses a fixed array of device memory
 *    that is part of the library's device code).
 *  - Matrices are row-major with an explicit leading dimension (in elements).
 *  - All work is enqueued on `stream` (NULL = the default stream); calls return
 *    without synchronizing.  Argument errors are detected on the host and
 *    returned synchronously before anything is enqueued.  Data-dependent
 *    errors (a non-positive pivot, a non-finite value) are written to a device
 *    int32 `info` (0 = ok), which the caller reads after synchronizing.
 *  - Calls on one stream are ordered; calls that share output or workspace
 *    buffers must not run concurrently on different streams.
 *  - Results are deterministic: the same inputs give bitwise-identical outputs.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPTQ_ABI_VERSION 0x00020005u /* major 2, minor 5 */

typedef enum gptq_status {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = 1, /* bad shape, pointer, stride or configuration     */
  GPTQ_ERR_NOT_PD = 2,      /* reported through `info` only (see gptq_prepare) */
  GPTQ_ERR_NONFINITE = 3,   /* reported through `info` only                    */
  GPTQ_ERR_EMPTY = 4,       /* no calibration tokens were accumulated          */
  GPTQ_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the query     */
  GPTQ_ERR_HIP = 6,         /* a HIP runtime call failed (launch error)        */
  GPTQ_ERR_UNSUPPORTED = 7  /* valid for the method, not built in this library */
} gptq_status;

typedef enum gptq_dtype { GPTQ_F32 = 0, GPTQ_BF16 = 1 } gptq_dtype;

/* Quantization settings.  The user-facing knobs of the pages: bits,
 * group_size, desc_act and damp_percent ("LLM quantization principles",
 * section 3.1; "GPTQ deep dive", section 3.3), and block_size, which must be a
 * multiple of group_size ("AWQ, MinMax, GPTQ calibration in Model Optimizer",
 * gtnt.cn news 115337, section 4). */
typedef struct gptq_config {
  int32_t bits;       /* 2..8                                                  */
  int32_t group_size; /* 8, 16, 32, 64 or 128 (dividing block_size), 256 or 512
                         (a multiple of block_size: computed as block_size =
                         group_size would, the group's parameters taken where it
                         starts); -1 = one group per row spanning all columns  */
  int32_t block_size; /* 128 (the only block width built)                      */
  float perc_damp;    /* damping fraction (default 0.01); used by gptq_prepare  */
  int32_t desc_act;   /* 0/1: columns in descending Hessian-diagonal order      */
  int32_t sym;        /* 0 = asymmetric min-max; 1 = symmetric (zero = 2^(b-1)) */
  int32_t static_groups; /* 0 = a group is group_size consecutive processing
                         positions, parameters from the current (compensated)
                         values at its first column; 1 = groups of group_size
                         consecutive ORIGINAL columns, parameters computed once
                         from the original weights (dead columns as 0), so that
                         with desc_act g_idx stays c / group_size.  Not on the
                         pages; the plain reading of the name.                  */
} gptq_config;

/* Version of this ABI (GPTQ_ABI_VERSION of the built library). */
uint32_t gptq_abi_version(void);

/* Static, NUL-terminated description of a status code; never NULL. */
const char* gptq_status_str(int32_t status);

/* ------------------------------------------------------------------------
 * Hessian accumulation -- "GPTQ deep dive", section 3.1, step 1.
 *
 * S[n, n] += X^T X for the calibration activations X[tokens, n] (row stride
 * ldx >= n elements, token-major as a layer sees them).  fp32 accumulation of
 * exact bf16 x bf16 (or fp32 x fp32) products.  Only the lower triangle
 * (i >= j) of S is read and written; the strict upper triangle is untouched.
 * S is the raw sum: H = 2S is formed by gptq_prepare.  Accumulation is
 * additive, so a caller may feed the calibration set in any number of calls
 * (S is the caller's resumable state).  tokens == 0 is a no-op.
 * Workspace: gptq_hessian_workspace_size(n, tokens) bytes (0 allowed -> ws may
 * be NULL).
 * ---------------------------------------------------------------------- */
gptq_status gptq_hessian_workspace_size(int64_t n, int64_t tokens, size_t* bytes);
gptq_status gptq_hessian_accumulate(float* S, int64_t n, int64_t lds, const void* X,
                                    gptq_dtype xdt, int64_t tokens, int64_t ldx, void* ws,
                                    size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Prepare -- "GPTQ deep dive", sections 3.1 (step 2) and 3.3, and 2.4 (the
 * Cholesky factorization replacing repeated inversion).
 *
 * From S (lower triangle, as accumulated above) over `tokens` calibration
 * tokens:  H = 2S; dead columns (H_ii == 0) get H_ii := 1 and dead[i] = 1;
 * with desc_act the processing order perm is the stable descending order of
 * diag(H) (else the identity); lambda = perc_damp * mean(diag H);
 * H_d = H + lambda I (permuted); and U[n, n] (row stride ldu) receives the
 * upper Cholesky factor of H_d^-1 in processing order (H_d^-1 = U^T U), with
 * zeros below the diagonal.  Computed in fp64 on the device, rounded to fp32.
 * U may alias S (same buffer, ldu == lds).
 * perm[n] (int32; processing position -> original column), dead[n] (uint8)
 * and lambda_out (one fp32) may each be NULL.  info: 0 ok, k > 0 = the
 * 1-based processing position of the first non-positive pivot (raise
 * perc_damp, as "GPTQ deep dive" section 3.3 advises), -1 = a non-finite
 * value in S.  Returns GPTQ_ERR_EMPTY synchronously when tokens == 0.
 * The factorization also runs on two library-owned streams of the device
 * (created on first use, default priority), ordered against `stream` by
 * events: the call behaves as work on `stream`.  Calls from several host
 * threads on one device are serialized while they enqueue.
 * ---------------------------------------------------------------------- */
gptq_status gptq_prepare_workspace_size(int64_t n, size_t* bytes);
gptq_status gptq_prepare(const float* S, int64_t n, int64_t lds, int64_t tokens,
                         float perc_damp, int32_t desc_act, float* U, int64_t ldu,
                         int32_t* perm, uint8_t* dead, float* lambda_out, int32_t* info,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Quantize one layer -- "GPTQ deep dive", section 3.1, step 3 (blocks of 128
 * columns; in each block, per column: group scale, rounding, error
 * accumulation; then one batched update of the later columns), section 2.2
 * (compensation through the inverse Hessian) and section 2.4 (fixed order,
 * lazy batched updates).
 *
 * W[m, n] (row stride ldw, fp32 or bf16) is read only.  U and perm come from
 * gptq_prepare (perm may be NULL = identity, dead may be NULL = none).
 * Outputs, all in ORIGINAL column order except where stated:
 *   codes[m, n]  uint8 in [0, 2^bits - 1], row stride n;
 *   scales[m, ngroups], zeros[m, ngroups] fp32 (zeros hold integers), groups
 *                numbered in processing order (static groups: in original
 *                order); ngroups = ceil(n / group_size) (1 when group_size == -1);
 *   g_idx[n]     int32 group of each original column (may be NULL);
 *   row_err[m]   fp32 sum over columns of e_c^2 = delta^T H_d delta for the
 *                row's error delta = W - dequant(Q) (may be NULL).
 * info (may be NULL): set to -1 if W holds a non-finite value.
 * Group parameters: range [min(0, min v), max(0, max v)] of the group's
 * current (compensated) values, scale = range / maxq,
 * zero = rne(-min * maxq / range), q = clamp(rne(w / scale) + zero, 0, maxq),
 * all in fp32 with IEEE division.
 * ---------------------------------------------------------------------- */
gptq_status gptq_quantize_workspace_size(int64_t m, int64_t n, const gptq_config* cfg,
                                         size_t* bytes);
gptq_status gptq_quantize_layer(const void* W, gptq_dtype wdt, int64_t m, int64_t n,
                                int64_t ldw, const float* U, int64_t ldu, const int32_t* perm,
                                const uint8_t* dead, const gptq_config* cfg, uint8_t* codes,
                                float* scales, float* zeros, int32_t* g_idx, float* row_err,
                                int32_t* info, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * gptq_quantize_layer without allocation.  For callers that cannot allocate
 * device memory or take a workspace from an allocator: code under HIP graph
 * capture, tight loops, harnesses that forbid hipMalloc.  Same arguments,
 * outputs and kernels as gptq_quantize_layer, minus the workspace: the
 * column loop's scratch is a fixed array of GPTQ_NOALLOC_SCRATCH_BYTES of
 * device memory owned by the library, one copy per GPU, held from the first
 * call on that GPU until the process ends.  The call allocates nothing and
 * frees nothing.
 * Limit: layers whose gptq_quantize_workspace_size exceeds
 * GPTQ_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. m * n up to about 11.7 M weights
 * without desc_act, 9.4 M with it; 4096 x 2048 fits, 4096 x 4096 does not)
 * return GPTQ_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that GPU's scratch (it keeps the last call's
 * contents; every part a call reads is written by the call first): calls
 * that overlap in time on one GPU -- on different streams, or from several
 * host threads without ordering -- race and must not be issued.
 * ---------------------------------------------------------------------- */
#define GPTQ_NOALLOC_SCRATCH_BYTES (64u << 20)
gptq_status gptq_quantize_layer_noalloc(const void* W, gptq_dtype wdt, int64_t m, int64_t n,
                                        int64_t ldw, const float* U, int64_t ldu,
                                        const int32_t* perm, const uint8_t* dead,
                                        const gptq_config* cfg, uint8_t* codes, float* scales,
                                        float* zeros, int32_t* g_idx, float* row_err,
                                        int32_t* info, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Bit packing.  The pages fix the storage cost (b bits per weight plus the
 * per-group scale and zero-point, "LLM quantization principles", section 4.2)
 * but not a layout; this library's layout: row r of codes[m, n] becomes one
 * little-endian bitstream of uint32 words, column c in bits [c*b, c*b + b)
 * (3-bit codes straddle words), zero-padded, packed[m, ceil(n*b/32)].
 * Codes must be < 2^bits (higher bits are masked off).
 * ---------------------------------------------------------------------- */
gptq_status gptq_pack(const uint8_t* codes, int64_t m, int64_t n, int32_t bits,
                      uint32_t* packed, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Packing in processing order: the layout of gptq_pack applied to the row
 * codes[r, perm[0]], codes[r, perm[1]], ..., so that stream position p holds
 * the code of original column perm[p] (perm as gptq_prepare returns it; NULL =
 * the identity, i.e. gptq_pack).  With desc_act the quantization groups are
 * runs of group_size consecutive processing positions ("GPTQ deep dive",
 * section 3.3), which is the form gptq_dequant_gemm reads.
 * ---------------------------------------------------------------------- */
gptq_status gptq_pack_ordered(const uint8_t* codes, int64_t m, int64_t n, int32_t bits,
                              const int32_t* perm, uint32_t* packed, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Dequantized-weight product -- "Quantized deployment, 1.5 TB to 250 GB"
 * (lmnt.cn news 123823), section 2.1 (a code q stands for (q - zero) * scale)
 * and "LLM quantization principles", section 5.2 (low-bit weights are
 * dequantized for the matrix product; fusing the two keeps the cost down):
 *
 *   Y[t, r] = sum_c X[t, c] * scale[r, g(c)] * (q[r, c] - zero[r, g(c)])
 *
 * X[tokens, n] bf16, row stride ldx >= n; without perm, ldx must be a
 * multiple of 8 and X 16-byte aligned (it is read in 16-byte vectors).
 * packed[m, ldp] uint32 (ldp >= ceil(n * bits / 32)): the codes packed in
 * processing order by gptq_pack_ordered with this same perm.  scales, zeros
 * [m, ngroups] fp32 as gptq_quantize_layer writes them: group k covers
 * processing positions [k * group_size, (k + 1) * group_size); group_size is
 * a multiple of 8, or -1 for one group per row.  perm[n] (may be NULL =
 * identity): processing position -> original column.  Y[tokens, ldy] fp32 or
 * bf16 (ydt); Y must not overlap the inputs.  bits 2..8; xdt must be BF16
 * (GPTQ_ERR_UNSUPPORTED otherwise).
 * Arithmetic: each weight is formed in fp32 as fma(q, scale, -(zero * scale)),
 * rounded to bf16 (nearest even), multiplied exactly by the bf16 activation,
 * and the products are summed in fp32 (in a fixed order: deterministic).
 * Workspace: gptq_dequant_gemm_workspace_size(tokens, m, n, perm != NULL)
 * bytes (may be 0; from 1024 tokens up, with n a multiple of 8, it holds the
 * dequantized bf16 weights, m * n * 2 bytes, which the call forms once and
 * multiplies as gptq_gemm_bf16 does -- the same weights, the same result
 * contract).  tokens == 0 or m == 0 is a no-op.
 * ---------------------------------------------------------------------- */
/* gptq_dequantize: W[m, n] bf16 (row stride ldw, a multiple of 8, 16-byte
 * aligned) = the weights gptq_dequant_gemm forms, bf16(fma(q, s, -(z s))) with
 * the fma in fp32 and round to nearest even ("Quantized deployment, 1.5 TB to
 * 250 GB" section 2.1: r = (q - zero) * scale), from codes packed in
 * processing order as gptq_dequant_gemm reads them (same packed, ldp, bits,
 * group_size, scales, zeros).  n a multiple of 8 (GPTQ_ERR_UNSUPPORTED
 * otherwise).  For products over many tokens the weights are dequantized
 * once and multiplied with gptq_gemm_bf16.
 *
 * gptq_gemm_bf16: Y[tokens, m] = X[tokens, n] W[m, n]^T, X and W bf16 device
 * (row strides multiples of 8 below 2^23, 16-byte aligned), products exact,
 * fp32 sums in a fixed order; Y fp32 or bf16 (round to nearest even), row
 * stride ldy >= m.  n a multiple of 8.  No workspace. */
gptq_status gptq_dequantize(const uint32_t* packed, int64_t ldp, int32_t bits,
                            int32_t group_size, const float* scales, const float* zeros,
                            int64_t m, int64_t n, void* W, int64_t ldw, hipStream_t stream);
gptq_status gptq_gemm_bf16(const void* X, int64_t tokens, int64_t n, int64_t ldx, const void* W,
                           int64_t m, int64_t ldw, void* Y, gptq_dtype ydt, int64_t ldy,
                           hipStream_t stream);

/* gptq_gather_columns: Xp[t, p] = X[t, perm[p]] for p < n, 0 for n <= p < ldxp --
 * the processing-order activations the product reads when perm is given,
 * formed once so that several layers with the same order (layers sharing an
 * input, hence a Hessian and its order: "GPTQ deep dive" section 3.1 step 4)
 * can be multiplied with perm = NULL.  X, Xp bf16 [tokens, *] device, row
 * strides ldx >= n and ldxp >= n (ldxp a multiple of 8, Xp 16-byte aligned);
 * perm int32 [n] device, a permutation of 0..n-1 (an entry outside it reads
 * as 0).  No workspace.  GPTQ_ERR_UNSUPPORTED for fp32 X. */
gptq_status gptq_gather_columns(const void* X, gptq_dtype xdt, int64_t tokens, int64_t n,
                                int64_t ldx, const int32_t* perm, void* Xp, int64_t ldxp,
                                hipStream_t stream);
gptq_status gptq_dequant_gemm_workspace_size(int64_t tokens, int64_t m, int64_t n,
                                             int32_t has_perm, size_t* bytes);
gptq_status gptq_dequant_gemm(const void* X, gptq_dtype xdt, int64_t tokens, int64_t n,
                              int64_t ldx, const uint32_t* packed, int64_t ldp, int32_t bits,
                              int32_t group_size, const float* scales, const float* zeros,
                              const int32_t* perm, int64_t m, void* Y, gptq_dtype ydt,
                              int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Forward steps between quantized layers -- "GPTQ deep dive", section 3.1
 * step 4, and "AWQ, MinMax, GPTQ calibration in Model Optimizer", section 4:
 * layers are quantized in order and each layer's calibration inputs are the
 * outputs of the layers already quantized.  In a Llama-style MLP block the
 * dequantized-weight products are joined by two elementwise steps:
 *
 *   gptq_swiglu:       h = bf16(silu(gate) * up), silu(g) = g / (1 + e^-g)
 *   gptq_residual_add: out = bf16(x + y)
 *
 * gate, up, y: fp32 [tokens, n] (row strides ldg, ldu, ldy >= n), as
 * gptq_dequant_gemm writes them; x, h, out: bf16 [tokens, n] (strides >= n).
 * fp32 arithmetic, rounded once to bf16 (nearest even).  out may alias x.
 * tokens == 0 or n == 0 is a no-op.
 * ---------------------------------------------------------------------- */
gptq_status gptq_swiglu(const float* gate, int64_t ldg, const float* up, int64_t ldu,
                        int64_t tokens, int64_t n, void* h, int64_t ldh, hipStream_t stream);
gptq_status gptq_residual_add(const void* x, int64_t ldx, const float* y, int64_t ldy,
                              int64_t tokens, int64_t n, void* out, int64_t ldo,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * AWQ-lite and awq_clip -- "AWQ, MinMax, GPTQ calibration in Model
 * Optimizer" (gtnt.cn news 115337), section 3, and "LLM quantization
 * principles", section 3.2.  The weights are multiplied per input channel by
 * s = x^alpha / w^(1 - alpha) and the activations divided by it (x, w: the
 * channel's mean |activation| and mean |weight|, floored at 1e-8); alpha is
 * searched on a grid of n_alpha points over [0, 1] (11 = steps of 0.1) for the
 * smallest output error ||X (W_eff - W)^T||^2, W_eff = dequant(Q(W diag(s)))
 * diag(1/s), Q the group min-max quantizer of rtn_minmax (groups of group_size
 * consecutive columns, -1 = whole row).  The error is computed through
 * S = X^T X (the lower triangle gptq_hessian_accumulate builds).  awq_clip
 * then searches, per row and group of W' = W diag(s), the clip value
 * c_k = (1 - 0.05 k) amax, k < n_steps (11 = down to 0.5 amax): the group's
 * parameters come from its values clamped to [-c_k, c_k]; the error of a
 * candidate is d S'_gg d^T, S' = diag(1/s) S diag(1/s), d the group's error
 * in the rescaled space.  Ties keep the first candidate (smallest alpha,
 * largest clip).  The quantized layer computes (X / s) dequant(codes)^T.
 *
 * awq_activation_absum: absum[n] += sum over tokens of |X[t, c]| (additive over
 *   calls, like the Hessian; each call sums in fp64 and rounds once into the
 *   fp32 absum); workspace awq_absum_workspace_size(n, tokens).
 * awq_lite: from W [m, n], S (lower, lds), absum over `tokens` tokens: s_out[n],
 *   alpha_out[1], losses[n_alpha] (fp32, device); workspace
 *   awq_lite_workspace_size(m, n) (holds a full copy of S and two m x n fp32
 *   matrices).  GPTQ_ERR_EMPTY when tokens == 0.  w is summed in fp64; s is
 *   computed in fp32 with powf.  Inputs are only read; every output is written.
 * awq_clip_quantize: codes[m, n] (uint8, of W diag(s)), scales/zeros
 *   [m, ceil(n / group_size)] fp32, clip_idx [m, ngroups] (uint8 k, may be
 *   NULL); s may be NULL (no rescaling: clip search on W itself).
 *   group_size 1..128 (GPTQ_ERR_UNSUPPORTED above).
 * ---------------------------------------------------------------------- */
gptq_status awq_absum_workspace_size(int64_t n, int64_t tokens, size_t* bytes);
gptq_status awq_activation_absum(const void* X, gptq_dtype xdt, int64_t tokens, int64_t n,
                                 int64_t ldx, float* absum, void* ws, size_t ws_bytes,
                                 hipStream_t stream);
gptq_status awq_lite_workspace_size(int64_t m, int64_t n, size_t* bytes);
gptq_status awq_lite(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                     const float* S, int64_t lds, const float* absum, int64_t tokens,
                     int32_t bits, int32_t group_size, int32_t sym, int32_t n_alpha,
                     float* s_out, float* alpha_out, float* losses, void* ws, size_t ws_bytes,
                     hipStream_t stream);
gptq_status awq_clip_quantize(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                              const float* S, int64_t lds, const float* s, int32_t bits,
                              int32_t group_size, int32_t sym, int32_t n_steps, uint8_t* codes,
                              float* scales, float* zeros, uint8_t* clip_idx,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Round-to-nearest baseline -- "GPTQ deep dive", section 1.2 (RTN rounds each
 * weight on its own, no compensation) with group-wise min-max parameters
 * ("Calibration algorithms guide", bhfrc.com news 5741, section 2.2): the
 * quantizer of gptq_quantize_layer applied to the original W, groups of
 * group_size consecutive original columns (-1 = whole row).
 * codes[m, n] (row stride n), scales/zeros[m, ceil(n / group_size)].
 * ---------------------------------------------------------------------- */
gptq_status rtn_minmax(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                       int32_t bits, int32_t group_size, int32_t sym, uint8_t* codes,
                       float* scales, float* zeros, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Layer reconstruction error -- "LLM quantization principles: GPTQ, AWQ,
 * GGUF" (0539edu.com news 6111416), section 3.1: the quantity GPTQ minimizes
 * layer by layer is the output error ||W X - W_q X||^2 over the calibration
 * inputs.  Through the raw second moments S = X^T X of gptq_hessian_accumulate
 * (lower triangle read, lds >= n):
 *   err[r] = delta_r S delta_r^T = sum over calibration tokens of (delta_r . x_t)^2,
 *   delta_r = W[r] - W_q[r],  W_q[r][c] = scales[r][g] * (codes[r][c] - zeros[r][g]),
 *   g = g_idx[c]
 * for W [m, n] (row stride ldw, fp32 or bf16) and the ORIGINAL-order outputs
 * of gptq_quantize_layer or rtn_minmax: codes [m, n] (row stride n),
 * scales/zeros [m, ngroups], g_idx [n] (for rtn_minmax, g_idx[c] =
 * c / group_size).  The sum over rows is the layer objective (half of
 * delta^T H delta with H = 2S, undamped).  err: double [m] on the device.
 * fp32 differences and products (the fp32 MFMA update product), each row
 * summed in fp64 in a fixed order: deterministic.  g_idx entries outside
 * [0, ngroups) are clamped.  m == 0 is a no-op.  Workspace:
 * gptq_layer_error_workspace_size(m, n) bytes (S made symmetric, the
 * differences and their product with S, in fp32).
 * ---------------------------------------------------------------------- */
gptq_status gptq_layer_error_workspace_size(int64_t m, int64_t n, size_t* bytes);
gptq_status gptq_layer_error(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                             const uint8_t* codes, const float* scales, const float* zeros,
                             int64_t ngroups, const int32_t* g_idx, const float* S, int64_t lds,
                             double* err, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
