// Internal launchers of the gfx950 kernels (C++ linkage, not part of the ABI).
#pragma once

#include "common.hpp"

namespace gptq {

// ---- rtn.hip --------------------------------------------------------------
hipError_t launch_rtn(const void* W, int dt, int64_t m, int64_t n, int64_t ldw, int bits,
                      int64_t G, int sym, uint8_t* codes, float* scales, float* zeros,
                      hipStream_t stream);

// ---- pack.hip -------------------------------------------------------------
// perm (may be null): position p of a row's stream takes codes[r, perm[p]]
hipError_t launch_pack(const uint8_t* codes, int64_t m, int64_t n, int bits,
                       const int32_t* perm, uint32_t* packed, hipStream_t stream);

// ---- hessian.hip ----------------------------------------------------------
size_t hessian_ws_bytes(int64_t n, int64_t tokens, int dt);
hipError_t launch_hessian(float* S, int64_t n, int64_t lds, const void* X, int dt, int64_t tokens,
                          int64_t ldx, void* ws, size_t ws_bytes, hipStream_t stream);

// ---- prepare.hip ----------------------------------------------------------
size_t prepare_ws_bytes(int64_t n);
hipError_t launch_prepare(const float* S, int64_t n, int64_t lds, float perc_damp, int desc_act,
                          float* U, int64_t ldu, int32_t* perm, uint8_t* dead, float* lambda_out,
                          int32_t* info, void* ws, hipStream_t stream);

// ---- quantize.hip ---------------------------------------------------------
struct QuantArgs {
  const void* W;
  int wdt;
  int64_t m, n, ldw;
  const float* U;
  int64_t ldu;
  const int32_t* perm;  // used only when desc_act
  const uint8_t* dead;  // may be null
  int bits, group_size, block_size, desc_act, sym, static_groups;
  uint8_t* codes;
  float* scales;
  float* zeros;
  int32_t* g_idx;
  float* row_err;
  int32_t* info;
  void* ws;
};
size_t quantize_ws_bytes(int64_t m, int64_t n, int desc_act);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
// gptq_quantize_layer's argument checks and launch, on the given workspace
gptq_status quantize_layer_checked(const void* W, gptq_dtype wdt, int64_t m, int64_t n,
                                   int64_t ldw, const float* U, int64_t ldu, const int32_t* perm,
                                   const uint8_t* dead, const gptq_config* cfg, uint8_t* codes,
                                   float* scales, float* zeros, int32_t* g_idx, float* row_err,
                                   int32_t* info, void* ws, size_t ws_bytes, hipStream_t stream);
// C[m, n] (row stride ldc) -= A[m, k] (row stride lda, a multiple of 4, A 16-byte
// aligned) B[k, n] (row stride ldb), fp32 MFMA
hipError_t gemm_f32_sub(float* C, int64_t ldc, int64_t m, int64_t n, const float* A, int64_t lda,
                        const float* B, int64_t ldb, int64_t k, hipStream_t stream);

// ---- awq.hip --------------------------------------------------------------
size_t awq_absum_ws_bytes(int64_t n, int64_t tokens);
hipError_t launch_awq_absum(const void* X, int dt, int64_t tokens, int64_t n, int64_t ldx,
                            float* absum, void* ws, hipStream_t stream);
size_t awq_lite_ws_bytes(int64_t m, int64_t n);
hipError_t launch_awq_lite(const void* W, int wdt, int64_t m, int64_t n, int64_t ldw,
                           const float* S, int64_t lds, const float* absum, int64_t tokens,
                           int bits, int64_t G, int sym, int nalpha, float* s_out,
                           float* alpha_out, float* losses, void* ws, hipStream_t stream);
hipError_t launch_awq_clip(const void* W, int wdt, int64_t m, int64_t n, int64_t ldw,
                           const float* S, int64_t lds, const float* s, int bits, int64_t G,
                           int sym, int nsteps, uint8_t* codes, float* scales, float* zeros,
                           uint8_t* clip_idx, hipStream_t stream);

// ---- dequant_gemm.hip -----------------------------------------------------
struct DequantArgs {
  const void* X;  // bf16 [tokens, ldx]
  int64_t tokens, n, ldx;
  const uint32_t* packed;  // [m, ldp], processing order
  int64_t ldp;
  int bits, group_size;
  const float* scales;
  const float* zeros;
  const int32_t* perm;  // may be null
  int64_t m;
  void* Y;
  int ydt;
  int64_t ldy;
  void* ws;
};
size_t dequant_gemm_ws_bytes(int64_t tokens, int64_t m, int64_t n, int has_perm);
// Y[tokens, m] = X W^T, X [tokens, n] and W [m, n] bf16 (n % 8 == 0, strides
// multiples of 8, 16-byte aligned, strides < 2^23); Y fp32 or bf16 (ybf16)
hipError_t launch_dense_gemm(const uint16_t* X, int64_t ldx, int64_t tokens, int64_t n,
                             const uint16_t* W, int64_t ldw, int64_t m, void* Y, int64_t ldy,
                             int ybf16, hipStream_t stream);
// W[m, n] bf16 = the product's weights from processing-order packed codes (n % 8 == 0)
hipError_t launch_dequantize(const uint32_t* P, int64_t ldp, int bits, int64_t m, int64_t n,
                             const float* scales, const float* zeros, int64_t group_size,
                             uint16_t* W, int64_t ldw, hipStream_t stream);
// Xp[t, p] = X[t, perm[p]] (p < n), 0 for n <= p < ldxp (bf16)
void launch_gather(const uint16_t* X, int64_t ldx, const int32_t* perm, int64_t tokens,
                   int64_t n, int64_t ldxp, uint16_t* Xp, hipStream_t stream);
hipError_t launch_dequant_gemm(const DequantArgs& d, hipStream_t stream);

// ---- error.hip ------------------------------------------------------------
size_t layer_error_ws_bytes(int64_t m, int64_t n);
hipError_t launch_layer_error(const void* W, int wdt, int64_t m, int64_t n, int64_t ldw,
                              const uint8_t* codes, const float* scales, const float* zeros,
                              int64_t ngroups, const int32_t* g_idx, const float* S, int64_t lds,
                              double* err, void* ws, hipStream_t stream);

// ---- forward.hip ----------------------------------------------------------
hipError_t launch_swiglu(const float* G, int64_t ldg, const float* U, int64_t ldu, int64_t rows,
                         int64_t n, void* H, int64_t ldh, hipStream_t stream);
hipError_t launch_residual_add(const void* X, int64_t ldx, const float* Y, int64_t ldy,
                               int64_t rows, int64_t n, void* O, int64_t ldo, hipStream_t stream);

}  // namespace gptq
