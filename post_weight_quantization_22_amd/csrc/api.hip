// extern "C" entry points: argument validation, workspace sizing, launches.
// Every check here runs on the host before anything is enqueued.
#include <cmath>

#include "kernels.hpp"

using namespace gptq;

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 24;  // sanity bound on m, n

inline bool bad_dim(int64_t v) { return v < 0 || v > kMaxDim; }

inline gptq_status hip_status(hipError_t e) { return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP; }

inline bool valid_dtype(int dt) { return dt == GPTQ_F32 || dt == GPTQ_BF16; }

inline bool quant_group_ok(int32_t g) {
  return g == -1 || g == 8 || g == 16 || g == 32 || g == 64 || g == 128 || g == 256 || g == 512;
}

gptq_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return GPTQ_OK;
  if (ws == nullptr || ws_bytes < need) return GPTQ_ERR_WORKSPACE;
  return GPTQ_OK;
}

}  // namespace

extern "C" {

uint32_t gptq_abi_version(void) { return GPTQ_ABI_VERSION; }

const char* gptq_status_str(int32_t status) {
  switch (status) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_INVALID_ARG: return "invalid argument";
    case GPTQ_ERR_NOT_PD: return "damped Hessian is not positive definite (raise perc_damp)";
    case GPTQ_ERR_NONFINITE: return "non-finite value in the input";
    case GPTQ_ERR_EMPTY: return "no calibration tokens";
    case GPTQ_ERR_WORKSPACE: return "workspace missing or too small";
    case GPTQ_ERR_HIP: return "HIP runtime error";
    case GPTQ_ERR_UNSUPPORTED: return "configuration not supported by this library";
    default: return "unknown status";
  }
}

gptq_status gptq_hessian_workspace_size(int64_t n, int64_t tokens, size_t* bytes) {
  if (!bytes || n <= 0 || bad_dim(n) || tokens < 0) return GPTQ_ERR_INVALID_ARG;
  *bytes = hessian_ws_bytes(n, tokens, GPTQ_BF16);
  return GPTQ_OK;
}

gptq_status gptq_hessian_accumulate(float* S, int64_t n, int64_t lds, const void* X,
                                    gptq_dtype xdt, int64_t tokens, int64_t ldx, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  if (!S || n <= 0 || bad_dim(n) || lds < n || tokens < 0 || !valid_dtype(xdt))
    return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0) return GPTQ_OK;
  if (!X || ldx < n) return GPTQ_ERR_INVALID_ARG;
  const gptq_status w = check_ws(ws, ws_bytes, hessian_ws_bytes(n, tokens, xdt));
  if (w != GPTQ_OK) return w;
  return hip_status(launch_hessian(S, n, lds, X, xdt, tokens, ldx, ws, ws_bytes, stream));
}

gptq_status gptq_prepare_workspace_size(int64_t n, size_t* bytes) {
  if (!bytes || n <= 0 || bad_dim(n)) return GPTQ_ERR_INVALID_ARG;
  *bytes = prepare_ws_bytes(n);
  return GPTQ_OK;
}

gptq_status gptq_prepare(const float* S, int64_t n, int64_t lds, int64_t tokens, float perc_damp,
                         int32_t desc_act, float* U, int64_t ldu, int32_t* perm, uint8_t* dead,
                         float* lambda_out, int32_t* info, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  if (!S || !U || !info || n <= 0 || bad_dim(n) || lds < n || ldu < n || tokens < 0 ||
      !(perc_damp >= 0.0f) || !std::isfinite(perc_damp) || (desc_act != 0 && desc_act != 1))
    return GPTQ_ERR_INVALID_ARG;
  if (U == S && ldu != lds) return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0) return GPTQ_ERR_EMPTY;
  const gptq_status w = check_ws(ws, ws_bytes, prepare_ws_bytes(n));
  if (w != GPTQ_OK) return w;
  return hip_status(launch_prepare(S, n, lds, perc_damp, desc_act, U, ldu, perm, dead, lambda_out,
                                   info, ws, stream));
}

gptq_status gptq_quantize_workspace_size(int64_t m, int64_t n, const gptq_config* cfg,
                                         size_t* bytes) {
  if (!bytes || !cfg || bad_dim(m) || bad_dim(n)) return GPTQ_ERR_INVALID_ARG;
  *bytes = quantize_ws_bytes(m, n, cfg->desc_act);
  return GPTQ_OK;
}

gptq_status gptq_quantize_layer(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                                const float* U, int64_t ldu, const int32_t* perm,
                                const uint8_t* dead, const gptq_config* cfg, uint8_t* codes,
                                float* scales, float* zeros, int32_t* g_idx, float* row_err,
                                int32_t* info, void* ws, size_t ws_bytes, hipStream_t stream) {
  return quantize_layer_checked(W, wdt, m, n, ldw, U, ldu, perm, dead, cfg, codes, scales, zeros,
                                g_idx, row_err, info, ws, ws_bytes, stream);
}

gptq_status gptq_pack(const uint8_t* codes, int64_t m, int64_t n, int32_t bits, uint32_t* packed,
                      hipStream_t stream) {
  if (bad_dim(m) || bad_dim(n) || bits < 1 || bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return GPTQ_OK;
  if (!codes || !packed) return GPTQ_ERR_INVALID_ARG;
  return hip_status(launch_pack(codes, m, n, bits, nullptr, packed, stream));
}

gptq_status gptq_pack_ordered(const uint8_t* codes, int64_t m, int64_t n, int32_t bits,
                              const int32_t* perm, uint32_t* packed, hipStream_t stream) {
  if (bad_dim(m) || bad_dim(n) || bits < 1 || bits > 8) return GPTQ_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return GPTQ_OK;
  if (!codes || !packed) return GPTQ_ERR_INVALID_ARG;
  return hip_status(launch_pack(codes, m, n, bits, perm, packed, stream));
}

gptq_status gptq_dequant_gemm_workspace_size(int64_t tokens, int64_t m, int64_t n,
                                             int32_t has_perm, size_t* bytes) {
  if (!bytes || tokens < 0 || bad_dim(tokens) || bad_dim(m) || bad_dim(n) ||
      (has_perm != 0 && has_perm != 1))
    return GPTQ_ERR_INVALID_ARG;
  *bytes = (tokens == 0 || m == 0 || n == 0) ? 0 : dequant_gemm_ws_bytes(tokens, m, n, has_perm);
  return GPTQ_OK;
}

gptq_status gptq_dequantize(const uint32_t* packed, int64_t ldp, int32_t bits,
                            int32_t group_size, const float* scales, const float* zeros,
                            int64_t m, int64_t n, void* W, int64_t ldw, hipStream_t stream) {
  if (bad_dim(m) || n <= 0 || bad_dim(n) || bits < 2 || bits > 8 ||
      !(group_size == -1 || (group_size >= 8 && group_size % 8 == 0)))
    return GPTQ_ERR_INVALID_ARG;
  if (n % 8 != 0) return GPTQ_ERR_UNSUPPORTED;
  if (m == 0) return GPTQ_OK;
  if (!packed || !scales || !zeros || !W || ldp < ceil_div(n * bits, 32) || ldw < n ||
      ldw % 8 != 0 || (reinterpret_cast<uintptr_t>(W) & 15) != 0)
    return GPTQ_ERR_INVALID_ARG;
  return hip_status(launch_dequantize(packed, ldp, bits, m, n, scales, zeros, group_size,
                                      static_cast<uint16_t*>(W), ldw, stream));
}

gptq_status gptq_gemm_bf16(const void* X, int64_t tokens, int64_t n, int64_t ldx, const void* W,
                           int64_t m, int64_t ldw, void* Y, gptq_dtype ydt, int64_t ldy,
                           hipStream_t stream) {
  if (tokens < 0 || bad_dim(tokens) || bad_dim(m) || n <= 0 || bad_dim(n) || !valid_dtype(ydt))
    return GPTQ_ERR_INVALID_ARG;
  if (n % 8 != 0) return GPTQ_ERR_UNSUPPORTED;
  if (tokens == 0 || m == 0) return GPTQ_OK;
  if (!X || !W || !Y || ldx < n || ldw < n || ldy < m || ldx % 8 != 0 || ldw % 8 != 0 ||
      (reinterpret_cast<uintptr_t>(X) & 15) != 0 || (reinterpret_cast<uintptr_t>(W) & 15) != 0)
    return GPTQ_ERR_INVALID_ARG;
  // the DMA offsets within a tile are 32-bit
  if (ldx >= (int64_t(1) << 23) || ldw >= (int64_t(1) << 23)) return GPTQ_ERR_UNSUPPORTED;
  return hip_status(launch_dense_gemm(static_cast<const uint16_t*>(X), ldx, tokens, n,
                                      static_cast<const uint16_t*>(W), ldw, m, Y, ldy,
                                      ydt == GPTQ_BF16 ? 1 : 0, stream));
}

gptq_status gptq_gather_columns(const void* X, gptq_dtype xdt, int64_t tokens, int64_t n,
                                int64_t ldx, const int32_t* perm, void* Xp, int64_t ldxp,
                                hipStream_t stream) {
  if (tokens < 0 || bad_dim(tokens) || n <= 0 || bad_dim(n) || !valid_dtype(xdt))
    return GPTQ_ERR_INVALID_ARG;
  if (xdt != GPTQ_BF16) return GPTQ_ERR_UNSUPPORTED;
  if (tokens == 0) return GPTQ_OK;
  if (!X || !perm || !Xp || ldx < n || ldxp < n || ldxp % 8 != 0 ||
      (reinterpret_cast<uintptr_t>(Xp) & 15) != 0)
    return GPTQ_ERR_INVALID_ARG;
  launch_gather(static_cast<const uint16_t*>(X), ldx, perm, tokens, n, ldxp,
                static_cast<uint16_t*>(Xp), stream);
  return hip_status(hipGetLastError());
}

gptq_status gptq_dequant_gemm(const void* X, gptq_dtype xdt, int64_t tokens, int64_t n,
                              int64_t ldx, const uint32_t* packed, int64_t ldp, int32_t bits,
                              int32_t group_size, const float* scales, const float* zeros,
                              const int32_t* perm, int64_t m, void* Y, gptq_dtype ydt,
                              int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (tokens < 0 || bad_dim(tokens) || bad_dim(m) || n <= 0 || bad_dim(n) || bits < 2 ||
      bits > 8 || !valid_dtype(xdt) || !valid_dtype(ydt) ||
      !(group_size == -1 || (group_size >= 8 && group_size % 8 == 0)))
    return GPTQ_ERR_INVALID_ARG;
  if (xdt != GPTQ_BF16) return GPTQ_ERR_UNSUPPORTED;
  if (tokens == 0 || m == 0) return GPTQ_OK;
  if (!X || !packed || !scales || !zeros || !Y || ldx < n || ldp < ceil_div(n * bits, 32) ||
      ldy < m)
    return GPTQ_ERR_INVALID_ARG;
  // X is read with 16-byte loads unless the permutation gathers it first
  if (!perm && (ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(X) & 15) != 0))
    return GPTQ_ERR_INVALID_ARG;
  const gptq_status w =
      check_ws(ws, ws_bytes, dequant_gemm_ws_bytes(tokens, m, n, perm != nullptr ? 1 : 0));
  if (w != GPTQ_OK) return w;
  DequantArgs d;
  d.X = X;
  d.tokens = tokens;
  d.n = n;
  d.ldx = ldx;
  d.packed = packed;
  d.ldp = ldp;
  d.bits = bits;
  d.group_size = group_size;
  d.scales = scales;
  d.zeros = zeros;
  d.perm = perm;
  d.m = m;
  d.Y = Y;
  d.ydt = ydt;
  d.ldy = ldy;
  d.ws = ws;
  return hip_status(launch_dequant_gemm(d, stream));
}

gptq_status gptq_swiglu(const float* gate, int64_t ldg, const float* up, int64_t ldu,
                        int64_t tokens, int64_t n, void* h, int64_t ldh, hipStream_t stream) {
  if (tokens < 0 || bad_dim(tokens) || n < 0 || bad_dim(n)) return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0 || n == 0) return GPTQ_OK;
  if (!gate || !up || !h || ldg < n || ldu < n || ldh < n) return GPTQ_ERR_INVALID_ARG;
  return hip_status(launch_swiglu(gate, ldg, up, ldu, tokens, n, h, ldh, stream));
}

gptq_status gptq_residual_add(const void* x, int64_t ldx, const float* y, int64_t ldy,
                              int64_t tokens, int64_t n, void* out, int64_t ldo,
                              hipStream_t stream) {
  if (tokens < 0 || bad_dim(tokens) || n < 0 || bad_dim(n)) return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0 || n == 0) return GPTQ_OK;
  if (!x || !y || !out || ldx < n || ldy < n || ldo < n) return GPTQ_ERR_INVALID_ARG;
  return hip_status(launch_residual_add(x, ldx, y, ldy, tokens, n, out, ldo, stream));
}

gptq_status awq_absum_workspace_size(int64_t n, int64_t tokens, size_t* bytes) {
  if (!bytes || n <= 0 || bad_dim(n) || tokens < 0) return GPTQ_ERR_INVALID_ARG;
  *bytes = awq_absum_ws_bytes(n, tokens);
  return GPTQ_OK;
}

gptq_status awq_activation_absum(const void* X, gptq_dtype xdt, int64_t tokens, int64_t n,
                                 int64_t ldx, float* absum, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  if (!absum || n <= 0 || bad_dim(n) || tokens < 0 || !valid_dtype(xdt))
    return GPTQ_ERR_INVALID_ARG;
  if (tokens == 0) return GPTQ_OK;
  if (!X || ldx < n) return GPTQ_ERR_INVALID_ARG;
  const gptq_status w = check_ws(ws, ws_bytes, awq_absum_ws_bytes(n, tokens));
  if (w != GPTQ_OK) return w;
  return hip_status(launch_awq_absum(X, xdt, tokens, n, ldx, absum, ws, stream));
}

gptq_status awq_lite_workspace_size(int64_t m, int64_t n, size_t* bytes) {
  if (!bytes || m <= 0 || n <= 0 || bad_dim(m) || bad_dim(n)) return GPTQ_ERR_INVALID_ARG;
  *bytes = awq_lite_ws_bytes(m, n);
  return GPTQ_OK;
}

gptq_status awq_lite(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                     const float* S, int64_t lds, const float* absum, int64_t tokens,
                     int32_t bits, int32_t group_size, int32_t sym, int32_t n_alpha,
                     float* s_out, float* alpha_out, float* losses, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (!W || !S || !absum || !s_out || !alpha_out || !losses || m <= 0 || n <= 0 ||
      bad_dim(m) || bad_dim(n) || ldw < n || lds < n || !valid_dtype(wdt) || bits < 2 ||
      bits > 8 || group_size == 0 || group_size < -1 || (sym != 0 && sym != 1) ||
      n_alpha < 2 || n_alpha > 101)
    return GPTQ_ERR_INVALID_ARG;
  if (tokens <= 0) return GPTQ_ERR_EMPTY;
  const gptq_status w = check_ws(ws, ws_bytes, awq_lite_ws_bytes(m, n));
  if (w != GPTQ_OK) return w;
  return hip_status(launch_awq_lite(W, wdt, m, n, ldw, S, lds, absum, tokens, bits, group_size,
                                    sym, n_alpha, s_out, alpha_out, losses, ws, stream));
}

gptq_status gptq_layer_error_workspace_size(int64_t m, int64_t n, size_t* bytes) {
  if (!bytes || bad_dim(m) || n <= 0 || bad_dim(n)) return GPTQ_ERR_INVALID_ARG;
  *bytes = layer_error_ws_bytes(m, n);
  return GPTQ_OK;
}

gptq_status gptq_layer_error(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                             const uint8_t* codes, const float* scales, const float* zeros,
                             int64_t ngroups, const int32_t* g_idx, const float* S, int64_t lds,
                             double* err, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!W || !codes || !scales || !zeros || !g_idx || !S || !err || bad_dim(m) || n <= 0 ||
      bad_dim(n) || ldw < n || lds < n || ngroups < 1 || ngroups > n || !valid_dtype(wdt))
    return GPTQ_ERR_INVALID_ARG;
  if (m == 0) return GPTQ_OK;
  const gptq_status w = check_ws(ws, ws_bytes, layer_error_ws_bytes(m, n));
  if (w != GPTQ_OK) return w;
  return hip_status(launch_layer_error(W, wdt, m, n, ldw, codes, scales, zeros, ngroups, g_idx, S,
                                       lds, err, ws, stream));
}

gptq_status awq_clip_quantize(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                              const float* S, int64_t lds, const float* s, int32_t bits,
                              int32_t group_size, int32_t sym, int32_t n_steps, uint8_t* codes,
                              float* scales, float* zeros, uint8_t* clip_idx,
                              hipStream_t stream) {
  if (!W || !S || !codes || !scales || !zeros || m < 0 || n <= 0 || bad_dim(m) || bad_dim(n) ||
      ldw < n || lds < n || !valid_dtype(wdt) || bits < 2 || bits > 8 || group_size < 1 ||
      (sym != 0 && sym != 1) || n_steps < 1 || n_steps > 11)
    return GPTQ_ERR_INVALID_ARG;
  if (group_size > 128) return GPTQ_ERR_UNSUPPORTED;
  if (m == 0) return GPTQ_OK;
  return hip_status(launch_awq_clip(W, wdt, m, n, ldw, S, lds, s, bits, group_size, sym, n_steps,
                                    codes, scales, zeros, clip_idx, stream));
}

gptq_status rtn_minmax(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                       int32_t bits, int32_t group_size, int32_t sym, uint8_t* codes,
                       float* scales, float* zeros, hipStream_t stream) {
  if (bad_dim(m) || bad_dim(n) || !valid_dtype(wdt) || bits < 2 || bits > 8 ||
      group_size == 0 || group_size < -1 || (sym != 0 && sym != 1))
    return GPTQ_ERR_INVALID_ARG;
  if (m == 0 || n == 0) return GPTQ_OK;
  if (!W || !codes || !scales || !zeros || ldw < n) return GPTQ_ERR_INVALID_ARG;
  return hip_status(launch_rtn(W, wdt, m, n, ldw, bits, group_size, sym, codes, scales, zeros,
                               stream));
}

}  // extern "C"

// Argument checks and launch of gptq_quantize_layer, shared with its
// no-allocation variant (which passes its static scratch as the workspace).
gptq_status gptq::quantize_layer_checked(const void* W, gptq_dtype wdt, int64_t m, int64_t n, int64_t ldw,
                                const float* U, int64_t ldu, const int32_t* perm,
                                const uint8_t* dead, const gptq_config* cfg, uint8_t* codes,
                                float* scales, float* zeros, int32_t* g_idx, float* row_err,
                                int32_t* info, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!cfg || bad_dim(m) || bad_dim(n) || !valid_dtype(wdt)) return GPTQ_ERR_INVALID_ARG;
  if (cfg->bits < 2 || cfg->bits > 8 || cfg->block_size <= 0 || cfg->group_size == 0 ||
      cfg->group_size < -1 ||
      (cfg->group_size > 0 && cfg->block_size % cfg->group_size != 0 &&
       cfg->group_size % cfg->block_size != 0) ||
      (cfg->desc_act != 0 && cfg->desc_act != 1) || (cfg->sym != 0 && cfg->sym != 1) ||
      (cfg->static_groups != 0 && cfg->static_groups != 1))
    return GPTQ_ERR_INVALID_ARG;
  if (cfg->block_size != 128 || !quant_group_ok(cfg->group_size)) return GPTQ_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return GPTQ_OK;
  if (!W || !U || !codes || !scales || !zeros || ldw < n || ldu < n) return GPTQ_ERR_INVALID_ARG;
  if (cfg->desc_act && !perm) return GPTQ_ERR_INVALID_ARG;
  const gptq_status w = check_ws(ws, ws_bytes, quantize_ws_bytes(m, n, cfg->desc_act));
  if (w != GPTQ_OK) return w;
  QuantArgs a;
  a.W = W;
  a.wdt = wdt;
  a.m = m;
  a.n = n;
  a.ldw = ldw;
  a.U = U;
  a.ldu = ldu;
  a.perm = perm;
  a.dead = dead;
  a.bits = cfg->bits;
  a.group_size = cfg->group_size;
  a.block_size = cfg->block_size;
  a.desc_act = cfg->desc_act;
  a.sym = cfg->sym;
  a.static_groups = cfg->group_size > 0 ? cfg->static_groups : 0;
  a.codes = codes;
  a.scales = scales;
  a.zeros = zeros;
  a.g_idx = g_idx;
  a.row_err = row_err;
  a.info = info;
  a.ws = ws;
  return hip_status(launch_quantize(a, stream));
}
