// Layer reconstruction error of a quantized layer, on gfx950.
//
// "LLM quantization principles: GPTQ, AWQ, GGUF" (0539edu.com news 6111416)
// section 3.1: the layer objective is the output error ||W X - W_q X||^2 over
// the calibration inputs.  Through the raw second moments S = X^T X that the
// Hessian step accumulates ("GPTQ deep dive", section 3.1 step 1), the error
// of row r is delta_r S delta_r^T = sum over tokens of (delta_r . x_t)^2, with
// delta_r = W[r] - W_q[r] and W_q[r][c] = scale * (q - zero) of column c's
// group g_idx[c] (original column order, as gptq_quantize_layer writes codes,
// scales, zeros and g_idx).  Summed over rows it is the layer objective.
//
// Three steps: D = W - W_q in fp32 (rows padded with zeros to a multiple of
// 4 floats); Z = -D S_sym on the fp32 MFMA update product (S_sym the whole
// symmetric S, built from S's lower triangle by 32 x 32 tiles and their
// transposes through LDS); err[r] = -sum_c Z[r][c] D[r][c], summed in fp64 in
// a fixed order by one workgroup per row (deterministic).  2 m n^2 flop.
#include "kernels.hpp"

namespace gptq {

namespace {

int64_t err_ld(int64_t n) { return ceil_div(n, (int64_t)4) * 4; }

__global__ __launch_bounds__(256) void delta_kernel(const void* __restrict__ W, int wdt,
                                                    int64_t ldw, const uint8_t* __restrict__ codes,
                                                    int64_t m, int64_t n,
                                                    const float* __restrict__ scales,
                                                    const float* __restrict__ zeros,
                                                    int64_t ngroups,
                                                    const int32_t* __restrict__ g_idx,
                                                    float* __restrict__ D, int64_t ldd) {
  // the dequantized weight is rounded on its own before the difference (the
  // compiler would otherwise fuse w - s (q - z) into one fma, even through
  // __fmul_rn)
#pragma clang fp contract(off)
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= ldd) return;
  int64_t g = 0;
  if (c < n) g = min<int64_t>(max<int64_t>(g_idx[c], 0), ngroups - 1);
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    float d = 0.0f;
    if (c < n) {
      const float s = scales[r * ngroups + g], z = zeros[r * ngroups + g];
      const float dq = s * ((float)codes[r * n + c] - z);
      d = load_elem(W, wdt, r * ldw + c) - dq;
    }
    D[r * ldd + c] = d;
  }
}

// F = S with its upper triangle filled from the lower one (n x n, stride ldf)
__global__ __launch_bounds__(256) void sym_full_kernel(const float* __restrict__ S, int64_t n,
                                                       int64_t lds, float* __restrict__ F,
                                                       int64_t ldf) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t i0 = (int64_t)blockIdx.y * 32, j0 = (int64_t)blockIdx.x * 32;
  if (j0 > i0) return;
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = i0 + r, j = j0 + tx;
    tile[r][tx] = (i < n && j <= i) ? S[i * lds + j] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t i = i0 + r, j = j0 + tx;
    if (i < n && j < n) F[i * ldf + j] = j <= i ? tile[r][tx] : tile[tx][r];
  }
  if (i0 == j0) return;
  for (int r = ty; r < 32; r += 8) {  // the transposed tile
    const int64_t j = j0 + r, i = i0 + tx;
    if (i < n && j < n) F[j * ldf + i] = tile[tx][r];
  }
}

__global__ __launch_bounds__(256) void zero_rows_kernel(float* __restrict__ p, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) p[i] = 0.0f;
}

// err[r] = -sum_c Z[r][c] D[r][c]: per-thread fp64 sums over a fixed stride,
// then a fixed tree
__global__ __launch_bounds__(256) void row_dot_kernel(const float* __restrict__ Z,
                                                      const float* __restrict__ D, int64_t ldd,
                                                      double* __restrict__ err) {
  __shared__ double red[256];
  const int64_t r = blockIdx.x;
  const float* z = Z + r * ldd;
  const float* d = D + r * ldd;
  double acc = 0.0;
  for (int64_t c = threadIdx.x; c < ldd; c += 256) acc += (double)z[c] * (double)d[c];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) err[r] = -red[0];
}

}  // namespace

size_t layer_error_ws_bytes(int64_t m, int64_t n) {
  const int64_t ldd = err_ld(n);
  return align_up((size_t)n * ldd * sizeof(float), 256) +
         2 * align_up((size_t)m * ldd * sizeof(float), 256);
}

hipError_t launch_layer_error(const void* W, int wdt, int64_t m, int64_t n, int64_t ldw,
                              const uint8_t* codes, const float* scales, const float* zeros,
                              int64_t ngroups, const int32_t* g_idx, const float* S, int64_t lds,
                              double* err, void* ws, hipStream_t stream) {
  if (m <= 0) return hipSuccess;
  const int64_t ldd = err_ld(n);
  char* p = static_cast<char*>(ws);
  float* F = reinterpret_cast<float*>(p);  // [n, ldd]: 16-byte rows for the product
  p += align_up((size_t)n * ldd * sizeof(float), 256);
  float* D = reinterpret_cast<float*>(p);
  p += align_up((size_t)m * ldd * sizeof(float), 256);
  float* Z = reinterpret_cast<float*>(p);
  {
    const dim3 grid((unsigned)ceil_div(n, (int64_t)32), (unsigned)ceil_div(n, (int64_t)32));
    hipLaunchKernelGGL(sym_full_kernel, grid, dim3(256), 0, stream, S, n, lds, F, ldd);
  }
  {
    const dim3 grid((unsigned)ceil_div(ldd, (int64_t)256), (unsigned)hmin(m, (int64_t)4096));
    hipLaunchKernelGGL(delta_kernel, grid, dim3(256), 0, stream, W, wdt, ldw, codes, m, n, scales,
                       zeros, ngroups, g_idx, D, ldd);
  }
  const int64_t total = m * ldd;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)ceil_div(total, (int64_t)256)), dim3(256), 0,
                     stream, Z, total);
  // Z = -D S in one launch (2 m n^2 flop; at 8192 x 28672 ~120 TFLOP/s, as
  // launches of K = 1024 adding to Z too)
  const hipError_t e = gemm_f32_sub(Z, ldd, m, n, D, ldd, F, ldd, n, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_dot_kernel, dim3((unsigned)m), dim3(256), 0, stream, Z, D, ldd, err);
  return hipGetLastError();
}

}  // namespace gptq
