// Elementwise steps of the forward pass that carries calibration activations
// from one quantized layer to the next.
//
// "GPTQ deep dive" (hncyxsy.com news 243429), section 3.1 step 4, and "AWQ,
// MinMax, GPTQ calibration in Model Optimizer" (gtnt.cn news 115337), section 4:
// layers are quantized in order, and the next layer's calibration inputs are
// what the already-quantized layers produce.  Between the dequantized-weight
// products of a Llama-style MLP block sit two elementwise steps, both HBM-bound:
//   h = bf16(silu(g) * u)            (gated activation; g, u fp32 products)
//   x' = bf16(x + y)                 (residual; x bf16, y fp32 product)
// silu(g) = g / (1 + e^-g), in fp32.  One thread per 4 consecutive elements of
// a row (16-byte fp32 loads, 8-byte bf16 stores) when the row strides allow.
#include "kernels.hpp"

namespace gptq {

namespace {

__device__ __forceinline__ uint16_t bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ G, int64_t ldg,
                                                     const float* __restrict__ U, int64_t ldu,
                                                     int64_t rows, int64_t n, int vec,
                                                     uint16_t* __restrict__ H, int64_t ldh) {
  const int64_t per_row = (n + 3) / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * per_row) return;
  const int64_t t = i / per_row, c0 = 4 * (i - t * per_row);
  const float* g = G + t * ldg + c0;
  const float* u = U + t * ldu + c0;
  uint16_t* h = H + t * ldh + c0;
  if (vec && c0 + 4 <= n) {
    const float4 gv = *reinterpret_cast<const float4*>(g);
    const float4 uv = *reinterpret_cast<const float4*>(u);
    const uint32_t lo = bf16_bits(silu(gv.x) * uv.x) | ((uint32_t)bf16_bits(silu(gv.y) * uv.y) << 16);
    const uint32_t hi = bf16_bits(silu(gv.z) * uv.z) | ((uint32_t)bf16_bits(silu(gv.w) * uv.w) << 16);
    *reinterpret_cast<uint2*>(h) = make_uint2(lo, hi);
  } else {
    for (int e = 0; e < 4 && c0 + e < n; ++e) h[e] = bf16_bits(silu(g[e]) * u[e]);
  }
}

__global__ __launch_bounds__(256) void residual_add_kernel(const uint16_t* __restrict__ X,
                                                           int64_t ldx, const float* __restrict__ Y,
                                                           int64_t ldy, int64_t rows, int64_t n,
                                                           int vec, uint16_t* __restrict__ O,
                                                           int64_t ldo) {
  const int64_t per_row = (n + 3) / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * per_row) return;
  const int64_t t = i / per_row, c0 = 4 * (i - t * per_row);
  const uint16_t* x = X + t * ldx + c0;
  const float* y = Y + t * ldy + c0;
  uint16_t* o = O + t * ldo + c0;
  if (vec && c0 + 4 <= n) {
    const uint2 xv = *reinterpret_cast<const uint2*>(x);
    const float4 yv = *reinterpret_cast<const float4*>(y);
    const float x0 = bf16_bits_to_f32(xv.x & 0xFFFFu), x1 = bf16_bits_to_f32(xv.x >> 16);
    const float x2 = bf16_bits_to_f32(xv.y & 0xFFFFu), x3 = bf16_bits_to_f32(xv.y >> 16);
    const uint32_t lo = bf16_bits(x0 + yv.x) | ((uint32_t)bf16_bits(x1 + yv.y) << 16);
    const uint32_t hi = bf16_bits(x2 + yv.z) | ((uint32_t)bf16_bits(x3 + yv.w) << 16);
    *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
  } else {
    for (int e = 0; e < 4 && c0 + e < n; ++e) o[e] = bf16_bits(bf16_bits_to_f32(x[e]) + y[e]);
  }
}

inline bool aligned(const void* p, int a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

hipError_t launch_swiglu(const float* G, int64_t ldg, const float* U, int64_t ldu, int64_t rows,
                         int64_t n, void* H, int64_t ldh, hipStream_t stream) {
  const int vec = aligned(G, 16) && aligned(U, 16) && aligned(H, 8) && ldg % 4 == 0 &&
                  ldu % 4 == 0 && ldh % 4 == 0;
  const int64_t total = rows * ceil_div(n, 4);
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream, G,
                     ldg, U, ldu, rows, n, vec, static_cast<uint16_t*>(H), ldh);
  return hipGetLastError();
}

hipError_t launch_residual_add(const void* X, int64_t ldx, const float* Y, int64_t ldy,
                               int64_t rows, int64_t n, void* O, int64_t ldo, hipStream_t stream) {
  const int vec = aligned(X, 8) && aligned(Y, 16) && aligned(O, 8) && ldx % 4 == 0 &&
                  ldy % 4 == 0 && ldo % 4 == 0;
  const int64_t total = rows * ceil_div(n, 4);
  hipLaunchKernelGGL(residual_add_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(X), ldx, Y, ldy, rows, n, vec,
                     static_cast<uint16_t*>(O), ldo);
  return hipGetLastError();
}

}  // namespace gptq
