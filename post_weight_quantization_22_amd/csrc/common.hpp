// Shared device helpers for the gfx950 GPTQ kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gptq_mi355x.h"

namespace gptq {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Load one weight as fp32 from an fp32 or bf16 matrix.
__device__ __forceinline__ float load_elem(const void* p, int dt, int64_t idx) {
  if (dt == GPTQ_BF16) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[idx]);
  }
  return reinterpret_cast<const float*>(p)[idx];
}

// Group parameters of the asymmetric min-max quantizer (range widened to
// include 0; an all-zero group uses [-1, 1]).  IEEE fp32 arithmetic, true
// division, round-half-even; the same sequence of fp32 operations as the
// method's definition, so that integer outcomes are reproducible.
__device__ __forceinline__ void minmax_params(float vmin, float vmax, float maxq, float& scale,
                                              float& zero) {
  float xmin = fminf(vmin, 0.0f);
  float xmax = fmaxf(vmax, 0.0f);
  if (xmin == xmax) {
    xmin = -1.0f;
    xmax = 1.0f;
  }
  const float span = xmax - xmin;
  scale = __fdiv_rn(span, maxq);
  zero = rintf(__fdiv_rn(__fmul_rn(-xmin, maxq), span));
}

// Symmetric variant: zero-point fixed at 2^(bits-1), scale = 2*max|v| / maxq.
__device__ __forceinline__ void sym_params(float amax, float maxq, float& scale, float& zero) {
  if (amax == 0.0f) amax = 1.0f;
  scale = __fdiv_rn(__fmul_rn(2.0f, amax), maxq);
  zero = floorf(__fmul_rn(maxq + 1.0f, 0.5f));
}

// q = clamp(rne(w / scale) + zero, 0, maxq)
__device__ __forceinline__ float quant_code(float w, float scale, float zero, float maxq) {
  float q = rintf(__fdiv_rn(w, scale)) + zero;
  return fminf(fmaxf(q, 0.0f), maxq);
}

// q = clamp(rne(w / scale) + zero, 0, maxq) with the IEEE quotient w / scale,
// computed as w * (1 / scale): that product is within 1.5 * 2^-23 |w / scale|
// of the quotient, so the two round to different integers only if a
// half-integer lies that close; then (rarely) the division itself decides.
// A non-finite t (w not finite, or 1 / scale overflowing for a subnormal
// scale) also takes the division: the test below is false only for a number.
__device__ __forceinline__ float quant_code_fast(float w, float scale, float rscale, float zero,
                                                 float maxq) {
  const float t = w * rscale;
  float q = rintf(t);
  const float tol = fmaxf(fabsf(t), 1.0f) * 3.6e-7f;
  if (!(fabsf(fabsf(t - floorf(t)) - 0.5f) > tol)) q = rintf(__fdiv_rn(w, scale));
  return fminf(fmaxf(q + zero, 0.0f), maxq);
}

__device__ __forceinline__ bool is_finite(float x) { return isfinite(x); }

// LDS DMA of 16 (4) bytes per lane: lane l's bytes land at lds + 16 l (4 l),
// read from sbase + voff (wave-uniform 64-bit base in SGPRs, per-lane 32-bit
// byte offset).  Issued from asm: the compiler cannot tell this LDS write from
// the LDS reads of other buffers and would otherwise wait for it before each
// of them; completion is awaited explicitly (vmcnt) before the barrier that
// publishes the data.  The instruction writes no VGPR (its data goes to LDS)
// and its address registers are consumed at issue.  M0, the LDS base of the
// transfer, is read at issue; it is saved and restored around it.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

__device__ __forceinline__ void lds_dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// LDS byte address of a __shared__ object (wave-uniform), for M0.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(p));
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t hmin(int64_t a, int64_t b) { return a < b ? a : b; }
inline int64_t hmax(int64_t a, int64_t b) { return a > b ? a : b; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace gptq
