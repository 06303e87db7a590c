// Group min-max round-to-nearest (the GPTQ quantizer with no compensation).
//
// "GPTQ deep dive" (hncyxsy.com news 243429) section 1.2: RTN rounds every
// weight to its nearest grid point on its own.  "Calibration algorithms
// guide" (bhfrc.com news 5741) section 2.2: one min/max, hence one scale and
// zero-point, per group of consecutive weights.
//
// HBM-bound: each lane owns 8 consecutive weights of a row (16 B bf16 or
// 32 B fp32 loaded at once) in each of two rows, a group spans G/8 lanes of
// one wave and its min/max is a butterfly over those lanes.  Whole-row groups (G == -1, or any
// G the wave path does not cover) take a workgroup-per-group path.
#include "kernels.hpp"

namespace gptq {

namespace {

struct Chunk8 {
  float v[8];
};

__device__ __forceinline__ Chunk8 load8(const void* W, int dt, int64_t row_off, int64_t c0,
                                        int64_t n) {
  Chunk8 ch;
  if (c0 + 8 <= n) {
    if (dt == GPTQ_BF16) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(W) + row_off + c0;
      if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
        uint4 u = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ch.v[2 * k] = __uint_as_float(w[k] << 16);
          ch.v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
        return ch;
      }
    } else {
      const float* p = reinterpret_cast<const float*>(W) + row_off + c0;
      if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        ch.v[0] = a.x; ch.v[1] = a.y; ch.v[2] = a.z; ch.v[3] = a.w;
        ch.v[4] = b.x; ch.v[5] = b.y; ch.v[6] = b.z; ch.v[7] = b.w;
        return ch;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) ch.v[k] = (c0 + k < n) ? load_elem(W, dt, row_off + c0 + k) : 0.0f;
  return ch;
}

__device__ __forceinline__ void store8_codes(uint8_t* codes, int64_t off, int64_t c0, int64_t n,
                                             const float* q) {
  uint8_t* p = codes + off + c0;
  if (c0 + 8 <= n && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= (uint32_t)q[k] << (8 * k);
      hi |= (uint32_t)q[k + 4] << (8 * k);
    }
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    return;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (c0 + k < n) p[k] = (uint8_t)q[k];
}

// Wave path: G is a power of two in [8, 512]; LPG = G / 8 lanes per group.
// A lane takes the same 8 columns of two rows, r and r + hm (hm = ceil(m / 2)),
// both loads in flight before either is quantized.
template <int LPG>
__device__ __forceinline__ void rtn_chunk(const Chunk8& ch, bool live, int64_t r, int64_t n,
                                          int64_t ngroups, int64_t g, int64_t k, int64_t c0,
                                          float maxq, int sym, uint8_t* __restrict__ codes,
                                          float* __restrict__ scales, float* __restrict__ zeros) {
  float vmin = ch.v[0], vmax = ch.v[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    vmin = fminf(vmin, ch.v[e]);
    vmax = fmaxf(vmax, ch.v[e]);
  }
  // columns past n were loaded as 0, which the 0-including range absorbs
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, off, LPG));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off, LPG));
  }
  float scale, zero;
  if (sym) sym_params(fmaxf(fabsf(vmin), fabsf(vmax)), maxq, scale, zero);
  else minmax_params(vmin, vmax, maxq, scale, zero);
  if (!live) return;
  // codes by the reciprocal, the IEEE quotient where a half-integer is near
  const float rscale = 1.0f / scale;
  float q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = quant_code_fast(ch.v[e], scale, rscale, zero, maxq);
  store8_codes(codes, r * n, c0, n, q);
  if ((k % LPG) == 0) {
    scales[r * ngroups + g] = scale;
    zeros[r * ngroups + g] = zero;
  }
}

template <int LPG>
__global__ __launch_bounds__(256) void rtn_wave_kernel(const void* __restrict__ W, int dt,
                                                       int64_t m, int64_t n, int64_t ldw,
                                                       int64_t ngroups, float maxq, int sym,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       float* __restrict__ zeros) {
  const int64_t slots_per_row = ngroups * LPG;
  const int64_t hm = (m + 1) / 2;
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live0 = slot < hm * slots_per_row;
  int64_t r;
  if (hm * slots_per_row <= INT32_MAX) {  // 32-bit division (a 64-bit one is a long sequence)
    r = live0 ? (int64_t)((uint32_t)slot / (uint32_t)slots_per_row) : 0;
  } else {
    r = live0 ? slot / slots_per_row : 0;
  }
  const int64_t k = live0 ? slot - r * slots_per_row : 0;
  const bool live1 = live0 && r + hm < m;
  const int64_t g = k / LPG;
  const int64_t c0 = g * (LPG * 8) + (k % LPG) * 8;
  Chunk8 ch0, ch1;
#pragma unroll
  for (int e = 0; e < 8; ++e) ch0.v[e] = ch1.v[e] = 0.0f;
  if (live0) ch0 = load8(W, dt, r * ldw, c0, n);
  if (live1) ch1 = load8(W, dt, (r + hm) * ldw, c0, n);
  rtn_chunk<LPG>(ch0, live0, r, n, ngroups, g, k, c0, maxq, sym, codes, scales, zeros);
  rtn_chunk<LPG>(ch1, live1, r + hm, n, ngroups, g, k, c0, maxq, sym, codes, scales, zeros);
}

// Workgroup path: one workgroup per (row, group) of any length.
__global__ __launch_bounds__(256) void rtn_block_kernel(const void* __restrict__ W, int dt,
                                                        int64_t n, int64_t ldw, int64_t G,
                                                        int64_t ngroups, float maxq, int sym,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales,
                                                        float* __restrict__ zeros) {
  __shared__ float smin[256 / kWave], smax[256 / kWave];
  const int64_t r = blockIdx.x / ngroups;
  const int64_t g = blockIdx.x % ngroups;
  const int64_t c0 = g * G, c1 = min(c0 + G, n);
  float vmin = 0.0f, vmax = 0.0f;
  for (int64_t c = c0 + threadIdx.x; c < c1; c += blockDim.x) {
    float v = load_elem(W, dt, r * ldw + c);
    vmin = fminf(vmin, v);
    vmax = fmaxf(vmax, v);
  }
  for (int off = 1; off < kWave; off <<= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, off));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  }
  const int wv = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
    smin[wv] = vmin;
    smax[wv] = vmax;
  }
  __syncthreads();
  vmin = smin[0];
  vmax = smax[0];
  for (int w = 1; w < (int)(blockDim.x / kWave); ++w) {
    vmin = fminf(vmin, smin[w]);
    vmax = fmaxf(vmax, smax[w]);
  }
  float scale, zero;
  if (sym) sym_params(fmaxf(fabsf(vmin), fabsf(vmax)), maxq, scale, zero);
  else minmax_params(vmin, vmax, maxq, scale, zero);
  for (int64_t c = c0 + threadIdx.x; c < c1; c += blockDim.x) {
    float v = load_elem(W, dt, r * ldw + c);
    codes[r * n + c] = (uint8_t)quant_code(v, scale, zero, maxq);
  }
  if (threadIdx.x == 0) {
    scales[r * ngroups + g] = scale;
    zeros[r * ngroups + g] = zero;
  }
}

}  // namespace

hipError_t launch_rtn(const void* W, int dt, int64_t m, int64_t n, int64_t ldw, int bits,
                      int64_t G, int sym, uint8_t* codes, float* scales, float* zeros,
                      hipStream_t stream) {
  const float maxq = (float)((1 << bits) - 1);
  const int64_t Ge = G > 0 ? G : n;
  const int64_t ngroups = ceil_div(n, Ge);
  const int64_t lpg = Ge / 8;
  const bool wave_path = G > 0 && (G & (G - 1)) == 0 && G >= 8 && G <= 512;
  if (wave_path) {
    const int64_t slots = (m + 1) / 2 * ngroups * lpg;  // a lane takes two rows
    const dim3 grid((unsigned)ceil_div(slots, 256));
#define GPTQ_RTN_CASE(L)                                                                     \
  case L:                                                                                  \
    hipLaunchKernelGGL(rtn_wave_kernel<L>, grid, dim3(256), 0, stream, W, dt, m, n, ldw,   \
                       ngroups, maxq, sym, codes, scales, zeros);                          \
    break;
    switch (lpg) {
      GPTQ_RTN_CASE(1)
      GPTQ_RTN_CASE(2)
      GPTQ_RTN_CASE(4)
      GPTQ_RTN_CASE(8)
      GPTQ_RTN_CASE(16)
      GPTQ_RTN_CASE(32)
      GPTQ_RTN_CASE(64)
      default:
        return hipErrorInvalidValue;
    }
#undef GPTQ_RTN_CASE
  } else {
    const dim3 grid((unsigned)(ngroups * m));
    hipLaunchKernelGGL(rtn_block_kernel, grid, dim3(256), 0, stream, W, dt, n, ldw, Ge, ngroups,
                       maxq, sym, codes, scales, zeros);
  }
  return hipGetLastError();
}

}  // namespace gptq
