// Bit packing of quantized codes.
//
// The storage cost is b bits per weight plus the group metadata ("LLM
// quantization principles", 0539edu.com news 6111416, section 4.2); the bit
// layout is this library's: row r is one little-endian stream of uint32
// words, column c in bits [c*b, c*b + b), zero-padded at the row's end.
//
// HBM-bound (reads 1 B and writes b/8 B per weight).  For b in {2, 4, 8} a
// word holds a whole number of codes: one lane produces one output word from
// one aligned vector load.  Other widths, and packing in processing order (a
// permutation of each row's columns, any width): one lane packs a run of 32
// consecutive stream positions into exactly b words (32 b bits), reading the
// run's codes with two 16-byte loads where aligned (or through the
// permutation, whose 32 entries it reads with 16-byte loads) and storing b
// consecutive words.
#include "kernels.hpp"

namespace gptq {

namespace {

template <int BITS>
__global__ __launch_bounds__(256) void pack_pow2_kernel(const uint8_t* __restrict__ codes,
                                                        int64_t m, int64_t n, int64_t nw,
                                                        uint32_t* __restrict__ packed) {
  constexpr int PER = 32 / BITS;  // codes per word
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= m * nw) return;
  const int64_t r = idx / nw, w = idx - r * nw;
  const int64_t c0 = w * PER;
  const uint8_t* src = codes + r * n + c0;
  uint32_t word = 0;
  if (c0 + PER <= n && (reinterpret_cast<uintptr_t>(src) % PER) == 0) {
    uint32_t v[PER / 4];
    if constexpr (PER == 16) {
      uint4 u = *reinterpret_cast<const uint4*>(src);
      v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    } else if constexpr (PER == 8) {
      uint2 u = *reinterpret_cast<const uint2*>(src);
      v[0] = u.x; v[1] = u.y;
    } else {
      v[0] = *reinterpret_cast<const uint32_t*>(src);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) word |= ((v[k / 4] >> (8 * (k % 4))) & MASK) << (k * BITS);
  } else {
    for (int k = 0; k < PER && c0 + k < n; ++k) word |= ((uint32_t)src[k] & MASK) << (k * BITS);
  }
  packed[idx] = word;
}

template <int BITS>
__global__ __launch_bounds__(256) void pack_run32_kernel(const uint8_t* __restrict__ codes,
                                                         int64_t m, int64_t n, int64_t nw,
                                                         const int32_t* __restrict__ perm,
                                                         uint32_t* __restrict__ packed) {
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int64_t runs = (n + 31) / 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= m * runs) return;
  const int64_t r = idx / runs, k = idx - r * runs;
  const int64_t c0 = 32 * k;
  const uint8_t* row = codes + r * n;
  uint32_t cv[32];
  if (c0 + 32 <= n) {
    if (perm && (reinterpret_cast<uintptr_t>(perm) & 15) == 0) {
      const int4* pp = reinterpret_cast<const int4*>(perm + c0);  // 128-byte steps
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int4 p4 = pp[q];
        cv[4 * q] = row[min(max(p4.x, 0), (int)n - 1)];
        cv[4 * q + 1] = row[min(max(p4.y, 0), (int)n - 1)];
        cv[4 * q + 2] = row[min(max(p4.z, 0), (int)n - 1)];
        cv[4 * q + 3] = row[min(max(p4.w, 0), (int)n - 1)];
      }
    } else if (perm) {
#pragma unroll
      for (int e = 0; e < 32; ++e) cv[e] = row[min(max((int64_t)perm[c0 + e], (int64_t)0), n - 1)];
    } else if ((reinterpret_cast<uintptr_t>(row + c0) & 15) == 0) {
      const uint4 u0 = *reinterpret_cast<const uint4*>(row + c0);
      const uint4 u1 = *reinterpret_cast<const uint4*>(row + c0 + 16);
      const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int e = 0; e < 32; ++e) cv[e] = (w[e >> 2] >> (8 * (e & 3))) & 0xFFu;
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) cv[e] = row[c0 + e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int64_t c = c0 + e;
      int64_t src = c;
      if (perm && c < n) src = min(max((int64_t)perm[c], (int64_t)0), n - 1);
      cv[e] = c < n ? row[src] : 0u;
    }
  }
  uint32_t out[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) out[j] = 0u;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const uint32_t v = cv[e] & MASK;
    const int bit = e * BITS, wi = bit >> 5, sh = bit & 31;
    out[wi] |= v << sh;
    if (sh + BITS > 32) out[wi + 1] |= v >> (32 - sh);
  }
  uint32_t* dst = packed + r * nw + k * BITS;
#pragma unroll
  for (int j = 0; j < BITS; ++j)
    if (k * BITS + j < nw) dst[j] = out[j];
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, int64_t m, int64_t n, int bits,
                       const int32_t* perm, uint32_t* packed, hipStream_t stream) {
  const int64_t nw = ceil_div(n * bits, 32);
  const int64_t total = m * nw;
  if (total == 0) return hipSuccess;
  if (!perm && (bits == 2 || bits == 4 || bits == 8)) {
    const dim3 grid((unsigned)ceil_div(total, 256));
    switch (bits) {
      case 2:
        hipLaunchKernelGGL(pack_pow2_kernel<2>, grid, dim3(256), 0, stream, codes, m, n, nw, packed);
        break;
      case 4:
        hipLaunchKernelGGL(pack_pow2_kernel<4>, grid, dim3(256), 0, stream, codes, m, n, nw, packed);
        break;
      default:
        hipLaunchKernelGGL(pack_pow2_kernel<8>, grid, dim3(256), 0, stream, codes, m, n, nw, packed);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)ceil_div(m * ceil_div(n, (int64_t)32), 256));
#define GPTQ_RUN32(B)                                                                          \
  hipLaunchKernelGGL(pack_run32_kernel<B>, grid, dim3(256), 0, stream, codes, m, n, nw, perm, \
                     packed)
  switch (bits) {
    case 1: GPTQ_RUN32(1); break;
    case 2: GPTQ_RUN32(2); break;
    case 3: GPTQ_RUN32(3); break;
    case 4: GPTQ_RUN32(4); break;
    case 5: GPTQ_RUN32(5); break;
    case 6: GPTQ_RUN32(6); break;
    case 7: GPTQ_RUN32(7); break;
    default: GPTQ_RUN32(8); break;
  }
#undef GPTQ_RUN32
  return hipGetLastError();
}

}  // namespace gptq
