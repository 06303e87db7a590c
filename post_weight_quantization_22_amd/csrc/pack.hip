// Bit packing of quantized codes.
//
// The storage cost is b bits per weight plus the group metadata ("LLM
// quantization principles", 0539edu.com news 6111416, section 4.2); the bit
// layout is this library's: row r is one little-endian stream of uint32
// words, column c in bits [c*b, c*b + b), zero-padded at the row's end.
//
// HBM-bound (reads 1 B and writes b/8 B per weight).  One lane produces one
// output word, so stores are fully coalesced.  For b in {2, 4, 8} a word holds
// a whole number of codes and the lane reads them with one aligned vector
// load; other widths (3, 5, 6, 7 bits) gather the <= 11 + 1 codes that touch
// the word.  Packing in processing order (a permutation of each row's columns)
// takes the gathering kernel for every width.
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

__global__ __launch_bounds__(256) void pack_any_kernel(const uint8_t* __restrict__ codes,
                                                       int64_t m, int64_t n, int64_t nw, int bits,
                                                       const int32_t* __restrict__ perm,
                                                       uint32_t* __restrict__ packed) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= m * nw) return;
  const int64_t r = idx / nw, w = idx - r * nw;
  const int64_t base = 32 * w;  // first bit of this word in the row's stream
  const int64_t cfirst = base / bits;
  const int64_t clast = min((base + 31) / bits, n - 1);
  const uint32_t mask = (1u << bits) - 1u;
  const uint8_t* row = codes + r * n;
  uint64_t acc = 0;
  for (int64_t c = cfirst; c <= clast; ++c) {
    const uint64_t v = (uint64_t)(row[perm ? perm[c] : c] & mask);
    const int64_t pos = c * bits - base;  // may be negative for a code entering from the left
    acc |= pos >= 0 ? (v << pos) : (v >> (-pos));
  }
  packed[idx] = (uint32_t)acc;
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, int64_t m, int64_t n, int bits,
                       const int32_t* perm, uint32_t* packed, hipStream_t stream) {
  const int64_t nw = ceil_div(n * bits, 32);
  const int64_t total = m * nw;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(total, 256));
  if (perm) {
    hipLaunchKernelGGL(pack_any_kernel, grid, dim3(256), 0, stream, codes, m, n, nw, bits, perm,
                       packed);
    return hipGetLastError();
  }
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(pack_pow2_kernel<2>, grid, dim3(256), 0, stream, codes, m, n, nw, packed);
      break;
    case 4:
      hipLaunchKernelGGL(pack_pow2_kernel<4>, grid, dim3(256), 0, stream, codes, m, n, nw, packed);
      break;
    case 8:
      hipLaunchKernelGGL(pack_pow2_kernel<8>, grid, dim3(256), 0, stream, codes, m, n, nw, packed);
      break;
    default:
      hipLaunchKernelGGL(pack_any_kernel, grid, dim3(256), 0, stream, codes, m, n, nw, bits,
                         nullptr, packed);
  }
  return hipGetLastError();
}

}  // namespace gptq
