// GPTQ column loop for one layer on gfx950.
//
// "GPTQ deep dive" (hncyxsy.com news 243429): section 3.1 step 3 (blocks of
// 128 columns; per column: group scale, rounding, error accumulation; then a
// batched update of the later columns), section 2.2 (a column's quantization
// error is compensated on the remaining weights through the inverse Hessian)
// and section 2.4 (fixed left-to-right order; lazy batched updates).  The
// inverse Hessian enters through U, the upper Cholesky factor of H_d^-1 in
// processing order, as produced by gptq_prepare.
//
// Per block [i0, i0 + 128):
//   block_quant_kernel: each row of W' is spread over 16 lanes (8 consecutive
//     columns per lane, so a wave holds 4 rows); the 128x128 diagonal block of
//     U is staged in LDS.  Column j is owned by lane j/8: it forms the code and
//     the scaled error e_j = (w_j - dq_j) / U_jj, which a DPP row broadcast
//     hands to the row's 16 lanes, and every lane applies
//     w_k -= e_j * U_jk to its own columns (U_jk = 0 for k < j).  Group
//     min/max is a butterfly over the G/8 lanes holding the group, taken from
//     the current (already compensated) values when the group's first column
//     is reached.
//   trailing_update_kernel: W'[:, i0+128:] -= E * U[i0:i0+128, i0+128:], an
//     fp32 GEMM with K = 128 on v_mfma_f32_16x16x4_f32.
#include <utility>

#include "kernels.hpp"

namespace gptq {

namespace {

constexpr int BLK = 128;  // block width in columns
constexpr int LPR = 16;   // lanes per row
constexpr int CPL = 8;    // columns per lane
constexpr int QROWS = 256 / LPR;  // rows per workgroup
constexpr int UPAD = 4;

template <int... Is, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// Broadcast lane SRC of each row of 16 lanes to the whole row (DPP row_newbcast).
template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + SRC, 0xF, 0xF, false));
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v) { *p = v; }

// W' = W[:, perm] as fp32 (processing order), dead columns zeroed, finiteness.
__global__ __launch_bounds__(256) void prep_weights_kernel(const void* __restrict__ W, int dt,
                                                           int64_t m, int64_t n, int64_t ldw,
                                                           const int32_t* __restrict__ perm,
                                                           const uint8_t* __restrict__ dead,
                                                           float* __restrict__ Wp,
                                                           int32_t* __restrict__ info) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  int64_t src = perm ? (int64_t)perm[c] : c;
  if (src < 0 || src >= n) src = c;  // a malformed permutation must not address out of range
  const bool is_dead = dead && dead[src];
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    float v = load_elem(W, dt, r * ldw + src);
    if (!isfinite(v) && info) *info = -1;
    Wp[r * n + c] = is_dead ? 0.0f : v;
  }
}

// One group per row: parameters from the whole row.
__global__ __launch_bounds__(256) void row_params_kernel(const float* __restrict__ Wp, int64_t m,
                                                         int64_t n, float maxq, int sym,
                                                         float* __restrict__ scales,
                                                         float* __restrict__ zeros) {
  __shared__ float smin[4], smax[4];
  for (int64_t r = blockIdx.x; r < m; r += gridDim.x) {
    float vmin = 0.0f, vmax = 0.0f;
    for (int64_t c = threadIdx.x; c < n; c += blockDim.x) {
      const float v = Wp[r * n + c];
      vmin = fminf(vmin, v);
      vmax = fmaxf(vmax, v);
    }
    for (int off = 1; off < kWave; off <<= 1) {
      vmin = fminf(vmin, __shfl_xor(vmin, off));
      vmax = fmaxf(vmax, __shfl_xor(vmax, off));
    }
    if ((threadIdx.x % kWave) == 0) {
      smin[threadIdx.x / kWave] = vmin;
      smax[threadIdx.x / kWave] = vmax;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < 4; ++w) {
        vmin = fminf(smin[0], smin[w]);
        vmax = fmaxf(smax[0], smax[w]);
        smin[0] = vmin;
        smax[0] = vmax;
      }
      float scale, zero;
      if (sym) sym_params(fmaxf(fabsf(smin[0]), fabsf(smax[0])), maxq, scale, zero);
      else minmax_params(smin[0], smax[0], maxq, scale, zero);
      scales[r] = scale;
      zeros[r] = zero;
    }
    __syncthreads();
  }
}

// One 128-column block.  G > 0: group size (8..128, divides 128); G < 0: one
// group per row with parameters already in scales/zeros (ngroups == 1).
template <int G>
__global__ __launch_bounds__(256) void block_quant_kernel(
    float* __restrict__ Wp, int64_t m, int64_t n, const float* __restrict__ U, int64_t ldu,
    int64_t i0, float maxq, int sym, uint8_t* __restrict__ codes, float* __restrict__ scales,
    float* __restrict__ zeros, int64_t ngroups, float* __restrict__ E,
    float* __restrict__ row_err, int first_block) {
  __shared__ float Us[BLK][BLK + UPAD];
  __shared__ float uinv[BLK];
  const int tid = threadIdx.x;
  const int bw = (int)min((int64_t)BLK, n - i0);

  // Stage the diagonal block of U: upper triangle of the block's columns.
  for (int idx = tid; idx < BLK * BLK; idx += blockDim.x) {
    const int j = idx / BLK, k = idx % BLK;
    float v = 0.0f;
    if (k >= j && k < bw) v = U[(i0 + j) * ldu + i0 + k];
    Us[j][k] = v;
  }
  __syncthreads();
  if (tid < BLK) uinv[tid] = tid < bw ? 1.0f / Us[tid][tid] : 0.0f;
  __syncthreads();

  const int l16 = tid & (LPR - 1);
  const int64_t r = (int64_t)blockIdx.x * QROWS + (tid >> 4);
  const bool rv = r < m;
  const int64_t cbase = i0 + CPL * l16;  // first column of this lane

  float w[CPL];
  if (rv && cbase + CPL <= n) {
    const float4* p = reinterpret_cast<const float4*>(Wp + r * n + cbase);
    if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      const float4 a = p[0], b = p[1];
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
#pragma unroll
      for (int s = 0; s < CPL; ++s) w[s] = Wp[r * n + cbase + s];
    }
  } else {
#pragma unroll
    for (int s = 0; s < CPL; ++s) w[s] = (rv && cbase + s < n) ? Wp[r * n + cbase + s] : 0.0f;
  }

  float scale = 1.0f, zero = 0.0f;
  if constexpr (G < 0) {
    if (rv) {
      scale = scales[r];
      zero = zeros[r];
    }
  }
  float e_own[CPL], q_own[CPL];
#pragma unroll
  for (int s = 0; s < CPL; ++s) {
    e_own[s] = 0.0f;
    q_own[s] = 0.0f;
  }

  static_for<BLK>([&](auto J) {
    constexpr int j = decltype(J)::value;
    constexpr int s = j % CPL;
    constexpr int owner = j / CPL;
    if constexpr (G > 0) {
      if constexpr (j % G == 0) {
        // parameters of the group starting at column j, for the lanes holding it
        float vmin = w[0], vmax = w[0];
#pragma unroll
        for (int t = 1; t < CPL; ++t) {
          vmin = fminf(vmin, w[t]);
          vmax = fmaxf(vmax, w[t]);
        }
#pragma unroll
        for (int off = 1; off < G / CPL; off <<= 1) {
          vmin = fminf(vmin, __shfl_xor(vmin, off, G / CPL));
          vmax = fmaxf(vmax, __shfl_xor(vmax, off, G / CPL));
        }
        if (sym) sym_params(fmaxf(fabsf(vmin), fabsf(vmax)), maxq, scale, zero);
        else minmax_params(vmin, vmax, maxq, scale, zero);
        if (l16 == owner && rv && i0 + j < n) {
          const int64_t g = (i0 + j) / G;
          scales[r * ngroups + g] = scale;
          zeros[r * ngroups + g] = zero;
        }
      }
    }
    const float wj = w[s];
    const float q = quant_code(wj, scale, zero, maxq);
    const float dq = scale * (q - zero);
    float e = (wj - dq) * uinv[j];
    e = row_bcast<owner>(e);
    if (l16 == owner) {
      e_own[s] = e;
      q_own[s] = q;
    }
    const float4 u0 = *reinterpret_cast<const float4*>(&Us[j][CPL * l16]);
    const float4 u1 = *reinterpret_cast<const float4*>(&Us[j][CPL * l16 + 4]);
    w[0] = fmaf(-e, u0.x, w[0]);
    w[1] = fmaf(-e, u0.y, w[1]);
    w[2] = fmaf(-e, u0.z, w[2]);
    w[3] = fmaf(-e, u0.w, w[3]);
    w[4] = fmaf(-e, u1.x, w[4]);
    w[5] = fmaf(-e, u1.y, w[5]);
    w[6] = fmaf(-e, u1.z, w[6]);
    w[7] = fmaf(-e, u1.w, w[7]);
  });

  // errors of columns past the end of the layer are zero (uinv = 0 there)
  float err = 0.0f;
#pragma unroll
  for (int s = 0; s < CPL; ++s) err = fmaf(e_own[s], e_own[s], err);
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) err += __shfl_xor(err, off, LPR);

  if (!rv) return;
  float* erow = E + r * BLK + CPL * l16;
  *reinterpret_cast<float4*>(erow) = make_float4(e_own[0], e_own[1], e_own[2], e_own[3]);
  *reinterpret_cast<float4*>(erow + 4) = make_float4(e_own[4], e_own[5], e_own[6], e_own[7]);
  uint8_t* crow = codes + r * n + cbase;
  if (cbase + CPL <= n && (reinterpret_cast<uintptr_t>(crow) & 7) == 0) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      lo |= (uint32_t)q_own[t] << (8 * t);
      hi |= (uint32_t)q_own[t + 4] << (8 * t);
    }
    *reinterpret_cast<uint2*>(crow) = make_uint2(lo, hi);
  } else {
#pragma unroll
    for (int t = 0; t < CPL; ++t)
      if (cbase + t < n) crow[t] = (uint8_t)q_own[t];
  }
  if (row_err && l16 == 0) row_err[r] = (first_block ? 0.0f : row_err[r]) + err;
}

// W'[:, c0:] -= E[:, 0:128] * U[i0:i0+128, c0:], c0 = i0 + 128.
// 128x128 output tile per workgroup, 4 waves of 64x64, K staged by 32.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int TT = 128;  // tile edge
constexpr int TK = 32;   // K chunk

__global__ __launch_bounds__(256) void trailing_update_kernel(float* __restrict__ Wp, int64_t m,
                                                              int64_t n,
                                                              const float* __restrict__ E,
                                                              const float* __restrict__ U,
                                                              int64_t ldu, int64_t i0,
                                                              int64_t tiles_n) {
  __shared__ float As[TT][TK + 1];
  __shared__ float Bs[TK][TT + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wr = wv >> 1, wc = wv & 1;
  const int64_t c0 = i0 + BLK;
  const int64_t tr = blockIdx.x / tiles_n, tc = blockIdx.x % tiles_n;
  const int64_t row0 = tr * TT, col0 = c0 + tc * TT;

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = row0 + 64 * wr + 16 * a + 4 * (lane >> 4) + q;
        const int64_t col = col0 + 64 * wc + 16 * b + (lane & 15);
        acc[a][b][q] = (row < m && col < n) ? Wp[row * n + col] : 0.0f;
      }

  for (int kc = 0; kc < BLK; kc += TK) {
    __syncthreads();
    for (int idx = tid; idx < TT * TK; idx += 256) {
      const int rr = idx / TK, kk = idx % TK;
      const int64_t row = row0 + rr;
      As[rr][kk] = row < m ? -E[row * BLK + kc + kk] : 0.0f;
    }
    for (int idx = tid; idx < TK * TT; idx += 256) {
      const int kk = idx / TT, cc = idx % TT;
      const int64_t col = col0 + cc;
      Bs[kk][cc] = col < n ? U[(i0 + kc + kk) * ldu + col] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < TK; ks += 4) {
      float af[4], bf[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) af[a] = As[64 * wr + 16 * a + (lane & 15)][ks + (lane >> 4)];
#pragma unroll
      for (int b = 0; b < 4; ++b) bf[b] = Bs[ks + (lane >> 4)][64 * wc + 16 * b + (lane & 15)];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
  }

#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = row0 + 64 * wr + 16 * a + 4 * (lane >> 4) + q;
        const int64_t col = col0 + 64 * wc + 16 * b + (lane & 15);
        if (row < m && col < n) Wp[row * n + col] = acc[a][b][q];
      }
}

__global__ void invert_perm_kernel(const int32_t* __restrict__ perm, int64_t n,
                                   int32_t* __restrict__ inv) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t p = perm[k];
  if (p >= 0 && p < n) inv[p] = (int32_t)k;
}

// codes[r, c] = codes_proc[r, inv[c]]; g_idx[c] = inv[c] / G.
__global__ __launch_bounds__(256) void unpermute_kernel(const uint8_t* __restrict__ cproc,
                                                        const int32_t* __restrict__ inv,
                                                        int64_t m, int64_t n, int64_t G,
                                                        uint8_t* __restrict__ codes,
                                                        int32_t* __restrict__ g_idx) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  int64_t k = inv ? inv[c] : c;
  if (k < 0 || k >= n) k = c;
  if (g_idx && blockIdx.y == 0) g_idx[c] = G > 0 ? (int32_t)(k / G) : 0;
  if (!codes) return;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) codes[r * n + c] = cproc[r * n + k];
}

}  // namespace

size_t quantize_ws_bytes(int64_t m, int64_t n, int desc_act) {
  size_t b = align_up((size_t)m * n * sizeof(float), 256);   // W'
  b += align_up((size_t)m * BLK * sizeof(float), 256);       // E
  if (desc_act) {
    b += align_up((size_t)m * n, 256);                       // codes, processing order
    b += align_up((size_t)n * sizeof(int32_t), 256);         // inverse permutation
  }
  return b;
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  const int64_t m = a.m, n = a.n;
  char* ws = reinterpret_cast<char*>(a.ws);
  float* Wp = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)m * n * sizeof(float), 256);
  float* E = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)m * BLK * sizeof(float), 256);
  uint8_t* cproc = a.codes;
  int32_t* inv = nullptr;
  if (a.desc_act) {
    cproc = reinterpret_cast<uint8_t*>(ws);
    ws += align_up((size_t)m * n, 256);
    inv = reinterpret_cast<int32_t*>(ws);
  }
  const float maxq = (float)((1 << a.bits) - 1);
  const int G = a.group_size;
  const int64_t ngroups = G > 0 ? ceil_div(n, G) : 1;

  if (a.info) hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(1), 0, stream, a.info, 0);
  {
    const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(m, 1024));
    hipLaunchKernelGGL(prep_weights_kernel, grid, dim3(256), 0, stream, a.W, a.wdt, m, n, a.ldw,
                       a.desc_act ? a.perm : nullptr, a.dead, Wp, a.info);
  }
  if (G < 0) {
    hipLaunchKernelGGL(row_params_kernel, dim3((unsigned)hmin(m, 4096)), dim3(256), 0,
                       stream, Wp, m, n, maxq, a.sym, a.scales, a.zeros);
  }
  const dim3 qgrid((unsigned)ceil_div(m, QROWS));
  for (int64_t i0 = 0; i0 < n; i0 += BLK) {
    const int first = i0 == 0;
#define GPTQ_BQ(GV)                                                                              \
  hipLaunchKernelGGL(block_quant_kernel<GV>, qgrid, dim3(256), 0, stream, Wp, m, n, a.U, a.ldu,  \
                     i0, maxq, a.sym, cproc, a.scales, a.zeros, ngroups, E, a.row_err, first)
    switch (G) {
      case 8: GPTQ_BQ(8); break;
      case 16: GPTQ_BQ(16); break;
      case 32: GPTQ_BQ(32); break;
      case 64: GPTQ_BQ(64); break;
      case 128: GPTQ_BQ(128); break;
      default: GPTQ_BQ(-1); break;
    }
#undef GPTQ_BQ
    if (i0 + BLK < n) {
      const int64_t tiles_n = ceil_div(n - i0 - BLK, TT);
      const int64_t tiles = tiles_n * ceil_div(m, TT);
      hipLaunchKernelGGL(trailing_update_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, Wp,
                         m, n, E, a.U, a.ldu, i0, tiles_n);
    }
  }
  if (a.desc_act) {
    hipLaunchKernelGGL(invert_perm_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream,
                       a.perm, n, inv);
    const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(m, 1024));
    hipLaunchKernelGGL(unpermute_kernel, grid, dim3(256), 0, stream, cproc, inv, m, n,
                       (int64_t)G, a.codes, a.g_idx);
  } else if (a.g_idx) {
    hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)ceil_div(n, 256), 1), dim3(256), 0, stream,
                       (const uint8_t*)nullptr, (const int32_t*)nullptr, (int64_t)0, n, (int64_t)G,
                       (uint8_t*)nullptr, a.g_idx);
  }
  return hipGetLastError();
}

}  // namespace gptq
