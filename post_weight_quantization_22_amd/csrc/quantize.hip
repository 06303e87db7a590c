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
//   The deferred update of the later columns is blocked twice: blocks of 128
//   columns form super-blocks of SB columns.  After each block, only the rest
//   of its super-block is updated (K = 128); after each super-block, every
//   column past it at once (K = SB), from the errors of the whole super-block.
//   Both are W'[:, c0:c1] -= E[:, k0:k1] U[k0:k1, c0:c1] on
//   v_mfma_f32_16x16x4_f32 (update_gemm_kernel); the second carries most of
//   the flops, with K long enough to keep the matrix cores busy instead of
//   re-streaming W' every 128 columns.
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

// The same for bf16 W in column order (no desc_act) with 16-byte aligned rows
// and n % 8 == 0: 8 columns per thread, 16-byte loads and stores.
__global__ __launch_bounds__(256) void prep_weights_bf16_kernel(const uint16_t* __restrict__ W,
                                                                int64_t m, int64_t n,
                                                                int64_t ldw,
                                                                const uint8_t* __restrict__ dead,
                                                                float* __restrict__ Wp,
                                                                int32_t* __restrict__ info) {
  const int64_t c = 8 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (c >= n) return;
  bool dz[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) dz[t] = dead && dead[c + t];
  bool bad = false;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    const uint4 v = *reinterpret_cast<const uint4*>(W + r * ldw + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f[2 * t] = __uint_as_float(w[t] << 16);
      f[2 * t + 1] = __uint_as_float(w[t] & 0xFFFF0000u);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bad |= !isfinite(f[t]);
      if (dz[t]) f[t] = 0.0f;
    }
    float4* o = reinterpret_cast<float4*>(Wp + r * n + c);
    o[0] = make_float4(f[0], f[1], f[2], f[3]);
    o[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
  if (bad && info) *info = -1;
}

// W' = W[:, perm] as fp32 for bf16 W with desc_act, a row at a time through
// LDS: the row comes in by coalesced 16-byte loads, is staged in LDS, and
// leaves in processing order by 16-byte stores of 8 fp32 values, the permuted
// reads served by the LDS.  One LDS row buffer (two barriers a row), so two
// workgroups share a CU and one's loads overlap the other's gather.  Each thread keeps
// the source columns of its output segments in registers for all its rows
// (16-bit entries: the column in bits 0-14, the dead flag in bit 15), so the
// permutation is read once per workgroup (512 threads).  Needs n % 8 == 0,
// n <= NCAP <= 32768, 16-byte aligned rows.  Every weight is checked for finiteness (dead
// columns included) before a dead column is zeroed.
template <int NCAP>
__global__ __launch_bounds__(512) void prep_rows_bf16_kernel(const uint16_t* __restrict__ W,
                                                             int64_t ldw,
                                                             const int32_t* __restrict__ perm,
                                                             const uint8_t* __restrict__ dead,
                                                             int64_t m, int64_t n,
                                                             int64_t rows_per_wg,
                                                             float* __restrict__ Wp,
                                                             int32_t* __restrict__ info) {
  constexpr int CH = NCAP / 8 / 512;  // 16-byte chunks (8 columns) of a row per thread
  static_assert(NCAP <= 32768, "15-bit column entries");
  __shared__ __align__(16) uint16_t buf[NCAP];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
  const int64_t r1 = min(m, r0 + rows_per_wg);
  if (r0 >= r1) return;
  const int nseg = (int)(n / 8);
  uint32_t pk[CH][4];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int sg = tid + 512 * i;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t p = 8 * (int64_t)sg + 2 * q + e;
        uint32_t v = 0;
        if (sg < nseg) {
          int64_t src = perm[p];
          if (src < 0 || src >= n) src = p;  // a malformed permutation must not address out of range
          v = (uint32_t)src | ((dead && dead[src]) ? 0x8000u : 0u);
        }
        h[e] = v;
      }
      pk[i][q] = h[0] | (h[1] << 16);
    }
  }
  bool bad = false;
  uint16_t* b = buf;
  for (int64_t r = r0; r < r1; ++r) {
    __syncthreads();  // every thread has gathered the previous row
    {
      // the row straight into LDS (no prefetch array: at 8 x 16 bytes a thread
      // the compiler keeps one in scratch memory)
      const uint4* src = reinterpret_cast<const uint4*>(W + r * ldw);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int idx = tid + 512 * c;
        if (idx < nseg) reinterpret_cast<uint4*>(b)[idx] = src[idx];
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int sg = tid + 512 * i;
      if (sg < nseg) {
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t h = (pk[i][q] >> (16 * e)) & 0xFFFFu;
            const float x = bf16_bits_to_f32(b[h & 0x7FFFu]);
            bad |= !isfinite(x);
            f[2 * q + e] = (h & 0x8000u) ? 0.0f : x;
          }
        float4* o = reinterpret_cast<float4*>(Wp + r * n + 8 * (int64_t)sg);
        o[0] = make_float4(f[0], f[1], f[2], f[3]);
        o[1] = make_float4(f[4], f[5], f[6], f[7]);
      }
    }
  }
  if (bad && info) *info = -1;
}

// Parameters of one group per row from the current values of columns
// [c0, c0 + len) of W': the whole row (one group per row), or a group that
// spans several blocks (its first column is a block start).  Written to
// scales/zeros[r * ngroups + g].
__global__ __launch_bounds__(256) void row_params_kernel(const float* __restrict__ Wp, int64_t m,
                                                         int64_t n, int64_t c0, int64_t len,
                                                         int64_t g, int64_t ngroups, float maxq,
                                                         int sym, float* __restrict__ scales,
                                                         float* __restrict__ zeros) {
  __shared__ float smin[4], smax[4];
  for (int64_t r = blockIdx.x; r < m; r += gridDim.x) {
    float vmin = 0.0f, vmax = 0.0f;
    for (int64_t c = c0 + threadIdx.x; c < c0 + len; c += blockDim.x) {
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
      scales[r * ngroups + g] = scale;
      zeros[r * ngroups + g] = zero;
    }
    __syncthreads();
  }
}

// Static groups: parameters of every group of G consecutive ORIGINAL columns
// from the original weights (dead columns as 0), before the loop.  One thread
// per (row, group).
__global__ __launch_bounds__(256) void static_params_kernel(const void* __restrict__ W, int dt,
                                                            int64_t m, int64_t n, int64_t ldw,
                                                            const uint8_t* __restrict__ dead,
                                                            int64_t G, int64_t ngroups,
                                                            float maxq, int sym,
                                                            float* __restrict__ scales,
                                                            float* __restrict__ zeros) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= m * ngroups) return;
  const int64_t r = i / ngroups, g = i - r * ngroups;
  float vmin = 0.0f, vmax = 0.0f;
  const int64_t c1 = min(n, (g + 1) * G);
  for (int64_t c = g * G; c < c1; ++c) {
    const float v = (dead && dead[c]) ? 0.0f : load_elem(W, dt, r * ldw + c);
    vmin = fminf(vmin, v);
    vmax = fmaxf(vmax, v);
  }
  float scale, zero;
  if (sym) sym_params(fmaxf(fabsf(vmin), fabsf(vmax)), maxq, scale, zero);
  else minmax_params(vmin, vmax, maxq, scale, zero);
  scales[i] = scale;
  zeros[i] = zero;
}

// One 128-column block.  G > 0: group size (8..128, divides 128), parameters
// computed here at each group's first column.  G < 0: parameters given in
// scales/zeros before the block; processing column k takes group
// (gperm ? gperm[k] : k) / gdiv (one group per row: gdiv = n; a group spanning
// several blocks: gdiv = its size; static groups: gperm = perm, gdiv = its size).
// Errors go to E[r, e0 + c] (row stride lde), c < 128.
template <int G>
__global__ __launch_bounds__(256) void block_quant_kernel(
    float* __restrict__ Wp, int64_t m, int64_t n, const float* __restrict__ U, int64_t ldu,
    int64_t i0, float maxq, int sym, uint8_t* __restrict__ codes, float* __restrict__ scales,
    float* __restrict__ zeros, int64_t ngroups, float* __restrict__ E, int64_t lde, int64_t e0,
    float* __restrict__ row_err, int first_block, const int32_t* __restrict__ gperm,
    int64_t gdiv) {
  __shared__ __align__(16) float Us[BLK][BLK + UPAD];
  __shared__ __align__(16) float uinv[BLK];
  const int tid = threadIdx.x;
  const int bw = (int)min((int64_t)BLK, n - i0);

  // this lane's 8 values of its row, in flight while U is staged
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

  // Stage the diagonal block of U (upper triangle of the block's columns):
  // 16 float4 per thread, all in flight before the first LDS store.
  {
    const bool vec = (ldu % 4 == 0) && ((reinterpret_cast<uintptr_t>(U) & 15) == 0);
    float4 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 256 * q;
      const int j = idx >> 5, k = 4 * (idx & 31);
      const int64_t row = i0 + (j < bw ? j : 0);
      const float* src = U + row * ldu + i0 + k;
      if (vec && k + 4 <= bw) {
        v[q] = *reinterpret_cast<const float4*>(src);
      } else {
        float t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = k + e < bw ? src[e] : 0.0f;
        v[q] = make_float4(t[0], t[1], t[2], t[3]);
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int idx = tid + 256 * q;
      const int j = idx >> 5, k = 4 * (idx & 31);
      float t[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = (j < bw && k + e >= j && k + e < bw) ? t[e] : 0.0f;
      *reinterpret_cast<float4*>(&Us[j][k]) = make_float4(t[0], t[1], t[2], t[3]);
    }
  }
  __syncthreads();
  if (tid < BLK) uinv[tid] = tid < bw ? 1.0f / Us[tid][tid] : 0.0f;
  __syncthreads();
  // 1 / U_jj of this lane's own columns (only the owner's error is broadcast)
  float uown[CPL];
  {
    const float4 a0 = *reinterpret_cast<const float4*>(&uinv[CPL * l16]);
    const float4 a1 = *reinterpret_cast<const float4*>(&uinv[CPL * l16 + 4]);
    uown[0] = a0.x; uown[1] = a0.y; uown[2] = a0.z; uown[3] = a0.w;
    uown[4] = a1.x; uown[5] = a1.y; uown[6] = a1.z; uown[7] = a1.w;
  }

  float scale = 1.0f, zero = 0.0f, rscale = 1.0f;
  // given parameters: each lane holds those of its own 8 columns (only the
  // owner lane's result of a column is used)
  float sc_own[CPL], z_own[CPL], rs_own[CPL];
  if constexpr (G < 0) {
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int64_t k = min(cbase + t, n - 1);
      const int64_t gi = (gperm ? (int64_t)gperm[k] : k) / gdiv;
      sc_own[t] = rv ? scales[r * ngroups + gi] : 1.0f;
      z_own[t] = rv ? zeros[r * ngroups + gi] : 0.0f;
      rs_own[t] = 1.0f / sc_own[t];
    }
  }
  float e_own[CPL], q_own[CPL];
#pragma unroll
  for (int s = 0; s < CPL; ++s) {
    e_own[s] = 0.0f;
    q_own[s] = 0.0f;
  }

  // row j of the U block for this lane's columns, one column ahead
  float4 uc0 = *reinterpret_cast<const float4*>(&Us[0][CPL * l16]);
  float4 uc1 = *reinterpret_cast<const float4*>(&Us[0][CPL * l16 + 4]);
  static_for<BLK>([&](auto J) {
    constexpr int j = decltype(J)::value;
    constexpr int s = j % CPL;
    constexpr int owner = j / CPL;
    float4 un0 = uc0, un1 = uc1;
    if constexpr (j + 1 < BLK) {
      un0 = *reinterpret_cast<const float4*>(&Us[j + 1][CPL * l16]);
      un1 = *reinterpret_cast<const float4*>(&Us[j + 1][CPL * l16 + 4]);
    }
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
        rscale = 1.0f / scale;
        if (l16 == owner && rv && i0 + j < n) {
          const int64_t g = (i0 + j) / G;
          scales[r * ngroups + g] = scale;
          zeros[r * ngroups + g] = zero;
        }
      }
    }
    if constexpr (G < 0) {
      scale = sc_own[s];
      zero = z_own[s];
      rscale = rs_own[s];
    }
    const float wj = w[s];
    const float q = quant_code_fast(wj, scale, rscale, zero, maxq);
    const float dq = scale * (q - zero);
    float e = (wj - dq) * uown[s];
    e = row_bcast<owner>(e);
    if (l16 == owner) {
      e_own[s] = e;
      q_own[s] = q;
    }
    // take the owner's select here: left to the compiler, the 16 selects of
    // a slot (one per owner) sink to the end of the block, keeping every
    // column's code and error live (~330 registers, one wave per SIMD)
    asm volatile("" : "+v"(e_own[s]), "+v"(q_own[s]));
    w[0] = fmaf(-e, uc0.x, w[0]);
    w[1] = fmaf(-e, uc0.y, w[1]);
    w[2] = fmaf(-e, uc0.z, w[2]);
    w[3] = fmaf(-e, uc0.w, w[3]);
    w[4] = fmaf(-e, uc1.x, w[4]);
    w[5] = fmaf(-e, uc1.y, w[5]);
    w[6] = fmaf(-e, uc1.z, w[6]);
    w[7] = fmaf(-e, uc1.w, w[7]);
    uc0 = un0;
    uc1 = un1;
  });

  // errors of columns past the end of the layer are zero (uinv = 0 there)
  float err = 0.0f;
#pragma unroll
  for (int s = 0; s < CPL; ++s) err = fmaf(e_own[s], e_own[s], err);
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) err += __shfl_xor(err, off, LPR);

  if (!rv) return;
  float* erow = E + r * lde + e0 + CPL * l16;
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

// W'[:, c0 + j] -= sum_{k < kc} E[i, k0 + k] U[u0 + k, c0 + j], j < nc.
// 128 x 128 output tile per workgroup (4 waves of 64 x 64, 4 x 4 MFMA tiles
// each), K in chunks of 32: the next chunk is loaded into registers while the
// current one is multiplied out of LDS (double-buffered, one barrier per
// chunk).  Tiles are numbered so that each XCD (every 8th workgroup) takes a
// contiguous range of them, sharing its L2 for the operands.
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int TK = 32;  // K chunk

struct UpdArgs {
  float* Wp;
  int64_t m, n;
  const float* E;
  int64_t lde, k0, kc;
  const float* U;
  int64_t ldu, u0, c0, nc;
  int64_t tiles_n, tiles;
  int vec_u;
};

// TT x TT output tile per workgroup of NW waves, 2 x NW/2 of them, each
// TT/2 rows x TT/(NW/2) columns of 16 x 16 MFMA tiles: TT = 128 with 8 waves
// (64 x 32 each, four waves per SIMD at two workgroups per CU) for the wide
// updates; TT = 64 with 4 waves for the narrow updates inside a super-block,
// where 128-wide tiles would leave most CUs idle.
template <int TT, int NW>
__global__ __launch_bounds__(64 * NW, NW / 2) void update_gemm_kernel(UpdArgs g) {
  constexpr int NT = 64 * NW;            // threads
  constexpr int HW = TT / 2;             // rows per wave
  constexpr int WC = TT / (NW / 2);      // columns per wave
  constexpr int SUBA = HW / 16, SUBB = WC / 16;  // MFMA tiles per wave edge
  constexpr int AQ = TT * TK / (4 * NT);  // float4 per thread per operand chunk
  // A rows of TK + 4 floats: the operand reads (16 rows x 4 k a wave) fall on
  // distinct banks and a thread's 4 k of a row go in one 16-byte store
  __shared__ __align__(16) float As[2][TT][TK + 4];
  __shared__ __align__(16) float Bs[2][TK][TT + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wr = wv / (NW / 2), wc = wv % (NW / 2);
  const int64_t T8 = (g.tiles / 8) * 8;
  const int64_t bid = blockIdx.x;
  const int64_t t = bid < T8 ? (bid % 8) * (T8 / 8) + bid / 8 : bid;
  // tiles in groups of 8 row blocks, column blocks outer and rows inner: the
  // workgroups in flight on an XCD (a contiguous range of t) share a few
  // column blocks of U and the group's rows of E, so U is read from beyond
  // the L2 about once per group instead of once per row block
  const int64_t tiles_m = g.tiles / g.tiles_n;
  const int64_t grp = t / (8 * g.tiles_n);
  const int64_t rig = min((int64_t)8, tiles_m - 8 * grp);  // row blocks in the group
  const int64_t idx = t - grp * 8 * g.tiles_n;
  const int64_t row0 = (grp * 8 + idx % rig) * TT, col0 = (idx / rig) * TT;  // col0 relative to c0

  f32x4 acc[SUBA][SUBB];
#pragma unroll
  for (int a = 0; a < SUBA; ++a)
#pragma unroll
    for (int b = 0; b < SUBB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = row0 + HW * wr + 16 * a + 4 * (lane >> 4) + q;
        const int64_t col = col0 + WC * wc + 16 * b + (lane & 15);
        acc[a][b][q] = (row < g.m && col < g.nc) ? g.Wp[row * g.n + g.c0 + col] : 0.0f;
      }

  // staging: A chunk TT x 32 (thread: rows tid/8 + (NT/8) q, k 4 (tid%8) .. +3),
  //          B chunk 32 x TT (thread: k (tid / (TT/4)) + (4 NT/TT) q, cols 4 (tid % (TT/4)) .. +3)
  float4 ra[AQ], rb[AQ];
  // whole chunks of a tile inside E and U take unchecked 16-byte loads
  const bool full_tile = row0 + TT <= g.m && col0 + TT <= g.nc && g.vec_u;
  auto fetch = [&](int64_t kk0) {
    if (full_tile && kk0 + TK <= g.kc) {  // uniform over the workgroup
#pragma unroll
      for (int q = 0; q < AQ; ++q) {
        const int rr = (tid >> 3) + (NT / 8) * q, kk = 4 * (tid & 7);
        ra[q] = *reinterpret_cast<const float4*>(g.E + (row0 + rr) * g.lde + g.k0 + kk0 + kk);
      }
#pragma unroll
      for (int q = 0; q < AQ; ++q) {
        const int kk = (tid / (TT / 4)) + (4 * NT / TT) * q, cc = 4 * (tid % (TT / 4));
        rb[q] = *reinterpret_cast<const float4*>(g.U + (g.u0 + kk0 + kk) * g.ldu + g.c0 + col0 +
                                                 cc);
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int rr = (tid >> 3) + (NT / 8) * q, kk = 4 * (tid & 7);
      const int64_t row = row0 + rr;
      const int64_t k = kk0 + kk;
      if (row < g.m && k + 4 <= g.kc) {
        ra[q] = *reinterpret_cast<const float4*>(g.E + row * g.lde + g.k0 + k);
      } else {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (row < g.m && k + e < g.kc) ? g.E[row * g.lde + g.k0 + k + e] : 0.0f;
        ra[q] = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int kk = (tid / (TT / 4)) + (4 * NT / TT) * q, cc = 4 * (tid % (TT / 4));
      const int64_t k = kk0 + kk;
      const int64_t col = col0 + cc;
      const float* src = g.U + (g.u0 + (k < g.kc ? k : 0)) * g.ldu + g.c0 + col;
      if (g.vec_u && k < g.kc && col + 4 <= g.nc) {
        rb[q] = *reinterpret_cast<const float4*>(src);
      } else {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (k < g.kc && col + e < g.nc) ? src[e] : 0.0f;
        rb[q] = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int rr = (tid >> 3) + (NT / 8) * q, kk = 4 * (tid & 7);
      *reinterpret_cast<float4*>(&As[buf][rr][kk]) =
          make_float4(-ra[q].x, -ra[q].y, -ra[q].z, -ra[q].w);
    }
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int kk = (tid / (TT / 4)) + (4 * NT / TT) * q, cc = 4 * (tid % (TT / 4));
      *reinterpret_cast<float4*>(&Bs[buf][kk][cc]) = rb[q];
    }
  };

  const int nchunks = (int)((g.kc + TK - 1) / TK);
  fetch(0);
  stash(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nchunks;
    if (more) fetch((int64_t)(c + 1) * TK);
    // the operands of k-step ks + 4 are read while those of ks multiply
    // (measured: 3-5 % over reading each step's operands just before its MFMAs)
    float af[2][SUBA], bf[2][SUBB];
#pragma unroll
    for (int a = 0; a < SUBA; ++a) af[0][a] = As[buf][HW * wr + 16 * a + (lane & 15)][(lane >> 4)];
#pragma unroll
    for (int b = 0; b < SUBB; ++b) bf[0][b] = Bs[buf][(lane >> 4)][WC * wc + 16 * b + (lane & 15)];
#pragma unroll
    for (int ks = 0; ks < TK; ks += 4) {
      const int cur = (ks >> 2) & 1;
      if (ks + 4 < TK) {
#pragma unroll
        for (int a = 0; a < SUBA; ++a)
          af[cur ^ 1][a] = As[buf][HW * wr + 16 * a + (lane & 15)][ks + 4 + (lane >> 4)];
#pragma unroll
        for (int b = 0; b < SUBB; ++b)
          bf[cur ^ 1][b] = Bs[buf][ks + 4 + (lane >> 4)][WC * wc + 16 * b + (lane & 15)];
      }
#pragma unroll
      for (int a = 0; a < SUBA; ++a)
#pragma unroll
        for (int b = 0; b < SUBB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[cur][a], bf[cur][b], acc[a][b], 0, 0,
                                                           0);
    }
    if (more) stash(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int a = 0; a < SUBA; ++a)
#pragma unroll
    for (int b = 0; b < SUBB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = row0 + HW * wr + 16 * a + 4 * (lane >> 4) + q;
        const int64_t col = col0 + WC * wc + 16 * b + (lane & 15);
        if (row < g.m && col < g.nc) g.Wp[row * g.n + g.c0 + col] = acc[a][b][q];
      }
}

void launch_update(float* Wp, int64_t m, int64_t n, const float* E, int64_t lde, int64_t k0,
                   int64_t kc, const float* U, int64_t ldu, int64_t u0, int64_t c0, int64_t nc,
                   hipStream_t stream) {
  if (nc <= 0 || kc <= 0 || m <= 0) return;
  UpdArgs g;
  g.Wp = Wp; g.m = m; g.n = n; g.E = E; g.lde = lde; g.k0 = k0; g.kc = kc;
  g.U = U; g.ldu = ldu; g.u0 = u0; g.c0 = c0; g.nc = nc;
  g.vec_u = (ldu % 4 == 0) && (c0 % 4 == 0) && ((reinterpret_cast<uintptr_t>(U) & 15) == 0);
  // 128-wide tiles when they fill the chip, else 64-wide ones
  if (ceil_div(nc, 128) * ceil_div(m, 128) >= 256) {
    g.tiles_n = ceil_div(nc, 128);
    g.tiles = g.tiles_n * ceil_div(m, 128);
    hipLaunchKernelGGL((update_gemm_kernel<128, 8>), dim3((unsigned)g.tiles), dim3(512), 0, stream,
                       g);
  } else {
    g.tiles_n = ceil_div(nc, 64);
    g.tiles = g.tiles_n * ceil_div(m, 64);
    hipLaunchKernelGGL((update_gemm_kernel<64, 4>), dim3((unsigned)g.tiles), dim3(256), 0, stream,
                       g);
  }
}

__global__ void invert_perm_kernel(const int32_t* __restrict__ perm, int64_t n,
                                   int32_t* __restrict__ inv) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t p = perm[k];
  if (p >= 0 && p < n) inv[p] = (int32_t)k;
}

// codes[r, c] = codes_proc[r, inv[c]] a row at a time through LDS: the
// processing-order row comes in by coalesced 16-byte loads (issued while the
// previous row is gathered) into one LDS row buffer (two barriers a row), and
// leaves in original order by 16-byte stores
// (16 codes), the permuted reads served by the LDS.  The source positions of
// a thread's two output segments (16-bit, two to a word) stay in registers,
// read once per workgroup (NCAP / 32 threads).  Needs n % 16 == 0, n <= NCAP <= 32768.  g_idx is
// written by unpermute_kernel's g_idx-only form.
template <int NCAP, int NT = NCAP / 32>
__global__ __launch_bounds__(NT) void unpermute_rows_kernel(const uint8_t* __restrict__ cproc,
                                                            const int32_t* __restrict__ inv,
                                                            int64_t m, int64_t n,
                                                            int64_t rows_per_wg,
                                                            uint8_t* __restrict__ codes) {
  constexpr int CH = NCAP / 16 / NT;  // 16-byte chunks (16 codes) of a row per thread (2)
  static_assert(NCAP <= 32768, "16-bit position entries");
  __shared__ __align__(16) uint8_t buf[NCAP];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
  const int64_t r1 = min(m, r0 + rows_per_wg);
  if (r0 >= r1) return;
  const int nseg = (int)(n / 16);
  uint32_t pk[CH][8];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int sg = tid + NT * i;
    int32_t kk[16];
    if ((reinterpret_cast<uintptr_t>(inv) & 15) == 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {  // a segment's 16 positions by four 16-byte loads
        const int4 t =
            sg < nseg ? reinterpret_cast<const int4*>(inv)[4 * sg + v] : int4{0, 0, 0, 0};
        kk[4 * v] = t.x; kk[4 * v + 1] = t.y; kk[4 * v + 2] = t.z; kk[4 * v + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) kk[v] = sg < nseg ? inv[16 * (int64_t)sg + v] : 0;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t h[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t c = 16 * (int64_t)sg + 2 * q + e;
        int64_t k = kk[2 * q + e];
        if (k < 0 || k >= n) k = c < n ? c : 0;  // a malformed permutation must not address out of range
        h[e] = (uint32_t)k;
      }
      pk[i][q] = h[0] | (h[1] << 16);
    }
  }
  // the next row's chunks are loaded into registers while this row is gathered
  uint4 nxt[CH];
  auto load_row = [&](int64_t r) {
    const uint4* src = reinterpret_cast<const uint4*>(cproc + r * n);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + NT * c;
      if (idx < nseg) nxt[c] = src[idx];
    }
  };
  load_row(r0);
  for (int64_t r = r0; r < r1; ++r) {
    __syncthreads();  // every thread has read the previous row
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + NT * c;
      if (idx < nseg) reinterpret_cast<uint4*>(buf)[idx] = nxt[c];
    }
    __syncthreads();
    if (r + 1 < r1) load_row(r + 1);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int sg = tid + NT * i;
      if (sg < nseg) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t a = pk[i][2 * q], c2 = pk[i][2 * q + 1];
          w[q] = (uint32_t)buf[a & 0xFFFFu] | ((uint32_t)buf[a >> 16] << 8) |
                 ((uint32_t)buf[c2 & 0xFFFFu] << 16) | ((uint32_t)buf[c2 >> 16] << 24);
        }
        *reinterpret_cast<uint4*>(codes + r * n + 16 * (int64_t)sg) =
            make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

// codes[r, c] = codes_proc[r, inv[c]]; g_idx[c] = inv[c] / G (static groups:
// c / G, the groups being runs of original columns).
__global__ __launch_bounds__(256) void unpermute_kernel(const uint8_t* __restrict__ cproc,
                                                        const int32_t* __restrict__ inv,
                                                        int64_t m, int64_t n, int64_t G,
                                                        int gstatic, uint8_t* __restrict__ codes,
                                                        int32_t* __restrict__ g_idx) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  int64_t k = inv ? inv[c] : c;
  if (k < 0 || k >= n) k = c;
  if (g_idx && blockIdx.y == 0) g_idx[c] = G > 0 ? (int32_t)((gstatic ? c : k) / G) : 0;
  if (!codes) return;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) codes[r * n + c] = cproc[r * n + k];
}

}  // namespace

// Super-block width: the K of the update past each super-block.
int64_t super_block(int64_t n) { return hmin(ceil_div(n, BLK) * BLK, 1024); }

size_t quantize_ws_bytes(int64_t m, int64_t n, int desc_act) {
  size_t b = align_up((size_t)m * n * sizeof(float), 256);              // W'
  b += align_up((size_t)m * super_block(n) * sizeof(float), 256);       // E
  if (desc_act) {
    b += align_up((size_t)m * n, 256);                       // codes, processing order
    b += align_up((size_t)n * sizeof(int32_t), 256);         // inverse permutation
  }
  return b;
}

hipError_t gemm_f32_sub(float* C, int64_t ldc, int64_t m, int64_t n, const float* A, int64_t lda,
                        const float* B, int64_t ldb, int64_t k, hipStream_t stream) {
  launch_update(C, m, ldc, A, lda, 0, k, B, ldb, 0, 0, n, stream);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  const int64_t m = a.m, n = a.n;
  char* ws = reinterpret_cast<char*>(a.ws);
  float* Wp = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)m * n * sizeof(float), 256);
  const int64_t SB = super_block(n);
  float* E = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)m * SB * sizeof(float), 256);
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
  if (a.wdt == GPTQ_BF16 && !a.desc_act && n % 8 == 0 && a.ldw % 8 == 0 &&
      reinterpret_cast<uintptr_t>(a.W) % 16 == 0) {
    const dim3 grid((unsigned)ceil_div(n, 8 * 256), (unsigned)hmin(m, 1024));
    hipLaunchKernelGGL(prep_weights_bf16_kernel, grid, dim3(256), 0, stream,
                       reinterpret_cast<const uint16_t*>(a.W), m, n, a.ldw, a.dead, Wp, a.info);
  } else if (a.wdt == GPTQ_BF16 && a.desc_act && n % 8 == 0 && a.ldw % 8 == 0 &&
             reinterpret_cast<uintptr_t>(a.W) % 16 == 0 && n <= 32768) {
    // permuted rows through LDS: 32 KB per workgroup up to 8192 columns, else 128 KB
    const int64_t wgs = hmin(m, (int64_t)512);  // two workgroups a CU
    const int64_t rpw = ceil_div(m, wgs);
    const dim3 grid((unsigned)ceil_div(m, rpw));
    if (n <= 8192)
      hipLaunchKernelGGL(prep_rows_bf16_kernel<8192>, grid, dim3(512), 0, stream,
                         reinterpret_cast<const uint16_t*>(a.W), a.ldw, a.perm, a.dead, m, n, rpw,
                         Wp, a.info);
    else
      hipLaunchKernelGGL(prep_rows_bf16_kernel<32768>, grid, dim3(512), 0, stream,
                         reinterpret_cast<const uint16_t*>(a.W), a.ldw, a.perm, a.dead, m, n, rpw,
                         Wp, a.info);
  } else {
    const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(m, 1024));
    hipLaunchKernelGGL(prep_weights_kernel, grid, dim3(256), 0, stream, a.W, a.wdt, m, n, a.ldw,
                       a.desc_act ? a.perm : nullptr, a.dead, Wp, a.info);
  }
  // where the parameters come from: computed in the block at each group's
  // first column (G divides the block), or given: from the whole row (G < 0),
  // from the original weights (static groups), or, for a group spanning
  // several blocks, from W' at the block where it starts
  const bool given = G < 0 || a.static_groups || G > BLK;
  const int64_t gdiv = G > 0 ? G : n;
  const int32_t* gperm = (a.static_groups && a.desc_act) ? a.perm : nullptr;
  if (G < 0) {
    hipLaunchKernelGGL(row_params_kernel, dim3((unsigned)hmin(m, 4096)), dim3(256), 0,
                       stream, Wp, m, n, (int64_t)0, n, (int64_t)0, (int64_t)1, maxq, a.sym,
                       a.scales, a.zeros);
  } else if (a.static_groups) {
    hipLaunchKernelGGL(static_params_kernel, dim3((unsigned)ceil_div(m * ngroups, 256)),
                       dim3(256), 0, stream, a.W, a.wdt, m, n, a.ldw, a.dead, (int64_t)G, ngroups,
                       maxq, a.sym, a.scales, a.zeros);
  }
  const dim3 qgrid((unsigned)ceil_div(m, QROWS));
  for (int64_t s0 = 0; s0 < n; s0 += SB) {
    const int64_t s1 = hmin(n, s0 + SB);
    for (int64_t i0 = s0; i0 < s1; i0 += BLK) {
      const int first = i0 == 0;
      if (!a.static_groups && G > BLK && i0 % G == 0) {
        // a group spanning several blocks starts here: every earlier error
        // has been applied to its columns (G divides the super-block)
        hipLaunchKernelGGL(row_params_kernel, dim3((unsigned)hmin(m, 4096)), dim3(256), 0,
                           stream, Wp, m, n, i0, hmin((int64_t)G, n - i0), i0 / G, ngroups, maxq,
                           a.sym, a.scales, a.zeros);
      }
#define GPTQ_BQ(GV)                                                                              \
  hipLaunchKernelGGL(block_quant_kernel<GV>, qgrid, dim3(256), 0, stream, Wp, m, n, a.U, a.ldu,  \
                     i0, maxq, a.sym, cproc, a.scales, a.zeros, ngroups, E, SB, i0 - s0,        \
                     a.row_err, first, gperm, gdiv)
      switch (given ? -1 : G) {
        case 8: GPTQ_BQ(8); break;
        case 16: GPTQ_BQ(16); break;
        case 32: GPTQ_BQ(32); break;
        case 64: GPTQ_BQ(64); break;
        case 128: GPTQ_BQ(128); break;
        default: GPTQ_BQ(-1); break;
      }
#undef GPTQ_BQ
      // the rest of this super-block, from this block's errors
      const int64_t i1 = i0 + BLK;
      if (i1 < s1) launch_update(Wp, m, n, E, SB, i0 - s0, BLK, a.U, a.ldu, i0, i1, s1 - i1, stream);
    }
    // every column past the super-block, from all of its errors
    if (s1 < n) launch_update(Wp, m, n, E, SB, 0, s1 - s0, a.U, a.ldu, s0, s1, n - s1, stream);
  }
  if (a.desc_act) {
    hipLaunchKernelGGL(invert_perm_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream,
                       a.perm, n, inv);
    if (n % 16 == 0 && n <= 32768) {
      // codes through LDS rows; g_idx by the per-column kernel alone
      // as many workgroups as fit on the GPU at once (2048 threads a CU), so
      // each reads its positions once and they run in one round
      const int64_t wgs = hmin(m, (int64_t)(n <= 16384 ? 1024 : 512));
      const int64_t rpw = ceil_div(m, wgs);
      const dim3 grid((unsigned)ceil_div(m, rpw));
      if (n <= 16384)
        hipLaunchKernelGGL(unpermute_rows_kernel<16384>, grid, dim3(512), 0, stream, cproc, inv,
                           m, n, rpw, a.codes);
      else
        hipLaunchKernelGGL(unpermute_rows_kernel<32768>, grid, dim3(1024), 0, stream, cproc, inv,
                           m, n, rpw, a.codes);
      if (a.g_idx)
        hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)ceil_div(n, 256), 1), dim3(256), 0,
                           stream, (const uint8_t*)nullptr, inv, (int64_t)0, n, (int64_t)G,
                           a.static_groups, (uint8_t*)nullptr, a.g_idx);
    } else {
      const dim3 grid((unsigned)ceil_div(n, 256), (unsigned)hmin(m, 1024));
      hipLaunchKernelGGL(unpermute_kernel, grid, dim3(256), 0, stream, cproc, inv, m, n,
                         (int64_t)G, a.static_groups, a.codes, a.g_idx);
    }
  } else if (a.g_idx) {
    hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)ceil_div(n, 256), 1), dim3(256), 0, stream,
                       (const uint8_t*)nullptr, (const int32_t*)nullptr, (int64_t)0, n, (int64_t)G,
                       a.static_groups, (uint8_t*)nullptr, a.g_idx);
  }
  return hipGetLastError();
}

}  // namespace gptq
