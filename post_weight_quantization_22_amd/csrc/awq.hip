// AWQ-lite channel scaling and awq_clip.
//
// "AWQ, MinMax, GPTQ calibration in Model Optimizer" (gtnt.cn news 115337),
// section 3: awq_lite rescales input channels and weights in opposite
// directions by s = x^alpha / w^(1 - alpha) (x, w: per-channel mean absolute
// values of the activations and of the weights), searching alpha over [0, 1] in
// steps of 0.1 for the smallest error between the rescaled, quantized layer's
// output and the true output; awq_clip then searches each group's clip value in
// [0.5 amax, amax] in steps of 0.05 amax.  "LLM quantization principles"
// section 3.2: the weights are multiplied by s and the activations divided.
//
// The output error of a candidate, ||X D^T||^2 with D = W_eff - W, is taken
// through the calibration second moments S = X^T X that the Hessian step
// accumulates: sum((D S) * D), one fp32 MFMA product per candidate alpha
// (the trailing-update GEMM), instead of a pass over the tokens.  The clip
// search is per (row, group) with the group's block of the rescaled S staged
// in LDS.  Both are deterministic (fixed summation orders).
#include <algorithm>

#include "kernels.hpp"

namespace gptq {

namespace {

constexpr float kFloor = 1e-8f;

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) p[i] = 0.0f;
}

// ---- per-channel mean absolute activation --------------------------------
// fp64 sums (a pass over X that is bound by its reads), so that the statistic
// is the correctly rounded sum whatever the token count
__global__ __launch_bounds__(256) void absum_partial_kernel(const void* __restrict__ X, int dt,
                                                            int64_t tokens, int64_t n,
                                                            int64_t ldx, int64_t per,
                                                            double* __restrict__ part) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  const int64_t t0 = (int64_t)blockIdx.y * per, t1 = min(tokens, t0 + per);
  double s = 0.0;
  for (int64_t t = t0; t < t1; ++t) s += (double)fabsf(load_elem(X, dt, t * ldx + c));
  part[(int64_t)blockIdx.y * n + c] = s;
}

// bf16 rows, 8 channels per lane (one 16-byte load), the workgroup's four waves
// on interleaved tokens of the slice, combined through LDS in a fixed order
__global__ __launch_bounds__(256) void absum_partial_bf16x8_kernel(
    const uint16_t* __restrict__ X, int64_t tokens, int64_t n, int64_t ldx, int64_t per,
    double* __restrict__ part) {
  __shared__ double red[3][64][8];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t c = ((int64_t)blockIdx.x * 64 + lane) * 8;
  const int64_t t0 = (int64_t)blockIdx.y * per, t1 = min(tokens, t0 + per);
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  if (c < n) {
    int64_t t = t0 + wv;
    for (; t + 12 < t1; t += 16) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = *reinterpret_cast<const uint4*>(X + (t + 4 * u) * ldx + c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += (double)fabsf(bf16_bits_to_f32(w[e] & 0xFFFFu));
          acc[2 * e + 1] += (double)fabsf(bf16_bits_to_f32(w[e] >> 16));
        }
      }
    }
    for (; t < t1; t += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(X + t * ldx + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)fabsf(bf16_bits_to_f32(w[e] & 0xFFFFu));
        acc[2 * e + 1] += (double)fabsf(bf16_bits_to_f32(w[e] >> 16));
      }
    }
  }
  if (wv > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wv - 1][lane][e] = acc[e];
  }
  __syncthreads();
  if (wv == 0 && c < n) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += red[w][lane][e];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[(int64_t)blockIdx.y * n + c + e] = acc[e];
  }
}

// out[c] = out[c] + sum (accumulate) or sum / div.  32 channels per workgroup,
// 8 threads per channel on interleaved partials, combined in a fixed order.
__global__ __launch_bounds__(256) void absum_reduce_kernel(const double* __restrict__ part,
                                                           int64_t P, int64_t n, int accumulate,
                                                           double div, float* __restrict__ out) {
  __shared__ double red[8][32];
  const int cl = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int64_t c = (int64_t)blockIdx.x * 32 + cl;
  double s = 0.0;
  if (c < n)
    for (int64_t p = grp; p < P; p += 8) s += part[p * n + c];
  red[grp][cl] = s;
  __syncthreads();
  if (grp == 0 && c < n) {
    for (int g = 1; g < 8; ++g) s += red[g][cl];
    out[c] = accumulate ? (float)((double)out[c] + s) : (float)(s / div);
  }
}

// s[c] = x^a / w^(1 - a), x = absum[c] / tokens, both floored; a from
// *alpha_dev when given (the searched value), else alpha
__global__ __launch_bounds__(256) void awq_scales_kernel(const float* __restrict__ absum,
                                                         float inv_tokens,
                                                         const float* __restrict__ wm,
                                                         int64_t n, const float* alpha_dev,
                                                         float alpha, float* __restrict__ s) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= n) return;
  const float a = alpha_dev ? *alpha_dev : alpha;
  const float x = fmaxf(absum[c] * inv_tokens, kFloor);
  const float w = fmaxf(wm[c], kFloor);
  s[c] = powf(x, a) / powf(w, 1.0f - a);
}

__global__ __launch_bounds__(256) void symmetrize_kernel(const float* __restrict__ S, int64_t lds,
                                                         int64_t n, float* __restrict__ F) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y)
    F[i * n + j] = j <= i ? S[i * lds + j] : S[j * lds + i];
}

// ---- one alpha: D = dequant(Q(W diag(s))) / s - W --------------------------
// One wave per (row, group); lanes stride the group's columns.
__global__ __launch_bounds__(256) void awq_qdq_kernel(const void* __restrict__ W, int dt,
                                                      int64_t m, int64_t n, int64_t ldw,
                                                      const float* __restrict__ s, int64_t G,
                                                      int64_t ngroups, float maxq, int sym,
                                                      float* __restrict__ D, int64_t ldd) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= m * ngroups) return;
  const int64_t r = pair / ngroups, g = pair - r * ngroups;
  const int64_t c0 = g * G, c1 = min(n, c0 + G);
  float vmin = 0.0f, vmax = 0.0f;
  for (int64_t c = c0 + lane; c < c1; c += 64) {
    const float v = __fmul_rn(load_elem(W, dt, r * ldw + c), s[c]);
    vmin = fminf(vmin, v);
    vmax = fmaxf(vmax, v);
  }
  for (int off = 1; off < 64; off <<= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, off));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  }
  float scale, zero;
  if (sym) sym_params(fmaxf(fabsf(vmin), fabsf(vmax)), maxq, scale, zero);
  else minmax_params(vmin, vmax, maxq, scale, zero);
  for (int64_t c = c0 + lane; c < c1; c += 64) {
    const float w = load_elem(W, dt, r * ldw + c);
    const float v = __fmul_rn(w, s[c]);
    const float q = quant_code(v, scale, zero, maxq);
    D[r * ldd + c] = (scale * (q - zero)) / s[c] - w;
  }
}

// sum of Z * D over the whole matrix: fixed per-block slices, then in order
__global__ __launch_bounds__(256) void dot_partial_kernel(const float* __restrict__ Z,
                                                          const float* __restrict__ D,
                                                          int64_t total, int64_t per,
                                                          float* __restrict__ part) {
  __shared__ float red[256];
  const int64_t i0 = (int64_t)blockIdx.x * per, i1 = min(total, i0 + per);
  float acc = 0.0f;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += 256) acc = fmaf(Z[i], D[i], acc);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// loss = -(sum of the partials), Z holding -(D S); one workgroup, fixed order
__global__ __launch_bounds__(256) void loss_final_kernel(const float* __restrict__ part,
                                                         int64_t np, float* __restrict__ loss) {
  __shared__ double red[256];
  const int64_t per = (np + 255) / 256;
  const int64_t p0 = (int64_t)threadIdx.x * per, p1 = min(np, p0 + per);
  double acc = 0.0;
  for (int64_t p = p0; p < p1; ++p) acc += (double)part[p];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)(-red[0]);
}

// alpha of the first smallest loss
__global__ void argmin_kernel(const float* __restrict__ losses, int na, float step,
                              float* __restrict__ alpha_out) {
  int best = 0;
  for (int i = 1; i < na; ++i)
    if (losses[i] < losses[best]) best = i;
  *alpha_out = (float)best * step;
}

// ---- awq_clip ---------------------------------------------------------------
// One group of columns per workgroup, its block of the rescaled second moments
// S'_gg in LDS; one row per wave at a time.  A wave forms the errors d_k of all
// the candidate clips of its row (lane j holds columns j and j + 64), stages them
// in LDS as [column][candidate], and then takes every quadratic form d_k S'_gg d_k
// in one sweep over the group's columns: each S' value read from LDS serves all
// the candidates.
constexpr int CLIP_MAXG = 128;
constexpr int CLIP_NK = 12;     // candidate slots (at most 11 used), three float4s
constexpr int CLIP_WAVES = 8;

__device__ __forceinline__ void clip_params(float amax, float vmin, float vmax, int k, float maxq,
                                            int sym, float& scale, float& zero) {
  const float c = __fmul_rn(amax, (float)(1.0 - 0.05 * k));
  if (sym) sym_params(fminf(amax, c), maxq, scale, zero);
  else minmax_params(fmaxf(vmin, -c), fminf(vmax, c), maxq, scale, zero);
}

__global__ __launch_bounds__(CLIP_WAVES * 64) void awq_clip_kernel(
    const void* __restrict__ W, int dt, int64_t m, int64_t n, int64_t ldw,
    const float* __restrict__ S, int64_t lds, const float* __restrict__ s, int64_t G,
    int64_t ngroups, float maxq, int sym, int nsteps, int64_t rows_per_wg,
    uint8_t* __restrict__ codes, float* __restrict__ scales, float* __restrict__ zeros,
    uint8_t* __restrict__ clip_idx) {
  __shared__ float Sg[CLIP_MAXG][CLIP_MAXG + 1];
  __shared__ float4 dsh[CLIP_WAVES][CLIP_MAXG][CLIP_NK / 4];
  const int64_t g = blockIdx.x;
  const int64_t c0 = g * G;
  const int gl = (int)min(G, n - c0);  // this group's width
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // rescaled second moments of the group, S_ij / (s_i s_j); zero outside it
  for (int idx = tid; idx < CLIP_MAXG * CLIP_MAXG; idx += CLIP_WAVES * 64) {
    const int i = idx / CLIP_MAXG, j = idx - i * CLIP_MAXG;
    float v = 0.0f;
    if (i < gl && j < gl) {
      const int64_t a = c0 + max(i, j), b = c0 + min(i, j);
      v = S[a * lds + b];
      if (s) v = v / (s[c0 + i] * s[c0 + j]);
    }
    Sg[i][j] = v;
  }
  __syncthreads();
  for (int64_t rbeg = (int64_t)blockIdx.y * rows_per_wg; rbeg < m;
       rbeg += (int64_t)gridDim.y * rows_per_wg) {
    const int64_t rend = min(m, rbeg + rows_per_wg);
    for (int64_t r = rbeg + wv; r < rend; r += CLIP_WAVES) {
      float v[2], amax = 0.0f, vmin = 0.0f, vmax = 0.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + 64 * h;
        float x = 0.0f;
        if (j < gl) {
          const float w = load_elem(W, dt, r * ldw + c0 + j);
          x = s ? __fmul_rn(w, s[c0 + j]) : w;
          vmin = fminf(vmin, x);
          vmax = fmaxf(vmax, x);
        }
        v[h] = x;
        amax = fmaxf(amax, fabsf(x));
      }
      for (int off = 1; off < 64; off <<= 1) {
        amax = fmaxf(amax, __shfl_xor(amax, off));
        vmin = fminf(vmin, __shfl_xor(vmin, off));
        vmax = fmaxf(vmax, __shfl_xor(vmax, off));
      }
      // the errors of every candidate, in the rescaled space
      float d0[CLIP_NK], d1[CLIP_NK];
#pragma unroll
      for (int k = 0; k < CLIP_NK; ++k) {
        d0[k] = 0.0f;
        d1[k] = 0.0f;
        if (k < nsteps) {
          float scale, zero;
          clip_params(amax, vmin, vmax, k, maxq, sym, scale, zero);
          if (lane < gl) d0[k] = scale * (quant_code(v[0], scale, zero, maxq) - zero) - v[0];
          if (lane + 64 < gl) d1[k] = scale * (quant_code(v[1], scale, zero, maxq) - zero) - v[1];
        }
      }
#pragma unroll
      for (int q = 0; q < CLIP_NK / 4; ++q) {
        dsh[wv][lane][q] = make_float4(d0[4 * q], d0[4 * q + 1], d0[4 * q + 2], d0[4 * q + 3]);
        dsh[wv][lane + 64][q] = make_float4(d1[4 * q], d1[4 * q + 1], d1[4 * q + 2], d1[4 * q + 3]);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      // t_k[j] = sum_i S'_ji d_k[i] for the lane's two columns, all k at once
      float t0[CLIP_NK], t1[CLIP_NK];
#pragma unroll
      for (int k = 0; k < CLIP_NK; ++k) {
        t0[k] = 0.0f;
        t1[k] = 0.0f;
      }
#pragma unroll 4
      for (int i = 0; i < gl; ++i) {
        const float s0 = Sg[lane][i], s1 = Sg[lane + 64][i];
#pragma unroll
        for (int q = 0; q < CLIP_NK / 4; ++q) {
          const float4 dk = dsh[wv][i][q];
          t0[4 * q] = fmaf(s0, dk.x, t0[4 * q]);
          t0[4 * q + 1] = fmaf(s0, dk.y, t0[4 * q + 1]);
          t0[4 * q + 2] = fmaf(s0, dk.z, t0[4 * q + 2]);
          t0[4 * q + 3] = fmaf(s0, dk.w, t0[4 * q + 3]);
          t1[4 * q] = fmaf(s1, dk.x, t1[4 * q]);
          t1[4 * q + 1] = fmaf(s1, dk.y, t1[4 * q + 1]);
          t1[4 * q + 2] = fmaf(s1, dk.z, t1[4 * q + 2]);
          t1[4 * q + 3] = fmaf(s1, dk.w, t1[4 * q + 3]);
        }
      }
      // e_k = sum_j d_k[j] t_k[j]; the first smallest wins
      float best = 0.0f;
      int bk = 0;
#pragma unroll
      for (int k = 0; k < CLIP_NK; ++k) {
        if (k < nsteps) {
          float e = fmaf(d1[k], t1[k], d0[k] * t0[k]);
          for (int off = 1; off < 64; off <<= 1) e += __shfl_xor(e, off);
          if (k == 0 || e < best) {
            best = e;
            bk = k;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();  // dsh is rewritten by the wave's next row
      float scale, zero;
      clip_params(amax, vmin, vmax, bk, maxq, sym, scale, zero);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + 64 * h;
        if (j < gl) codes[r * n + c0 + j] = (uint8_t)quant_code(v[h], scale, zero, maxq);
      }
      if (lane == 0) {
        scales[r * ngroups + g] = scale;
        zeros[r * ngroups + g] = zero;
        if (clip_idx) clip_idx[r * ngroups + g] = (uint8_t)bk;
      }
    }
  }
}

}  // namespace

constexpr int64_t kAbsumSplit = 256;  // token slices of the activation statistics

size_t awq_absum_ws_bytes(int64_t n, int64_t tokens) {
  (void)tokens;
  return (size_t)kAbsumSplit * (size_t)n * sizeof(double);
}

namespace {
// out[c] (+)= sum over rows of |A[r, c]| (accumulate), or that sum / div
void launch_colsum(const void* X, int dt, int64_t tokens, int64_t n, int64_t ldx, double* part,
                   float* out, int accumulate, double div, hipStream_t stream) {
  const int64_t per = ceil_div(tokens, kAbsumSplit);
  const int64_t P = ceil_div(tokens, per);
  const bool vec = dt == GPTQ_BF16 && n % 8 == 0 && ldx % 8 == 0 &&
                   (reinterpret_cast<uintptr_t>(X) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(absum_partial_bf16x8_kernel, dim3((unsigned)ceil_div(n, 512), (unsigned)P),
                       dim3(256), 0, stream, static_cast<const uint16_t*>(X), tokens, n, ldx, per,
                       part);
  else
    hipLaunchKernelGGL(absum_partial_kernel, dim3((unsigned)ceil_div(n, 256), (unsigned)P),
                       dim3(256), 0, stream, X, dt, tokens, n, ldx, per, part);
  hipLaunchKernelGGL(absum_reduce_kernel, dim3((unsigned)ceil_div(n, 32)), dim3(256), 0, stream,
                     part, P, n, accumulate, div, out);
}
}  // namespace

hipError_t launch_awq_absum(const void* X, int dt, int64_t tokens, int64_t n, int64_t ldx,
                            float* absum, void* ws, hipStream_t stream) {
  launch_colsum(X, dt, tokens, n, ldx, static_cast<double*>(ws), absum, 1, 1.0, stream);
  return hipGetLastError();
}

namespace {
constexpr int64_t kDotBlocks = 1024;
inline size_t al(size_t b) { return align_up(b, 256); }
}  // namespace

// D and Z rows padded to a multiple of 4 floats (the product's A operand is read
// in float4s)
inline int64_t lite_ld(int64_t n) { return (int64_t)align_up((size_t)n, 4); }

size_t awq_lite_ws_bytes(int64_t m, int64_t n) {
  return al((size_t)n * 4) + al((size_t)n * n * 4) + 2 * al((size_t)m * lite_ld(n) * 4) +
         al((size_t)kDotBlocks * 4) + al(awq_absum_ws_bytes(n, m));
}

hipError_t launch_awq_lite(const void* W, int wdt, int64_t m, int64_t n, int64_t ldw,
                           const float* S, int64_t lds, const float* absum, int64_t tokens,
                           int bits, int64_t G, int sym, int nalpha, float* s_out,
                           float* alpha_out, float* losses, void* ws, hipStream_t stream) {
  char* p = static_cast<char*>(ws);
  float* wm = reinterpret_cast<float*>(p);
  p += al((size_t)n * 4);
  float* F = reinterpret_cast<float*>(p);
  p += al((size_t)n * n * 4);
  const int64_t ldd = lite_ld(n);
  float* D = reinterpret_cast<float*>(p);
  p += al((size_t)m * ldd * 4);
  float* Z = reinterpret_cast<float*>(p);
  p += al((size_t)m * ldd * 4);
  float* part = reinterpret_cast<float*>(p);
  p += al((size_t)kDotBlocks * 4);
  double* colpart = reinterpret_cast<double*>(p);
  const int64_t Geff = G > 0 ? G : n;
  const int64_t ngroups = ceil_div(n, Geff);
  const float maxq = (float)((1 << bits) - 1);
  const float inv_tokens = 1.0f / (float)tokens;
  const float step = 1.0f / (float)(nalpha - 1);
  const dim3 cgrid((unsigned)ceil_div(n, 256));
  launch_colsum(W, wdt, m, n, ldw, colpart, wm, 0, (double)m, stream);
  hipLaunchKernelGGL(symmetrize_kernel,
                     dim3((unsigned)ceil_div(n, 256), (unsigned)std::min<int64_t>(n, 65535)),
                     dim3(256), 0, stream, S, lds, n, F);
  // the padding columns of D stay zero (they meet zero columns of Z in the dot)
  const int64_t total = m * ldd;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream,
                     D, total);
  const int64_t per = ceil_div(total, kDotBlocks);
  const int64_t nblk = ceil_div(total, per);
  for (int a = 0; a < nalpha; ++a) {
    hipLaunchKernelGGL(awq_scales_kernel, cgrid, dim3(256), 0, stream, absum, inv_tokens, wm, n,
                       (const float*)nullptr, step * (float)a, s_out);
    hipLaunchKernelGGL(awq_qdq_kernel, dim3((unsigned)ceil_div(m * ngroups, 4)), dim3(256), 0,
                       stream, W, wdt, m, n, ldw, s_out, Geff, ngroups, maxq, sym, D, ldd);
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)ceil_div(total, 256)), dim3(256), 0, stream,
                       Z, total);
    const hipError_t e = gemm_f32_sub(Z, ldd, m, n, D, ldd, F, n, n, stream);  // Z = -D S
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dot_partial_kernel, dim3((unsigned)nblk), dim3(256), 0, stream, Z, D, total,
                       per, part);
    hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(256), 0, stream, part, nblk, losses + a);
  }
  hipLaunchKernelGGL(argmin_kernel, dim3(1), dim3(1), 0, stream, losses, nalpha, step, alpha_out);
  hipLaunchKernelGGL(awq_scales_kernel, cgrid, dim3(256), 0, stream, absum, inv_tokens, wm, n,
                     (const float*)alpha_out, 0.0f, s_out);
  return hipGetLastError();
}

hipError_t launch_awq_clip(const void* W, int wdt, int64_t m, int64_t n, int64_t ldw,
                           const float* S, int64_t lds, const float* s, int bits, int64_t G,
                           int sym, int nsteps, uint8_t* codes, float* scales, float* zeros,
                           uint8_t* clip_idx, hipStream_t stream) {
  const int64_t ngroups = ceil_div(n, G);
  const float maxq = (float)((1 << bits) - 1);
  const int64_t rows_per_wg = 64;
  const dim3 grid((unsigned)ngroups, (unsigned)std::min<int64_t>(ceil_div(m, rows_per_wg), 65535));
  hipLaunchKernelGGL(awq_clip_kernel, grid, dim3(CLIP_WAVES * 64), 0, stream, W, wdt, m, n, ldw, S, lds, s, G,
                     ngroups, maxq, sym, nsteps, rows_per_wg, codes, scales, zeros, clip_idx);
  return hipGetLastError();
}

}  // namespace gptq
