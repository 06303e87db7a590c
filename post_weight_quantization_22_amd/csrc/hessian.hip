// Layer Hessian accumulation S += X^T X on gfx950.
//
// "GPTQ deep dive" (hncyxsy.com news 243429) section 3.1 step 1: the layer
// Hessian is built from the layer's calibration inputs X as 2 X X^T (the
// factor 2 and the damping are applied by gptq_prepare).  X arrives
// token-major, X[tokens, n], so X X^T = sum over tokens of x_t x_t^T: a SYRK
// whose reduction axis is the token axis.
//
// bf16 path (the dense contraction, on MFMA): lower-triangle 128x128 output
// tiles, 4 waves each holding a 64x64 sub-tile as 2x2
// v_mfma_f32_32x32x16_bf16 accumulators.  A stage covers 32 tokens.  Both
// operands need the token axis in the per-lane k slots, while X is contiguous
// along channels, so the stage is transposed on its way into LDS: a lane loads
// two token rows x 8 channels (2 x 16 B, coalesced along channels), pairs the
// two tokens of each channel into one 32-bit word and stores it at
// [channel][token pair]; an MFMA operand is then one 16-byte LDS read.
// bf16 x bf16 products are exact in fp32; accumulation is fp32.
//
// Tiles are few when n is small, so the token axis is split P ways; each
// split writes its partial tile to the workspace and a reduction kernel adds
// the P partials to S in a fixed order (deterministic, no atomics).  With
// P == 1 the tile is added to S directly.
//
// fp32 path (fp32 activations; small layers): a SIMT fp32 SYRK, lower tiles.
#include "kernels.hpp"

namespace gptq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int HT = 128;    // output tile edge
constexpr int HK = 32;     // tokens per stage
constexpr int HKP = HK + 8;  // LDS row length in bf16 (padding vs bank conflicts)

__device__ __forceinline__ void tile_coords(int64_t L, int64_t& ti, int64_t& tj) {
  // lower-triangle tile L -> (ti >= tj), row-major over the triangle
  int64_t t = (int64_t)((sqrt(8.0 * (double)L + 1.0) - 1.0) * 0.5);
  while (t * (t + 1) / 2 > L) --t;
  while ((t + 1) * (t + 2) / 2 <= L) ++t;
  ti = t;
  tj = L - t * (t + 1) / 2;
}

struct Rows2 {
  uint4 a, b;  // two token rows x 8 channels (bf16)
};

__device__ __forceinline__ Rows2 load_rows2(const uint16_t* __restrict__ X, int64_t ldx,
                                            int64_t tokens, int64_t n, int64_t t, int64_t c,
                                            bool vec_ok) {
  Rows2 r;
  const bool full_c = c + 8 <= n;
  if (vec_ok && full_c) {
    r.a = t < tokens ? *reinterpret_cast<const uint4*>(X + t * ldx + c) : make_uint4(0, 0, 0, 0);
    r.b = t + 1 < tokens ? *reinterpret_cast<const uint4*>(X + (t + 1) * ldx + c)
                         : make_uint4(0, 0, 0, 0);
    return r;
  }
  uint32_t wa[4], wb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t lo = 0, hi = 0, lo2 = 0, hi2 = 0;
    if (t < tokens) {
      if (c + 2 * k < n) lo = X[t * ldx + c + 2 * k];
      if (c + 2 * k + 1 < n) hi = X[t * ldx + c + 2 * k + 1];
    }
    if (t + 1 < tokens) {
      if (c + 2 * k < n) lo2 = X[(t + 1) * ldx + c + 2 * k];
      if (c + 2 * k + 1 < n) hi2 = X[(t + 1) * ldx + c + 2 * k + 1];
    }
    wa[k] = lo | (hi << 16);
    wb[k] = lo2 | (hi2 << 16);
  }
  r.a = make_uint4(wa[0], wa[1], wa[2], wa[3]);
  r.b = make_uint4(wb[0], wb[1], wb[2], wb[3]);
  return r;
}

// Write the 8 channels x 2 tokens held in r into T[channel][token pair].
__device__ __forceinline__ void store_transposed(uint32_t* __restrict__ T, int ch0, int tp,
                                                 const Rows2& r) {
  const uint32_t a[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
  const uint32_t b[4] = {r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // channel 2k: low halves of token t and t+1; channel 2k+1: high halves
    T[(ch0 + 2 * k) * (HKP / 2) + tp] = (a[k] & 0xFFFFu) | (b[k] << 16);
    T[(ch0 + 2 * k + 1) * (HKP / 2) + tp] = (a[k] >> 16) | (b[k] & 0xFFFF0000u);
  }
}

__global__ __launch_bounds__(256) void syrk_bf16_kernel(const uint16_t* __restrict__ X,
                                                        int64_t ldx, int64_t tokens, int64_t n,
                                                        int64_t tok_per_split,
                                                        float* __restrict__ S, int64_t lds,
                                                        float* __restrict__ part,
                                                        int64_t ntiles) {
  __shared__ uint32_t At[HT * HKP / 2];
  __shared__ uint32_t Bt[HT * HKP / 2];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wr = wv >> 1, wc = wv & 1;
  const int64_t L = blockIdx.x;
  const int64_t p = blockIdx.y;
  int64_t ti, tj;
  tile_coords(L, ti, tj);
  const int64_t i0 = ti * HT, j0 = tj * HT;
  const bool diag = ti == tj;
  const int64_t t_begin = p * tok_per_split;
  const int64_t t_end = min(tokens, t_begin + tok_per_split);
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(X) & 15) == 0) && (ldx % 8 == 0);

  // loader mapping: token pair tp (0..15), channel chunk cc (0..15)
  const int tp = tid >> 4, cc = tid & 15;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[a][b][q] = 0.0f;

  Rows2 ra, rb;
  if (t_begin < t_end) {
    ra = load_rows2(X, ldx, t_end, n, t_begin + 2 * tp, i0 + 8 * cc, vec_ok);
    if (!diag) rb = load_rows2(X, ldx, t_end, n, t_begin + 2 * tp, j0 + 8 * cc, vec_ok);
  }
  for (int64_t t0 = t_begin; t0 < t_end; t0 += HK) {
    __syncthreads();
    store_transposed(At, 8 * cc, tp, ra);
    if (!diag) store_transposed(Bt, 8 * cc, tp, rb);
    __syncthreads();
    if (t0 + HK < t_end) {  // prefetch the next stage into registers
      ra = load_rows2(X, ldx, t_end, n, t0 + HK + 2 * tp, i0 + 8 * cc, vec_ok);
      if (!diag) rb = load_rows2(X, ldx, t_end, n, t0 + HK + 2 * tp, j0 + 8 * cc, vec_ok);
    }
    const uint32_t* Bsrc = diag ? At : Bt;
#pragma unroll
    for (int kk = 0; kk < HK / 16; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int row = 64 * wr + 32 * a + (lane & 31);
        af[a] = *reinterpret_cast<const bf16x8*>(&At[row * (HKP / 2) + 8 * kk + 4 * (lane >> 5)]);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int col = 64 * wc + 32 * b + (lane & 31);
        bfr[b] = *reinterpret_cast<const bf16x8*>(&Bsrc[col * (HKP / 2) + 8 * kk + 4 * (lane >> 5)]);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
  }

  // D layout of the 32x32 MFMA: lane l, register q -> row 8*(q/4) + 4*(l/32) + q%4, col l%32
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int ii = 64 * wr + 32 * a + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        const int jj = 64 * wc + 32 * b + (lane & 31);
        if (part) {
          part[((p * ntiles + L) * HT + ii) * HT + jj] = acc[a][b][q];
        } else {
          const int64_t gi = i0 + ii, gj = j0 + jj;
          if (gi < n && gj <= gi) S[gi * lds + gj] += acc[a][b][q];
        }
      }
}

// S[lower] += sum over splits of the partial tiles, splits in order.
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ part,
                                                              int64_t P, int64_t ntiles,
                                                              int64_t n, float* __restrict__ S,
                                                              int64_t lds) {
  const int64_t L = blockIdx.x;
  int64_t ti, tj;
  tile_coords(L, ti, tj);
  for (int e = threadIdx.x; e < HT * HT; e += blockDim.x) {
    const int ii = e / HT, jj = e % HT;
    const int64_t gi = ti * HT + ii, gj = tj * HT + jj;
    if (gi >= n || gj > gi) continue;
    float s = 0.0f;
    for (int64_t p = 0; p < P; ++p) s += part[(p * ntiles + L) * HT * HT + e];
    S[gi * lds + gj] += s;
  }
}

// fp32 activations: SIMT SYRK, 64x64 lower tiles, 256 threads x 4x4 outputs.
constexpr int FT = 64, FK = 16;
__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ X, int64_t ldx,
                                                       int64_t tokens, int64_t n,
                                                       float* __restrict__ S, int64_t lds) {
  __shared__ float As[FK][FT + 1];
  __shared__ float Bs[FK][FT + 1];
  int64_t ti, tj;
  tile_coords(blockIdx.x, ti, tj);
  const int64_t i0 = ti * FT, j0 = tj * FT;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int64_t t0 = 0; t0 < tokens; t0 += FK) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < FK * FT; idx += 256) {
      const int kk = idx / FT, cc = idx % FT;
      const int64_t t = t0 + kk;
      As[kk][cc] = (t < tokens && i0 + cc < n) ? X[t * ldx + i0 + cc] : 0.0f;
      Bs[kk][cc] = (t < tokens && j0 + cc < n) ? X[t * ldx + j0 + cc] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = As[kk][ty + 16 * u];
        b[u] = Bs[kk][tx + 16 * u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t gi = i0 + ty + 16 * u, gj = j0 + tx + 16 * v;
      if (gi < n && gj <= gi) S[gi * lds + gj] += acc[u][v];
    }
}

struct HessPlan {
  int64_t ntiles, P, tok_per_split;
  size_t ws;
};

HessPlan plan_bf16(int64_t n, int64_t tokens) {
  HessPlan pl;
  const int64_t T = ceil_div(n, HT);
  pl.ntiles = T * (T + 1) / 2;
  // aim for >= ~2048 workgroups; each split keeps at least 2048 tokens
  int64_t P = ceil_div(2048, pl.ntiles);
  P = hmax(1, hmin(P, tokens / 2048));
  pl.tok_per_split = ceil_div(ceil_div(tokens, P), HK) * HK;
  P = hmax(1, ceil_div(tokens, pl.tok_per_split));
  pl.P = P;
  pl.ws = P > 1 ? (size_t)P * pl.ntiles * HT * HT * sizeof(float) : 0;
  return pl;
}

}  // namespace

size_t hessian_ws_bytes(int64_t n, int64_t tokens, int dt) {
  if (dt != GPTQ_BF16 || tokens <= 0 || n <= 0) return 0;
  return plan_bf16(n, tokens).ws;
}

hipError_t launch_hessian(float* S, int64_t n, int64_t lds, const void* X, int dt, int64_t tokens,
                          int64_t ldx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (tokens <= 0 || n <= 0) return hipSuccess;
  if (dt == GPTQ_F32) {
    const int64_t T = ceil_div(n, FT);
    hipLaunchKernelGGL(syrk_f32_kernel, dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0, stream,
                       reinterpret_cast<const float*>(X), ldx, tokens, n, S, lds);
    return hipGetLastError();
  }
  const HessPlan pl = plan_bf16(n, tokens);
  if (ws_bytes < pl.ws) return hipErrorInvalidValue;
  float* part = pl.P > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)pl.ntiles, (unsigned)pl.P), dim3(256), 0,
                     stream, reinterpret_cast<const uint16_t*>(X), ldx, tokens, n,
                     pl.tok_per_split, S, lds, part, pl.ntiles);
  if (pl.P > 1) {
    hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)pl.ntiles), dim3(256), 0, stream,
                       part, pl.P, pl.ntiles, n, S, lds);
  }
  return hipGetLastError();
}

}  // namespace gptq
